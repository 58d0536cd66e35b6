"""HIP graph capture of the library's launches (through torch.cuda.CUDAGraph):
the decode step, the fused prefill and the sliced prefill (with a caller
workspace, so nothing is allocated while capturing). Every replay is checked
bit for bit against the same calls made eagerly, with eager work between the
replays."""
import numpy as np
import pytest

import workloads as W
from gpu_util import log, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def capture(fn, n=1):
    import torch
    fn()                                   # warm: nothing lazily set up inside the capture
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for _ in range(n):
                fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return g


def test_decode_steps_in_a_graph():
    """Three in-place decode steps captured once; each replay advances the state
    by three more steps, exactly as three eager calls do."""
    import torch
    import gated_delta_rule_63_amd as kda
    cfg = W.variant("T8192_H96", B=4, T=1, H=8, h0=True, name="decode graph")
    t = to_device(W.make_inputs(cfg, 21), "bf16")
    s_graph = t["h0"].clone()
    o_graph = torch.empty((4, 1, 8, 128), dtype=torch.float32, device=s_graph.device)
    step = lambda: kda.decode_step(t["q"], t["k"], t["v"], t["g"], t["beta"], state=s_graph, out=o_graph, in_place=True)
    g = capture(step, n=3)                 # capture() ran one eager step first
    s_eager = t["h0"].clone()
    o_eager = torch.empty_like(o_graph)
    eager = lambda: kda.decode_step(t["q"], t["k"], t["v"], t["g"], t["beta"], state=s_eager, out=o_eager, in_place=True)
    eager()
    for rep in range(3):
        g.replay()
        for _ in range(3):
            eager()
        torch.cuda.synchronize()
        log(f"[graph] decode replay {rep}: max|ds| {float((s_graph - s_eager).abs().max()):.3e}")
        assert torch.equal(s_graph, s_eager) and torch.equal(o_graph, o_eager)


@pytest.mark.parametrize("what,kw,sliced", [
    ("fused T=1000 H=4", dict(T=1000, H=4, h0=True), False),
    ("sliced T=12320 H=4", dict(T=12320, H=4, h0=True), True),
])
def test_prefill_in_a_graph(what, kw, sliced):
    import torch
    import gated_delta_rule_63_amd as kda
    cfg = W.variant("T8192_H96", name=what, **kw)
    t = to_device(W.make_inputs(cfg, 22), "bf16")
    o = torch.empty((1, cfg.T, cfg.H, 128), dtype=torch.float32, device=t["q"].device)
    hT = torch.empty((1, cfg.H, 128, 128), dtype=torch.float32, device=t["q"].device)
    # kda_fwd's own workspace (the sliced path's states), so nothing is allocated while capturing
    nws = kda.fwd_workspace_size(t["q"])
    assert (nws > 0) == sliced
    ws = torch.empty(nws, dtype=torch.uint8, device=t["q"].device) if nws else None
    run = lambda oo, hh: kda.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], initial_state=t["h0"], out=oo,
                                 final_state=hh, workspace=ws)
    g = capture(lambda: run(o, hT))
    o_ref, h_ref = torch.empty_like(o), torch.empty_like(hT)
    run(o_ref, h_ref)
    for rep in range(3):
        o.zero_()
        hT.zero_()
        g.replay()
        torch.cuda.synchronize()
        log(f"[graph] {what} replay {rep}: equal o {torch.equal(o, o_ref)} hT {torch.equal(hT, h_ref)}")
        assert torch.equal(o, o_ref) and torch.equal(hT, h_ref)
