"""Properties of the HIP path that hold at any size (GPU).

Chunking is sequence-local, every (sequence, head, V-block) is owned by one
workgroup, and the state is carried in fp32, so several of these hold bitwise.
"""
import numpy as np
import pytest

import workloads as W
from gpu_util import TOL, log, rel_err, run_gpu, run_oracle, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def fwd(t, **kw):
    import torch
    import gated_delta_rule_63_amd as kda
    o, hT = kda.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], cu_seqlens=t.get("cu"),
                    initial_state=t.get("h0"), **kw)
    torch.cuda.synchronize()
    return o, hT


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_run_to_run_bitwise(dtype):
    cfg = W.variant("varlen6_T8192_H96", T=2000, H=4, seq_lens=(700, 1, 299, 1000), name="det")
    t = to_device(W.make_inputs(cfg, 1, dtype=dtype), dtype)
    o1, h1 = fwd(t)
    o2, h2 = fwd(t)
    assert bool((o1 == o2).all()) and bool((h1 == h2).all())


def test_h0_hT_alias():
    import torch
    cfg = W.variant("T8192_H96", T=500, H=3, h0=True, gate="mild", name="alias")
    t = to_device(W.make_inputs(cfg, 2), "bf16")
    o_ref, h_ref = fwd(t)
    state = t["h0"].clone()
    t2 = dict(t, h0=state)
    o, h = fwd(t2, final_state=state)
    assert h.data_ptr() == state.data_ptr()
    assert bool((o == o_ref).all()) and bool((state == h_ref).all())


def test_varlen_equals_per_sequence_runs():
    import torch
    lens = (65, 0, 1, 32, 33, 300)
    cfg = W.variant("varlen6_T8192_H96", T=sum(lens), H=3, seq_lens=lens, name="split")
    inp = W.make_inputs(cfg, 3)
    t = to_device(inp, "bf16")
    o, h = fwd(t)
    for n, (_, a, b) in enumerate(inp.seq_bounds()):
        if a == b:
            assert bool((h[n] == t["h0"][n]).all())
            continue
        sub = {k: (v[:, a:b].contiguous() if k in ("q", "k", "v", "g", "beta") else v) for k, v in t.items()}
        sub["cu"] = None
        sub["h0"] = t["h0"][n:n + 1].contiguous()
        on, hn = fwd(sub)
        if b - a == 1:
            # a one-token call without cu_seqlens runs the fp32 decode kernel,
            # not the chunked kernel with its fp16/bf16 operands: the two agree
            # to the parity bars, not bitwise
            tol_o, tol_s = TOL["bf16"]
            assert rel_err(o[:, a:b].cpu().numpy(), on.cpu().numpy()) <= tol_o, f"sequence {n}"
            assert rel_err(h[n].cpu().numpy(), hn[0].cpu().numpy()) <= tol_s, f"sequence {n} state"
            continue
        assert bool((on == o[:, a:b]).all()), f"sequence {n}"
        assert bool((hn[0] == h[n]).all()), f"sequence {n} state"


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_handoff_at_chunk_boundary_is_bitwise(dtype):
    """Two halves with hT handed over as h0 equal one run when the split is a multiple of 32."""
    cfg = W.variant("T8192_H96", T=2048, H=3, h0=True, gate="mild", name="handoff")
    t = to_device(W.make_inputs(cfg, 4, dtype=dtype), dtype)
    o, h = fwd(t)
    m = 1024
    first = {k: (v[:, :m].contiguous() if k in ("q", "k", "v", "g", "beta") else v) for k, v in t.items()}
    second = {k: (v[:, m:].contiguous() if k in ("q", "k", "v", "g", "beta") else v) for k, v in t.items()}
    oa, ha = fwd(first)
    second["h0"] = ha
    ob, hb = fwd(second)
    assert bool((oa == o[:, :m]).all()) and bool((ob == o[:, m:]).all()) and bool((hb == h).all())


def test_many_short_sequences():
    rng = np.random.default_rng(5)
    lens = tuple(int(x) for x in rng.integers(1, 10, size=1000))
    cfg = W.variant("varlen6_T8192_H96", T=sum(lens), H=2, seq_lens=lens, name="1000 short sequences")
    inp = W.make_inputs(cfg, 5)
    o, h = run_gpu(inp)
    ro, rs = run_oracle(inp)
    eo, es = rel_err(o, ro), rel_err(h, rs)
    log(f"[inv] 1000 sequences: err_o {eo:.2e} err_hT {es:.2e}")
    assert eo <= TOL["bf16"][0] and es <= TOL["bf16"][1]


def test_linear_in_q():
    import torch
    cfg = W.variant("T8192_H96", T=700, H=2, h0=True, name="lin")
    t = to_device(W.make_inputs(cfg, 6), "bf16")
    o1, _ = fwd(t)
    t2 = dict(t, q=(t["q"].float() * 2.0).to(torch.bfloat16))   # exact in bf16
    o2, _ = fwd(t2)
    # exact up to operand rounding: fp16 subnormals have a fixed spacing, so
    # rounding 2x is not always twice the rounding of x
    assert rel_err(o2.cpu().numpy(), 2.0 * o1.cpu().numpy()) <= 1e-4


def test_split_over_workgroups_is_bitwise():
    """The number of workgroups a head is split over (1, 2, 4 or 8, chosen from
    the number of chains on a 256-CU chip) does not change any value: a 160-head
    run (one workgroup per head, sixteen waves) equals the same heads run as an
    80-head (two-way split), a 40-head (four-way) and a 20-head (eight-way)
    problem."""
    import torch
    cfg = W.variant("T8192_H96", T=300, H=160, h0=True, gate="mild", name="split-ways")
    t = to_device(W.make_inputs(cfg, 8), "bf16")
    o160, h160 = fwd(t)
    for H in (20, 40, 80):
        sub = {k: (v[:, :, :H].contiguous() if k in ("q", "k", "v", "g", "beta") else v) for k, v in t.items()}
        sub["h0"] = t["h0"][:, :H].contiguous()
        o, h = fwd(sub)
        log(f"[split] H={H}: max|o - o160| = {float((o - o160[:, :, :H]).abs().max()):.3g}")
        assert bool((o == o160[:, :, :H]).all()), f"H={H} output"
        assert bool((h == h160[:, :H]).all()), f"H={H} state"
