"""Intra-GPU segment scan (few long chains): kda_fwd cuts each chain into slices
when the chains are few and long (bf16, fixed length, T >= 12288 and at most
one sixth as many chains as compute units). A slice's state map is affine,
S_end = Pmap S_start + R, and so are its outputs. With a workspace of
fwd_workspace_size bytes kda_fwd takes the one-pass route (every slice in one
launch, one workgroup per run, then the output corrections S_j^T ell); without
one, the three-slice route (two passes).
These tests run both routes against the fp64 oracle."""
import numpy as np
import pytest

import workloads as W
from gpu_util import TOL, log, rel_err, run_oracle, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


ROUTES = ["one_pass", "three"]


def fwd(t, route, final_state=None, gdn=None):
    import torch
    import gated_delta_rule_63_amd as kda
    ws = None
    if route == "one_pass":
        n = kda.fwd_workspace_size(t["q"])
        assert n > 0
        ws = torch.empty(n, dtype=torch.uint8, device=t["q"].device)
    f = kda.gdn_fwd if gdn is not None else kda.fwd
    o, hT = f(t["q"], t["k"], t["v"], gdn if gdn is not None else t["g"], t["beta"], cu_seqlens=t["cu"],
              initial_state=t["h0"], final_state=final_state, workspace=ws)
    torch.cuda.synchronize()
    return o, hT


# g = 0 keeps the whole history in the state (only the delta correction forgets),
# so the slices' start states matter everywhere; "mild" spans about 120 tokens.
@pytest.mark.parametrize("route", ROUTES)
@pytest.mark.parametrize("gate,h0", [("zero", True), ("mild", True), ("bj", False)])
def test_sliced_chain_matches_oracle(gate, h0, route):
    cfg = W.variant("T131072_H32", T=12320, H=4, gate=gate, h0=h0, name=f"slices {gate}")
    inp = W.make_inputs(cfg, 11)
    t = to_device(inp, "bf16")
    o, hT = fwd(t, route)
    ro, rs = run_oracle(inp)
    eo, es = rel_err(o.cpu().numpy(), ro), rel_err(hT.cpu().numpy(), rs)
    tol_o, tol_s = TOL["bf16"]
    log(f"[slices] {route} T=12320 H=4 gate={gate} h0={h0}: err_o {eo:.2e} err_hT {es:.2e}")
    assert eo <= tol_o and es <= tol_s


@pytest.mark.parametrize("route", ROUTES)
def test_sliced_batch_with_ragged_tail(route):
    """Two batch rows (six chains) whose length is not a whole number of chunks:
    the slices' chain index covers the batch row, and the last slice ends in a
    partial chunk."""
    cfg = W.variant("T131072_H32", B=2, T=12301, H=3, gate="mild", h0=True, name="slices B=2 ragged")
    inp = W.make_inputs(cfg, 13)
    t = to_device(inp, "bf16")
    o, hT = fwd(t, route)
    ro, rs = run_oracle(inp)
    eo, es = rel_err(o.cpu().numpy(), ro), rel_err(hT.cpu().numpy(), rs)
    tol_o, tol_s = TOL["bf16"]
    log(f"[slices] {route} B=2 T=12301 H=3: err_o {eo:.2e} err_hT {es:.2e}")
    assert eo <= tol_o and es <= tol_s


@pytest.mark.parametrize("route", ROUTES)
def test_sliced_chain_state_alias(route):
    """h0 == hT (in place) through the sliced paths: the first pass reads h0 before
    the last step writes hT."""
    import torch
    cfg = W.variant("T131072_H32", T=12288, H=2, gate="zero", h0=True, name="slices alias")
    inp = W.make_inputs(cfg, 12)
    t = to_device(inp, "bf16")
    o_ref, h_ref = fwd(t, route)
    state = t["h0"].clone()
    o, h = fwd(dict(t, h0=state), route, final_state=state)
    assert h.data_ptr() == state.data_ptr()
    assert bool((o == o_ref).all()) and bool((state == h_ref).all())


@pytest.mark.parametrize("route", ROUTES)
def test_sliced_chain_scalar_gate(route):
    import torch
    import oracle
    cfg = W.variant("T131072_H32", T=12288, H=3, gate="scalar_mild", h0=True, name="slices gdn")
    inp = W.make_inputs(cfg, 13)
    t = to_device(inp, "bf16")
    gs = torch.from_numpy(inp.g_scalar()).to(t["q"].device)
    o, hT = fwd(t, route, gdn=gs)
    ro, rs = oracle.gdn_ref_fwd(inp.q, inp.k, inp.v, inp.g_scalar(), inp.beta, h0=inp.h0)
    eo, es = rel_err(o.cpu().numpy(), ro), rel_err(hT.cpu().numpy(), rs)
    log(f"[slices] {route} gdn T=12288 H=3: err_o {eo:.2e} err_hT {es:.2e}")
    tol_o, tol_s = TOL["bf16"]
    assert eo <= tol_o and es <= tol_s


def test_one_pass_route_without_final_state():
    """The one-pass slice route with no final state requested: the last combine
    is skipped, the other combines and the output corrections still run."""
    import torch
    import gated_delta_rule_63_amd as kda
    cfg = W.variant("T131072_H32", T=12352, H=2, gate="mild", h0=True, name="one pass, no hT")
    inp = W.make_inputs(cfg, 14)
    t = to_device(inp, "bf16")
    ws = torch.empty(kda.fwd_workspace_size(t["q"]), dtype=torch.uint8, device=t["q"].device)
    o, hT = kda.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], initial_state=t["h0"],
                    output_final_state=False, workspace=ws)
    torch.cuda.synchronize()
    assert hT is None
    ro, _ = run_oracle(inp)
    eo = rel_err(o.cpu().numpy(), ro)
    log(f"[slices] one pass, no hT, T=12352 H=2: err_o {eo:.2e}")
    assert eo <= TOL["bf16"][0]
