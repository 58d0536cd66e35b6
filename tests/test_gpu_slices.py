"""Intra-GPU segment scan (few long chains): kda_fwd cuts each chain into three
slices when the chains are few and long (bf16, fixed length, T >= 12288 and at
most one sixth as many chains as compute units). The middle slice's affine map
S_end = Pmap S_start + R is formed on the GPU; these tests run such shapes
against the fp64 oracle."""
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


def fwd(t, final_state=None, gdn=None):
    import torch
    import gated_delta_rule_63_amd as kda
    f = kda.gdn_fwd if gdn is not None else kda.fwd
    o, hT = f(t["q"], t["k"], t["v"], gdn if gdn is not None else t["g"], t["beta"], cu_seqlens=t["cu"],
              initial_state=t["h0"], final_state=final_state)
    torch.cuda.synchronize()
    return o, hT


# g = 0 keeps the whole history in the state (only the delta correction forgets),
# so the slices' start states matter everywhere; "mild" spans about 120 tokens.
@pytest.mark.parametrize("gate,h0", [("zero", True), ("mild", True), ("bj", False)])
def test_sliced_chain_matches_oracle(gate, h0):
    cfg = W.variant("T131072_H32", T=12320, H=4, gate=gate, h0=h0, name=f"slices {gate}")
    inp = W.make_inputs(cfg, 11)
    t = to_device(inp, "bf16")
    o, hT = fwd(t)
    ro, rs = run_oracle(inp)
    eo, es = rel_err(o.cpu().numpy(), ro), rel_err(hT.cpu().numpy(), rs)
    tol_o, tol_s = TOL["bf16"]
    log(f"[slices] T=12320 H=4 gate={gate} h0={h0}: err_o {eo:.2e} err_hT {es:.2e}")
    assert eo <= tol_o and es <= tol_s


def test_sliced_batch_with_ragged_tail():
    """Two batch rows (six chains) whose length is not a whole number of chunks:
    the slices' chain index covers the batch row, and the last slice ends in a
    partial chunk."""
    cfg = W.variant("T131072_H32", B=2, T=12301, H=3, gate="mild", h0=True, name="slices B=2 ragged")
    inp = W.make_inputs(cfg, 13)
    t = to_device(inp, "bf16")
    o, hT = fwd(t)
    ro, rs = run_oracle(inp)
    eo, es = rel_err(o.cpu().numpy(), ro), rel_err(hT.cpu().numpy(), rs)
    tol_o, tol_s = TOL["bf16"]
    log(f"[slices] B=2 T=12301 H=3: err_o {eo:.2e} err_hT {es:.2e}")
    assert eo <= tol_o and es <= tol_s


def test_sliced_chain_state_alias():
    """h0 == hT (in place) through the sliced path: the first pass reads h0 before
    the last one writes hT."""
    import torch
    cfg = W.variant("T131072_H32", T=12288, H=2, gate="zero", h0=True, name="slices alias")
    inp = W.make_inputs(cfg, 12)
    t = to_device(inp, "bf16")
    o_ref, h_ref = fwd(t)
    state = t["h0"].clone()
    o, h = fwd(dict(t, h0=state), final_state=state)
    assert h.data_ptr() == state.data_ptr()
    assert bool((o == o_ref).all()) and bool((state == h_ref).all())


def test_sliced_chain_scalar_gate():
    import torch
    import oracle
    cfg = W.variant("T131072_H32", T=12288, H=3, gate="scalar_mild", h0=True, name="slices gdn")
    inp = W.make_inputs(cfg, 13)
    t = to_device(inp, "bf16")
    gs = torch.from_numpy(inp.g_scalar()).to(t["q"].device)
    o, hT = fwd(t, gdn=gs)
    ro, rs = oracle.gdn_ref_fwd(inp.q, inp.k, inp.v, inp.g_scalar(), inp.beta, h0=inp.h0)
    eo, es = rel_err(o.cpu().numpy(), ro), rel_err(hT.cpu().numpy(), rs)
    log(f"[slices] gdn T=12288 H=3: err_o {eo:.2e} err_hT {es:.2e}")
    tol_o, tol_s = TOL["bf16"]
    assert eo <= tol_o and es <= tol_s
