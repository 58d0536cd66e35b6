"""The long-context workload, T = 131072 and H = 32 with an initial state,
against the fp64 oracle on every head: as one call, and as two calls of 65536
tokens with the first call's final state handed over as the second's initial
state. Both the pages' gate draw and a mild gate (g x 0.01, memory of about
120 tokens) are run: with the pages' draw the state forgets within about 20
tokens, so only the mild gate makes h0, the handover and the slice routes'
affine combines (three slices: starting at tokens 43680 and 87360, or 21824
and 43680 within each half; one pass: four slices starting at tokens 32768,
65536 and 98304, or 16384, 32768 and 49152 within each half, their outputs
corrected by S_j^T ell) matter at full length."""
import numpy as np
import pytest

import workloads as W
from gpu_util import TOL, log, rel_err, run_oracle, to_device

pytestmark = pytest.mark.gpu

HALF = 65536


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


_cache = {}


def case(gate):
    """Inputs and the oracle's result for one gate draw, computed once per module."""
    if gate not in _cache:
        _cache.clear()      # one workload in host memory at a time
        cfg = W.variant("T131072_H32", gate=gate, name=f"T131072_H32 gate={gate}")
        log(f"[long] generating {cfg.name}")
        inp = W.make_inputs(cfg, 0)
        log(f"[long] oracle on all 32 heads")
        ro, rs = run_oracle(inp)
        _cache[gate] = (inp, ro, rs)
    return _cache[gate]


def fwd(t, route="three"):
    """route "three": no workspace (the three-slice route); "one_pass": a
    workspace of fwd_workspace_size bytes (every slice in one launch, then the
    combines and the output corrections)."""
    import torch
    import gated_delta_rule_63_amd as kda
    ws = None
    if route == "one_pass":
        ws = torch.empty(kda.fwd_workspace_size(t["q"]), dtype=torch.uint8, device=t["q"].device)
    o, hT = kda.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], initial_state=t["h0"], workspace=ws)
    torch.cuda.synchronize()
    return o, hT


def halves(t):
    first = {k: (v[:, :HALF].contiguous() if k in ("q", "k", "v", "g", "beta") else v) for k, v in t.items()}
    second = {k: (v[:, HALF:].contiguous() if k in ("q", "k", "v", "g", "beta") else v) for k, v in t.items()}
    return first, second


@pytest.mark.parametrize("route", ["one_pass", "three"])
@pytest.mark.parametrize("gate", ["bj", "mild"])
def test_long_context_all_heads(gate, route):
    inp, ro, rs = case(gate)
    t = to_device(inp, "bf16")
    o, hT = fwd(t, route)
    eo, es = rel_err(o.cpu().numpy(), ro), rel_err(hT.cpu().numpy(), rs)
    tol_o, tol_s = TOL["bf16"]
    log(f"[long] T=131072 H=32 gate={gate} {route} slices, all heads: err_o {eo:.3e} (tol {tol_o:.0e}) "
        f"err_hT {es:.3e} (tol {tol_s:.0e})")
    assert np.isfinite(eo) and np.isfinite(es)
    assert eo <= tol_o and es <= tol_s


@pytest.mark.parametrize("gate", ["bj", "mild"])
def test_long_context_handoff_all_heads(gate):
    """2 x 65536 with hT -> h0: each half's output and the final state against
    the oracle's single run. The halves take the three-slice route themselves,
    so their slice boundaries differ from the single call's and the two agree to
    rounding, not bit for bit."""
    inp, ro, rs = case(gate)
    t = to_device(inp, "bf16")
    first, second = halves(t)
    oa, ha = fwd(first)
    second["h0"] = ha
    ob, hb = fwd(second)
    # the handed-over state is the oracle's state after token 65536
    import oracle
    sl = lambda x: np.ascontiguousarray(x[:, :HALF])
    _, rmid = oracle.kda_ref_fwd(sl(inp.q), sl(inp.k), sl(inp.v), sl(inp.g), sl(inp.beta), h0=inp.h0)
    tol_o, tol_s = TOL["bf16"]
    rms_o = W.rms(ro)
    ea = float(np.max(np.abs(oa.cpu().numpy() - ro[:, :HALF]))) / rms_o
    eb = float(np.max(np.abs(ob.cpu().numpy() - ro[:, HALF:]))) / rms_o
    em = rel_err(ha.cpu().numpy(), rmid)
    es = rel_err(hb.cpu().numpy(), rs)
    log(f"[long] 2 x 65536 gate={gate}: err_o first {ea:.3e} second {eb:.3e} (tol {tol_o:.0e}), "
        f"handed-over state {em:.3e}, final state {es:.3e} (tol {tol_s:.0e})")
    assert ea <= tol_o and eb <= tol_o and em <= tol_s and es <= tol_s
