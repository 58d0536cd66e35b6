"""Gated DeltaNet (one scalar gate per (token, head)) on the GPU: kda_gdn_fwd
against the fp64 oracle gdn_ref_fwd, and bitwise against kda_fwd with the gate
repeated over the 128 channels."""
import numpy as np
import pytest

import workloads as W
from gpu_util import TOL, log, rel_err, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def gdn_gpu(t, gs, heads=None):
    import torch
    import gated_delta_rule_63_amd as kda
    o, hT = kda.gdn_fwd(t["q"], t["k"], t["v"], gs, t["beta"], cu_seqlens=t["cu"], initial_state=t["h0"])
    torch.cuda.synchronize()
    return o, hT


def gdn_oracle(inp, heads=None):
    import oracle
    q, k, v, gs, beta, h0 = inp.q, inp.k, inp.v, inp.g_scalar(), inp.beta, inp.h0
    if heads is not None:
        sl = lambda x: np.ascontiguousarray(x[:, :, heads])
        q, k, v, gs, beta = sl(q), sl(k), sl(v), sl(gs), sl(beta)
        h0 = None if h0 is None else np.ascontiguousarray(h0[:, heads])
    return oracle.gdn_ref_fwd(q, k, v, gs, beta, cu_seqlens=inp.cu_seqlens, h0=h0)


def check(inp, dtype, what, heads=None):
    import torch
    t = to_device(inp, dtype)
    gs = torch.from_numpy(inp.g_scalar()).to(t["q"].device)
    o, hT = gdn_gpu(t, gs)
    o, hT = o.cpu().numpy(), hT.cpu().numpy()
    ro, rs = gdn_oracle(inp, heads)
    if heads is not None:
        o, hT = o[:, :, heads], hT[:, heads]
    eo, es = rel_err(o, ro), rel_err(hT, rs)
    tol_o, tol_s = TOL[dtype]
    log(f"[gdn] {what} dtype={dtype} err_o={eo:.3e} (tol {tol_o:.0e}) err_hT={es:.3e} (tol {tol_s:.0e})")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(hT))
    assert eo <= tol_o and es <= tol_s


CASES = [
    ("fixed T=1000 (ragged)", dict(T=1000, H=3)),
    ("batch 2 T=333", dict(B=2, T=333, H=2)),
    ("mild gate with h0", dict(T=700, H=2, h0=True, gate="scalar_mild")),
    ("varlen edge lengths", dict(T=130, H=2, seq_lens=(1, 32, 0, 33, 64), h0=True)),
    ("single token", dict(T=1, H=4, h0=True)),
]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("what,kw", CASES, ids=[c[0] for c in CASES])
def test_gdn_matches_oracle(what, kw, dtype):
    kw = dict(kw)
    kw.setdefault("gate", "scalar")
    cfg = W.variant("T8192_H96", name="gdn " + what, **kw)
    check(W.make_inputs(cfg, 5, dtype=dtype), dtype, what)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_gdn_equals_kda_with_repeated_gate(dtype):
    """The scalar-gate kernels read one gate per (token, head) and otherwise run
    the KDA arithmetic unchanged: bitwise equal to kda_fwd with the gate repeated."""
    import torch
    import gated_delta_rule_63_amd as kda
    cfg = W.variant("varlen6_T8192_H96", T=400, H=3, seq_lens=(100, 37, 0, 263), gate="scalar_mild", name="gdn=kda")
    inp = W.make_inputs(cfg, 6, dtype=dtype)
    t = to_device(inp, dtype)
    gs = torch.from_numpy(inp.g_scalar()).to(t["q"].device)
    o1, h1 = gdn_gpu(t, gs)
    o2, h2 = kda.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], cu_seqlens=t["cu"], initial_state=t["h0"])
    torch.cuda.synchronize()
    assert bool((o1 == o2).all()) and bool((h1 == h2).all())


def test_gdn_headline_shape_all_heads():
    """T = 8192, H = 96 with a scalar gate, every head compared with the oracle."""
    cfg = W.variant("T8192_H96", gate="scalar", name="gdn T8192_H96")
    check(W.make_inputs(cfg, 0), "bf16", "T=8192 H=96, all heads")


def test_gdn_rejects_channel_gate_shape():
    import torch
    import gated_delta_rule_63_amd as kda
    cfg = W.variant("T8192_H96", T=40, H=2, name="gdn shape")
    t = to_device(W.make_inputs(cfg, 1), "bf16")
    with pytest.raises(ValueError):
        kda.gdn_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"])
