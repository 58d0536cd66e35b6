"""Helpers for the GPU tests: move seeded inputs to the device, run the HIP path
through its C ABI, and compare with the oracle."""
from __future__ import annotations

import sys
import time

import numpy as np

import workloads as W

TOL = {"bf16": (2e-2, 1e-2), "fp32": (1e-4, 1e-4)}   # (o, hT) as max|err| / RMS(oracle)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_device(inp: W.Inputs, dtype: str):
    import torch
    dev = torch.device("cuda:0")
    if dtype == "bf16":
        cvt = lambda x: torch.from_numpy(W.bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        cvt = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev)
    t = dict(q=cvt(inp.q), k=cvt(inp.k), v=cvt(inp.v),
             g=torch.from_numpy(inp.g).to(dev), beta=torch.from_numpy(inp.beta).to(dev))
    t["cu"] = torch.from_numpy(inp.cu_seqlens).to(dev) if inp.cu_seqlens is not None else None
    t["h0"] = torch.from_numpy(inp.h0).to(dev) if inp.h0 is not None else None
    return t


def run_gpu(inp: W.Inputs, dtype: str = None, t=None, **kw):
    """Returns (o, hT) as numpy fp32 arrays."""
    import torch
    import gated_delta_rule_63_amd as kda
    dtype = dtype or inp.cfg.dtype
    t = t or to_device(inp, dtype)
    o, hT = kda.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], cu_seqlens=t["cu"],
                    initial_state=t["h0"], **kw)
    torch.cuda.synchronize()
    return o.cpu().numpy(), (hT.cpu().numpy() if hT is not None else None)


def run_oracle(inp: W.Inputs, heads=None):
    import oracle
    q, k, v, g, beta, h0 = inp.q, inp.k, inp.v, inp.g, inp.beta, inp.h0
    if heads is not None:
        sl = lambda x: np.ascontiguousarray(x[:, :, heads])
        q, k, v, g, beta = sl(q), sl(k), sl(v), sl(g), sl(beta)
        h0 = None if h0 is None else np.ascontiguousarray(h0[:, heads])
    return oracle.kda_ref_fwd(q, k, v, g, beta, cu_seqlens=inp.cu_seqlens, h0=h0)


def rel_err(got, ref):
    ref = np.asarray(ref, np.float64)
    r = W.rms(ref)
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref))) / max(r, 1e-300)


def check(inp: W.Inputs, dtype: str = None, heads=None, tol=None, what=""):
    dtype = dtype or inp.cfg.dtype
    tol_o, tol_s = tol or TOL[dtype]
    t0 = time.time()
    o, hT = run_gpu(inp, dtype)
    t1 = time.time()
    ro, rs = run_oracle(inp, heads)
    t2 = time.time()
    if heads is not None:
        o, hT = o[:, :, heads], hT[:, heads]
    eo, es = rel_err(o, ro), rel_err(hT, rs)
    log(f"[parity] {what or inp.cfg.name} dtype={dtype} err_o={eo:.3e} (tol {tol_o:.0e}) "
        f"err_hT={es:.3e} (tol {tol_s:.0e}) gpu={t1 - t0:.1f}s oracle={t2 - t1:.1f}s")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(hT))
    assert eo <= tol_o, f"o: {eo:.3e} > {tol_o:.0e}"
    assert es <= tol_s, f"hT: {es:.3e} > {tol_s:.0e}"
    return eo, es
