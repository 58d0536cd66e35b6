"""Stage-by-stage parity of the staged path (a0 chunk map, a1 gate scan,
a2 intra-chunk, a3 recurrence, a4 output) with the fp64 chunk algebra of the
oracle (oracle/chunk_ref.py, 32-token chunks), and of kda_fwd_staged with the
fp64 recurrence.

The stage kernels compute in fp32, so their intermediates are held to
1e-4 x RMS of the reference quantity; the end-to-end bar is the product's.
"""
import numpy as np
import pytest

import workloads as W
from gpu_util import TOL, log, rel_err, run_oracle, to_device
from oracle.chunk_ref import chunk_fwd

pytestmark = pytest.mark.gpu
C = 32
STAGE_TOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def expected_map(inp):
    rows = []
    for n, (b, t0, t1) in enumerate(inp.seq_bounds()):
        for c0 in range(t0, t1, C):
            rows.append((n, c0, min(C, t1 - c0), b))
    return rows


def close(got, ref, what, tol=STAGE_TOL):
    e = rel_err(got, ref)
    log(f"[stage] {what}: max|err|/rms = {e:.2e}")
    assert e <= tol, f"{what}: {e:.2e} > {tol:.0e}"


CASES = [
    W.variant("T8192_H96", T=1 + 31 + 32 + 33 + 0 + 70 + 5, H=3, seq_lens=(1, 31, 32, 33, 0, 70, 5), h0=True,
              gate="mild", name="varlen edge lengths, mild decay"),
    W.variant("T8192_H96", B=2, T=100, H=2, name="batch 2 ragged"),
    W.variant("tiny_fp32", T=96, name="fp32 inputs", h0=True),
]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_stages_against_chunk_algebra(cfg):
    import torch
    import gated_delta_rule_63_amd as kda
    inp = W.make_inputs(cfg, 11)
    t = to_device(inp, cfg.dtype)
    st = kda.Staged(t["q"], t["k"], t["v"], t["g"], t["beta"], cu_seqlens=t["cu"], initial_state=t["h0"])
    # a0: bit-exact chunk map
    st.chunk_map()
    torch.cuda.synchronize()
    want = expected_map(inp)
    got = st.map.cpu().numpy()
    assert [tuple(r) for r in got[:len(want)]] == want
    assert np.all(got[len(want):, 0] == -1) and np.all(got[len(want):, 2] == 0)
    first = np.cumsum([0] + [(t1 - t0 + C - 1) // C for (_, t0, t1) in inp.seq_bounds()])
    si = st.seqinfo.cpu().numpy()
    assert np.array_equal(si[:, 0], first[:-1]) and np.array_equal(si[:, 1], np.diff(first))

    st.gate_scan()
    st.intra()
    hT = torch.empty((cfg.N, cfg.H, 128, 128), device="cuda")
    st.recurrence(hT)
    o = torch.zeros((cfg.B, cfg.T, cfg.H, 128), device="cuda")
    st.output(o)
    torch.cuda.synchronize()

    _, hT_ref, stages = chunk_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta, cu_seqlens=inp.cu_seqlens,
                                  h0=inp.h0, C=C, keep=True)
    G, Wt, U, Kt, Qg, Dl = (x.cpu().numpy() for x in (st.Gamma, st.W, st.U, st.Kt, st.Qg, st.Delta))
    M, hc, gl = st.M.cpu().numpy(), st.hc.cpu().numpy(), st.gl.cpu().numpy()
    ref = {k: [] for k in ["Gamma", "W", "U", "Kt", "Qg", "Delta", "M", "S_in", "gamma_last"]}
    got = {k: [] for k in ref}
    for s, (n, c0, nv, b) in enumerate(want):
        for h in range(cfg.H):
            r = stages[(n, h)][(c0 - inp.seq_bounds()[n][1]) // C]
            assert r["t0"] == c0
            for key, arr in (("Gamma", G), ("W", Wt), ("U", U), ("Kt", Kt), ("Qg", Qg), ("Delta", Dl)):
                got[key].append(arr[b, c0:c0 + nv, h])
                ref[key].append(r[key])
            got["M"].append(M[s, h, :nv, :nv])
            ref["M"].append(r["M"])
            got["S_in"].append(hc[s, h])
            ref["S_in"].append(r["S_in"])
            got["gamma_last"].append(gl[s, h])
            ref["gamma_last"].append(r["gamma_last"])
    for key in ref:
        close(np.concatenate([x.ravel() for x in got[key]]), np.concatenate([x.ravel() for x in ref[key]]),
              f"{cfg.name} {key}")
    ro, rs = run_oracle(inp)
    close(o.cpu().numpy(), ro, f"{cfg.name} o", STAGE_TOL)
    close(hT.cpu().numpy(), rs, f"{cfg.name} hT", STAGE_TOL)
    close(hT.cpu().numpy(), hT_ref, f"{cfg.name} hT vs chunk algebra", STAGE_TOL)


@pytest.mark.parametrize("name", ["tiny_fp32", "T8192_H96", "varlen6_T8192_H96"])
def test_staged_end_to_end(name):
    import torch
    import gated_delta_rule_63_amd as kda
    cfg = W.CONFIGS[name]
    inp = W.make_inputs(cfg, 0)
    t = to_device(inp, cfg.dtype)
    o, hT, st = kda.fwd_staged(t["q"], t["k"], t["v"], t["g"], t["beta"], cu_seqlens=t["cu"],
                               initial_state=t["h0"])
    torch.cuda.synchronize()
    del st
    ro, rs = run_oracle(inp)
    eo, es = rel_err(o.cpu().numpy(), ro), rel_err(hT.cpu().numpy(), rs)
    log(f"[staged] {name}: err_o {eo:.2e} err_hT {es:.2e}")
    tol_o, tol_s = TOL[cfg.dtype]
    assert eo <= tol_o and es <= tol_s
