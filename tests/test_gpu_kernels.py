"""Each forward kernel by name (kda_fwd_kernel) against the fp64 oracle: the
pipelined 32-token kernel, the one-phase-at-a-time 32-token kernel and the
16-token-chunk kernel (the chunk-length ablation). Chunk boundaries differ
between them, so ragged lengths around 16 and 32 are covered."""
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


def run_kernel(inp, dtype, kernel):
    import torch
    import gated_delta_rule_63_amd as kda
    t = to_device(inp, dtype)
    o, hT = kda.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], cu_seqlens=t["cu"], initial_state=t["h0"],
                    kernel=kernel)
    torch.cuda.synchronize()
    return o.cpu().numpy(), hT.cpu().numpy()


def check(inp, dtype, kernel, what, heads=None):
    o, hT = run_kernel(inp, dtype, kernel)
    ro, rs = run_oracle(inp, heads)
    if heads is not None:
        o, hT = o[:, :, heads], hT[:, heads]
    eo, es = rel_err(o, ro), rel_err(hT, rs)
    tol_o, tol_s = TOL[dtype]
    log(f"[kernel {kernel}] {what} dtype={dtype} err_o={eo:.3e} (tol {tol_o:.0e}) err_hT={es:.3e} (tol {tol_s:.0e})")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(hT))
    assert eo <= tol_o and es <= tol_s


CASES = [
    ("fixed T=1000 (ragged)", dict(T=1000, H=3)),
    ("batch 2 T=333", dict(B=2, T=333, H=2)),
    ("mild decay with h0", dict(T=700, H=2, h0=True, gate="mild")),
    ("g = 0", dict(T=300, H=2, gate="zero")),
    ("one-hot keys", dict(T=300, H=2, keys="onehot", h0=True, gate="mild")),
    ("gate repeated over channels", dict(T=400, H=2, gate="scalar", h0=True)),
    ("varlen around 16 and 32", dict(T=1 + 15 + 16 + 17 + 0 + 31 + 32 + 33 + 100, H=3,
                                      seq_lens=(1, 15, 16, 17, 0, 31, 32, 33, 100), h0=True)),
    ("single token", dict(T=1, H=2, h0=True)),
]


@pytest.mark.parametrize("what,kw", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("kernel", ["pipe", "serial", "chunk16"])
def test_kernel_matches_oracle(kernel, what, kw):
    cfg = W.variant("T8192_H96", name=what, **kw)
    check(W.make_inputs(cfg, 11), "bf16", kernel, what)


def test_serial_fp32():
    cfg = W.variant("tiny_fp32", T=500, H=2, h0=True, gate="mild", name="serial fp32")
    check(W.make_inputs(cfg, 12, dtype="fp32"), "fp32", "serial", "fp32 T=500")


def test_chunk16_headline_shape_all_heads():
    """T = 8192, H = 96 through the 16-token kernel, every head compared with the oracle."""
    cfg = W.CONFIGS["T8192_H96"]
    check(W.make_inputs(cfg, 0), "bf16", "chunk16", "T=8192 H=96, all heads")


def test_fp32_rejected_by_bf16_kernels():
    import gated_delta_rule_63_amd as kda
    cfg = W.variant("tiny_fp32", T=40, H=2, name="fp32 reject")
    t = to_device(W.make_inputs(cfg, 1, dtype="fp32"), "fp32")
    for kernel in ("pipe", "chunk16", "two_pass"):
        with pytest.raises(kda.KDAError):
            kda.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], kernel=kernel)
    with pytest.raises(ValueError):
        kda.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], kernel="chunk64")


TWO_PASS_CASES = [
    ("fixed T=1000 (ragged)", dict(T=1000, H=3)),
    ("batch 2 T=333", dict(B=2, T=333, H=2, h0=True)),
    ("mild decay with h0", dict(T=700, H=2, h0=True, gate="mild")),
    ("17 chunks: one full preparation group and one of a single chunk", dict(T=530, H=2, h0=True)),
    ("single token", dict(T=1, H=2, h0=True)),
    ("T=8192 H=96", dict()),
]


@pytest.mark.parametrize("what,kw", TWO_PASS_CASES, ids=[c[0] for c in TWO_PASS_CASES])
def test_two_pass_equals_pipe_bitwise(what, kw):
    """The two-kernel form runs the pipelined kernel's arithmetic with the
    operands parked in device memory between the halves: identical o and hT."""
    import torch
    cfg = W.variant("T8192_H96", name=what, **kw)
    inp = W.make_inputs(cfg, 13)
    o1, h1 = run_kernel(inp, "bf16", "pipe")
    o2, h2 = run_kernel(inp, "bf16", "two_pass")
    log(f"[kernel two_pass] {what}: max|o - o_pipe| = {np.abs(o1 - o2).max():.3e}")
    np.testing.assert_array_equal(o2, o1)
    np.testing.assert_array_equal(h2, h1)
    if cfg.T <= 1000:
        ro, rs = run_oracle(inp)
        assert rel_err(o2, ro) <= TOL["bf16"][0] and rel_err(h2, rs) <= TOL["bf16"][1]


def test_two_pass_with_caller_workspace():
    """A large enough desc->workspace is used instead of an allocation; the result is the same."""
    import torch
    import gated_delta_rule_63_amd as kda
    cfg = W.variant("T8192_H96", T=600, H=3, h0=True, name="two_pass workspace")
    inp = W.make_inputs(cfg, 14)
    t = to_device(inp, "bf16")
    nbytes = kda.kernel_workspace_size(t["q"], "two_pass")
    assert nbytes == 3 * ((600 + 31) // 32) * 53248
    ws = torch.empty(nbytes, dtype=torch.uint8, device=t["q"].device)
    o1, h1 = kda.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], initial_state=t["h0"], kernel="two_pass", workspace=ws)
    o2, h2 = kda.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], initial_state=t["h0"], kernel="two_pass")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
