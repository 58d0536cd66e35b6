"""Decode step (one token per sequence) against the fp64 oracle (GPU).

kda_decode_step runs one recurrence step per (sequence, head) in fp32, so it
is held to 1e-5 x RMS against the oracle on the same (bf16-rounded) inputs,
tighter than the prefill bars. A prefill followed by decode steps is held to
the prefill bars, since it carries the prefill's state.
"""
import ctypes

import numpy as np
import pytest

import workloads as W
from gpu_util import TOL, log, rel_err, run_oracle, to_device

pytestmark = pytest.mark.gpu
DEC_TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def step_inputs(N, H, seed, dtype="bf16", h0=True):
    cfg = W.variant("T8192_H96", B=N, T=1, H=H, h0=h0, name=f"decode N={N} H={H}")
    if dtype == "fp32":
        cfg = W.variant(cfg, dtype="fp32")
    return W.make_inputs(cfg, seed, dtype=dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("N,H,h0", [(1, 1, True), (16, 4, True), (7, 3, False), (64, 96, True)])
def test_decode_step_matches_oracle(dtype, N, H, h0):
    import torch
    import gated_delta_rule_63_amd as kda
    inp = step_inputs(N, H, 3, dtype, h0)
    t = to_device(inp, dtype)
    o, S = kda.decode_step(t["q"], t["k"], t["v"], t["g"], t["beta"], state=t["h0"])
    torch.cuda.synchronize()
    ro, rs = run_oracle(inp)
    eo, es = rel_err(o.cpu().numpy(), ro), rel_err(S.cpu().numpy(), rs)
    log(f"[decode] N={N} H={H} h0={h0} {dtype}: err_o {eo:.2e} err_state {es:.2e}")
    assert eo <= DEC_TOL and es <= DEC_TOL


def test_decode_in_place_equals_out_of_place():
    import torch
    import gated_delta_rule_63_amd as kda
    inp = step_inputs(8, 5, 4)
    t = to_device(inp, "bf16")
    o1, S1 = kda.decode_step(t["q"], t["k"], t["v"], t["g"], t["beta"], state=t["h0"])
    state = t["h0"].clone()
    o2, S2 = kda.decode_step(t["q"], t["k"], t["v"], t["g"], t["beta"], state=state, in_place=True)
    torch.cuda.synchronize()
    assert S2.data_ptr() == state.data_ptr()
    assert bool((o1 == o2).all()) and bool((S1 == S2).all())


def test_fwd_with_one_token_uses_the_same_step():
    """kda_fwd with T = 1 and no cu_seqlens runs the decode kernel: bitwise equal."""
    import torch
    import gated_delta_rule_63_amd as kda
    inp = step_inputs(6, 4, 5)
    t = to_device(inp, "bf16")
    o1, S1 = kda.decode_step(t["q"], t["k"], t["v"], t["g"], t["beta"], state=t["h0"])
    o2, S2 = kda.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], initial_state=t["h0"])
    torch.cuda.synchronize()
    assert bool((o1 == o2).all()) and bool((S1 == S2).all())


def test_prefill_then_decode_steps():
    """Prefill 300 tokens, then decode 8 more one at a time with the state updated
    in place; o of the decoded tokens and the final state match the oracle run
    over all 308 tokens."""
    import torch
    import gated_delta_rule_63_amd as kda
    P, S_ = 300, 8
    cfg = W.variant("T8192_H96", B=3, T=P + S_, H=4, h0=True, name="prefill+decode")
    inp = W.make_inputs(cfg, 6)
    t = to_device(inp, "bf16")
    pre = {k: (v[:, :P].contiguous() if k in ("q", "k", "v", "g", "beta") else v) for k, v in t.items()}
    _, state = kda.fwd(pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], initial_state=pre["h0"])
    outs = []
    for s in range(P, P + S_):
        sl = {k: t[k][:, s:s + 1].contiguous() for k in ("q", "k", "v", "g", "beta")}
        o, _ = kda.decode_step(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], state=state, in_place=True)
        outs.append(o)
    torch.cuda.synchronize()
    o_dec = torch.cat(outs, dim=1).cpu().numpy()
    ro, rs = run_oracle(inp)
    eo = rel_err(o_dec, ro[:, P:])
    es = rel_err(state.cpu().numpy(), rs)
    log(f"[decode] prefill {P} + {S_} decode steps: err_o {eo:.2e} err_state {es:.2e}")
    tol_o, tol_s = TOL["bf16"]
    assert eo <= tol_o and es <= tol_s


def test_decode_rejects_before_launch():
    import torch
    import gated_delta_rule_63_amd as kda
    from gated_delta_rule_63_amd._lib import lib, Desc, KDA_BF16, KDA_F32
    inp = step_inputs(2, 2, 7)
    t = to_device(inp, "bf16")
    with pytest.raises(ValueError):
        kda.decode_step(t["q"].repeat(1, 2, 1, 1), t["k"].repeat(1, 2, 1, 1), t["v"].repeat(1, 2, 1, 1),
                        t["g"].repeat(1, 2, 1, 1), t["beta"].repeat(1, 2, 1))
    P = ctypes.c_void_p
    d = Desc(2, 1, 2, 128, 128, 2, KDA_BF16, KDA_F32, None, 0)
    o = torch.empty((2, 1, 2, 128), device="cuda")
    ptrs = [P(x.data_ptr()) for x in (t["q"], t["k"], t["v"], t["g"], t["beta"])]
    mis = P(t["h0"].data_ptr() + 4)   # misaligned state
    assert lib().kda_decode_step(*ptrs, mis, P(o.data_ptr()), None, ctypes.byref(d), None) == -3
