"""kda_fwd_noalloc (the entry point for callers that cannot allocate) against
kda_fwd and the fp64 oracle, through the C ABI: two calls in a row on the
three-slice route (which uses the static workspace; the one-pass slice route's
workspace does not fit there), the second with a smaller input, then one on
the one-pass slice route (small enough to fit), then a shape that needs no
workspace. The slice routes write every workspace value before reading it, so
a call cannot see an earlier call's leftovers. On the CPU: a descriptor whose
smallest slice workspace exceeds the static array is refused before anything
is enqueued."""
import ctypes

import numpy as np
import pytest

import workloads as W


def test_noalloc_rejects_oversized_workspace():
    import gated_delta_rule_63_amd as kda
    L = kda.lib()
    mx = L.kda_fwd_noalloc_max_workspace()
    assert mx == 8 << 20
    P = ctypes.c_void_p(0x1000)
    # 40 chains on the slice routes: the one-pass route (what kda_fwd_workspace_size
    # reports; three slices here) takes 3 states per chain and later slice and
    # ell for slices 1 and 2, the three-slice route 4 states per chain
    # (10 MiB): both exceed the 8 MiB array
    d = kda.Desc(1, 12288, 40, 128, 128, 1, 0, 1, None, 0)
    assert L.kda_fwd_workspace_size(ctypes.byref(d)) == 40 * 3 * 2 * 128 * 128 * 4 + 8192 * 40 * 128 * 4
    assert 40 * 4 * 128 * 128 * 4 > mx
    assert L.kda_fwd_noalloc(P, P, P, P, P, None, None, P, P, ctypes.byref(d), None) == -5
    # variable-length batches never take the slice route: the same descriptor
    # with cu_seqlens is not refused for its size (a null q makes kda_fwd stop
    # with KDA_ERR_NULL before any launch)
    cu = ctypes.c_void_p(0x2000)
    assert L.kda_fwd_noalloc(None, P, P, P, P, cu, None, P, P, ctypes.byref(d), None) == -1
    d = kda.Desc(1, 64, 2, 64, 128, 1, 0, 1, None, 0)       # argument errors as kda_fwd
    assert L.kda_fwd_noalloc(P, P, P, P, P, None, None, P, P, ctypes.byref(d), None) == -3
    assert L.kda_fwd_noalloc(P, P, P, P, P, None, None, P, P, None, None) == -1


@pytest.mark.gpu
def test_noalloc_matches_kda_fwd():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_63_amd as kda
    from gpu_util import TOL, log, rel_err, run_oracle, to_device
    # (shape, route kda_fwd_noalloc takes): three-slice when the one-pass
    # route's workspace exceeds the static array, one-pass when it fits
    cases = [
        (W.variant("T131072_H32", T=12320, H=4, gate="mild", h0=True, name="sliced T=12320 H=4"), "three"),
        (W.variant("T131072_H32", T=12288, H=3, gate="zero", h0=True, name="sliced T=12288 H=3 (smaller)"), "three"),
        (W.variant("T131072_H32", T=12288, H=1, gate="mild", h0=True, name="sliced T=12288 H=1"), "one_pass"),
        (W.variant("T8192_H96", T=1000, H=3, h0=True, name="one launch T=1000 H=3"), None),
    ]
    for i, (cfg, route) in enumerate(cases):
        inp = W.make_inputs(cfg, 30 + i)
        t = to_device(inp, "bf16")
        need = kda.fwd_workspace_size(t["q"])   # the one-pass route's
        assert (need > 0) == (route is not None)
        assert (need > kda.noalloc_max_workspace()) == (route == "three")
        o = torch.empty((1, cfg.T, cfg.H, 128), dtype=torch.float32, device=t["q"].device)
        h = torch.empty((1, cfg.H, 128, 128), dtype=torch.float32, device=t["q"].device)
        o.fill_(float("nan"))
        h.fill_(float("nan"))
        kda.fwd_noalloc(t["q"], t["k"], t["v"], t["g"], t["beta"], initial_state=t["h0"], out=o, final_state=h)
        # kda_fwd on the same route: a workspace of `need` bytes selects the one-pass route
        ws = torch.empty(need, dtype=torch.uint8, device=t["q"].device) if route == "one_pass" else None
        o_ref, h_ref = kda.fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], initial_state=t["h0"], workspace=ws)
        torch.cuda.synchronize()
        same = torch.equal(o, o_ref) and torch.equal(h, h_ref)
        ro, rs = run_oracle(inp)
        eo, es = rel_err(o.cpu().numpy(), ro), rel_err(h.cpu().numpy(), rs)
        log(f"[noalloc] {cfg.name} ({route} slices): one-pass workspace {need} B, bitwise equal to kda_fwd: {same}, "
            f"err_o {eo:.2e} err_hT {es:.2e}")
        assert same
        assert eo <= TOL["bf16"][0] and es <= TOL["bf16"][1]
