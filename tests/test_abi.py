"""The C ABI without a GPU: the library loads, exports every function that
include/kda.h declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


@pytest.fixture(scope="module")
def K():
    import gated_delta_rule_63_amd as kda
    return kda


def declared_functions():
    txt = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", txt)))


def test_exports_every_declared_function(K):
    names = declared_functions()
    assert len(names) >= 12, names
    lib = ctypes.CDLL(K._lib.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/kda.h but not exported"
    assert sorted(K._lib.EXPORTS) == names


def test_version_and_status_strings(K):
    assert K.version() == 100
    for code in [0, -1, -2, -3, -4, -5, -6]:
        assert K.status_string(code)
    assert "unknown" in K.status_string(-99)


def desc(K, B=1, T=64, H=2, Kd=128, V=128, N=None, in_dt=0, out_dt=1):
    return K.Desc(B, T, H, Kd, V, B if N is None else N, in_dt, out_dt, None, 0)


P = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails or succeeds before any launch


def check(K, d, cu=None, q=P, o=P):
    return K.lib().kda_fwd_check(q, P, P, P, P, cu, None, o, None, ctypes.byref(d))


def test_validation_codes(K):
    assert check(K, desc(K)) == 0
    assert K.lib().kda_fwd_check(P, P, P, P, P, None, None, P, None, None) == -1          # NULL desc
    assert check(K, desc(K, Kd=64)) == -3 and check(K, desc(K, V=256)) == -3              # K, V != 128
    assert check(K, desc(K, in_dt=7)) == -4 and check(K, desc(K, out_dt=9)) == -4
    assert check(K, desc(K, out_dt=0)) == -3                                              # bf16 o not built
    assert check(K, desc(K, B=0)) == -2 and check(K, desc(K, T=-1)) == -2
    assert check(K, desc(K, B=2, N=3)) == -2                                              # N != B without cu
    assert check(K, desc(K, B=2, N=3), cu=P) == -2                                        # varlen needs B == 1
    assert check(K, desc(K, N=5), cu=P) == 0
    assert check(K, desc(K), q=None) == -1 and check(K, desc(K), o=None) == -1
    assert check(K, desc(K, T=0), q=None, o=None) == 0                                    # empty: no data needed


def test_fwd_rejects_before_launch(K):
    """Argument errors return without touching the device (this machine has none)."""
    d = desc(K, Kd=64)
    assert K.lib().kda_fwd(P, P, P, P, P, None, None, P, None, ctypes.byref(d), None) == -3
    d = desc(K)
    assert K.lib().kda_fwd_staged(P, P, P, P, P, None, None, P, None, ctypes.byref(d), None) == -5   # no workspace
    for fn, n in (("kda_stage_gate_scan", 1), ("kda_stage_intra", 4), ("kda_stage_recurrence", 2),
                  ("kda_stage_output", 1)):
        assert getattr(K.lib(), fn)(*([P] * n), ctypes.byref(d), None) == -5
    assert K.lib().kda_stage_chunk_map(None, ctypes.byref(d), None) == -5
    d.workspace, d.workspace_bytes = P, 16
    assert K.lib().kda_stage_output(P, ctypes.byref(d), None) == -5                       # too small


def test_fwd_kernel_rejects_before_launch(K):
    """kda_fwd_kernel: an unknown kernel, or a bf16-only kernel with fp32 inputs,
    is KDA_ERR_UNSUPPORTED; shape errors as kda_fwd. All before any launch."""
    L = K.lib()
    run = lambda d, kern: L.kda_fwd_kernel(P, P, P, P, P, None, None, P, None, ctypes.byref(d), kern, None)
    assert run(desc(K), 5) == -3 and run(desc(K), -1) == -3
    assert run(desc(K, in_dt=1), K.KERNELS["two_pass"]) == -3
    cu = ctypes.c_void_p(0x2000)
    assert L.kda_fwd_kernel(P, P, P, P, P, cu, None, P, None, ctypes.byref(desc(K, N=3)), K.KERNELS["two_pass"],
                            None) == -3                                   # two_pass takes no cu_seqlens
    # one 53,248-byte operand record per (sequence, head, 32-token chunk)
    size = lambda d, kern: L.kda_fwd_kernel_workspace_size(ctypes.byref(d), kern)
    assert size(desc(K, B=2, T=100, H=3), K.KERNELS["two_pass"]) == 2 * 3 * 4 * 53248
    assert size(desc(K), K.KERNELS["pipe"]) == 0 and size(desc(K, Kd=64), K.KERNELS["two_pass"]) == 0
    assert run(desc(K, in_dt=1), K.KERNELS["pipe"]) == -3
    assert run(desc(K, in_dt=1), K.KERNELS["chunk16"]) == -3
    assert run(desc(K, Kd=64), K.KERNELS["serial"]) == -3
    assert run(desc(K, N=3), K.KERNELS["chunk16"]) == -2


def test_decode_rejects_before_launch(K):
    """kda_decode_step: shape, null and alignment errors return before any launch."""
    L = K.lib()
    A = ctypes.c_void_p(0x10000)                    # 16-byte aligned stand-in pointer
    M = ctypes.c_void_p(0x10004)                    # misaligned
    d = desc(K, B=4, T=2, N=4)
    assert L.kda_decode_step(A, A, A, A, A, None, A, None, ctypes.byref(d), None) == -2   # T != 1
    d = desc(K, B=4, T=1, N=3)
    assert L.kda_decode_step(A, A, A, A, A, None, A, None, ctypes.byref(d), None) == -2   # N != B
    d = desc(K, B=4, T=1, N=4)
    assert L.kda_decode_step(None, A, A, A, A, None, A, None, ctypes.byref(d), None) == -1
    assert L.kda_decode_step(A, A, A, A, A, M, A, None, ctypes.byref(d), None) == -3      # misaligned state
    assert L.kda_decode_step(A, A, A, A, A, None, M, None, ctypes.byref(d), None) == -3   # misaligned o
    assert L.kda_decode_step(A, A, A, A, A, None, A, None, None, None) == -1


def test_staged_layout(K):
    L = K.Layout()
    d = desc(K, B=1, T=8192, H=96)
    assert K.lib().kda_staged_layout(ctypes.byref(d), ctypes.byref(L)) == 0
    assert L.chunk == 32 and L.nslots == 257
    offs = [L.map, L.seqinfo, L.Gamma, L.gl, L.W, L.U, L.Kt, L.Qg, L.M, L.hc, L.Delta]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    tok = 8192 * 96 * 128 * 4
    assert L.U - L.W >= tok and L.Delta - L.hc >= 257 * 96 * 128 * 128 * 4 and L.total - L.Delta >= tok
    assert K.lib().kda_staged_workspace_size(ctypes.byref(d)) == L.total
    d2 = desc(K, T=100, N=7)       # varlen: ceil(100/32) + 7 slots
    assert K.lib().kda_staged_layout(ctypes.byref(d2), ctypes.byref(L)) == 0 and L.nslots == 4 + 7
    assert K.lib().kda_staged_workspace_size(ctypes.byref(desc(K, Kd=64))) == 0


def test_fwd_workspace_size(K):
    """kda_fwd_workspace_size reports what kda_fwd itself uses: nothing for the
    single fused launch; for few long chains the one-pass slice route's three
    64 KiB fp32 states per (sequence, head) and later slice and its fp32 ell for
    every slice after the first [B, T - (first token of slice 1), H, 128]. The
    slice count S is the largest that puts all 2S - 1 runs of every chain on the
    chip at once (one workgroup each), at most 4 and at most T / 4096 (this
    machine has no GPU, so the library assumes the MI355X's 256 compute
    units)."""
    size = lambda d: K.lib().kda_fwd_workspace_size(ctypes.byref(d))

    def one_pass(B, T, H):
        S = max(2, min(4, (256 // (B * H) + 1) // 2, T // 4096))
        b1 = (T // S) // 32 * 32
        return B * H * 3 * (S - 1) * 128 * 128 * 4 + B * (T - b1) * H * 128 * 4
    assert size(desc(K, T=8192, H=96)) == 0                          # headline shape: one fused launch
    assert size(desc(K, T=8192, H=64)) == 0
    assert size(desc(K, T=8192, N=6, H=96)) == 0                     # varlen: never sliced
    assert size(desc(K, T=131072, H=32)) == one_pass(1, 131072, 32)   # four slices: 18 MiB + 1.5 GiB
    assert size(desc(K, T=131072, H=32)) == (18 << 20) + (3 << 29)
    assert size(desc(K, T=65536, H=32)) == one_pass(1, 65536, 32)     # each half of the 2 x 65536 handoff
    assert size(desc(K, T=12301, B=2, H=3)) == one_pass(2, 12301, 3)  # three slices, from tokens 4096 and 8192
    assert size(desc(K, T=12301, B=2, H=3)) == 6 * 3 * 2 * 65536 + 2 * (12301 - 4096) * 3 * 512
    assert size(desc(K, T=131072, H=42)) == one_pass(1, 131072, 42)   # 42 chains: three slices
    assert size(desc(K, T=12287, H=32)) == 0                         # too short to slice
    assert size(desc(K, T=131072, H=48)) == 0                        # more than one chain per six CUs
    assert size(desc(K, T=131072, H=32, in_dt=1)) == 0               # fp32 inputs run whole
    assert size(desc(K, T=1, B=4, H=32)) == 0                        # decode route
    assert size(desc(K, Kd=64)) == 0 and K.lib().kda_fwd_workspace_size(None) == 0
