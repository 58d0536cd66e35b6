"""ctypes binding of libkda.so: argument marshalling only."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkda.so")

KDA_BF16, KDA_F32 = 0, 1
# kda_kernel_t
KERNELS = {"auto": 0, "pipe": 1, "serial": 2, "chunk16": 3, "two_pass": 4}
STATUS = {0: "KDA_OK", -1: "KDA_ERR_NULL", -2: "KDA_ERR_SHAPE", -3: "KDA_ERR_UNSUPPORTED",
          -4: "KDA_ERR_DTYPE", -5: "KDA_ERR_WORKSPACE", -6: "KDA_ERR_HIP"}

# every symbol include/kda.h declares
EXPORTS = ["kda_status_string", "kda_version", "kda_fwd_check", "kda_fwd", "kda_gdn_fwd", "kda_fwd_kernel",
           "kda_fwd_kernel_workspace_size", "kda_fwd_workspace_size", "kda_fwd_noalloc",
           "kda_fwd_noalloc_max_workspace",
           "kda_decode_step", "kda_staged_layout",
           "kda_staged_workspace_size", "kda_stage_chunk_map", "kda_stage_gate_scan", "kda_stage_intra",
           "kda_stage_recurrence", "kda_stage_output", "kda_fwd_staged"]


class Desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("K", ctypes.c_int32), ("V", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
                ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class Layout(ctypes.Structure):
    _fields_ = [("nslots", ctypes.c_int32), ("chunk", ctypes.c_int32)] + [
        (n, ctypes.c_size_t) for n in ("map", "seqinfo", "Gamma", "gl", "W", "U", "Kt", "Qg", "M", "hc",
                                       "Delta", "total")]


class KDAError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {STATUS.get(code, code)} ({status_string(code)})")


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"HIP library {LIB_PATH} is not built; run __graft_entry__.build() "
                              "(or python gated_delta_rule_63_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        L.kda_status_string.argtypes = [ctypes.c_int]
        L.kda_status_string.restype = ctypes.c_char_p
        L.kda_version.restype = ctypes.c_int32
        L.kda_fwd_check.argtypes = [P] * 9 + [ctypes.POINTER(Desc)]
        L.kda_fwd_check.restype = ctypes.c_int
        L.kda_fwd.argtypes = [P] * 9 + [ctypes.POINTER(Desc), P]
        L.kda_fwd.restype = ctypes.c_int
        L.kda_fwd_noalloc.argtypes = [P] * 9 + [ctypes.POINTER(Desc), P]
        L.kda_fwd_noalloc.restype = ctypes.c_int
        L.kda_fwd_noalloc_max_workspace.argtypes = []
        L.kda_fwd_noalloc_max_workspace.restype = ctypes.c_size_t
        L.kda_gdn_fwd.argtypes = [P] * 9 + [ctypes.POINTER(Desc), P]
        L.kda_gdn_fwd.restype = ctypes.c_int
        L.kda_fwd_kernel.argtypes = [P] * 9 + [ctypes.POINTER(Desc), ctypes.c_int32, P]
        L.kda_fwd_kernel.restype = ctypes.c_int
        L.kda_fwd_kernel_workspace_size.argtypes = [ctypes.POINTER(Desc), ctypes.c_int32]
        L.kda_fwd_kernel_workspace_size.restype = ctypes.c_size_t
        L.kda_decode_step.argtypes = [P] * 8 + [ctypes.POINTER(Desc), P]
        L.kda_decode_step.restype = ctypes.c_int
        L.kda_fwd_workspace_size.argtypes = [ctypes.POINTER(Desc)]
        L.kda_fwd_workspace_size.restype = ctypes.c_size_t
        L.kda_staged_workspace_size.argtypes = [ctypes.POINTER(Desc)]
        L.kda_staged_workspace_size.restype = ctypes.c_size_t
        L.kda_staged_layout.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(Layout)]
        L.kda_staged_layout.restype = ctypes.c_int
        D = ctypes.POINTER(Desc)
        for name, n in (("kda_stage_chunk_map", 1), ("kda_stage_gate_scan", 1), ("kda_stage_intra", 4),
                        ("kda_stage_recurrence", 2), ("kda_stage_output", 1)):
            fn = getattr(L, name)
            fn.argtypes = [P] * n + [D, P]
            fn.restype = ctypes.c_int
        L.kda_fwd_staged.argtypes = [P] * 9 + [D, P]
        L.kda_fwd_staged.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().kda_status_string(int(code)).decode()
