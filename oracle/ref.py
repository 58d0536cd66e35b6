"""ctypes wrapper of the fp64 recurrence oracle (kda_ref.c). Test infrastructure only."""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

from . import build as _build

_lib = None


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        lib.kda_ref_fwd.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, P, P, P]
        lib.kda_ref_fwd.restype = ctypes.c_int
        lib.gdn_ref_fwd.argtypes = lib.kda_ref_fwd.argtypes
        lib.gdn_ref_fwd.restype = ctypes.c_int
        lib.kda_ref_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def threads() -> int:
    return int(load().kda_ref_threads())


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def kda_ref_fwd(q, k, v, g, beta, cu_seqlens: Optional[np.ndarray] = None,
                h0: Optional[np.ndarray] = None, want_state: bool = True):
    """fp64 recurrence. q, k, v, g: [B, T, H, 128]; beta [B, T, H]; h0 [N, H, 128, 128].

    Returns (o [B, T, H, V] fp64, hT [N, H, K, V] fp64 or None).
    """
    return _run("kda_ref_fwd", q, k, v, g, beta, cu_seqlens, h0, want_state)


def gdn_ref_fwd(q, k, v, g, beta, cu_seqlens: Optional[np.ndarray] = None,
                h0: Optional[np.ndarray] = None, want_state: bool = True):
    """The same fp64 recurrence with a scalar gate per (token, head): g [B, T, H]
    (Gated DeltaNet). Other arguments and results as kda_ref_fwd."""
    return _run("gdn_ref_fwd", q, k, v, g, beta, cu_seqlens, h0, want_state)


def _run(fn, q, k, v, g, beta, cu_seqlens, h0, want_state):
    f = lambda x: np.ascontiguousarray(x, dtype=np.float32)
    q, k, v, g, beta = f(q), f(k), f(v), f(g), f(beta)
    B, T, H, K = q.shape
    V = v.shape[-1]
    gshape = q.shape if fn == "kda_ref_fwd" else q.shape[:3]
    assert k.shape == q.shape and g.shape == gshape and v.shape[:3] == q.shape[:3]
    assert beta.shape == (B, T, H)
    cu = None
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
        N = len(cu) - 1
        assert B == 1 and cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    else:
        N = B
    if h0 is not None:
        h0 = np.ascontiguousarray(h0, dtype=np.float64)
        assert h0.shape == (N, H, K, V)
    o = np.zeros((B, T, H, V), np.float64)
    hT = np.zeros((N, H, K, V), np.float64) if want_state else None
    rc = getattr(load(), fn)(_p(q), _p(k), _p(v), _p(g), _p(beta), _p(cu), N, B, T, H, K, V,
                             _p(h0), _p(o), _p(hT))
    if rc != 0:
        raise RuntimeError(f"{fn} failed with code {rc}")
    return o, hT
