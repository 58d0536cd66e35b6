"""fp64 chunk algebra of the KDA recurrence (numpy). TEST INFRASTRUCTURE ONLY.

The chunked prefill evaluates the same recurrence as kda_ref.c a chunk of C
tokens at a time with matrix products; chunking is an exact re-association.
The pages credit this chunked form with the prefill speed-up and name its chunk
length (16 in FlashKDA v1, 64 in flash-linear-attention) and its two-kernel
split (toolarium.ru page, §"Где ограничения прямо сейчас"). The algebra below
is derived from the recurrence, not printed on the pages.

For a chunk of n tokens entering with state S0 (g in natural-log units):
    Gamma_r   = sum_{j <= r} g_j                      (inclusive, per channel)
    A_ri      = beta_r sum_c k_rc k_ic exp(Gamma_rc - Gamma_ic)    for i < r, else 0
    Tinv      = (I + A)^{-1}                          (unit lower triangular)
    W         = Tinv Diag(beta) (K * exp(Gamma))      U = Tinv Diag(beta) V
    Delta     = U - W S0                              (row r = beta_r times the
                                                       delta-rule error of token r)
    M_ri      = sum_c q_rc k_ic exp(Gamma_rc - Gamma_ic)           for i <= r, else 0
    O         = (Q * exp(Gamma)) S0 + M Delta
    S_next    = Diag(exp(Gamma_last)) S0 + (K * exp(Gamma_last - Gamma))^T Delta
Every exponent above is <= 0 (i <= r), so the plain evaluation cannot overflow.

Chunks restart at each sequence start; the last chunk of a sequence may be short.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np
from scipy.linalg import solve_triangular


def chunk_step(q, k, v, g, beta, S0):
    """One chunk. q, k, g: [n, K]; v: [n, V]; beta: [n]; S0: [K, V]. fp64 in, dict out."""
    q, k, v, g, beta, S0 = (np.asarray(x, np.float64) for x in (q, k, v, g, beta, S0))
    n, K = k.shape
    Gam = np.cumsum(g, axis=0)                                   # [n, K]
    diff = Gam[:, None, :] - Gam[None, :, :]                     # [r, i, c] = Gamma_rc - Gamma_ic
    lower = np.tril(np.ones((n, n), dtype=bool))
    strict = np.tril(np.ones((n, n), dtype=bool), -1)
    gate = np.where(lower[:, :, None], np.exp(np.where(lower[:, :, None], diff, 0.0)), 0.0)
    KK = np.einsum("rc,ic,ric->ri", k, k, gate)
    A = np.where(strict, beta[:, None] * KK, 0.0)
    Tinv = solve_triangular(np.eye(n) + A, np.eye(n), lower=True, unit_diagonal=True)
    gam = np.exp(Gam)
    W = Tinv @ (beta[:, None] * (k * gam))
    U = Tinv @ (beta[:, None] * v)
    Delta = U - W @ S0
    M = np.where(lower, np.einsum("rc,ic,ric->ri", q, k, gate), 0.0)
    O = (q * gam) @ S0 + M @ Delta
    Kt = k * np.exp(Gam[-1][None, :] - Gam)
    S1 = np.exp(Gam[-1])[:, None] * S0 + Kt.T @ Delta
    return dict(Gamma=Gam, A=A, Tinv=Tinv, W=W, U=U, Delta=Delta, M=M, O=O,
                Kt=Kt, Qg=q * gam, Kg=k * gam, gamma_last=np.exp(Gam[-1]), S_in=S0, S_out=S1)


def chunk_fwd(q, k, v, g, beta, cu_seqlens: Optional[np.ndarray] = None,
              h0: Optional[np.ndarray] = None, C: int = 64, keep: bool = False):
    """Chunked forward over [B, T, H, *] inputs, same layouts as kda_ref_fwd.

    Returns (o, hT, stages) where stages[(n, h)] lists the per-chunk dicts when keep=True.
    """
    q, k, v, g = (np.asarray(x, np.float64) for x in (q, k, v, g))
    beta = np.asarray(beta, np.float64)
    B, T, H, K = q.shape
    V = v.shape[-1]
    if cu_seqlens is not None:
        bounds = [(0, int(cu_seqlens[i]), int(cu_seqlens[i + 1])) for i in range(len(cu_seqlens) - 1)]
    else:
        bounds = [(b, 0, T) for b in range(B)]
    N = len(bounds)
    o = np.zeros((B, T, H, V))
    hT = np.zeros((N, H, K, V))
    stages = {}
    for n, (b, t0, t1) in enumerate(bounds):
        for h in range(H):
            S = np.zeros((K, V)) if h0 is None else np.asarray(h0[n, h], np.float64)
            lst: List[dict] = []
            for c0 in range(t0, t1, C):
                c1 = min(t1, c0 + C)
                st = chunk_step(q[b, c0:c1, h], k[b, c0:c1, h], v[b, c0:c1, h], g[b, c0:c1, h],
                                beta[b, c0:c1, h], S)
                o[b, c0:c1, h] = st["O"]
                S = st["S_out"]
                if keep:
                    st["t0"] = c0
                    lst.append(st)
            hT[n, h] = S
            if keep:
                stages[(n, h)] = lst
    return o, hT, stages
