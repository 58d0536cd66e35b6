"""Pins for the CPU oracle (runs without a GPU).

The pages print no formula and no worked example for KDA, so every pin here
comes from the mathematics of the recurrence
    S_t = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T,  o_t = S_t^T q_t
(KDA as a channel-wise-gated refinement of Gated DeltaNet: toolarium.ru page
"FlashKDA: Moonshot открыла ядра Kimi Delta Attention для H20",
§"Почему это новость про инфраструктуру"; donniechu.com page, §"Số liệu kỹ thuật").

Each pin is a function of an implementation with the oracle's signature. The
oracle must pass them all; each planted mistake (a mutated copy of the
recurrence, at the bottom) must fail at least one, which shows the pins can see
a dropped term, a wrong sign or index, or a transposed operand.
"""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as W
from oracle.chunk_ref import chunk_fwd, chunk_step

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng


# ----------------------------------------------------------------------------- helpers
def unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def rand_inputs(T, H, seed, K=128, V=128, B=1, gate="bj", h0=False, N=None):
    r = RNG(seed)
    q = unit_rows(r.standard_normal((B, T, H, K))).astype(np.float32)
    k = unit_rows(r.standard_normal((B, T, H, K))).astype(np.float32)
    v = r.standard_normal((B, T, H, V)).astype(np.float32)
    beta = (1 / (1 + np.exp(-r.standard_normal((B, T, H))))).astype(np.float32)
    g = np.maximum(-np.logaddexp(0, r.standard_normal((B, T, H, K))), -5)
    if gate == "mild":
        g = 0.01 * g
    g = g.astype(np.float32)
    hh = 0.1 * r.standard_normal((N or B, H, K, V)) if h0 else None
    return q, k, v, g, beta, hh


def close(a, b, tol, what=""):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    scale = max(float(np.sqrt(np.mean(b * b))), 1e-300)
    err = float(np.max(np.abs(a - b))) / scale if a.size else 0.0
    assert err <= tol, f"{what}: max|err|/rms = {err:.3e} > {tol:.1e}"


# ----------------------------------------------------------------------------- pins
def pin_worked_example(impl):
    """Hand-worked K = V = 2 example (tests/golden/worked_example_2x2.txt)."""
    rec = {}
    for line in open(os.path.join(GOLDEN, "worked_example_2x2.txt")):
        line = line.split("#")[0].split()
        if line:
            rec[line[0]] = np.array([float(x) for x in line[1:]])
    T = 3
    k = rec["k"].reshape(1, T, 1, 2)
    v = rec["v"].reshape(1, T, 1, 2)
    q = rec["q"].reshape(1, T, 1, 2)
    beta = rec["beta"].reshape(1, T, 1)
    g = np.log(rec["alpha"]).reshape(1, T, 1, 2)
    o, hT = impl(q, k, v, g, beta)
    np.testing.assert_allclose(o.reshape(T, 2), rec["o"].reshape(T, 2), rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(hT.reshape(2, 2), rec["hT"].reshape(2, 2), rtol=1e-6, atol=1e-6)


def pin_single_token(impl):
    """T = 1 from a zero state: S_1 = beta k v^T, so o = beta (q.k) v (decay acts on zero)."""
    q, k, v, g, beta, _ = rand_inputs(1, 3, 1)
    o, hT = impl(q, k, v, g, beta)
    qk = np.sum(q.astype(np.float64) * k, axis=-1)                     # [1, 1, H]
    close(o, (beta * qk)[..., None] * v, 1e-12, "o")
    close(hT[:, :], np.einsum("bh,bhk,bhv->bhkv", beta[:, 0], k[:, 0].astype(np.float64), v[:, 0]), 1e-12, "hT")


def pin_onehot_rows(impl):
    """One-hot keys k_t = e_j: row j follows (1 - beta) alpha_j row + beta v, other rows decay.

    Every row of S is then an independent exponential moving average, evaluated
    here row by row with scalar recurrences (no matrices).
    """
    T, H, K, V = 40, 2, 128, 128
    r = RNG(2)
    q, _, v, g, beta, h0 = rand_inputs(T, H, 3, h0=True)
    idx = r.integers(0, 8, size=(1, T, H))         # few distinct keys so rows get rewritten
    k = np.zeros((1, T, H, K), np.float32)
    np.put_along_axis(k, idx[..., None], 1.0, axis=-1)
    o, hT = impl(q, k, v, g, beta, h0=h0)
    for h in range(H):
        rows = h0[0, h].astype(np.float64).copy()
        for t in range(T):
            a = np.exp(g[0, t, h].astype(np.float64))
            j = idx[0, t, h]
            b = float(beta[0, t, h])
            for c in range(K):
                if c == j:
                    rows[c] = (1.0 - b) * a[c] * rows[c] + b * v[0, t, h].astype(np.float64)
                else:
                    rows[c] = a[c] * rows[c]
            want_o = np.zeros(V)
            for c in range(K):
                want_o += float(q[0, t, h, c]) * rows[c]
            close(o[0, t, h], want_o, 1e-10, f"o t={t} h={h}")
        close(hT[0, h], rows, 1e-10, f"hT h={h}")


def pin_delta_store(impl):
    """g = 0, beta = 1, one-hot keys: S becomes a key -> latest value store (exact)."""
    T, H, K = 50, 2, 128
    r = RNG(4)
    v = r.standard_normal((1, T, H, K)).astype(np.float32)
    kid = r.integers(0, 6, size=(1, T, H))
    qid = r.integers(0, 6, size=(1, T, H))
    k = np.zeros((1, T, H, K), np.float32)
    q = np.zeros((1, T, H, K), np.float32)
    np.put_along_axis(k, kid[..., None], 1.0, axis=-1)
    np.put_along_axis(q, qid[..., None], 1.0, axis=-1)
    g = np.zeros((1, T, H, K), np.float32)
    beta = np.ones((1, T, H), np.float32)
    o, hT = impl(q, k, v, g, beta)
    for h in range(H):
        store = {}
        for t in range(T):
            store[kid[0, t, h]] = v[0, t, h].astype(np.float64)
            want = store.get(qid[0, t, h], np.zeros(K))
            np.testing.assert_allclose(o[0, t, h], want, rtol=0, atol=1e-12)


def pin_pure_decay(impl):
    """beta = 0: hT = Diag(exp(sum_t g_t)) h0 and o_t = (Diag(exp Gamma_t) h0)^T q_t (mild gate)."""
    T, H = 37, 2
    q, k, v, g, beta, h0 = rand_inputs(T, H, 5, gate="mild", h0=True)
    beta = np.zeros_like(beta)
    o, hT = impl(q, k, v, g, beta, h0=h0)
    Gam = np.cumsum(g.astype(np.float64), axis=1)                      # [1, T, H, K]
    want_hT = np.exp(Gam[0, -1])[:, :, None] * h0[0]
    close(hT[0], want_hT, 1e-12, "hT")
    want_o = np.einsum("thk,hkv,thk->thv", np.exp(Gam[0]), h0[0], q[0].astype(np.float64))
    close(o[0], want_o, 1e-12, "o")
    assert np.sqrt(np.mean(want_o ** 2)) > 1e-3, "the decayed state must stay visible"


def pin_linearity(impl):
    """o is linear in q; (o, hT) are jointly linear in (v, h0)."""
    T, H = 30, 2
    q1, k, v1, g, beta, h01 = rand_inputs(T, H, 6, h0=True)
    q2, _, v2, _, _, h02 = rand_inputs(T, H, 7, h0=True)
    # dyadic grids keep q1 + 2 q2 and v1 - 3 v2 exact in float32
    grid = lambda x, step: (np.round(x / step) * step).astype(np.float32)
    q1, q2, v1, v2 = grid(q1, 2.0 ** -8), grid(q2, 2.0 ** -8), grid(v1, 2.0 ** -6), grid(v2, 2.0 ** -6)
    oa, _ = impl(q1, k, v1, g, beta, h0=h01)
    ob, _ = impl(q2, k, v1, g, beta, h0=h01)
    oc, _ = impl(q1 + 2 * q2, k, v1, g, beta, h0=h01)
    close(oc, oa + 2 * ob, 1e-12, "linear in q")
    o1, s1 = impl(q1, k, v1, g, beta, h0=h01)
    o2, s2 = impl(q1, k, v2, g, beta, h0=h02)
    o3, s3 = impl(q1, k, v1 - 3 * v2, g, beta, h0=h01 - 3 * h02)
    close(o3, o1 - 3 * o2, 1e-12, "o linear in (v, h0)")
    close(s3, s1 - 3 * s2, 1e-12, "hT linear in (v, h0)")


def pin_v_permutation(impl):
    """Permuting the V columns of v and h0 permutes those of o and hT."""
    T, H = 25, 2
    q, k, v, g, beta, h0 = rand_inputs(T, H, 8, h0=True)
    p = RNG(9).permutation(v.shape[-1])
    o, hT = impl(q, k, v, g, beta, h0=h0)
    op, hTp = impl(q, k, v[..., p], g, beta, h0=h0[..., p])
    close(op, o[..., p], 1e-13, "o")
    close(hTp, hT[..., p], 1e-13, "hT")


def pin_rotation(impl):
    """Scalar gate (g_t,c = g_t): rotating q, k, h0 by an orthogonal R leaves o and maps hT -> R hT."""
    T, H, K = 30, 2, 128
    q, k, v, g, beta, h0 = rand_inputs(T, H, 10, h0=True)
    g = np.repeat(g[..., :1], K, axis=-1)
    R, _ = np.linalg.qr(RNG(11).standard_normal((K, K)))
    o, hT = impl(q, k, v, g, beta, h0=h0)
    rot = lambda x: np.einsum("ij,...j->...i", R, x.astype(np.float64))
    o2, hT2 = impl(rot(q), rot(k), v, g, beta, h0=np.einsum("ij,nhjv->nhiv", R, h0))
    # the rotated q, k reach the oracle rounded to float32 (relative 6e-8), hence 1e-5
    close(o2, o, 1e-5, "o")
    close(hT2, np.einsum("ij,nhjv->nhiv", R, hT), 1e-5, "hT")


def pin_varlen(impl):
    """A packed batch equals independent per-sequence runs (zero-length sequences included)."""
    lens = [5, 0, 17, 1, 9]
    T, H = sum(lens), 2
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q, k, v, g, beta, h0 = rand_inputs(T, H, 12, h0=True, N=len(lens))
    o, hT = impl(q, k, v, g, beta, cu_seqlens=cu, h0=h0)
    for n, L in enumerate(lens):
        s = slice(cu[n], cu[n + 1])
        if L == 0:
            close(hT[n], h0[n], 0.0, "empty sequence keeps h0")
            continue
        on, hn = impl(q[:, s], k[:, s], v[:, s], g[:, s], beta[:, s], h0=h0[n:n + 1])
        close(o[:, s], on, 1e-13, f"o seq {n}")
        close(hT[n], hn[0], 1e-13, f"hT seq {n}")


def pin_handoff(impl):
    """Two halves with hT handed over as h0 equal one run."""
    T, H = 44, 2
    q, k, v, g, beta, h0 = rand_inputs(T, H, 13, gate="mild", h0=True)
    o, hT = impl(q, k, v, g, beta, h0=h0)
    m = 19
    oa, ha = impl(q[:, :m], k[:, :m], v[:, :m], g[:, :m], beta[:, :m], h0=h0)
    ob, hb = impl(q[:, m:], k[:, m:], v[:, m:], g[:, m:], beta[:, m:], h0=ha)
    close(np.concatenate([oa, ob], axis=1), o, 1e-13, "o")
    close(hb, hT, 1e-13, "hT")


PINS = [pin_worked_example, pin_single_token, pin_onehot_rows, pin_delta_store, pin_pure_decay,
        pin_linearity, pin_v_permutation, pin_rotation, pin_varlen, pin_handoff]


def oracle_impl(q, k, v, g, beta, cu_seqlens=None, h0=None):
    return oracle.kda_ref_fwd(q, k, v, g, beta, cu_seqlens=cu_seqlens, h0=h0)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle_impl)


# ----------------------------------------------------------------------------- planted mistakes
def mutant(kind):
    """A copy of the recurrence with one planted mistake (numpy, fp64)."""
    def impl(q, k, v, g, beta, cu_seqlens=None, h0=None):
        q, k, v, g, beta = (np.asarray(x, np.float64) for x in (q, k, v, g, beta))
        B, T, H, K = q.shape
        V = v.shape[-1]
        bounds = ([(0, int(cu_seqlens[i]), int(cu_seqlens[i + 1])) for i in range(len(cu_seqlens) - 1)]
                  if cu_seqlens is not None else [(b, 0, T) for b in range(B)])
        o = np.zeros((B, T, H, V))
        hT = np.zeros((len(bounds), H, K, V))
        for n, (b, t0, t1) in enumerate(bounds):
            for h in range(H):
                S = np.zeros((K, V)) if h0 is None else np.array(h0[n, h], np.float64)
                if kind == "h0_transposed" and h0 is not None:
                    S = S.T.copy()
                if kind == "h0_ignored":
                    S = np.zeros((K, V))
                for t in range(t0, t1):
                    kt, qt, vt, bt = k[b, t, h], q[b, t, h], v[b, t, h], beta[b, t, h]
                    a = np.exp(-g[b, t, h]) if kind == "exp_neg" else np.exp(g[b, t, h])
                    if kind == "pre_update_output":
                        o[b, t, h] = S.T @ qt
                    if kind == "decay_after":
                        e = vt - S.T @ kt
                        S = S + bt * np.outer(kt, e)
                        S = a[:, None] * S
                    else:
                        pred_state = S if kind == "undecayed_prediction" else None
                        S = (S * a[None, :]) if kind == "decay_columns" else (a[:, None] * S)
                        ps = S if pred_state is None else pred_state
                        if kind == "transposed_prediction":
                            e = vt - ps @ kt
                        elif kind == "sign":
                            e = vt + ps.T @ kt
                        else:
                            e = vt - ps.T @ kt
                        w = kt if kind == "no_beta" else bt * kt
                        S = S + np.outer(w, e)
                    if kind == "transposed_output":
                        o[b, t, h] = S @ qt
                    elif kind == "scaled_output":
                        o[b, t, h] = (S.T @ qt) / np.sqrt(K)
                    elif kind != "pre_update_output":
                        o[b, t, h] = S.T @ qt
                hT[n, h] = S
        return o, hT
    return impl


MUTANTS = ["decay_after", "no_beta", "pre_update_output", "decay_columns", "sign",
           "transposed_prediction", "exp_neg", "scaled_output", "undecayed_prediction",
           "transposed_output", "h0_ignored", "h0_transposed"]


def test_mutant_carrier_is_correct():
    """The unmutated numpy copy passes every pin, so a mutant failure is due to its mistake."""
    for pin in PINS:
        pin(mutant("none"))


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_catch_planted_mistake(kind):
    impl = mutant(kind)
    caught = []
    for pin in PINS:
        try:
            pin(impl)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake '{kind}'"


# ----------------------------------------------------------------------------- chunk algebra
@pytest.mark.parametrize("C", [1, 7, 16, 32, 64])
def test_chunk_algebra_equals_recurrence(C):
    """The chunked form is an exact re-association: brute-force equality at T <= 128,
    including partial chunks, varlen restarts and initial states."""
    lens = [100, 3, 0, 25]
    T, H = sum(lens), 2
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q, k, v, g, beta, h0 = rand_inputs(T, H, 20 + C, h0=True, N=len(lens))
    o_ref, hT_ref = oracle.kda_ref_fwd(q, k, v, g, beta, cu_seqlens=cu, h0=h0)
    o, hT, _ = chunk_fwd(q, k, v, g, beta, cu_seqlens=cu, h0=h0, C=C)
    close(o, o_ref, 1e-11, "o")
    close(hT, hT_ref, 1e-11, "hT")
    # mild gate: the inter-chunk terms carry weight
    q, k, v, g, beta, h0 = rand_inputs(128, 1, 40 + C, gate="mild", h0=True)
    o_ref, hT_ref = oracle.kda_ref_fwd(q, k, v, g, beta, h0=h0)
    o, hT, _ = chunk_fwd(q, k, v, g, beta, h0=h0, C=C)
    close(o, o_ref, 1e-11, "o mild")
    close(hT, hT_ref, 1e-11, "hT mild")


def test_chunk_intermediates():
    """(I + A) Tinv = I; Delta row r = beta_r times the delta-rule error of token r;
    the chunk's state map is affine: S_next = (Diag(gamma_last) - Kt^T W) S0 + Kt^T U."""
    T, C = 40, 40
    q, k, v, g, beta, h0 = rand_inputs(T, 1, 30, gate="mild", h0=True)
    st = chunk_step(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], beta[0, :, 0], h0[0, 0])
    close((np.eye(T) + st["A"]) @ st["Tinv"], np.eye(T), 1e-13, "(I+A) Tinv")
    for r in [0, 1, 7, 39]:
        if r == 0:
            S_prev = h0[0, 0]
        else:
            _, hp = oracle.kda_ref_fwd(q[:, :r], k[:, :r], v[:, :r], g[:, :r], beta[:, :r], h0=h0)
            S_prev = hp[0, 0]
        decayed = np.exp(g[0, r, 0].astype(np.float64))[:, None] * S_prev
        err = v[0, r, 0] - decayed.T @ k[0, r, 0]
        close(st["Delta"][r], beta[0, r, 0] * err, 1e-11, f"Delta row {r}")
    Pm = np.diag(st["gamma_last"]) - st["Kt"].T @ st["W"]
    close(Pm @ h0[0, 0] + st["Kt"].T @ st["U"], st["S_out"], 1e-12, "affine map")


def test_gate_range_of_workloads():
    """Gate values stay in [-5, 0] (the documented input range) and beta in (0, 1)."""
    inp = W.make_inputs(W.CONFIGS["tiny_fp32"], 0)
    assert inp.g.min() >= -5.0 and inp.g.max() <= 0.0
    assert inp.beta.min() > 0.0 and inp.beta.max() < 1.0


def test_workloads_match_pages_table():
    """The varlen mixes and shapes match the H20 table (tests/golden/h20_workloads.json)."""
    tab = json.load(open(os.path.join(GOLDEN, "h20_workloads.json")))
    rows = {(r["H"], tuple(r["seq_lens"]) if r["seq_lens"] else None) for r in tab["rows"]}
    for name in ["T8192_H64", "T8192_H96", "varlen6_T8192_H96", "varlen8x1024_H96"]:
        c = W.CONFIGS[name]
        assert c.T == 8192 and (c.H, c.seq_lens) in rows, name
    assert tab["protocol"] == {"warmup": 30, "iters": 200, "repeats": 5}


def test_bf16_rounding():
    """Round-to-nearest-even to bfloat16, checked on hand-picked bit patterns."""
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -7, -2.5, 1.0 - 2 ** -10], np.float32)
    want = np.array([1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.5, 1.0], np.float32)
    np.testing.assert_array_equal(W.bf16_round(x), want)
    assert W.bf16_bits(np.array([1.0], np.float32))[0] == 0x3F80


# ----------------------------------------------------------------------------- scalar gate (GDN)
def gdn_inputs(T, H, seed, **kw):
    q, k, v, g, beta, h0 = rand_inputs(T, H, seed, **kw)
    return q, k, v, np.ascontiguousarray(g[..., 0]), beta, h0


@pytest.mark.parametrize("case", ["fixed", "varlen", "h0"])
def test_gdn_equals_kda_with_repeated_gate(case):
    """One gate per (token, head) is KDA with that gate on every channel: the two
    oracle entries agree bitwise (same operations in the same order)."""
    if case == "varlen":
        q, k, v, gs, beta, h0 = gdn_inputs(70, 3, 20, h0=True, N=3)
        cu = np.array([0, 33, 33, 70], np.int64)
    else:
        q, k, v, gs, beta, h0 = gdn_inputs(45, 2, 21, B=2, h0=(case == "h0"))
        cu = None
    g = np.repeat(gs[..., None], q.shape[-1], axis=-1)
    o1, h1 = oracle.gdn_ref_fwd(q, k, v, gs, beta, cu_seqlens=cu, h0=h0)
    o2, h2 = oracle.kda_ref_fwd(q, k, v, g, beta, cu_seqlens=cu, h0=h0)
    assert np.array_equal(o1, o2) and np.array_equal(h1, h2)


def test_gdn_single_step_closed_form():
    """T = 1 from h0 with a scalar gate a = exp(g): S_1 = a h0 + beta k (v - a h0^T k)^T, o = S_1^T q."""
    q, k, v, gs, beta, h0 = gdn_inputs(1, 3, 22, h0=True)
    o, hT = oracle.gdn_ref_fwd(q, k, v, gs, beta, h0=h0)
    for h in range(3):
        a = np.exp(np.float64(gs[0, 0, h]))
        kk, qq, vv = (x[0, 0, h].astype(np.float64) for x in (k, q, v))
        D0 = a * h0[0, h]
        S1 = D0 + beta[0, 0, h] * np.outer(kk, vv - D0.T @ kk)
        close(hT[0, h], S1, 1e-13, "hT")
        close(o[0, 0, h], S1.T @ qq, 1e-13, "o")


def test_gdn_rotation_invariance():
    """Scalar gate: rotating q, k and h0 by an orthogonal R leaves o unchanged and maps
    hT -> R hT. With a channel-wise gate the same rotation changes o (the pin can tell
    the two gates apart)."""
    T, H, K = 40, 2, 128
    q, k, v, gs, beta, h0 = gdn_inputs(T, H, 23, h0=True)
    R, _ = np.linalg.qr(RNG(24).standard_normal((K, K)))
    rot = lambda x: np.einsum("ij,...j->...i", R, x.astype(np.float64))
    h0r = np.einsum("ij,nhjv->nhiv", R, h0)
    o, hT = oracle.gdn_ref_fwd(q, k, v, gs, beta, h0=h0)
    o2, hT2 = oracle.gdn_ref_fwd(rot(q), rot(k), v, gs, beta, h0=h0r)
    close(o2, o, 1e-5, "o")
    close(hT2, np.einsum("ij,nhjv->nhiv", R, hT), 1e-5, "hT")
    _, _, _, gc, _, _ = rand_inputs(T, H, 23)
    oc, _ = oracle.kda_ref_fwd(q, k, v, gc, beta, h0=h0)
    oc2, _ = oracle.kda_ref_fwd(rot(q), rot(k), v, gc, beta, h0=h0r)
    with pytest.raises(AssertionError):
        close(oc2, oc, 1e-5, "o (channel-wise gate)")


def test_scalar_gate_workload():
    cfg = W.variant("T8192_H96", T=64, H=2, gate="scalar", name="gdn")
    inp = W.make_inputs(cfg, 0)
    gs = inp.g_scalar()
    assert gs.shape == (1, 64, 2) and np.all(gs <= 0) and np.all(gs >= -5)
    base = W.make_inputs(W.variant("T8192_H96", T=64, H=2, name="kda"), 0)
    assert np.array_equal(base.q, inp.q) and np.array_equal(base.beta, inp.beta)
    assert np.array_equal(gs, base.g[..., 0])    # channel 0 of the same draw
