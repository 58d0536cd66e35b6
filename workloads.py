"""Seeded synthetic inputs for the KDA chunked prefill.

This module is shared by the tests, the benchmark and the smoke check. It draws
the inputs and rounds them to the precision the device receives. It holds none
of the method's arithmetic: no decay, no delta rule, no output.

Workload shapes follow the H20 benchmark table on the toolarium.ru page
"FlashKDA: Moonshot открыла ядра Kimi Delta Attention для H20"
(§"Что показывают H20-бенчмарки"): T = 8192 tokens, H in {64, 96},
D = K = V = 128, fixed-length and two variable-length mixes. The donniechu.com
page "FlashKDA … Kimi Delta Attention" (§"Số liệu kỹ thuật") fixes K = V = 128,
bf16 + fp32 precision, cu_seqlens and initial/final states.

Value distributions (the pages give none, so these are stated readings):
  q, k ~ N(0, 1), then L2-normalised over the 128 channels of each (token, head)
  in fp32; v ~ N(0, 1); beta = sigmoid(N(0, 1)); g = max(-softplus(N(0, 1)), -5)
  per channel, softplus evaluated stably in fp64 and stored as fp32;
  h0 = 0.1 * N(0, 1) per (sequence, head) when a config asks for it.
  q, k, v are rounded to bf16 (round-to-nearest-even) except on fp32 configs.

Draw order with numpy.random.Generator(PCG64(seed)): q, k, v (float32
standard_normal, full [B, T, H, 128] shapes), beta pre-activation [B, T, H],
g pre-activation [B, T, H, 128], then h0 [N, H, 128, 128] if used.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

D = 128  # K = V = 128, the only head size the method supports


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return the uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = np.isnan(x)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = (r >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 value, returned as float32."""
    return bf16_to_f32(bf16_bits(x))


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    B: int
    T: int                      # tokens per batch row (packed total when varlen)
    H: int
    dtype: str = "bf16"         # dtype of q, k, v: "bf16" or "fp32"
    seq_lens: Optional[tuple] = None   # varlen mix (B must be 1); None = fixed length
    h0: bool = False            # draw an initial state per (sequence, head)
    gate: str = "bj"            # "bj" | "mild" | "zero" | "floor" | "scalar" | "scalar_mild" (all but "bj" test-only)
    beta: str = "bj"            # "bj" | "zero" | "one"
    keys: str = "gauss"         # "gauss" | "onehot" | "same"
    note: str = ""

    @property
    def N(self) -> int:
        return len(self.seq_lens) if self.seq_lens is not None else self.B

    @property
    def token_heads(self) -> int:
        return self.B * self.T * self.H


# The workloads: the pages' benchmark shapes (the headline is T=8192, H=96) and a
# tiny fp32 case.
VARLEN_MIX = (1300, 547, 2048, 963, 271, 3063)
CONFIGS = {
    "tiny_fp32": Config("tiny_fp32", 1, 256, 2, dtype="fp32", note="tiny fixed, fp32 inputs, h0 = 0"),
    "T8192_H64": Config("T8192_H64", 1, 8192, 64, note="fixed-length prefill, H=64"),
    "T8192_H96": Config("T8192_H96", 1, 8192, 96, note="fixed-length prefill, H=96 (headline)"),
    "varlen6_T8192_H96": Config("varlen6_T8192_H96", 1, 8192, 96, seq_lens=VARLEN_MIX, h0=True, note="varlen 6-sequence mix"),
    "varlen8x1024_H96": Config("varlen8x1024_H96", 1, 8192, 96, seq_lens=(1024,) * 8, h0=True, note="varlen 8 x 1024"),
    "T131072_H32": Config("T131072_H32", 1, 131072, 32, h0=True, note="long-context stateful prefill"),
}


def cu_seqlens_of(seq_lens: Sequence[int]) -> np.ndarray:
    cu = np.zeros(len(seq_lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(seq_lens, dtype=np.int64))
    return cu


@dataclasses.dataclass
class Inputs:
    cfg: Config
    q: np.ndarray          # float32 [B, T, H, 128], values exactly as the device receives them
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray          # float32 [B, T, H, 128]
    beta: np.ndarray       # float32 [B, T, H]
    h0: Optional[np.ndarray]          # float32 [N, H, 128, 128] or None
    cu_seqlens: Optional[np.ndarray]  # int32 [N + 1] or None

    def device_bits(self, name: str) -> np.ndarray:
        """bf16 bit pattern of q/k/v for bf16 configs (exact: values are already bf16)."""
        return bf16_bits(getattr(self, name))

    def g_scalar(self) -> np.ndarray:
        """The per-(token, head) gate [B, T, H] of a scalar-gate input."""
        assert np.all(self.g == self.g[..., :1]), "gate is not scalar"
        return np.ascontiguousarray(self.g[..., 0])

    def seq_bounds(self):
        """(batch row, start, end) per sequence."""
        if self.cu_seqlens is None:
            return [(b, 0, self.cfg.T) for b in range(self.cfg.B)]
        cu = self.cu_seqlens
        return [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]


def _softplus64(z: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, z.astype(np.float64))


def make_inputs(cfg: Config, seed: int, dtype: Optional[str] = None) -> Inputs:
    dtype = dtype or cfg.dtype
    B, T, H = cfg.B, cfg.T, cfg.H
    if cfg.seq_lens is not None:
        assert B == 1 and sum(cfg.seq_lens) == T, "varlen configs pack into one row of T tokens"
    rng = np.random.Generator(np.random.PCG64(seed))
    shp = (B, T, H, D)
    q = rng.standard_normal(shp, dtype=np.float32)
    k = rng.standard_normal(shp, dtype=np.float32)
    v = rng.standard_normal(shp, dtype=np.float32)
    bz = rng.standard_normal((B, T, H), dtype=np.float32)
    gz = rng.standard_normal(shp, dtype=np.float32)
    h0 = None
    if cfg.h0:
        h0 = (np.float32(0.1) * rng.standard_normal((cfg.N, H, D, D), dtype=np.float32)).astype(np.float32)

    # L2 normalisation per (token, head) in fp32, before rounding to the device dtype.
    q /= np.sqrt(np.sum(q * q, axis=-1, keepdims=True, dtype=np.float32))
    k /= np.sqrt(np.sum(k * k, axis=-1, keepdims=True, dtype=np.float32))

    if cfg.keys == "onehot":
        idx = rng.integers(0, D, size=(B, T, H))
        k = np.zeros(shp, np.float32)
        np.put_along_axis(k, idx[..., None], 1.0, axis=-1)
    elif cfg.keys == "same":
        k[:] = k[:, :1]          # every token of a row shares the first token's key

    beta = (1.0 / (1.0 + np.exp(-bz.astype(np.float64)))).astype(np.float32)
    if cfg.beta == "zero":
        beta[:] = 0.0
    elif cfg.beta == "one":
        beta[:] = 1.0

    if cfg.gate in ("scalar", "scalar_mild"):
        # one gate per (token, head) (the Gated DeltaNet form): channel 0's draw,
        # repeated over the channels
        gz = np.repeat(gz[..., :1], D, axis=-1)
    g = np.maximum(-_softplus64(gz), -5.0)
    if cfg.gate in ("mild", "scalar_mild"):
        g = 0.01 * g
    elif cfg.gate == "zero":
        g = np.zeros_like(g)
    elif cfg.gate == "floor":
        # every channel at the floor of the draws' range, -5 per token: the
        # strongest in-chunk decay the generator produces
        g = np.full_like(g, -5.0)
    g = g.astype(np.float32)
    del gz

    if dtype == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    else:
        assert dtype == "fp32"
    cu = cu_seqlens_of(cfg.seq_lens) if cfg.seq_lens is not None else None
    return Inputs(cfg, q, k, v, g, beta, h0, cu)


def variant(base: str | Config, **kw) -> Config:
    """A test-only variant of a config (mild decay, zero gate, edge lengths, ...)."""
    cfg = CONFIGS[base] if isinstance(base, str) else base
    name = kw.pop("name", cfg.name + "+" + ",".join(f"{a}={b}" for a, b in sorted(kw.items())))
    return dataclasses.replace(cfg, name=name, **kw)


def rms(x: np.ndarray) -> float:
    x = np.asarray(x, dtype=np.float64)
    return float(np.sqrt(np.mean(x * x))) if x.size else 0.0
