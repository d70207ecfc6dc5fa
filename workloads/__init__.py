"""Seeded synthetic inputs for block-causal ReLU linear attention.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It holds no arithmetic of the method itself: it only draws random
numbers, rounds them to the storage type and describes the five workload
shapes.  The shapes come from the video sizes the SANA-Video pages quote
(the abstract's "up to 720x1280 and minute-length"; the SANA-Video 2.0
model page's hidden size 2560 and (8,32,32) VAE compression):

  c1  tiny, fp32 parity case        B1 H2  d32   4 blocks x 256 tokens
  c2  480p non-causal (CFG pair)    B2 H70 d32   1 block  x 8190 (21 frames x 15x26)
  c3  720p 5 s block-causal         B1 H70 d32   7 blocks x 2640 (3 frames x 22x40)
  c4  minute-long 480p streaming    B1 H70 d32  80 blocks x 1170 (3 frames x 15x26), 3D RoPE
  c5  2.0-style gated               B1 H20 d128  8 blocks x 1760 (2 frames x 22x40), decay g

Recipe (identical for every consumer): ``numpy.random.default_rng(seed)``,
seed = config number; draw Q, K, V in that order with
``standard_normal(float32)`` in [B,H,N,d] C-order, round to bf16 with
round-to-nearest-even (c1 stays fp32); then, for gated configs, draw
g_raw ~ N(2,1) in float64 of shape [B,H,nb] and store sigmoid(g_raw) as fp32.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "ConvConfig", "CONV_CONFIGS", "make_conv_inputs",
    "Rope", "Config", "CONFIGS", "get_config", "bf16_round", "bf16_bits", "fp8_bits",
    "fp8_from_bits", "fp8_round", "make_grad_output",
    "bf16_from_bits", "make_inputs", "scaled_config",
]


@dataclasses.dataclass(frozen=True)
class Rope:
    """3D rotary positions: (t, h, w) dims split dt/dh/dw, raster t-h-w order.

    Token p of a call sits at frame t0 + p // (grid_h*grid_w), row
    (p // grid_w) % grid_h and column p % grid_w.
    """
    dt_dims: int = 8
    dh_dims: int = 12
    dw_dims: int = 12
    grid_h: int = 15
    grid_w: int = 26
    t0: int = 0
    base: float = 10000.0

    def with_t0(self, t0: int) -> "Rope":
        return dataclasses.replace(self, t0=t0)


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    B: int
    H: int
    d: int
    nb: int
    n: int
    dtype: str            # "f32", "bf16" or "fp8" (OCP E4M3 inputs)
    seed: int
    eps: float = 1e-6
    rope: Optional[Rope] = None
    gated: bool = False
    streaming: bool = False   # the nb blocks are fed one block step at a time
    description: str = ""

    @property
    def N(self) -> int:
        return self.nb * self.n

    @property
    def tokens_heads(self) -> int:
        return self.B * self.H * self.N


CONFIGS = {
    "c1": Config("c1", B=1, H=2, d=32, nb=4, n=256, dtype="f32", seed=1,
                 description="tiny block-causal, fp32, brute-force checked"),
    "c2": Config("c2", B=2, H=70, d=32, nb=1, n=8190, dtype="bf16", seed=2,
                 description="480p non-causal, 21 frames x 15x26, CFG pair"),
    "c3": Config("c3", B=1, H=70, d=32, nb=7, n=2640, dtype="bf16", seed=3,
                 description="720p 5 s block-causal, 7 blocks of 3 frames x 22x40"),
    "c4": Config("c4", B=1, H=70, d=32, nb=80, n=1170, dtype="bf16", seed=4,
                 rope=Rope(8, 12, 12, 15, 26, 0, 10000.0), streaming=True,
                 description="minute-long 480p streaming, 80 steps of 3 frames x 15x26, 3D RoPE"),
    "c5": Config("c5", B=1, H=20, d=128, nb=8, n=1760, dtype="bf16", seed=5,
                 gated=True,
                 description="2.0-style gated, 8 blocks of 2 frames x 22x40, g=sigmoid(N(2,1))"),
}


def get_config(name: str) -> Config:
    return CONFIGS[name.lower()]


def scaled_config(cfg: Config, **overrides) -> Config:
    """The same workload family with some sizes replaced (for small parity cases)."""
    return dataclasses.replace(cfg, **overrides)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round-to-nearest-even, NaN kept quiet."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # in uint32: the sum stays below 2^32 for every non-NaN pattern (at most
    # 0xFF7FFFFF + 0x8000); NaN patterns, which may wrap, are replaced below
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return out


def bf16_from_bits(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> the exact float32 values."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def fp8_from_bits(b: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 ("fn": 1 sign, 4 exponent bits of bias 7, 3 mantissa bits,
    no infinities, S.1111.111 is NaN) bit patterns (uint8) -> exact float32."""
    b = np.ascontiguousarray(b, dtype=np.uint8).astype(np.int32)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    out = (sign * mag).astype(np.float32)
    out[(b & 0x7F) == 0x7F] = np.nan
    return out


def fp8_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> OCP FP8 E4M3 bit patterns, round to nearest, ties to even
    mantissa; magnitudes past the largest finite value (448) saturate to it;
    NaN -> 0x7F with its sign."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    ax = np.abs(x).astype(np.float64)
    out = np.zeros(x.shape, dtype=np.int32)
    # the 127 non-negative finite codes, their values in increasing order
    codes = np.arange(0x7F, dtype=np.int32)
    vals = fp8_from_bits(codes.astype(np.uint8)).astype(np.float64)
    idx = np.clip(np.searchsorted(vals, ax), 1, len(vals) - 1)   # vals[idx-1] <= ax <= vals[idx]
    lo, hi = vals[idx - 1], vals[idx]
    up = (ax - lo > hi - ax) | ((ax - lo == hi - ax) & ((idx - 1) % 2 == 1))
    out = np.where(up, idx, idx - 1)
    out = np.where(ax >= vals[-1], len(vals) - 1, out)           # saturate at 448
    out = out | np.where(np.signbit(x), 0x80, 0)
    out = np.where(np.isnan(x), 0x7F | np.where(np.signbit(x), 0x80, 0), out)
    return out.astype(np.uint8)


def fp8_round(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest OCP FP8 E4M3 value, as float32."""
    return fp8_from_bits(fp8_bits(x))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 values rounded (RNE) to the nearest bf16, returned as float32."""
    return bf16_from_bits(bf16_bits(x))


def _gate(rng: np.random.Generator, shape) -> np.ndarray:
    raw = rng.standard_normal(shape, dtype=np.float64) + 2.0
    return (1.0 / (1.0 + np.exp(-raw))).astype(np.float32)


def make_inputs(cfg: Config, seed: Optional[int] = None, *, B=None, H=None,
                nb=None, n=None) -> dict:
    """Draw the inputs of ``cfg`` (sizes optionally overridden).

    Returns a dict with ``Q, K, V`` as float32 arrays of shape [B,H,N,d]
    holding exactly representable values of the storage type (bf16-exact for
    bf16 configs), ``g`` ([B,H,nb] float32, or None), plus the config, the
    sizes and ``rope``.  For bf16 configs ``Q_bits`` etc. hold the raw bf16
    bit patterns (uint16) that a device buffer should contain.
    """
    B = cfg.B if B is None else B
    H = cfg.H if H is None else H
    nb = cfg.nb if nb is None else nb
    n = cfg.n if n is None else n
    d = cfg.d
    N = nb * n
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    out = {"cfg": cfg, "B": B, "H": H, "nb": nb, "n": n, "N": N, "d": d,
           "eps": cfg.eps, "rope": cfg.rope, "dtype": cfg.dtype}
    for name in ("Q", "K", "V"):
        x = rng.standard_normal((B, H, N, d), dtype=np.float32)
        if cfg.dtype == "bf16":
            bits = bf16_bits(x)
            out[name + "_bits"] = bits
            out[name] = bf16_from_bits(bits)
        elif cfg.dtype == "fp8":
            bits = fp8_bits(x)
            out[name + "_bits"] = bits
            out[name] = fp8_from_bits(bits)
        else:
            out[name] = x
    out["g"] = _gate(rng, (B, H, nb)) if cfg.gated else None
    return out


def make_grad_output(x: dict, seed: int) -> np.ndarray:
    """dO for a backward case of the inputs ``x`` (from ``make_inputs``):
    standard normal [B,H,N,d] float32 from its own generator (seed ``seed``),
    rounded to the inputs' storage type as Q, K and V are."""
    rng = np.random.default_rng(seed)
    dO = rng.standard_normal((x["B"], x["H"], x["N"], x["d"]), dtype=np.float32)
    return bf16_round(dO) if x["dtype"] == "bf16" else dO


def step_slice(x: np.ndarray, step: int, n: int) -> np.ndarray:
    """Tokens of block ``step`` of a [B,H,N,d] array, as a contiguous copy."""
    return np.ascontiguousarray(x[:, :, step * n:(step + 1) * n, :])


# ---------------------------------------------------------------------------
# the causal temporal convolution of the Mix-FFN (block-boundary cache)
# ---------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class ConvConfig:
    """X [B, T, P, C]: T = nb * F latent frames in blocks of F, P = grid_h *
    grid_w positions, C channels (C fastest)."""
    name: str
    B: int
    nb: int
    F: int
    grid_h: int
    grid_w: int
    C: int
    dtype: str
    seed: int
    streaming: bool = False
    description: str = ""

    @property
    def T(self) -> int:
        return self.nb * self.F

    @property
    def P(self) -> int:
        return self.grid_h * self.grid_w


# C = 2240 is the model width of the attention workloads above (70 heads x 32)
CONV_CONFIGS = {
    "t1": ConvConfig("t1", B=1, nb=2, F=2, grid_h=3, grid_w=4, C=24, dtype="f32", seed=11,
                     description="tiny fp32 parity case, 2 blocks of 2 frames x 3x4, 24 channels"),
    "t3": ConvConfig("t3", B=1, nb=7, F=3, grid_h=22, grid_w=40, C=2240, dtype="bf16", seed=13,
                     description="720p 5 s one call, 7 blocks of 3 frames x 22x40, 2240 channels"),
    "t4": ConvConfig("t4", B=1, nb=80, F=3, grid_h=15, grid_w=26, C=2240, dtype="bf16", seed=14,
                     streaming=True,
                     description="minute-long 480p stream, 80 steps of 3 frames x 15x26, 2240 channels"),
}


def make_conv_inputs(cfg: ConvConfig, seed: Optional[int] = None, *, B=None, nb=None, F=None,
                     P=None, C=None) -> dict:
    """Draw X ~ N(0,1) [B, T, P, C] (bf16-exact for bf16 configs; raw bits in
    X_bits), depthwise taps w [C, 3] ~ N(0, 1/3) and bias [C] ~ N(0, 0.01) as
    fp32, and a cache frame [B, P, C] ~ N(0,1) (storage-type exact), in that
    order, from default_rng(seed)."""
    B = cfg.B if B is None else B
    nb = cfg.nb if nb is None else nb
    F = cfg.F if F is None else F
    P = cfg.P if P is None else P
    C = cfg.C if C is None else C
    T = nb * F
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    out = {"cfg": cfg, "B": B, "nb": nb, "F": F, "T": T, "P": P, "C": C, "dtype": cfg.dtype}
    x = rng.standard_normal((B, T, P, C), dtype=np.float32)
    w = (rng.standard_normal((C, 3)) / np.sqrt(3.0)).astype(np.float32)
    bias = (rng.standard_normal(C) * 0.1).astype(np.float32)
    cache = rng.standard_normal((B, P, C), dtype=np.float32)
    if cfg.dtype == "bf16":
        out["X_bits"] = bf16_bits(x)
        out["X"] = bf16_from_bits(out["X_bits"])
        out["cache_bits"] = bf16_bits(cache)
        out["cache"] = bf16_from_bits(out["cache_bits"])
    else:
        out["X"], out["cache"] = x, cache
    out["w"], out["bias"] = w, bias
    return out
