"""Seeded synthetic workloads for fused linear cross-entropy.

This module only draws inputs: the configuration table, seeded random
streams, round-to-nearest-even quantisation of the drawn values to the
storage type, targets and prompt masks.  It holds none of the loss
arithmetic, so both the CPU oracle and the GPU library can be fed from it
without sharing any code of the method itself.

Shapes follow the workloads the pages discuss: the per-rank shape of the
long-sequence write-up (65,536 local tokens, 124,160 vocab columns after a
two-way vocab split; "Long-Sequence MoE RL Training: From First Principles
to MI300X", section 3, and the Megatron-Lite / bumblebee write-up, section
2.3 step 1), plus smaller and longer cases of the same family.

Input recipe (all seeded, no dataset):
  * H ~ N(0, 1) drawn in float32, W ~ N(0, sigma_w^2) drawn in float32; for
    bf16 configs both are rounded to bf16 by round-to-nearest-even.
  * targets uniform on [0, V) or truncated Zipf(s) over ranks 1..V with
    id = rank - 1 (no permutation).
  * prompt masking: contiguous prefixes of each sequence set to
    ignore_index.
  * seeds: numpy SeedSequence(1234 + config_index).spawn(5) gives the
    streams for H, W, targets, mask and the parity row sample.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

IGNORE_INDEX = -100

DTYPE_F32 = "f32"
DTYPE_BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    T: int
    d: int
    V: int
    dtype: str                 # "f32" or "bf16": storage and input precision
    sigma_w: float
    targets: str               # "uniform" or "zipf"
    zipf_s: float = 1.1
    # prompt masking: n_seq sequences of T // n_seq tokens, the first
    # `masked_prefix` tokens of each set to IGNORE_INDEX
    n_seq: int = 1
    masked_prefix: int = 0
    reduction: str = "none"    # "none", "mean" (over T) or "mean_valid"
    seed_base: int = 1234

    @property
    def index(self) -> int:
        return CONFIGS.index(self)

    @property
    def n_ignored(self) -> int:
        return self.n_seq * self.masked_prefix

    @property
    def n_valid(self) -> int:
        return self.T - self.n_ignored

    def scales(self) -> tuple[float, float]:
        """(loss scale, grad scale) of the reduction.

        "mean" divides by T, "mean_valid" by the number of non-ignored
        tokens, "none" keeps per-token values (scale 1)."""
        if self.reduction == "mean":
            s = 1.0 / self.T
        elif self.reduction == "mean_valid":
            s = 1.0 / max(self.n_valid, 1)
        else:
            s = 1.0
        return s, s

    def counted_flops(self) -> int:
        """Forward 2*T*d*V plus backward 6*T*d*V (recompute included)."""
        return 8 * self.T * self.d * self.V


CONFIGS = [
    Config("tiny_f32_T256_d128_V1000", 256, 128, 1000, DTYPE_F32, 0.02, "uniform"),
    Config("small_bf16_T4096_d2048_V32000", 4096, 2048, 32000, DTYPE_BF16, 0.02, "uniform",
           reduction="mean"),
    Config("mid_bf16_T16384_d2048_V151936", 16384, 2048, 151936, DTYPE_BF16, 0.02, "zipf",
           n_seq=4, masked_prefix=1024, reduction="mean_valid"),
    Config("pages_bf16_T65536_d2048_V124160", 65536, 2048, 124160, DTYPE_BF16, 0.02, "uniform"),
    Config("long_bf16_T131072_d4096_V124160", 131072, 4096, 124160, DTYPE_BF16, 0.01, "zipf",
           n_seq=1, masked_prefix=39321),
]


def config_by_index(i: int) -> Config:
    return CONFIGS[i]


# ---------------------------------------------------------------- quantisation

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even); returns uint16 bits.

    Inputs are finite draws, so NaN/Inf handling is not needed here."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


# ------------------------------------------------------------------- streams

def streams(seed: int):
    """Five independent PCG64 generators: H, W, targets, mask, row sample."""
    ss = np.random.SeedSequence(seed)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(5)]


def _normal_matrix(rng, rows: int, cols: int, sigma: float, dtype: str,
                   chunk_rows: int = 4096) -> np.ndarray:
    """rows x cols draws of N(0, sigma^2) in float32, stored as float32 or bf16 bits."""
    out = np.empty((rows, cols), dtype=np.float32 if dtype == DTYPE_F32 else np.uint16)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        x = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        out[r0:r1] = x if dtype == DTYPE_F32 else f32_to_bf16_bits(x)
    return out


def zipf_targets(rng, n: int, V: int, s: float) -> np.ndarray:
    """Truncated Zipf over ranks 1..V, P(k) proportional to k^-s, id = k - 1."""
    w = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = rng.random(n)
    ids = np.searchsorted(cdf, u, side="right")
    return np.minimum(ids, V - 1).astype(np.int64)


def uniform_targets(rng, n: int, V: int) -> np.ndarray:
    return rng.integers(0, V, size=n, dtype=np.int64)


def prefix_mask(T: int, n_seq: int, masked_prefix: int) -> np.ndarray:
    """Boolean [T], True where the token is ignored (a prompt prefix)."""
    m = np.zeros(T, dtype=bool)
    if masked_prefix:
        L = T // n_seq
        for s in range(n_seq):
            m[s * L: s * L + masked_prefix] = True
    return m


@dataclasses.dataclass
class Inputs:
    """H [T,d], W [V,d] as float32 arrays or bf16 bit arrays (uint16), targets int64."""
    H: np.ndarray
    W: np.ndarray
    y: np.ndarray
    dtype: str
    ignore_index: int = IGNORE_INDEX

    @property
    def T(self):
        return self.H.shape[0]

    @property
    def d(self):
        return self.H.shape[1]

    @property
    def V(self):
        return self.W.shape[0]

    def H_f32(self) -> np.ndarray:
        return self.H if self.dtype == DTYPE_F32 else bf16_bits_to_f32(self.H)

    def W_f32(self) -> np.ndarray:
        return self.W if self.dtype == DTYPE_F32 else bf16_bits_to_f32(self.W)

    def rows(self, idx: np.ndarray) -> "Inputs":
        """The sub-batch of the given token rows (order kept)."""
        return Inputs(self.H[idx], self.W, self.y[idx], self.dtype, self.ignore_index)


def make_inputs(T: int, d: int, V: int, dtype: str, seed: int, sigma_w: float = 0.02,
                targets: str = "uniform", zipf_s: float = 1.1, n_seq: int = 1,
                masked_prefix: int = 0, ignore_frac: float = 0.0) -> Inputs:
    """Seeded inputs of any shape.  `ignore_frac` adds an i.i.d. Bernoulli mask."""
    gH, gW, gy, gm, _ = streams(seed)
    H = _normal_matrix(gH, T, d, 1.0, dtype)
    W = _normal_matrix(gW, V, d, sigma_w, dtype)
    if targets == "zipf":
        y = zipf_targets(gy, T, V, zipf_s)
    else:
        y = uniform_targets(gy, T, V)
    mask = prefix_mask(T, n_seq, masked_prefix)
    if ignore_frac > 0:
        mask |= gm.random(T) < ignore_frac
    y[mask] = IGNORE_INDEX
    return Inputs(H, W, y, dtype)


def config_inputs(cfg: Config | int) -> Inputs:
    if isinstance(cfg, int):
        cfg = CONFIGS[cfg]
    return make_inputs(cfg.T, cfg.d, cfg.V, cfg.dtype, cfg.seed_base + cfg.index,
                       sigma_w=cfg.sigma_w, targets=cfg.targets, zipf_s=cfg.zipf_s,
                       n_seq=cfg.n_seq, masked_prefix=cfg.masked_prefix)


def sample_rows(cfg: Config | int, n: int, T: Optional[int] = None) -> np.ndarray:
    """Seeded sample of n distinct token rows, ascending (the fifth stream)."""
    if isinstance(cfg, int):
        cfg = CONFIGS[cfg]
    T = cfg.T if T is None else T
    g = streams(cfg.seed_base + cfg.index)[4]
    return np.sort(g.choice(T, size=min(n, T), replace=False)).astype(np.int64)
