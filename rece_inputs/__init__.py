"""Seeded synthetic workloads for the RECE / SCE reduced cross-entropy loss.

This module is shared by the CPU oracle (``oracle/``), the tests and ``bench.py``.
It holds none of the loss's arithmetic: it only draws the inputs (hidden states X,
item table Y, positive ids, random projections B) and rounds them to the input
dtype.  The random projections that RECE draws inside the loss (RECE page,
Algorithm 1, the randn step) are drawn here and passed in, so that the oracle and
the GPU path see identical B.

Recipe (one ``numpy.random.SeedSequence(seed)`` per workload, spawned into six
independent streams: X, Y, B, item permutation, positives, spare):

* X[s, d] and Y[C, d] ~ N(0, variance 1/sqrt(d)), drawn in float64 row-major,
  rounded once to the input dtype (round-to-nearest-even; bf16 straight from
  float64, no double rounding).  Logits x.y then have unit variance.
* B[r, d, n_b] ~ N(0, 1), rounded the same way (one independent slice per round).
* positives: uniform on [0, C) or a finite-support Zipf(alpha) over ranks 1..C
  (p(rank) proportional to rank**-alpha, inverse-CDF sampling), mapped through a
  seeded permutation pi of the catalogue: item = pi[rank - 1].
* optional popular-item boost: the rows pi[0 : C // 100] of Y (the most popular
  items) are multiplied by a factor before rounding.
* positions are flattened sequence-major (sequence 0's positions first); no padding.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, loss hyper-parameters and input recipe."""

    name: str
    seqs: int            # number of sequences in the batch
    seqlen: int          # positions per sequence; s = seqs * seqlen
    C: int               # catalogue size
    d: int               # embedding dimension
    dtype: str           # "f32" or "bf16" for X, Y and B
    n_b: int             # random vectors (buckets) per round
    n_c: int             # chunks (RECE); unused by SCE
    k: int               # negatives kept per position (per round for RECE)
    rounds: int          # RECE rounds r
    variant: str = "rece"          # "rece" or "sce"
    b_x: int = 0                   # SCE: positions taken per bucket
    b_y: int = 0                   # SCE: items taken per bucket
    positives: str = "uniform"     # "uniform" or "zipf"
    zipf_alpha: float = 1.0
    popular_scale: float = 1.0     # factor applied to the C//100 most popular rows of Y
    seed: int = 0
    b_seed: Optional[int] = None   # separate seed for B only (None: same stream as the rest)
    n_ec: int = 1                  # RECE: neighbouring chunks on each side of a window
    window_wrap: bool = True       # RECE: window chunk indices modulo n_c (else clipped)

    @property
    def s(self) -> int:
        return self.seqs * self.seqlen

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads the loss is specified on, plus the degenerate full-CE case.
WORKLOADS = {
    "tiny": Workload("tiny", 4, 64, 2000, 64, F32, 16, 16, 32, 1,
                     positives="uniform", seed=1),
    "tiny_fullce": Workload("tiny_fullce", 4, 64, 2000, 64, F32, 1, 1, 1999, 1,
                            positives="uniform", seed=1, b_seed=101),
    "sasrec": Workload("sasrec", 256, 200, 30000, 64, BF16, 64, 64, 128, 2,
                       positives="zipf", zipf_alpha=1.1, seed=2),
    "million": Workload("million", 128, 200, 1_000_000, 64, BF16, 256, 256, 256, 2,
                        positives="zipf", zipf_alpha=1.05, popular_scale=3.0, seed=3),
    "tenmillion": Workload("tenmillion", 128, 256, 10_000_000, 128, BF16, 1024, 1024, 256, 3,
                           positives="zipf", zipf_alpha=1.0, seed=4),
    "sce": Workload("sce", 256, 256, 876_000, 256, BF16, 512, 0, 128, 1, variant="sce",
                    b_x=256, b_y=2048, positives="zipf", zipf_alpha=1.1, seed=5),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    Returns float64 values that are exactly representable in bfloat16 (8
    significant bits, 8 exponent bits).  Rounding is done once, from float64.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    # bfloat16 keeps 8 significant bits; below its normal range the spacing is 2**-133.
    e_eff = np.maximum(e, -125)
    q = np.rint(np.ldexp(x, 8 - e_eff))          # integer significand, half to even
    return np.ldexp(q, e_eff - 8)


def to_bf16_bits(x_bf16_exact: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 encodings of values that are exactly bfloat16-representable."""
    f = np.asarray(x_bf16_exact, dtype=np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


def _round_dtype(x64: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 draws to the input dtype; returns float32 arrays (exact values)."""
    if dtype == BF16:
        return round_to_bf16(x64).astype(np.float32)
    if dtype == F32:
        return x64.astype(np.float32)
    raise ValueError(f"unknown dtype {dtype}")


def _normal_rows(rng: np.random.Generator, n: int, d: int, std: float, dtype: str,
                 block_rows: int = 1 << 18) -> np.ndarray:
    """Row-major N(0, std**2) draws, rounded to dtype, produced in row blocks."""
    out = np.empty((n, d), dtype=np.float32)
    for r0 in range(0, n, block_rows):
        r1 = min(n, r0 + block_rows)
        out[r0:r1] = _round_dtype(rng.standard_normal((r1 - r0, d)) * std, dtype)
    return out


def zipf_ranks(rng: np.random.Generator, n: int, C: int, alpha: float) -> np.ndarray:
    """n draws of a rank in 1..C with P(rank) proportional to rank**-alpha."""
    ranks = np.arange(1, C + 1, dtype=np.float64)
    p = ranks ** (-alpha)
    cdf = np.cumsum(p)
    cdf /= cdf[-1]
    u = rng.random(n)
    r = np.searchsorted(cdf, u, side="right") + 1
    return np.minimum(r, C).astype(np.int64)


@dataclass
class Inputs:
    """Generated arrays.  X, Y, B hold float32 values exactly representable in the dtype."""

    w: Workload
    X: np.ndarray        # [s, d] float32
    Y: np.ndarray        # [C, d] float32
    pos: np.ndarray      # [s] int32
    B: np.ndarray        # [rounds, d, n_b] float32 (RECE) or [1, d, n_b] (SCE)
    perm: np.ndarray = field(repr=False, default=None)   # item popularity permutation pi

    def device_arrays(self):
        """Arrays in the layout the library consumes: bf16 as uint16 bits, else float32."""
        if self.w.dtype == BF16:
            return (to_bf16_bits(self.X), to_bf16_bits(self.Y), self.pos,
                    to_bf16_bits(self.B))
        return self.X, self.Y, self.pos, self.B


def make_inputs(w: Workload, seed: Optional[int] = None) -> Inputs:
    """Draw the inputs of workload ``w`` (seed defaults to ``w.seed``)."""
    seed = w.seed if seed is None else seed
    sx, sy, sb, spi, spos, _spare = np.random.SeedSequence(seed).spawn(6)
    std = float(w.d) ** -0.25            # variance 1/sqrt(d)
    s, C, d = w.s, w.C, w.d

    X = _normal_rows(np.random.default_rng(sx), s, d, std, w.dtype)

    pi = np.random.default_rng(spi).permutation(C).astype(np.int64)
    rng_y = np.random.default_rng(sy)
    if w.popular_scale != 1.0:
        popular = np.zeros(C, dtype=bool)
        popular[pi[: C // 100]] = True
        Y = np.empty((C, d), dtype=np.float32)
        block = 1 << 18
        for r0 in range(0, C, block):
            r1 = min(C, r0 + block)
            v = rng_y.standard_normal((r1 - r0, d)) * std
            v[popular[r0:r1]] *= w.popular_scale
            Y[r0:r1] = _round_dtype(v, w.dtype)
    else:
        Y = _normal_rows(rng_y, C, d, std, w.dtype)

    n_slices = w.rounds if w.variant == "rece" else 1
    b_ss = np.random.SeedSequence(w.b_seed) if w.b_seed is not None else sb
    B = _round_dtype(np.random.default_rng(b_ss).standard_normal((n_slices, d, w.n_b)), w.dtype)

    rng_pos = np.random.default_rng(spos)
    if w.positives == "uniform":
        pos = rng_pos.integers(0, C, size=s)
    elif w.positives == "zipf":
        pos = pi[zipf_ranks(rng_pos, s, C, w.zipf_alpha) - 1]
    else:
        raise ValueError(w.positives)
    return Inputs(w, X, Y, pos.astype(np.int32), B, pi)


def scaled(name: str, **overrides) -> Workload:
    """A named workload with some fields replaced (smaller test cases of the same recipe)."""
    return WORKLOADS[name].with_(**overrides)
