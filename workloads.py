"""Seeded synthetic workloads for the smoothed W8A8 linear layer.

This module only draws random numbers. It holds none of the method's
arithmetic (no maxima, no smoothing factors, no quantization), so both the
oracle and the HIP path can take their inputs from here without sharing any
computation.

Shapes and value structure follow the pages:
  * X is tokens x input channels and W is input channels x output channels
    ("Move activation scale without changing the real linear map", para. 1).
  * Activation outliers sit in a handful of fixed channels ("Quantization",
    learn-kernels.com, para. 2); down-projection layers carry massive
    token-specific outliers on a small channel set (Pith review of arXiv
    2506.01967, one-line summary and referee major comment 3).
  * Calibration statistics come from a small representative set (SmoothQuant
    glossary entry, "What calibration data does SmoothQuant need?"); the held-out
    split follows the Pith skeptic's concrete test.

The LLaMA2-7B activations recorded on WikiText-2 in the Pith review are not
available here; these draws stand in for them with the same shapes (hidden
4096, down_proj 11008) and outlier structure.

Recipe (fixed per workload, all draws float64 from numpy's PCG64
``default_rng(seed)``, then cast to float16 with round-half-even):
  1. outlier channels: sorted ``rng.choice(K, n_ch, replace=False)`` (or a
     fixed list, drawn from nothing)
  2. per-channel factors (constant, or ``rng.uniform(lo, hi, n_ch)``)
  3. outlier tokens of X, then of X_cal (only for token-specific outliers)
  4. X ~ N(0, 1), M x K, drawn row-chunk by row-chunk
  5. X_cal ~ N(0, 1), T x K (skipped when calibrating in-sample)
  6. each consumer's W ~ N(0, sigma^2), K x N_i, in consumer order
Counts are rounded to the nearest integer (1% of 4096 -> 41, 0.5% of 8192 ->
41, 2% of 2048 -> 41, 2% of 512 -> 10).
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import List, Optional, Tuple

import numpy as np

_CHUNK_ROWS = 1024


@dataclass(frozen=True)
class Workload:
    name: str
    M: int                     # tokens of the batch that is served
    K: int                     # input channels
    Ns: Tuple[int, ...]        # output channels of each consumer of X
    alpha: float
    seed: int
    sigma_w: float             # std of W
    n_outlier_ch: int
    factor: Tuple[float, float]  # (lo, hi); lo == hi means a constant factor
    token_frac: float = 0.0    # > 0: outliers only on this fraction of tokens
    T_cal: int = 512           # calibration tokens; 0 means in-sample (X itself)
    fixed_channels: Tuple[int, ...] = ()  # outlier channels named outright (no draw)
    description: str = ""

    @property
    def N(self) -> int:
        return int(sum(self.Ns))

    def with_m(self, m: int) -> "Workload":
        return replace(self, name=self.name + f"_m{m}", M=int(m))

    def with_alpha(self, a: float) -> "Workload":
        return replace(self, name=self.name + f"_a{a}", alpha=float(a))


WORKLOADS = {
    "tiny": Workload("tiny", 16, 64, (64,), 0.5, 0, 0.02, 2, (60.0, 60.0), T_cal=0,
                     fixed_channels=(3, 41),
                     description="16x64x64, channels {3,41} x60, in-sample calibration"),
    "qkv4096": Workload("qkv4096", 2048, 4096, (4096,), 0.5, 2, 0.02, 41, (50.0, 100.0),
                        description="LLaMA-7B q/k/v-style 2048x4096x4096, 1% channels x U(50,100)"),
    "down11008": Workload("down11008", 2048, 11008, (4096,), 0.5, 3, 0.02, 4, (1000.0, 1000.0),
                          token_frac=0.02,
                          description="LLaMA-7B down_proj-style 2048x11008x4096, 4 channels x1000 on 2% of tokens"),
    "decode8192": Workload("decode8192", 16, 8192, (28672,), 0.5, 4, 0.02, 82, (80.0, 80.0),
                           description="decode M in {1,4,16} x 8192 x 28672, 1% channels x80"),
    "prefill8192x3": Workload("prefill8192x3", 8192, 8192, (8192, 8192, 8192), 0.5, 5, 0.015, 41,
                              (100.0, 100.0),
                              description="8192x8192 shared X feeding three 8192x8192 projections, 0.5% channels x100"),
    # The Smooth Rotation study needs a power-of-two width (the Sylvester
    # matrix); this is the down_proj outlier structure at d = 4096.
    "massive4096": Workload("massive4096", 2048, 4096, (4096,), 0.5, 6, 0.02, 4, (1000.0, 1000.0),
                            token_frac=0.02,
                            description="down_proj-style 2048x4096x4096, 4 channels x1000 on 2% of tokens"),
}


@dataclass
class Inputs:
    x: np.ndarray            # float16 [M][K]
    x_cal: np.ndarray        # float16 [T][K] (the same array as x when in-sample)
    ws: List[np.ndarray]     # float16 [K][N_i] per consumer
    outlier_channels: np.ndarray
    outlier_tokens: Optional[np.ndarray]
    outlier_tokens_cal: Optional[np.ndarray]

    @property
    def w(self) -> np.ndarray:
        """All consumers' weights concatenated along the output channels (K x sum N_i)."""
        return self.ws[0] if len(self.ws) == 1 else np.concatenate(self.ws, axis=1)


def _normal_f16(rng: np.random.Generator, rows: int, cols: int, scale: float = 1.0) -> np.ndarray:
    """rows x cols float16 draws of N(0, scale^2), drawn in row chunks of float64.

    Drawing in chunks consumes the generator exactly as one large draw would,
    but keeps the float64 staging buffer small.
    """
    out = np.empty((rows, cols), dtype=np.float16)
    for r0 in range(0, rows, _CHUNK_ROWS):
        r1 = min(rows, r0 + _CHUNK_ROWS)
        blk = rng.standard_normal((r1 - r0, cols))
        if scale != 1.0:
            blk *= scale
        out[r0:r1] = blk.astype(np.float16)
    return out


def generate(wl: Workload, m: Optional[int] = None, with_w: bool = True) -> Inputs:
    """Draws the inputs of workload ``wl`` (optionally with a different token count m)."""
    M = wl.M if m is None else int(m)
    rng = np.random.default_rng(wl.seed)
    if wl.fixed_channels:
        ch = np.array(wl.fixed_channels, dtype=np.int64)
    else:
        ch = np.sort(rng.choice(wl.K, wl.n_outlier_ch, replace=False))
    lo, hi = wl.factor
    fac = np.full(wl.n_outlier_ch, lo) if lo == hi else rng.uniform(lo, hi, wl.n_outlier_ch)
    tok = tok_cal = None
    if wl.token_frac > 0:
        tok = np.sort(rng.choice(M, max(1, int(round(wl.token_frac * M))), replace=False))
        if wl.T_cal > 0:
            tok_cal = np.sort(rng.choice(wl.T_cal, max(1, int(round(wl.token_frac * wl.T_cal))),
                                         replace=False))
    # Raw N(0,1) draws are staged in float64 and rounded once after the outlier factor.
    x64 = rng.standard_normal((M, wl.K))
    rows = np.arange(M) if tok is None else tok
    x64[np.ix_(rows, ch)] *= fac[None, :]
    x = x64.astype(np.float16)
    del x64
    if wl.T_cal > 0:
        c64 = rng.standard_normal((wl.T_cal, wl.K))
        rows = np.arange(wl.T_cal) if tok_cal is None else tok_cal
        c64[np.ix_(rows, ch)] *= fac[None, :]
        x_cal = c64.astype(np.float16)
        del c64
    else:
        x_cal = x
    ws = []
    if with_w:
        for n in wl.Ns:
            ws.append(_normal_f16(rng, wl.K, n, wl.sigma_w))
    return Inputs(x, x_cal, ws, ch, tok, tok_cal)


def random_f16(seed: int, rows: int, cols: int, scale: float = 1.0) -> np.ndarray:
    """Plain N(0, scale^2) float16 matrix, for ragged-shape and edge-case tests."""
    return _normal_f16(np.random.default_rng(seed), rows, cols, scale)


def random_i8(seed: int, rows: int, cols: int, lo: int = -127, hi: int = 127) -> np.ndarray:
    """Uniform int8 codes in [lo, hi], for direct GEMM tests."""
    return np.random.default_rng(seed).integers(lo, hi + 1, size=(rows, cols), dtype=np.int64).astype(np.int8)


def random_scales(seed: int, n: int, lo: float = 1e-3, hi: float = 1e-1) -> np.ndarray:
    """Positive float32 scales, for direct GEMM epilogue tests."""
    return np.random.default_rng(seed).uniform(lo, hi, n).astype(np.float32)


# ---- inputs of the normalization in front of the layer --------------------
#
# The fold of S^-1 into a preceding RMS normalization takes the hidden state h
# (the normalization's input) instead of X.  Recipe: h is the workload's X
# draw itself (same outlier channels and factors), the normalization weight
# gamma is drawn from U(0.5, 1.5) by its own generator (seed + 1000, so the
# draws above are unchanged) and rounded to float16; eps is the common 1e-5.
NORM_EPS = 1e-5


def norm_weight(wl: Workload) -> np.ndarray:
    """float16 [K] weight of the normalization in front of workload wl."""
    rng = np.random.default_rng(wl.seed + 1000)
    return rng.uniform(0.5, 1.5, wl.K).astype(np.float16)
