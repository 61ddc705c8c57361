"""CPU oracle for the SmoothQuant-smoothed W8A8 linear layer Y = (X S^-1)(S W).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark use this package; the product library never imports, links
or runs it.  It shares no code with the HIP path; the only common module is
``workloads``, which draws random inputs and holds none of the method's
arithmetic.

The quantized path (calibration statistics, smoothing factors, fold,
per-token quantization, int32 product, dequantization) is the plain C in
``sq_oracle.c``; this module marshals numpy arrays into it.  The exact-
arithmetic checks of the method (the identity, the wrong-dimension control,
the unquantized fp16 rewrite) are written here in float64 numpy.

Pages cited:
  [P1] "Move activation scale without changing the real linear map"
  [P4] Pith review of arXiv 2506.01967 ("Smooth Rotation")
  [P5] "Quantization" (learn-kernels.com)

``quant_error_report`` (layer-wise error) is pinned by hand-worked one-token
cases and by an exact-grid case with zero error; the pages print no values for
it on real layers.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import build as _build

_LIB = None

_f16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i8p = np.ctypeslib.ndpointer(dtype=np.int8, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64
_f16p1 = np.ctypeslib.ndpointer(dtype=np.uint16, ndim=1, flags="C_CONTIGUOUS")


def lib():
    """Loads the compiled oracle, building it first only if it is missing
    (SQ_ORACLE_LIB names another build of the same source, e.g. the
    sanitized one the tests run the pins against)."""
    global _LIB
    if _LIB is None:
        path = os.environ.get("SQ_ORACLE_LIB") or _build.LIB_PATH
        if not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        L.oracle_half_to_float.restype = ctypes.c_float
        L.oracle_half_to_float.argtypes = [ctypes.c_uint16]
        L.oracle_calibrate_absmax.restype = None
        L.oracle_calibrate_absmax.argtypes = [_f16p, _i64, _i64, _i64, _f32p, ctypes.c_int]
        L.oracle_row_absmax.restype = None
        L.oracle_row_absmax.argtypes = [_f16p, _i64, _i64, _i64, _f32p]
        L.oracle_smoothing_factors.restype = ctypes.c_int
        L.oracle_smoothing_factors.argtypes = [_f32p, _f32p, _i64, ctypes.c_float, _f32p, _f32p]
        L.oracle_fold_quant_weights.restype = None
        L.oracle_fold_quant_weights.argtypes = [_f16p, _i64, _i64, _i64, _f32p, _i8p, _f32p]
        L.oracle_quant_act_per_token.restype = None
        L.oracle_quant_act_per_token.argtypes = [_f16p, _i64, _i64, _i64, _f32p, _i8p, _f32p]
        L.oracle_gemm_i32.restype = ctypes.c_int64
        L.oracle_gemm_i32.argtypes = [_i8p, _i8p, _i64, _i64, _i64, _i32p]
        L.oracle_dequant.restype = None
        L.oracle_dequant.argtypes = [_i32p, _f32p, _f32p, _i64, _i64, _f64p]
        L.oracle_fold_norm_weight.restype = None
        L.oracle_fold_norm_weight.argtypes = [_f16p1, _i64, _f32p, _f32p]
        L.oracle_row_sum_squares.restype = ctypes.c_double
        L.oracle_row_sum_squares.argtypes = [_f16p1, _i64]
        L.oracle_rmsnorm_quant_per_token.restype = None
        L.oracle_rmsnorm_quant_per_token.argtypes = [_f16p, _i64, _i64, _i64, _f32p,
                                                     ctypes.c_float, _i8p, _f32p]
        L.oracle_fwht_f32.restype = None
        L.oracle_fwht_f32.argtypes = [_f32p, _i64]
        L.oracle_quant4_rows.restype = None
        L.oracle_quant4_rows.argtypes = [_f16p, _i64, _i64, _i64, _f32p, ctypes.c_int,
                                         ctypes.c_float, _i8p, _f32p, _f32p]
        L.oracle_layer.restype = None
        L.oracle_layer.argtypes = [_f16p, _i64, _i64, _i64, _f32p, _i8p, _f32p, _i64,
                                   _i8p, _f32p, _i32p, _f64p]
        _LIB = L
    return _LIB


def _bits(a: np.ndarray) -> np.ndarray:
    assert a.dtype == np.float16 and a.ndim == 2
    return np.ascontiguousarray(a).view(np.uint16)


def half_to_float(h: int) -> float:
    return float(lib().oracle_half_to_float(int(h)))


# ---- quantized path (C) ----------------------------------------------------

def calibrate_absmax(x_cal: np.ndarray, ax: Optional[np.ndarray] = None) -> np.ndarray:
    """A1: per-input-channel max |X| over calibration tokens; with ``ax`` given,
    the running maximum continues from it ([P4] key machinery: max|X_j|)."""
    T, K = x_cal.shape
    out = np.zeros(K, np.float32) if ax is None else np.array(ax, np.float32, copy=True)
    lib().oracle_calibrate_absmax(_bits(x_cal), T, K, K, out, 0 if ax is None else 1)
    return out


def row_absmax(w: np.ndarray) -> np.ndarray:
    """A2 (weights): max |W[j, :]| of each input channel j."""
    K, N = w.shape
    out = np.empty(K, np.float32)
    lib().oracle_row_absmax(_bits(w), K, N, N, out)
    return out


def smoothing_factors(ax: np.ndarray, aw: np.ndarray, alpha: float):
    """A2: s_j = ax_j^alpha / aw_j^(1-alpha) in double, rounded to float; returns (s, inv_s, status)."""
    K = ax.shape[0]
    s = np.empty(K, np.float32)
    inv = np.empty(K, np.float32)
    st = lib().oracle_smoothing_factors(np.ascontiguousarray(ax, np.float32),
                                        np.ascontiguousarray(aw, np.float32), K,
                                        float(alpha), s, inv)
    return s, inv, int(st)


def fold_quant_weights(w: np.ndarray, s: np.ndarray):
    """A3: Wq [N][K] int8 and per-output-channel scales of (S W)."""
    K, N = w.shape
    wq = np.empty((N, K), np.int8)
    ws = np.empty(N, np.float32)
    lib().oracle_fold_quant_weights(_bits(w), K, N, N, np.ascontiguousarray(s, np.float32), wq, ws)
    return wq, ws


def quant_act_per_token(x: np.ndarray, inv_s: np.ndarray):
    """A4: Xq [M][K] int8 and per-token scales of (X S^-1)."""
    M, K = x.shape
    xq = np.empty((M, K), np.int8)
    xs = np.empty(M, np.float32)
    lib().oracle_quant_act_per_token(_bits(x), M, K, K, np.ascontiguousarray(inv_s, np.float32), xq, xs)
    return xq, xs


def gemm_i32(xq: np.ndarray, wq: np.ndarray) -> np.ndarray:
    """A5: int32 acc[m][n] = sum_j Xq[m][j] Wq[n][j]."""
    M, K = xq.shape
    N, K2 = wq.shape
    assert K == K2
    acc = np.empty((M, N), np.int32)
    ovf = lib().oracle_gemm_i32(np.ascontiguousarray(xq), np.ascontiguousarray(wq), M, N, K, acc)
    assert ovf == 0, "int32 accumulator overflow"
    return acc


def dequant(acc: np.ndarray, x_scale: np.ndarray, w_scale: np.ndarray) -> np.ndarray:
    """A6: acc * x_scale[m] * w_scale[n] in float64."""
    M, N = acc.shape
    y = np.empty((M, N), np.float64)
    lib().oracle_dequant(np.ascontiguousarray(acc), np.ascontiguousarray(x_scale, np.float32),
                         np.ascontiguousarray(w_scale, np.float32), M, N, y)
    return y


def to_f16(y: np.ndarray) -> np.ndarray:
    """Rounds float64 values once to float16 (numpy's round-half-even conversion)."""
    return np.asarray(y, np.float64).astype(np.float16)


def layer_block(x: np.ndarray, inv_s: np.ndarray, wq: np.ndarray, w_scale: np.ndarray) -> np.ndarray:
    """A4+A5+A6 in one C call on a block of tokens (the CPU-baseline unit); float64 y."""
    M, K = x.shape
    N = wq.shape[0]
    xq = np.empty((M, K), np.int8)
    xs = np.empty(M, np.float32)
    acc = np.empty((M, N), np.int32)
    y = np.empty((M, N), np.float64)
    lib().oracle_layer(_bits(x), M, K, K, np.ascontiguousarray(inv_s, np.float32),
                       np.ascontiguousarray(wq), np.ascontiguousarray(w_scale, np.float32), N,
                       xq, xs, acc, y)
    return y


# ---- next row: S^-1 folded into the preceding RMS normalization (C) ---------

def fold_norm_weight(gamma: np.ndarray, inv_s: np.ndarray) -> np.ndarray:
    """g_j = float(gamma_j) * inv_s_j: the normalization's weight divided by the
    smoothing factor, so that its output is already X S^-1 ([P1 para. 3])."""
    gb = np.ascontiguousarray(np.asarray(gamma, np.float16)).view(np.uint16)
    K = gb.shape[0]
    g = np.empty(K, np.float32)
    lib().oracle_fold_norm_weight(gb, K, np.ascontiguousarray(inv_s, np.float32), g)
    return g


def row_sum_squares(h_row: np.ndarray) -> float:
    """sum_j h_j^2 of one fp16 row, exact and rounded once to double."""
    hb = np.ascontiguousarray(np.asarray(h_row, np.float16)).view(np.uint16)
    return float(lib().oracle_row_sum_squares(hb, hb.shape[0]))


def rmsnorm_quant_per_token(h: np.ndarray, g: np.ndarray, eps: float):
    """RMS normalization with the folded weight g and per-token int8
    quantization in one step: Xq [M][K] int8 and x_scale [M]."""
    M, K = h.shape
    xq = np.empty((M, K), np.int8)
    xs = np.empty(M, np.float32)
    lib().oracle_rmsnorm_quant_per_token(_bits(h), M, K, K, np.ascontiguousarray(g, np.float32),
                                         float(eps), xq, xs)
    return xq, xs


# ---- next row: Smooth Rotation at 4 bits ([P4]) (C) ---------------------------

def fwht_f32(v: np.ndarray) -> np.ndarray:
    """v H_d (unnormalized Sylvester Hadamard) by the fast transform in float,
    strides 1, 2, 4, ... in that order; returns a new float32 vector."""
    out = np.array(v, np.float32, copy=True)
    d = out.shape[0]
    assert d & (d - 1) == 0, "d must be a power of two"
    lib().oracle_fwht_f32(out, d)
    return out


def quant4_rows(x: np.ndarray, mult: np.ndarray, rotate: bool, post: float = 1.0):
    """4-bit symmetric round-to-nearest quantization of the rows of x (fp16)
    times mult, rotated by H first when asked: (codes int8 [M][K], scale [M])."""
    M, K = x.shape
    if rotate:
        assert K & (K - 1) == 0
    q = np.empty((M, K), np.int8)
    sc = np.empty(M, np.float32)
    work = np.empty(K, np.float32)
    lib().oracle_quant4_rows(_bits(x), M, K, K, np.ascontiguousarray(mult, np.float32),
                             1 if rotate else 0, float(post), q, sc, work)
    return q, sc


def quant4_act_per_token(x: np.ndarray, inv_s: np.ndarray, rotate: bool):
    """A4 at 4 bits: per-token codes in [-7, 7] of (x * inv_s) H (or of x * inv_s)."""
    return quant4_rows(x, inv_s, rotate, 1.0)


def fold4_weights(w: np.ndarray, s: np.ndarray, rotate: bool):
    """A3 at 4 bits: per-output-channel codes [N][K] in [-7, 7] of H (s * W)
    (or of s * W); with the rotation the scale carries the 1/d of the two
    unnormalized transforms."""
    K = w.shape[0]
    return quant4_rows(np.ascontiguousarray(w.T), s, rotate, 1.0 / K if rotate else 1.0)


def hadamard_fp64(d: int) -> np.ndarray:
    """Sylvester H_d in float64, H[i][j] = (-1)^popcount(i & j)."""
    i = np.arange(d)
    bits = np.bitwise_and(i[:, None], i[None, :])
    pop = np.zeros_like(bits)
    while bits.any():
        pop += bits & 1
        bits >>= 1
    return np.where(pop % 2 == 0, 1.0, -1.0)


@dataclass
class Chain:
    ax: np.ndarray
    aw: np.ndarray
    s: np.ndarray
    inv_s: np.ndarray
    status: int
    wq: np.ndarray
    w_scale: np.ndarray
    xq: np.ndarray
    x_scale: np.ndarray
    acc: Optional[np.ndarray]
    y64: Optional[np.ndarray]

    @property
    def y16(self) -> np.ndarray:
        return to_f16(self.y64)


def smoothed_linear(x: np.ndarray, x_cal: np.ndarray, w: np.ndarray, alpha: float,
                    rows: Optional[np.ndarray] = None) -> Chain:
    """The whole chain A1..A6.  ``rows`` restricts A5/A6 to a subset of tokens
    (A4 still quantizes every token)."""
    ax = calibrate_absmax(x_cal)
    aw = row_absmax(w)
    s, inv_s, st = smoothing_factors(ax, aw, alpha)
    wq, wsc = fold_quant_weights(w, s)
    xq, xsc = quant_act_per_token(x, inv_s)
    sel = slice(None) if rows is None else rows
    acc = gemm_i32(np.ascontiguousarray(xq[sel]), wq)
    y = dequant(acc, xsc[sel], wsc)
    return Chain(ax, aw, s, inv_s, st, wq, wsc, xq, xsc, acc, y)


# ---- exact-arithmetic checks of the method (float64 numpy) -----------------

def matmul_fp64(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Y = X W in float64 (the unsmoothed reference)."""
    return np.asarray(x, np.float64) @ np.asarray(w, np.float64)


def smoothed_matmul_fp64(x: np.ndarray, w: np.ndarray, s: np.ndarray) -> np.ndarray:
    """(X S^-1)(S W) in float64: column j of X divided by s_j, row j of W
    multiplied by s_j ([P1 para. 1])."""
    s64 = np.asarray(s, np.float64)
    xs = np.asarray(x, np.float64) / s64[None, :]
    ws = np.asarray(w, np.float64) * s64[:, None]
    return xs @ ws


def rmsnorm_fp64(h: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """The unfused normalization output h / sqrt(mean_j h^2 + eps) * gamma in
    float64 (what the layer's X is before smoothing)."""
    h64 = np.asarray(h, np.float64)
    rstd = 1.0 / np.sqrt(np.mean(h64 * h64, axis=1) + float(eps))
    return h64 * rstd[:, None] * np.asarray(gamma, np.float64)[None, :]


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    """||a - b||_F / ||b||_F."""
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / np.linalg.norm(b))


def unquantized_fp16_rewrite(x: np.ndarray, w: np.ndarray, s: np.ndarray, inv_s: np.ndarray):
    """The check the pages ask for before quantizing ([P1 para. 5]): the
    smoothed operands stored in fp16, X~ = fp16(float(X) * inv_s) and
    W~ = fp16(float(W) * s), multiplied in float64.  Returns (Y_s, ok), where
    ok is False when a smoothed value does not fit fp16 (representability,
    [P1 paras. 1 and 5])."""
    xt = np.asarray(x, np.float32) * np.asarray(inv_s, np.float32)[None, :]
    wt = np.asarray(w, np.float32) * np.asarray(s, np.float32)[:, None]
    with np.errstate(over="ignore"):
        xt16 = xt.astype(np.float16)
        wt16 = wt.astype(np.float16)
    ok = bool(np.isfinite(xt16).all() and np.isfinite(wt16).all())
    return xt16.astype(np.float64) @ wt16.astype(np.float64), ok


def quant_error_report(x: np.ndarray, x_cal: np.ndarray, w: np.ndarray, alpha: Optional[float]):
    """Layer-wise squared-Frobenius error ||Y_q - XW||^2 / ||XW||^2 of the W8A8
    layer, smoothed with strength alpha, or unsmoothed (S = I) for None
    ([P4] core discovery measures this quantity).  The pages print no values
    for it; tests pin it on hand-worked one-token cases (S = I and alpha = 0,
    1/2, 1) and on inputs on the int8 grid, where it is exactly 0."""
    ref = matmul_fp64(x, w)
    if alpha is None:
        K = x.shape[1]
        s = np.ones(K, np.float32)
        inv = np.ones(K, np.float32)
    else:
        s, inv, st = smoothing_factors(calibrate_absmax(x_cal), row_absmax(w), alpha)
        assert st == 0
    wq, wsc = fold_quant_weights(w, s)
    xq, xsc = quant_act_per_token(x, inv)
    y = dequant(gemm_i32(xq, wq), xsc, wsc)
    return float(np.sum((y - ref) ** 2) / np.sum(ref ** 2))
