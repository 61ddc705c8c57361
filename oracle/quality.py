"""Quality measures of the smoothed W8A8 layer, for the alpha sweep.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle``): the tests use these
to score the layer; the product library never imports them.

What is measured, and where the pages speak of it:
  * layer error ||Y_q - XW||_F^2 / ||XW||_F^2 -- the layer-wise squared
    Frobenius quantization error ([P4] core discovery);
  * quantization difficulty -- the standard deviation of the channel
    magnitudes ([P4] key machinery: the secondary device), taken for the
    activations X S^-1 (magnitude of input channel j = max over tokens) and
    for the weights S W (magnitude of input channel j = max over outputs),
    the axis along which smoothing moves the difficulty ([P1] para. 2);
  * weight reconstruction error ||S W - dequant(Wq)||_F^2 / ||S W||_F^2 of
    the per-output-channel int8 weights;
  * activation clipping under a static per-tensor scale fixed on the
    calibration tokens: the share of entries of X S^-1 above the largest
    calibration magnitude (the per-token dynamic scale never clips);
  * in-sample versus held-out calibration ([P4] skeptic critique, concrete
    test): the factors from the evaluated tokens themselves or from a
    separate calibration draw.
Readings: the magnitudes use the same float32 products as the quantizer
(x * inv_s_j, W * s_j); the statistics are taken in float64; the standard
deviation is the population one (divide by the channel count).
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from . import (calibrate_absmax, dequant, fold_quant_weights, gemm_i32, matmul_fp64,
               quant_act_per_token, row_absmax, smoothing_factors, to_f16)


def scaled_activations(x: np.ndarray, inv_s: np.ndarray) -> np.ndarray:
    """float32(x) * inv_s_j, one float32 product per entry (the quantizer's x~)."""
    return x.astype(np.float32) * inv_s.astype(np.float32)[None, :]


def scaled_weights(w: np.ndarray, s: np.ndarray) -> np.ndarray:
    """float32(W[j, n]) * s_j, one float32 product per entry (the fold's W~)."""
    return w.astype(np.float32) * s.astype(np.float32)[:, None]


def difficulty(magnitudes: np.ndarray) -> float:
    """Population standard deviation of the channel magnitudes, in float64."""
    m = np.asarray(magnitudes, np.float64)
    return float(np.sqrt(np.mean((m - m.mean()) ** 2)))


def activation_difficulty(x: np.ndarray, inv_s: np.ndarray) -> float:
    return difficulty(np.abs(scaled_activations(x, inv_s)).max(axis=0))


def weight_difficulty(w: np.ndarray, s: np.ndarray) -> float:
    return difficulty(np.abs(scaled_weights(w, s)).max(axis=1))


def weight_recon_error(w: np.ndarray, s: np.ndarray, wq: Optional[np.ndarray] = None,
                       w_scale: Optional[np.ndarray] = None) -> float:
    """||W~ - q * dw||_F^2 / ||W~||_F^2 with W~ = W * s, codes q[n][j] and
    scales dw[n] (from the oracle's fold unless given)."""
    if wq is None or w_scale is None:
        wq, w_scale = fold_quant_weights(w, s)
    wt = scaled_weights(w, s).astype(np.float64)
    rec = (wq.astype(np.float64) * w_scale.astype(np.float64)[:, None]).T   # [K][N]
    return float(np.sum((wt - rec) ** 2) / np.sum(wt ** 2))


def static_clip_fraction(x: np.ndarray, x_cal: np.ndarray, inv_s: np.ndarray) -> float:
    """Share of entries of x~ whose magnitude exceeds the largest magnitude of
    the calibration tokens' x~ (one static scale for the whole tensor)."""
    bound = np.abs(scaled_activations(x_cal, inv_s)).max()
    return float(np.mean(np.abs(scaled_activations(x, inv_s)) > bound))


def layer_error(y: np.ndarray, ref: np.ndarray) -> float:
    """||y - ref||_F^2 / ||ref||_F^2 in float64."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.sum((y - ref) ** 2) / np.sum(ref ** 2))


def factors(x_stat: np.ndarray, w: np.ndarray, alpha: Optional[float]):
    """(s, inv_s) from the statistics of x_stat, or ones for alpha None (S = I)."""
    K = w.shape[0]
    if alpha is None:
        one = np.ones(K, np.float32)
        return one, one.copy()
    s, inv, st = smoothing_factors(calibrate_absmax(x_stat), row_absmax(w), alpha)
    assert st == 0
    return s, inv


def sweep(x: np.ndarray, x_cal: np.ndarray, w: np.ndarray, alphas: Sequence[Optional[float]],
          rows: Optional[np.ndarray] = None) -> Dict[str, Dict[str, float]]:
    """Every measure for each alpha (None: S = I), with held-out calibration
    (x_cal) and in-sample calibration (x itself).  The layer error compares
    the layer's fp16 output on the token rows `rows` (all if None) with the
    float64 product XW."""
    rows = np.arange(x.shape[0]) if rows is None else np.asarray(rows)
    ref = matmul_fp64(x[rows], w)
    out: Dict[str, Dict[str, float]] = {}
    for alpha in alphas:
        for tag, stat in (("held_out", x_cal), ("in_sample", x)):
            s, inv = factors(stat, w, alpha)
            wq, wsc = fold_quant_weights(w, s)
            xq, xsc = quant_act_per_token(x[rows], inv)
            y = to_f16(dequant(gemm_i32(xq, wq), xsc, wsc))   # the layer's fp16 output
            key = f"{'I' if alpha is None else alpha}/{tag}"
            out[key] = {
                "layer_error": layer_error(y, ref),
                "weight_recon_error": weight_recon_error(w, s, wq, wsc),
                "act_difficulty": activation_difficulty(x, inv),
                "weight_difficulty": weight_difficulty(w, s),
                "static_clip_fraction": static_clip_fraction(x, x_cal, inv),
            }
    return out


# ---- Smooth Rotation at 4 bits: the comparison of [P4] core discovery ---------

W4A4_METHODS = {            # name: (smoothing strength or None for S = I, rotate)
    "original": (None, False),
    "smooth": (0.5, False),
    "rotate": (None, True),
    "smooth_rotate": (0.5, True),
}


def w4a4_layer(x: np.ndarray, w: np.ndarray, s: np.ndarray, inv_s: np.ndarray, rotate: bool,
               rows: np.ndarray):
    """The 4-bit layer on token rows `rows`: per-token codes of (x / s) [H],
    per-output-channel codes of [H] (s W), int32 product, fp16 output.
    Returns (y16 as float64, activation scales)."""
    from . import fold4_weights, quant4_act_per_token
    xq, xs = quant4_act_per_token(x[rows], inv_s, rotate)
    wq, ws = fold4_weights(w, s, rotate)
    y = to_f16(dequant(gemm_i32(xq, wq), xs, ws)).astype(np.float64)
    return y, xs


def act_step(x_scale: np.ndarray, d: int, rotate: bool) -> float:
    """Mean activation step size in the orthonormal convention.  The 4-bit
    quantizer's scale is max|v| / 7 of v = (x / s) H with the unnormalized H,
    whose entries are +-1; the rotation of [P4] key machinery is R = H / sqrt(d)
    (entries +-1/sqrt(d)), so the step of (x / s) R is scale / sqrt(d).
    Unrotated, the step is the scale itself."""
    step = np.asarray(x_scale, np.float64) / (np.sqrt(d) if rotate else 1.0)
    return float(np.mean(step))


def w4a4_compare(x: np.ndarray, x_cal: np.ndarray, w: np.ndarray,
                 rows: Optional[np.ndarray] = None) -> Dict[str, Dict[str, float]]:
    """Original, smoothing alone (alpha 1/2), rotation alone and smoothing then
    rotation, each at 4 bits on both operands, with held-out (x_cal) and
    in-sample (x) smoothing statistics ([P4] core discovery; skeptic's
    concrete test).  Measures: layer error of the fp16 output against the
    float64 XW, and the mean activation step size in the orthonormal
    convention (scale / sqrt(d) when rotated, since the transform here is
    unnormalized)."""
    rows = np.arange(x.shape[0]) if rows is None else np.asarray(rows)
    ref = matmul_fp64(x[rows], w)
    d = x.shape[1]
    out: Dict[str, Dict[str, float]] = {}
    for name, (alpha, rot) in W4A4_METHODS.items():
        for tag, stat in (("held_out", x_cal), ("in_sample", x)):
            if alpha is None and tag == "in_sample":
                continue        # no statistics involved
            s, inv = factors(stat, w, alpha)
            y, xs = w4a4_layer(x, w, s, inv, rot, rows)
            out[f"{name}/{tag}"] = {"layer_error": layer_error(y, ref),
                                    "act_step": act_step(xs, d, rot)}
    return out
