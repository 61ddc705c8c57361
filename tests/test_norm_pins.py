"""Pins of the oracle's fold of S^-1 into the preceding RMS normalization.

The oracle's normalization-plus-quantization step must agree with things
fixed outside it:
  * the exact sum of squares, against exact rational arithmetic;
  * the unfused, textbook form -- RMS-normalize h in float64, divide by s,
    quantize with the scale max/127 -- which the fused codes and scales must
    reconstruct to within half a quantization step and the scale's rounding;
  * exact invariants: doubling a token leaves its codes and (with eps = 0)
    its scale bit-identical; a constant token has codes +-127 and scale 1/127;
  * degenerate tokens (all zero, NaN, infinite);
  * the multi-consumer rule ("Move activation scale without changing the real
    linear map", para. 3): with one s shared by every consumer of the
    normalized activation, each consumer's output matches the unquantized
    layer; a consumer that does not receive the compensation is far off.
"""
from fractions import Fraction

import numpy as np
import pytest

import workloads as W


def exact_sum_squares(row16):
    tot = Fraction(0)
    for v in row16.astype(np.float64):
        f = Fraction(float(v))
        tot += f * f
    return float(tot)     # Fraction -> float rounds to nearest even


def test_row_sum_squares_is_exact(orc):
    rng = np.random.default_rng(11)
    rows = [
        np.array([1, 2, 3, 4], np.float16),
        # the largest and the smallest magnitude together: a double sum would drop the small ones
        np.array([65504.0] * 3 + [2.0 ** -24] * 5 + [-6.1e-5, 3.0e-8], np.float16),
        # every finite bit pattern class: random bits with the exponent field below 31
        (rng.integers(0, 0x7c00, 512) | (rng.integers(0, 2, 512) << 15)).astype(np.uint16)
        .view(np.float16),
        (rng.standard_normal(4096) * 30).astype(np.float16),
        np.zeros(64, np.float16),
    ]
    for r in rows:
        assert orc.row_sum_squares(r) == exact_sum_squares(r)
    # sums that need more than 53 bits: 2^-24 added to 2^30 is lost in a double sum
    r = np.array([32768.0, 2.0 ** -24], np.float16)
    want = Fraction(2 ** 30) + Fraction(1, 2 ** 48)
    assert orc.row_sum_squares(r) == float(want)
    assert np.isnan(orc.row_sum_squares(np.array([1.0, np.nan, np.inf], np.float16)))
    assert orc.row_sum_squares(np.array([1.0, -np.inf], np.float16)) == np.inf


def norm_case(name, rows=None):
    wl = W.WORKLOADS[name]
    inp = W.generate(wl)
    h = inp.x if rows is None else inp.x[rows]
    return wl, inp, h, W.norm_weight(wl)


@pytest.mark.parametrize("name,eps,scale", [("tiny", W.NORM_EPS, 1.0), ("qkv4096", W.NORM_EPS, 1.0),
                                            ("tiny", W.NORM_EPS, 1e-3), ("qkv4096", 0.0, 1.0)])
def test_fused_matches_textbook_rmsnorm(orc, name, eps, scale):
    rows = None if name == "tiny" else np.arange(0, 2048, 97)
    wl, inp, h, gamma = norm_case(name, rows)
    # scale 1e-3 puts mean(h^2) near eps, so where eps enters matters
    h = (h.astype(np.float64) * scale).astype(np.float16)
    # factors from the calibration tokens' normalized activations
    xc = orc.to_f16(orc.rmsnorm_fp64(inp.x_cal, gamma, eps))
    s, inv, st = orc.smoothing_factors(orc.calibrate_absmax(xc), orc.row_absmax(inp.w), wl.alpha)
    assert st == 0
    g = orc.fold_norm_weight(gamma, inv)
    xq, xs = orc.rmsnorm_quant_per_token(h, g, eps)
    # unfused, float64: normalize, divide by s, take the per-token scale max/127
    xbar = orc.rmsnorm_fp64(h, gamma, eps) / s.astype(np.float64)[None, :]
    want_scale = np.abs(xbar).max(axis=1) / 127.0
    # the fused scale differs only by float roundings: gamma*inv_s and h*g (3),
    # the final rounding (1), each at most 2^-24 relative
    np.testing.assert_array_less(np.abs(xs - want_scale), 2.0 ** -22 * want_scale + 1e-30)
    # every code is the unfused value divided by the scale, to within half a step
    err = np.abs(xq.astype(np.float64) * xs[:, None] - xbar)
    assert np.all(err <= xs[:, None] * (0.5 + 1e-4)), err.max()


def test_doubling_a_token_changes_nothing(orc):
    wl, inp, h, gamma = norm_case("qkv4096", np.arange(0, 64))
    inv = np.random.default_rng(3).uniform(0.05, 2.0, wl.K).astype(np.float32)
    g = orc.fold_norm_weight(gamma, inv)
    h2 = (h.astype(np.float32) * 2).astype(np.float16)
    assert np.isfinite(h2.astype(np.float32)).all()
    q1, s1 = orc.rmsnorm_quant_per_token(h, g, 0.0)
    q2, s2 = orc.rmsnorm_quant_per_token(h2, g, 0.0)
    np.testing.assert_array_equal(q1, q2)
    np.testing.assert_array_equal(s1, s2)


def test_constant_token_and_degenerate_tokens(orc):
    K = 64
    g = orc.fold_norm_weight(np.ones(K, np.float16), np.ones(K, np.float32))
    h = np.zeros((5, K), np.float16)
    h[0] = 0.25
    h[1] = -8.0
    h[3, 7] = np.nan
    h[4, 9] = np.inf
    q, s = orc.rmsnorm_quant_per_token(h, g, 0.0)
    # rstd = 1/|c|, the maximum is |c|: the scale is 1/127, the codes +-127
    assert s[0] == np.float32(1.0 / 127.0) and s[1] == np.float32(1.0 / 127.0)
    assert (q[0] == 127).all() and (q[1] == -127).all()
    assert s[2] == 0.0 and (q[2] == 0).all()                     # all-zero token
    assert np.isnan(s[3]) and np.isnan(s[4]) and (q[3:] == 0).all()
    # eps > 0: a zero token still has scale 0
    q, s = orc.rmsnorm_quant_per_token(h[2:3], g, 1e-5)
    assert s[0] == 0.0 and (q == 0).all()


def test_gamma_fold_is_gamma_over_s(orc):
    gamma = np.array([0.5, 1.0, 1.25, -2.0] * 4, np.float16)
    s = np.array([2.0, 4.0, 0.5, 8.0] * 4, np.float32)
    g = orc.fold_norm_weight(gamma, (1.0 / s).astype(np.float32))
    np.testing.assert_array_equal(g, (gamma.astype(np.float64) / s).astype(np.float32))


def test_multi_consumer_rule(orc):
    """One normalized activation feeding three projections: one s over all
    three (the concatenated fold), the normalization's weight folded once."""
    wl = W.WORKLOADS["tiny"]
    rng = np.random.default_rng(5)
    K, M = wl.K, 48
    inp = W.generate(W.Workload("tiny3", M, K, (64, 32, 96), 0.5, 9, 0.02, 2, (60.0, 60.0),
                                T_cal=0, fixed_channels=(3, 41)))
    gamma = rng.uniform(0.5, 1.5, K).astype(np.float16)
    eps = W.NORM_EPS
    h = inp.x
    xbar = orc.rmsnorm_fp64(h, gamma, eps)
    s, inv, st = orc.smoothing_factors(orc.calibrate_absmax(orc.to_f16(xbar)),
                                       orc.row_absmax(inp.w), 0.5)
    assert st == 0
    g = orc.fold_norm_weight(gamma, inv)
    xq, xs = orc.rmsnorm_quant_per_token(h, g, eps)
    wq, wsc = orc.fold_quant_weights(inp.w, s)          # all three consumers at once
    n0 = 0
    for w_i in inp.ws:
        n1 = n0 + w_i.shape[1]
        y = orc.dequant(orc.gemm_i32(xq, np.ascontiguousarray(wq[n0:n1])), xs, wsc[n0:n1])
        ref = xbar @ w_i.astype(np.float64)
        assert orc.rel_fro(y, ref) < 0.02
        # control: this consumer left without the compensation (its weights not
        # multiplied by s) while reading the folded normalization's output
        wq0, wsc0 = orc.fold_quant_weights(w_i, np.ones(K, np.float32))
        bad = orc.dequant(orc.gemm_i32(xq, wq0), xs, wsc0)
        assert orc.rel_fro(bad, ref) > 0.3
        n0 = n1
