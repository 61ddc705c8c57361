"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test ties an oracle function to something other than itself: values the
pages print (the matrix-lab example, stored under tests/golden/), closed forms
(the alpha = 1/2 smoothed maximum sqrt(|o| max|W|) of the Pith review),
exact-arithmetic identities, brute force with an independent library routine,
and provable error bounds of round-to-nearest quantization.  The mutations a
plausible mistake would make (a dropped factor, the wrong axis, a truncating
rounding, a sign error) fail at least one of them.
"""
import json
import os

import numpy as np
import pytest

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32_ulp(x):
    return np.spacing(np.abs(np.asarray(x, np.float32))).astype(np.float64)


# ---- fp16 decoding -----------------------------------------------------------

def test_half_to_float_exhaustive(orc):
    """Every one of the 65536 binary16 patterns decodes to numpy's value."""
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    x = bits.reshape(256, 256).view(np.float16)
    # Row maxima are not what is tested here; decode through calibrate on one
    # token per row so that every pattern passes through the C decoder.
    got = np.array([orc.half_to_float(int(b)) for b in bits[::97]], np.float32)
    r = ref[::97]
    assert np.array_equal(np.isnan(got), np.isnan(r))
    m = ~np.isnan(r)
    assert np.array_equal(got[m].view(np.uint32), r[m].view(np.uint32))
    # full sweep: each column of a one-token calibration is |value| of one pattern
    ax = orc.calibrate_absmax(x.reshape(1, 65536))
    rabs = np.abs(ref)
    assert np.array_equal(np.isnan(ax), np.isnan(rabs))
    m = ~np.isnan(rabs)
    assert np.array_equal(ax[m].view(np.uint32), rabs[m].view(np.uint32))


# ---- A1 / A2 statistics --------------------------------------------------------

def test_calibrate_bruteforce_and_accumulate(orc):
    x = W.random_f16(11, 37, 96, scale=3.0)          # T != K catches a swapped axis
    ref = np.abs(x.astype(np.float32)).max(axis=0)
    ax = orc.calibrate_absmax(x)
    assert np.array_equal(ax, ref)
    # streaming two batches equals one pass over their concatenation
    ax2 = orc.calibrate_absmax(x[20:], orc.calibrate_absmax(x[:20]))
    assert np.array_equal(ax2, ref)
    # every statistic is exactly the magnitude of some entry of its column
    for j in range(96):
        assert ax[j] in np.abs(x[:, j].astype(np.float32))


def test_calibrate_nan_is_sticky(orc):
    x = W.random_f16(12, 8, 32)
    x[5, 7] = np.nan
    x[2, 9] = np.inf
    ax = orc.calibrate_absmax(x)
    assert np.isnan(ax[7]) and np.isinf(ax[9])
    assert np.isfinite(np.delete(ax, [7, 9])).all()
    prev = np.zeros(32, np.float32)
    prev[3] = np.nan
    assert np.isnan(orc.calibrate_absmax(W.random_f16(13, 4, 32), prev)[3])


def test_row_absmax_bruteforce(orc):
    w = W.random_f16(14, 48, 80, scale=0.02)         # K != N catches a swapped axis
    assert np.array_equal(orc.row_absmax(w), np.abs(w.astype(np.float32)).max(axis=1))


# ---- A2 smoothing factors: closed forms -------------------------------------

def _tiny():
    wl = W.WORKLOADS["tiny"]
    return wl, W.generate(wl)


@pytest.mark.parametrize("alpha", [0.5, 0.8, 0.25, 1.0, 0.0])
def test_smoothed_maxima_closed_forms(orc, alpha):
    """In-sample calibration (X_cal = X, the tiny workload): the smoothed
    activation maximum of channel j is ax_j / s_j = ax_j^(1-a) aw_j^(1-a) and
    the smoothed weight maximum is aw_j s_j = ax_j^a aw_j^a; their product is
    ax_j aw_j for every alpha, and at alpha = 1/2 both equal sqrt(ax_j aw_j),
    the Pith review's sqrt(|o| max|W|).  alpha = 1 flattens every activation
    channel to 1, alpha = 0 every weight row to 1."""
    wl, inp = _tiny()
    ax = orc.calibrate_absmax(inp.x)
    aw = orc.row_absmax(inp.w)
    s, inv, st = orc.smoothing_factors(ax, aw, alpha)
    assert st == 0
    xm = np.abs(inp.x.astype(np.float64) * inv.astype(np.float64)[None, :]).max(axis=0)
    wm = np.abs(inp.w.astype(np.float64) * s.astype(np.float64)[:, None]).max(axis=1)
    ax64, aw64 = ax.astype(np.float64), aw.astype(np.float64)
    a = float(np.float32(alpha))
    tol = 8 * 2.0 ** -24
    np.testing.assert_allclose(xm, ax64 ** (1 - a) * aw64 ** (1 - a), rtol=tol)
    np.testing.assert_allclose(wm, ax64 ** a * aw64 ** a, rtol=tol)
    np.testing.assert_allclose(xm * wm, ax64 * aw64, rtol=tol)
    if alpha == 0.5:
        np.testing.assert_allclose(xm, np.sqrt(ax64 * aw64), rtol=tol)
        np.testing.assert_allclose(wm, np.sqrt(ax64 * aw64), rtol=tol)
        # the outlier channels {3, 41}: the smoothed maximum is sqrt(|o| max|W|)
        for j in (3, 41):
            assert abs(xm[j] - np.sqrt(ax64[j] * aw64[j])) <= tol * xm[j]
    if alpha == 1.0:
        np.testing.assert_allclose(xm, 1.0, rtol=tol)
        assert np.array_equal(s, ax)                # ax^1 / aw^0
    if alpha == 0.0:
        np.testing.assert_allclose(wm, 1.0, rtol=tol)


def test_smoothing_direction_shrinks_outliers(orc):
    """Dividing activations by s moves the range into the weights: the outlier
    channels' share of the activation range drops, the matching weight rows
    grow ("Move activation scale ..." para. 2)."""
    wl, inp = _tiny()
    ax = orc.calibrate_absmax(inp.x)
    aw = orc.row_absmax(inp.w)
    s, inv, _ = orc.smoothing_factors(ax, aw, 0.5)
    xm = np.abs(inp.x.astype(np.float64) * inv[None, :]).max(axis=0)
    assert ax.max() / np.median(ax) > 20
    assert xm.max() / np.median(xm) < 0.5 * ax.max() / np.median(ax)
    assert (s[[3, 41]] > np.median(s)).all()


def test_smoothing_factor_edge_cases(orc):
    ax = np.array([0.0, 2.0, 0.0, 8.0, 1.0], np.float32)
    aw = np.array([1.0, 0.0, 0.0, 2.0, 1.0], np.float32)
    s, inv, st = orc.smoothing_factors(ax, aw, 0.5)
    assert st == 0
    assert s[0] == 1.0 and s[1] == 1.0 and s[2] == 1.0   # dead channel / zero row
    assert s[3] == 2.0 and inv[3] == 0.5                   # sqrt(8 / 2)
    assert s[4] == 1.0
    for bad in (np.nan, np.inf, -1.0):
        a2 = ax.copy()
        a2[1] = bad
        assert orc.smoothing_factors(a2, aw, 0.5)[2] == 1
    # alpha = 1 with a huge statistic: 1/s underflows to a subnormal
    s, inv, st = orc.smoothing_factors(np.array([3e38], np.float32), np.array([1.0], np.float32), 1.0)
    assert st == 2
    # alpha = 1/2 agrees with the correctly rounded sqrt of the ratio (to 1 ulp)
    rng = np.random.default_rng(3)
    ax = rng.uniform(0.01, 500, 1000).astype(np.float16).astype(np.float32)
    aw = rng.uniform(1e-3, 0.2, 1000).astype(np.float16).astype(np.float32)
    s, _, _ = orc.smoothing_factors(ax, aw, 0.5)
    ref = np.sqrt(ax.astype(np.float64) / aw.astype(np.float64))
    assert np.all(np.abs(s - ref) <= f32_ulp(s))


# ---- the identity (X S^-1)(S W) = X W -------------------------------------------

def test_identity_power_of_two_bit_exact(orc):
    rng = np.random.default_rng(5)
    x = W.random_f16(21, 33, 64)
    w = W.random_f16(22, 64, 48, 0.02)
    s = np.exp2(rng.integers(-6, 7, 64)).astype(np.float32)
    assert np.array_equal(orc.smoothed_matmul_fp64(x, w, s), orc.matmul_fp64(x, w))


def test_identity_general_s(orc):
    wl, inp = _tiny()
    s, _, _ = orc.smoothing_factors(orc.calibrate_absmax(inp.x), orc.row_absmax(inp.w), 0.5)
    ref = orc.matmul_fp64(inp.x, inp.w)
    assert orc.rel_fro(orc.smoothed_matmul_fp64(inp.x, inp.w, s), ref) <= 1e-12


def test_wrong_dimension_is_a_different_map(orc):
    """Planted mistake: scale the output-channel dimension of W (its columns)
    instead of the input-channel rows.  With the tiny workload's non-uniform s
    (about 8x between outlier and ordinary channels) that is a different
    linear map, and the identity check must report it."""
    wl, inp = _tiny()
    s, _, _ = orc.smoothing_factors(orc.calibrate_absmax(inp.x), orc.row_absmax(inp.w), 0.5)
    s64 = s.astype(np.float64)
    wrong = (inp.x.astype(np.float64) / s64[None, :]) @ (inp.w.astype(np.float64) * s64[None, :])
    ref = orc.matmul_fp64(inp.x, inp.w)
    assert orc.rel_fro(wrong, ref) >= 0.1
    assert orc.rel_fro(orc.smoothed_matmul_fp64(inp.x, inp.w, s), ref) <= 1e-12
    # the same mistake inside the quantized chain (rows of Wq scaled by the
    # column's factor) also fails the end-to-end error bound used below
    s_uniform = np.full_like(s, float(np.median(s)))
    wrong2 = (inp.x.astype(np.float64) / s64[None, :]) @ (inp.w.astype(np.float64) * s_uniform.astype(np.float64)[:, None])
    assert orc.rel_fro(wrong2, ref) >= 0.1


def test_matrix_lab_worked_example(orc):
    """The page's matrix lab: a = 0.25, b = 0 has determinant 0.25, maps e1 to
    a quarter of itself, leaves e2 alone, and the compensating factor 4 sits on
    the matching weight channel."""
    g = json.load(open(os.path.join(GOLDEN, "matrix_lab.json")))
    # alpha = 1 makes s = ax; choose channel statistics (4, 1) so S^-1 = diag(a, 1)
    s, inv, st = orc.smoothing_factors(np.array([4.0, 1.0], np.float32),
                                       np.array([1.0, 1.0], np.float32), 1.0)
    assert st == 0
    lab = np.array([[inv[0], g["b"]], [0.0, inv[1]]], np.float64)
    assert inv[0] == g["a"]
    assert np.linalg.det(lab) == pytest.approx(g["determinant"], abs=0)
    assert np.array_equal(np.array([1.0, 0.0]) @ lab, np.array(g["image_of_e1"]))
    assert np.array_equal(np.array([0.0, 1.0]) @ lab, np.array(g["image_of_e2"]))
    assert s[g["compensated_weight_channel"]] == g["compensating_scale"]
    # the fold puts the 4 on weight row 0: Wq row-0 entries dequantize to 4 W[0, :]
    w = np.array([[0.5, -0.25, 0.125], [0.5, 0.75, -1.0]], np.float16)
    wq, wsc = orc.fold_quant_weights(w, s)
    deq = wq.astype(np.float64).T * wsc.astype(np.float64)[None, :]
    np.testing.assert_allclose(deq[0], 4 * w[0].astype(np.float64), atol=np.max(wsc) / 2 + 1e-12)
    np.testing.assert_allclose(deq[1], w[1].astype(np.float64), atol=np.max(wsc) / 2 + 1e-12)
    x = np.array([[1.0, 2.0], [-3.0, 0.5], [0.25, -1.0]], np.float16)
    assert np.array_equal(orc.smoothed_matmul_fp64(x, w, s), orc.matmul_fp64(x, w))
    # the factor on the wrong side (column 0 of W) is not the same map
    s64 = s.astype(np.float64)
    w2 = np.array([[0.5, -0.25], [0.5, 0.75]], np.float16)
    x2 = x[:, :2]
    wrong = (x2.astype(np.float64) / s64[None, :]) @ (w2.astype(np.float64) * s64[None, :])
    assert not np.allclose(wrong, orc.matmul_fp64(x2, w2))


# ---- A3 / A4 quantizers -----------------------------------------------------------

def _check_rowwise_quant(vals64, q, scale):
    """Symmetric round-to-nearest properties of one quantized row set:
    codes in [-127, 127]; the largest magnitude maps to +-127; every value is
    within half a step of its code; the step is max|v| / 127."""
    assert q.min() >= -127 and q.max() <= 127
    amax = np.abs(vals64).max(axis=1)
    nz = amax > 0
    assert np.all(np.abs(q[nz]).max(axis=1) == 127)
    st = scale.astype(np.float64)
    np.testing.assert_allclose(st[nz] * 127, amax[nz], rtol=3 * 2.0 ** -24)
    err = np.abs(vals64[nz] - q[nz].astype(np.float64) * st[nz, None])
    # half a step, plus the float32 rounding of the scaled value and of the step
    bound = st[nz, None] * 0.5 + np.abs(vals64[nz]) * 2.0 ** -21
    assert np.all(err <= bound)
    assert np.all(q[~nz] == 0) and np.all(scale[~nz] == 0)


def test_activation_quantizer_properties(orc):
    wl = W.WORKLOADS["qkv4096"]
    inp = W.generate(wl, m=64, with_w=False)
    ax = orc.calibrate_absmax(inp.x_cal)
    inv = (1.0 / np.sqrt(np.maximum(ax, 1e-3))).astype(np.float32)   # any positive inv_s
    xq, xs = orc.quant_act_per_token(inp.x, inv)
    xt = inp.x.astype(np.float64) * inv.astype(np.float64)[None, :]
    _check_rowwise_quant(xt, xq, xs)


def test_weight_quantizer_properties(orc):
    w = W.random_f16(31, 96, 40, 0.02)
    s = np.exp(np.random.default_rng(4).normal(0, 1.5, 96)).astype(np.float32)
    wq, wsc = orc.fold_quant_weights(w, s)
    wt = w.astype(np.float64) * s.astype(np.float64)[:, None]    # row j times s_j
    _check_rowwise_quant(wt.T, wq, wsc)


def test_round_half_even_ties(orc):
    """With 1/s = 1 and a row maximum of 127 the step is exactly 1, so codes
    are the values rounded half to even: 2.5 -> 2, 3.5 -> 4, -2.5 -> -2."""
    row = np.array([[127, 2.5, 3.5, -2.5, 0.5, 1.5, -0.5, 126.5,
                     -126.5, 5.5, -5.5, 0.25, 7.5, -7.5, 64.5, 0]], np.float16)
    xq, xs = orc.quant_act_per_token(row, np.ones(16, np.float32))
    assert xs[0] == 1.0
    assert xq[0].tolist() == [127, 2, 4, -2, 0, 2, 0, 126, -126, 6, -6, 0, 8, -8, 64, 0]
    wq, ws = orc.fold_quant_weights(row.T.copy(), np.ones(16, np.float32))
    assert ws[0] == 1.0 and wq[0].tolist() == xq[0].tolist()


def test_quantizer_degenerate_rows(orc):
    x = W.random_f16(41, 5, 32)
    x[1] = 0
    x[3, 4] = np.nan
    x[4, 9] = -np.inf
    xq, xs = orc.quant_act_per_token(x, np.ones(32, np.float32))
    assert xs[1] == 0 and np.all(xq[1] == 0)
    assert np.isnan(xs[3]) and np.all(xq[3] == 0)
    assert np.isnan(xs[4]) and np.all(xq[4] == 0)
    assert np.isfinite(xs[[0, 2]]).all() and np.abs(xq[[0, 2]]).max() == 127


def overflow_rows(K, seed):
    """Three fp16 rows with every magnitude in [2^-6, 2^-2] or zero (row 0 has
    zeros, row 1 negative zeros, row 2 none): times 2^-120 every value is a
    normal float, the row maximum is at most 2^-122, and 127 / max overflows."""
    rng = np.random.default_rng(seed)
    mag = 2.0 ** rng.uniform(-6, -2, size=(3, K))
    x = (mag * rng.choice([-1.0, 1.0], size=(3, K))).astype(np.float16)
    x[0, ::7] = 0.0
    x[1, 3::5] = -0.0
    return x


def test_rows_whose_multiplier_overflows(orc):
    """For a maximum a below QMAX / FLT_MAX the float multiplier QMAX / a is
    infinite: nonzero values take the clamp's +-QMAX and zeros the code 0, in
    every quantizer (8-bit activations, the fused norm, weights, 4-bit)."""
    K = 64
    x = overflow_rows(K, 5)
    inv = np.full(K, 2.0 ** -120, np.float32)
    xt = x.astype(np.float32) * inv
    a = np.abs(xt).max(axis=1)
    assert np.all(np.abs(xt[xt != 0]) >= np.float32(2.0 ** -126))      # normal floats
    with np.errstate(over="ignore"):
        assert np.all(np.isinf(np.float32(127.0) / a))
    sign = np.sign(xt).astype(np.int8)
    assert (sign == 0).sum() > 0
    xq, xs = orc.quant_act_per_token(x, inv)
    assert np.array_equal(xq, sign * 127)
    assert np.array_equal(xs.view(np.uint32), (a / np.float32(127.0)).view(np.uint32))
    xq2, _ = orc.rmsnorm_quant_per_token(x, inv, 1e-5)
    assert np.array_equal(xq2, sign * 127)
    wq, ws = orc.fold_quant_weights(np.ascontiguousarray(x.T), inv)
    assert np.array_equal(wq, sign * 127) and np.array_equal(ws, xs)
    # 4 bits: 7 / a overflows only for a <= 2^-126 (the smallest normal float)
    x4 = (np.sign(x.astype(np.float32)) * 0.25).astype(np.float16)
    q4, s4 = orc.quant4_act_per_token(x4, np.full(K, 2.0 ** -124, np.float32), False)
    assert np.array_equal(q4, sign * 7)
    assert np.all(s4 == np.float32(2.0 ** -126) / np.float32(7.0))
    # rotated: a single nonzero 2^-126 at channel 1 spreads to +-2^-126 on
    # every output, with the signs of row 1 of the Sylvester matrix
    e1 = np.zeros((1, K), np.float16)
    e1[0, 1] = 0.25
    q4r, s4r = orc.quant4_act_per_token(e1, np.full(K, 2.0 ** -124, np.float32), True)
    assert q4r[0].tolist() == [7 if i % 2 == 0 else -7 for i in range(K)]
    assert s4r[0] == np.float32(2.0 ** -126) / np.float32(7.0)


# ---- A5 / A6 ---------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(1, 1, 16), (7, 13, 48), (33, 65, 160), (3, 5, 4096)])
def test_gemm_matches_int64_bruteforce(orc, shape):
    M, N, K = shape
    xq = W.random_i8(51, M, K, -128, 127)
    wq = W.random_i8(52, N, K, -128, 127)
    ref = xq.astype(np.int64) @ wq.astype(np.int64).T
    assert np.array_equal(orc.gemm_i32(xq, wq).astype(np.int64), ref)


def test_gemm_extremes(orc):
    K = 133136                      # largest multiple of 16 with K * 127^2 < 2^31
    xq = np.full((1, K), 127, np.int8)
    wq = np.full((2, K), -127, np.int8)
    wq[1] = 127
    acc = orc.gemm_i32(xq, wq)
    assert acc.tolist() == [[-K * 16129, K * 16129]]


def test_dequant_exact_cases(orc):
    acc = np.array([[1, -2, 2047], [-2048, 0, 5]], np.int32)
    y = orc.dequant(acc, np.ones(2, np.float32), np.ones(3, np.float32))
    assert np.array_equal(orc.to_f16(y).astype(np.float64), acc.astype(np.float64))
    y = orc.dequant(acc, np.array([0.5, 4.0], np.float32), np.array([0.25, 2.0, 1.0], np.float32))
    exp = acc * np.array([0.5, 4.0])[:, None] * np.array([0.25, 2.0, 1.0])[None, :]
    assert np.array_equal(y, exp)
    # fp16 conversion: overflow to inf at 65520, ties to even
    assert np.isinf(orc.to_f16(np.array([65520.0]))[0])
    assert orc.to_f16(np.array([65519.0]))[0] == 65504
    assert orc.to_f16(np.array([2049.0]))[0] == 2048 and orc.to_f16(np.array([2051.0]))[0] == 2052


# ---- end to end -------------------------------------------------------------------

def _chain_bound(orc, x, w, c):
    """Provable bound on |y - X W| for the quantized chain: with
    x~ = dx (qx + ex), W~ = dw (qw + ew) and |ex|, |ew| <= 1/2,
    |sum x~ W~ - dx dw sum qx qw| <= dx dw sum_j (|qx| + |qw| + 1/2) / 2;
    plus the float32 roundings of x~, W~, s and 1/s (a few 2^-24 relative per
    term) and the float64 evaluation of y."""
    dx = c.x_scale.astype(np.float64)
    dw = c.w_scale.astype(np.float64)
    qx = np.abs(c.xq.astype(np.float64))
    qw = np.abs(c.wq.astype(np.float64))
    K = x.shape[1]
    qsum = qx.sum(1)[:, None] + qw.sum(1)[None, :] + K / 2
    b = dx[:, None] * dw[None, :] * qsum / 2
    b += (np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64))) * 2.0 ** -20
    return b


@pytest.mark.parametrize("name", ["tiny", "qkv4096", "down11008"])
def test_chain_error_bound(orc, name):
    """Y_q of the whole chain A1..A6 stays within the provable quantization
    bound of the exact X W.  A wrong axis, a dropped 1/s, a truncating
    rounding or a scale error breaks this on these workloads."""
    wl = W.WORKLOADS[name]
    inp = W.generate(wl, m=min(wl.M, 24))
    w = inp.w if name == "tiny" else np.ascontiguousarray(inp.w[:, :256])
    c = orc.smoothed_linear(inp.x, inp.x_cal, w, wl.alpha)
    assert c.status == 0
    ref = orc.matmul_fp64(inp.x, w)
    b = _chain_bound(orc, inp.x, w, c)
    assert np.all(np.abs(c.y64 - ref) <= b)
    # and the rounded fp16 output within half an fp16 ulp more
    y16 = c.y16.astype(np.float64)
    assert np.all(np.abs(y16 - ref) <= b + np.abs(c.y64) * 2.0 ** -11 + 2.0 ** -25)


def test_chain_bound_catches_planted_mistakes(orc):
    """The bound above is tight enough to fail a plausible oracle mistake:
    truncation instead of rounding, and a fold that forgets s."""
    wl = W.WORKLOADS["qkv4096"]
    inp = W.generate(wl, m=16)
    w = np.ascontiguousarray(inp.w[:, :128])
    c = orc.smoothed_linear(inp.x, inp.x_cal, w, wl.alpha)
    ref = orc.matmul_fp64(inp.x, w)
    # fold without s: codes of W instead of S W, combined with X / s
    wq_bad, wsc_bad = orc.fold_quant_weights(w, np.ones_like(c.s))
    y_bad = orc.dequant(orc.gemm_i32(c.xq, wq_bad), c.x_scale, wsc_bad)
    b = _chain_bound(orc, inp.x, w, c)
    assert np.any(np.abs(y_bad - ref) > b)
    # truncation toward zero of the activation codes
    xt = inp.x.astype(np.float32) * c.inv_s[None, :]
    r = (np.float32(127.0) / (c.x_scale * np.float32(127.0)))[:, None]
    xq_tr = np.trunc(xt * r).astype(np.int8)
    y_tr = orc.dequant(orc.gemm_i32(xq_tr, c.wq), c.x_scale, c.w_scale)
    assert orc.rel_fro(y_tr, ref) > 1.5 * orc.rel_fro(c.y64, ref)


def _layer_inputs(orc, name, rows):
    wl = W.WORKLOADS[name]
    inp = W.generate(wl, m=rows)
    s, inv, st = orc.smoothing_factors(orc.calibrate_absmax(inp.x_cal), orc.row_absmax(inp.w),
                                       wl.alpha)
    assert st == 0
    wq, wsc = orc.fold_quant_weights(inp.w, s)
    return np.ascontiguousarray(inp.x), s, inv, wq, wsc


def _layer_equals_staged(orc, block, x, inv, wq, wsc):
    """block(x, inv_s, wq, w_scale) against A4, A5 and A6 called one by one
    (each pinned on its own above), bit for bit in float64."""
    xq, xs = orc.quant_act_per_token(x, inv)
    staged = orc.dequant(orc.gemm_i32(xq, wq), xs, wsc)
    got = block(x, inv, wq, wsc)
    return got.shape == staged.shape and np.array_equal(got.view(np.uint64),
                                                        staged.view(np.uint64))


@pytest.mark.parametrize("name,rows", [("tiny", None), ("qkv4096", 64)])
def test_layer_block_equals_the_staged_chain(orc, name, rows):
    """The CPU baseline's unit of work (quantization + int32 product +
    dequantization in one C call, on a block of tokens) is exactly the
    per-stage oracle chain: the tiny workload, and a 64-token block of the
    2048 x 4096 x 4096 layer with its real folded weights."""
    x, s, inv, wq, wsc = _layer_inputs(orc, name, rows)
    assert _layer_equals_staged(orc, orc.layer_block, x, inv, wq, wsc)


@pytest.mark.parametrize("mutant", ["s_for_inv_s", "scales_reversed", "tokens_rolled",
                                    "unsmoothed_codes"])
def test_layer_block_pin_catches_swapped_arguments(orc, mutant):
    """A block computed from the wrong arguments (s where 1/s belongs, the
    weight scales out of order, the token rows shifted, codes folded without
    s) fails the comparison above."""
    x, s, inv, wq, wsc = _layer_inputs(orc, "tiny", None)
    wq_plain, wsc_plain = orc.fold_quant_weights(W.generate(W.WORKLOADS["tiny"]).w,
                                                 np.ones_like(s))

    def bad(x_, inv_, wq_, wsc_):
        if mutant == "s_for_inv_s":
            return orc.layer_block(x_, s, wq_, wsc_)
        if mutant == "scales_reversed":
            return orc.layer_block(x_, inv_, wq_, np.ascontiguousarray(wsc_[::-1]))
        if mutant == "tokens_rolled":
            return orc.layer_block(np.ascontiguousarray(np.roll(x_, 1, axis=0)), inv_, wq_, wsc_)
        return orc.layer_block(x_, inv_, wq_plain, wsc_plain)
    assert not _layer_equals_staged(orc, bad, x, inv, wq, wsc)


@pytest.mark.parametrize("name", ["tiny", "qkv4096"])
def test_unquantized_fp16_rewrite(orc, name):
    """Before quantizing, the smoothed graph in fp16 matches fp64 X W within
    relative Frobenius 1e-3 and every smoothed value fits fp16."""
    wl = W.WORKLOADS[name]
    inp = W.generate(wl, m=min(wl.M, 64))
    w = inp.w if name == "tiny" else np.ascontiguousarray(inp.w[:, :512])
    s, inv, st = orc.smoothing_factors(orc.calibrate_absmax(inp.x_cal), orc.row_absmax(w), wl.alpha)
    ys, ok = orc.unquantized_fp16_rewrite(inp.x, w, s, inv)
    assert ok
    assert orc.rel_fro(ys, orc.matmul_fp64(inp.x, w)) <= 1e-3


def test_multi_consumer_fold_slices(orc):
    """One smoothed X feeds three projections: folding the concatenation
    [W1|W2|W3] with the shared s equals folding each consumer with that s,
    and each consumer's identity holds ("Move activation scale ..." para. 3)."""
    K = 96
    ws = [W.random_f16(60 + i, K, 40 + 8 * i, 0.015) for i in range(3)]
    wcat = np.concatenate(ws, axis=1)
    x = W.random_f16(64, 12, K)
    ax = orc.calibrate_absmax(x)
    aw = orc.row_absmax(wcat)
    assert np.array_equal(aw, np.maximum.reduce([orc.row_absmax(w) for w in ws]))
    s, inv, _ = orc.smoothing_factors(ax, aw, 0.5)
    wq, wsc = orc.fold_quant_weights(wcat, s)
    off = 0
    for w in ws:
        q1, s1 = orc.fold_quant_weights(w, s)
        n = w.shape[1]
        assert np.array_equal(q1, wq[off:off + n]) and np.array_equal(s1, wsc[off:off + n])
        assert orc.rel_fro(orc.smoothed_matmul_fp64(x, w, s), orc.matmul_fp64(x, w)) <= 1e-12
        off += n


def test_quality_report_smoothing_helps_on_outliers(orc):
    """Reported, not a parity claim (the pages print no error values): on the
    outlier workloads smoothing lowers the layer's squared-Frobenius error."""
    wl = W.WORKLOADS["qkv4096"]
    inp = W.generate(wl, m=32)
    w = np.ascontiguousarray(inp.w[:, :256])
    e_id = orc.quant_error_report(inp.x, inp.x_cal, w, None)
    e_sq = orc.quant_error_report(inp.x, inp.x_cal, w, 0.5)
    assert e_sq < e_id


def test_quality_report_hand_cases(orc):
    """The layer error ||Y_q - XW||^2 / ||XW||^2 on one token x = [1, 0.5] and one
    output channel w = [1, 1], worked by hand from the definitions (x_cal = x):
    - S = I, and alpha = 0 (s_j = 1 / max|W_j| = 1): 0.5 * 127 = 63.5 rounds to
      64 (ties to even), the weights are exact, Y_q = (127 + 64) / 127;
    - alpha = 1 (s = max|X_j| = [1, 0.5]): the activation codes become exact
      [127, 127] and the weight row 0.5 takes the same tie, so the same error;
    - alpha = 1/2 (s = [1, sqrt(1/2)]): 0.7071 * 127 = 89.80 rounds to 90 on both
      sides, Y_q = (127^2 + 90^2) / 127^2 = 24229 / 16129.
    The scales 1/127 are float32, so the values hold to ~1e-5 relative."""
    x = np.array([[1.0, 0.5]], np.float16)
    w = np.array([[1.0], [1.0]], np.float16)
    ref = 1.5 ** 2
    tie = (191.0 / 127.0 - 1.5) ** 2 / ref            # = 1 / 145161
    half = (24229.0 / 16129.0 - 1.5) ** 2 / ref
    for alpha in (None, 0.0, 1.0):
        assert orc.quant_error_report(x, x, w, alpha) == pytest.approx(tie, rel=1e-4)
    assert orc.quant_error_report(x, x, w, 0.5) == pytest.approx(half, rel=1e-4)
    assert half < tie / 3


def test_quality_report_zero_on_the_grid(orc):
    """Tokens and weight columns that are multiples of 2^-7 with a largest
    magnitude of exactly 127 * 2^-7 quantize without error when S = I
    (r = 127 / (127 * 2^-7) = 128 exactly), so the layer error is exactly 0."""
    rng = np.random.default_rng(21)
    M, K, N = 6, 64, 5
    xc = rng.integers(-126, 127, size=(M, K))
    xc[:, 7] = 127
    wc = rng.integers(-126, 127, size=(K, N))
    wc[9, :] = -127
    x = (xc * 2.0 ** -7).astype(np.float16)
    w = (wc * 2.0 ** -7).astype(np.float16)
    assert orc.quant_error_report(x, x, w, None) == 0.0


# ---- the input generator ------------------------------------------------------------

def test_generator_chunked_draws_match_single_draw():
    rng1 = np.random.default_rng(9)
    a = W._normal_f16(rng1, 2500, 7, 0.5)
    b = (np.random.default_rng(9).standard_normal((2500, 7)) * 0.5).astype(np.float16)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_generator_structure():
    wl = W.WORKLOADS["down11008"]
    inp = W.generate(wl, m=256, with_w=False)
    assert len(inp.outlier_channels) == 4 and len(inp.outlier_tokens) == 5
    big = np.abs(inp.x[np.ix_(inp.outlier_tokens, inp.outlier_channels)].astype(np.float32))
    assert np.median(big) > 100
    assert inp.x_cal.shape == (512, 11008) and len(inp.outlier_tokens_cal) == 10
