"""Pins of the oracle's Smooth Rotation at 4 bits (Pith review of arXiv
2506.01967: key machinery, core discovery, referee major comment 1).

  * the fast transform against the Sylvester matrix written from its closed
    form H[i][j] = (-1)^popcount(i & j): unit vectors give its rows, random
    vectors its product within the float error bound, applying it twice
    gives d times the input exactly;
  * the rotation keeps the linear map: (X S^-1 H)(H S W) / d = X W;
  * the 4-bit quantizer: codes in [-7, 7], the maximum at +-7, half a step of
    error, ties to even, zero and non-finite rows, the 1/d in the weight
    scale (a W4A4 layer reproduces X W, not d X W);
  * Eq. (8) and Eq. (9) on a synthetic massive-outlier token: the largest
    rotated outlier term is sum|o_i| / sqrt(d) exactly when a Hadamard column
    aligns with the outlier signs; after in-sample smoothing it is
    sum sqrt(|o_i| max|W_i|) / sqrt(d) -- sqrt(d) times the value the printed
    Eq. (9), with denominator d, gives.
"""
import numpy as np
import pytest

import workloads as W


@pytest.mark.parametrize("d", [16, 64, 256])
def test_fwht_of_unit_vectors_gives_the_sylvester_rows(orc, d):
    H = orc.hadamard_fp64(d)
    for i in range(d):
        e = np.zeros(d, np.float32)
        e[i] = 1.0
        np.testing.assert_array_equal(orc.fwht_f32(e), H[i])
    np.testing.assert_array_equal(H @ H, d * np.eye(d))


@pytest.mark.parametrize("d", [64, 1024, 4096])
def test_fwht_matches_the_dense_product(orc, d):
    rng = np.random.default_rng(d)
    H = orc.hadamard_fp64(d)
    for scale in (1.0, 1000.0):
        v = (rng.standard_normal(d) * scale).astype(np.float32)
        v[rng.integers(0, d, 3)] *= 500.0          # a few outliers
        got = orc.fwht_f32(v).astype(np.float64)
        want = v.astype(np.float64) @ H
        n = int(np.log2(d))
        u = 2.0 ** -24
        bound = (n * u / (1 - n * u)) * np.abs(v.astype(np.float64)).sum()
        assert np.all(np.abs(got - want) <= bound)
    # twice = d * identity, exactly for small integers
    iv = rng.integers(-50, 50, d).astype(np.float32)
    np.testing.assert_array_equal(orc.fwht_f32(orc.fwht_f32(iv)), d * iv)


def test_rotation_keeps_the_linear_map(orc):
    rng = np.random.default_rng(1)
    d, M, N = 256, 24, 40
    H = orc.hadamard_fp64(d)
    x = rng.standard_normal((M, d))
    w = rng.standard_normal((d, N))
    s = rng.uniform(0.1, 10.0, d)
    y = ((x / s[None, :]) @ H) @ (H @ (w * s[:, None])) / d
    np.testing.assert_allclose(y, x @ w, rtol=0, atol=1e-10 * np.abs(x @ w).max())


def test_quant4_rows_grid_ties_and_degenerate_rows(orc):
    K = 16
    one = np.ones(K, np.float32)
    x = np.zeros((5, K), np.float16)
    x[0] = [7, 2.5, 3.5, -2.5, 0.5, 1.5, -0.5, 6.5, -6.5, 5.5, -5.5, 0.25, 4.5, -4.5, 1, 0]
    x[2] = x[0]
    x[2, 4] = np.nan
    x[3] = x[0]
    x[3, 0] = np.inf
    x[4] = -x[0]
    q, sc = orc.quant4_rows(x, one, rotate=False)
    # a = 7, so the step is 1 and the codes are the values rounded half to even
    assert q[0].tolist() == [7, 2, 4, -2, 0, 2, 0, 6, -6, 6, -6, 0, 4, -4, 1, 0]
    assert sc[0] == np.float32(1.0) and sc[1] == 0.0 and (q[1] == 0).all()
    assert np.isnan(sc[2]) and np.isnan(sc[3]) and (q[2:4] == 0).all()
    assert (q[4] == -q[0]).all()
    # rotated: a NaN or an infinity spreads to every coordinate
    q, sc = orc.quant4_rows(x, one, rotate=True)
    assert np.isnan(sc[2]) and np.isnan(sc[3]) and (q[2:4] == 0).all() and sc[1] == 0.0


@pytest.mark.parametrize("rotate", [False, True])
def test_quant4_rows_bounds(orc, rotate):
    wl = W.WORKLOADS["qkv4096"]
    x = W.generate(wl, m=64, with_w=False).x
    mult = W.random_scales(3, wl.K, 0.05, 2.0)
    q, sc = orc.quant4_rows(x, mult, rotate)
    v = x.astype(np.float32) * mult[None, :]
    if rotate:
        v = np.stack([orc.fwht_f32(r) for r in v])
    a = np.abs(v).max(axis=1)
    assert np.array_equal(sc, (a / np.float32(7.0)).astype(np.float32))
    assert np.abs(q).max() == 7 and (np.abs(q).max(axis=1) == 7).all()
    err = np.abs(q.astype(np.float64) * (a[:, None] / 7.0) - v)
    assert np.all(err <= a[:, None] / 14.0 * (1 + 1e-6))


@pytest.mark.parametrize("rotate", [False, True])
def test_w4a4_layer_reproduces_xw(orc, rotate):
    """The 1/d sits in the weight scale: the 4-bit layer approximates X W
    (a missing or doubled 1/d is off by a factor d)."""
    wl = W.WORKLOADS["tiny"]
    inp = W.generate(wl)
    ax = orc.calibrate_absmax(inp.x_cal)
    s, inv, st = orc.smoothing_factors(ax, orc.row_absmax(inp.w), 0.5)
    xq, xs = orc.quant4_act_per_token(inp.x, inv, rotate)
    wq, ws = orc.fold4_weights(inp.w, s, rotate)
    y = orc.dequant(orc.gemm_i32(xq, wq), xs, ws)
    ref = orc.matmul_fp64(inp.x, inp.w)
    e = orc.rel_fro(y, ref)
    assert e < 0.35, e            # 4-bit grid on both operands: a coarse but finite error
    assert orc.rel_fro(y * wl.K, ref) > 10


def gf2_rank(idx):
    rows = [int(i) for i in idx]
    rank = 0
    for bit in reversed(range(32)):
        piv = next((r for r in rows if (r >> bit) & 1), None)
        if piv is None:
            continue
        rows = [r ^ piv if (r >> bit) & 1 else r for r in rows if r != piv]
        rank += 1
    return rank


def outlier_token(d, rng, n_out=4, mag=1000.0):
    ch = np.sort(rng.choice(d, n_out, replace=False))
    o = np.zeros(d)
    o[ch] = mag * rng.choice([-1.0, 1.0], n_out)
    eps = rng.standard_normal(d)
    eps[ch] = 0.0
    return ch, o, eps


@pytest.mark.parametrize("d", [4096, 8192])
def test_eq8_and_eq9_on_a_massive_outlier_token(orc, d):
    rng = np.random.default_rng(d + 7)
    H = None if d > 4096 else orc.hadamard_fp64(d)
    ch, o, eps = outlier_token(d, rng)

    def rot(v):   # v R with R = H / sqrt(d), in float64
        if H is not None:
            return v @ H / np.sqrt(d)
        return orc.fwht_f32(v.astype(np.float32)).astype(np.float64) / np.sqrt(d)

    # the outlier indices are independent over GF(2) here, so a column of H
    # has every sign pattern on them: the outlier term reaches sum |o_i|
    assert gf2_rank(ch) == len(ch)
    eq8 = np.abs(o).sum() / np.sqrt(d)
    assert np.max(np.abs(rot(o))) == pytest.approx(eq8, rel=1e-6)
    t = o + eps
    assert abs(np.max(np.abs(rot(t))) - eq8) <= np.max(np.abs(rot(eps))) * (1 + 1e-6)
    # smoothing first, in sample: s_j = sqrt(max|X_j| / max|W_j|) on the token
    # itself turns o_i into sign(o_i) sqrt(|o_i| max|W_i|)
    wmax = rng.uniform(0.05, 0.1, d)
    s = np.sqrt(np.abs(t) / wmax)
    s[np.abs(t) == 0] = 1.0
    so = o / s
    np.testing.assert_allclose(np.abs(so[ch]), np.sqrt(np.abs(o[ch]) * wmax[ch]), rtol=1e-12)
    eq9_fixed = np.sqrt(np.abs(o[ch]) * wmax[ch]).sum() / np.sqrt(d)
    eq9_printed = np.sqrt(np.abs(o[ch]) * wmax[ch]).sum() / d
    got = np.max(np.abs(rot(so)))
    assert got == pytest.approx(eq9_fixed, rel=1e-6)
    assert got == pytest.approx(eq9_printed * np.sqrt(d), rel=1e-6)


# ---- the activation step of the four-way comparison ---------------------------------
#
# One token worked by hand (d = 16): x = 8 e_0, calibration on the token itself,
# weight row 0 with maximum 0.5 and every other row zero.  Channels other than
# 0 have a zero statistic and take s = 1; s_0 = sqrt(8 / 0.5) = 4, so x / s is
# 2 e_0 exactly.  e_0 H is row 0 of the Sylvester matrix, all ones, so the
# rotated token is 2 (or 8 without smoothing) in every channel and its maximum
# is that value; the quantizer's scale is max / 7 in float, and the step in the
# orthonormal convention R = H / sqrt(d) is scale / 4.

def _hand_case_steps():
    d = 16
    x = np.zeros((1, d), np.float16)
    x[0, 0] = 8.0
    w = np.zeros((d, 3), np.float16)
    w[0] = [0.5, -0.25, 0.125]
    return d, x, w


def _hand_case_expected():
    sev = np.float32(7.0)
    smooth = float(np.float32(2.0) / sev)       # max of x / s = 2
    plain = float(np.float32(8.0) / sev)        # max of x = 8
    return {"original": plain, "smooth": smooth, "rotate": plain / 4.0,
            "smooth_rotate": smooth / 4.0}


def _steps_match_hand_case(q):
    d, x, w = _hand_case_steps()
    got = q.w4a4_compare(x, x, w)
    want = _hand_case_expected()
    for key, meas in got.items():
        if meas["act_step"] != want[key.split("/")[0]]:
            return False
    return True


def test_w4a4_activation_step_hand_case():
    from oracle import quality as q
    d, x, w = _hand_case_steps()
    got = q.w4a4_compare(x, x, w)
    assert set(k.split("/")[0] for k in got) == set(q.W4A4_METHODS)
    want = _hand_case_expected()
    for key, meas in got.items():
        assert meas["act_step"] == want[key.split("/")[0]], key
    assert _steps_match_hand_case(q)


@pytest.mark.parametrize("mutant", ["divide_by_d", "no_rotation_factor", "always_rotated"])
def test_w4a4_activation_step_catches_planted_mistakes(monkeypatch, mutant):
    """The step measure with a plausible mistake planted in the oracle (the
    printed Eq. (9)'s d instead of sqrt(d); the unnormalized transform's scale
    taken as the step; every method treated as rotated) fails the hand case."""
    from oracle import quality as q

    def bad(x_scale, d, rotate):
        xs = np.asarray(x_scale, np.float64)
        if mutant == "divide_by_d":
            return float(np.mean(xs / (d if rotate else 1.0)))
        if mutant == "no_rotation_factor":
            return float(np.mean(xs))
        return float(np.mean(xs / np.sqrt(d)))
    monkeypatch.setattr(q, "act_step", bad)
    assert not _steps_match_hand_case(q)
