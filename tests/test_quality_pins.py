"""Pins of the quality measures used by the alpha sweep (oracle/quality.py),
each against a value fixed by construction or by the method's closed forms."""
import numpy as np
import pytest

import workloads as W


@pytest.fixture(scope="module")
def q():
    from oracle import quality
    return quality


def test_difficulty_is_population_std(q):
    assert q.difficulty([1.0, 3.0]) == 1.0
    assert q.difficulty([2.0, 2.0, 2.0]) == 0.0
    assert q.difficulty([0.0, 0.0, 3.0, 3.0]) == 1.5


def test_weight_recon_error_zero_on_the_grid(q):
    # every column holds multiples of 2^-7 up to +-127 * 2^-7 (its maximum), so
    # with s = 1 the codes reproduce the weights exactly
    rng = np.random.default_rng(5)
    K, N = 32, 8
    codes = rng.integers(-126, 127, size=(K, N))
    codes[3, :] = 127
    w = (codes * 2.0 ** -7).astype(np.float16)
    assert q.weight_recon_error(w, np.ones(K, np.float32)) == 0.0
    # one value moved off the grid by half a step: error = (step/2)^2 / ||W||^2
    w2 = w.astype(np.float64)
    w2[0, 0] += 2.0 ** -8
    w2 = w2.astype(np.float16)
    err = q.weight_recon_error(w2, np.ones(K, np.float32))
    assert 0 < err <= (2.0 ** -8) ** 2 / np.sum(w2.astype(np.float64) ** 2) * (1 + 1e-9)


def test_static_clip_fraction_by_construction(q):
    x_cal = np.array([[0.5, -1.0], [0.25, 0.75]], np.float16)   # largest magnitude 1
    x = np.array([[0.5, 1.5], [-2.0, 1.0]], np.float16)          # 1.5 and -2 exceed it
    inv = np.ones(2, np.float32)
    assert q.static_clip_fraction(x, x_cal, inv) == 0.5
    # halving every factor halves both sides: same share
    assert q.static_clip_fraction(x, x_cal, inv * np.float32(0.5)) == 0.5


def test_in_sample_closed_forms_of_the_migration(q, orc):
    """With the factors fitted on the evaluated tokens: alpha = 1 leaves every
    activation channel at magnitude 1 (difficulty 0), alpha = 0 every weight
    row at magnitude 1; for any alpha the two magnitudes multiply to
    ax_j * aw_j (the difficulty moves, the product stays)."""
    wl = W.WORKLOADS["tiny"]
    inp = W.generate(wl)
    x, w = inp.x, inp.w
    s1, inv1 = q.factors(x, w, 1.0)
    assert q.activation_difficulty(x, inv1) <= 4 * 2.0 ** -23
    s0, inv0 = q.factors(x, w, 0.0)
    assert q.weight_difficulty(w, s0) <= 4 * 2.0 ** -23
    ax = orc.calibrate_absmax(x).astype(np.float64)
    aw = orc.row_absmax(w).astype(np.float64)
    for alpha in (0.25, 0.5, 0.8):
        s, inv = q.factors(x, w, alpha)
        am = np.abs(q.scaled_activations(x, inv)).max(axis=0).astype(np.float64)
        wm = np.abs(q.scaled_weights(w, s)).max(axis=1).astype(np.float64)
        assert np.allclose(am * wm, ax * aw, rtol=8 * 2.0 ** -24, atol=0)


def test_unsmoothed_identity_factors(q):
    wl = W.WORKLOADS["tiny"]
    inp = W.generate(wl)
    s, inv = q.factors(inp.x, inp.w, None)
    assert np.all(s == 1.0) and np.all(inv == 1.0)


def test_layer_error_definition(q):
    ref = np.array([[3.0, 4.0]])
    assert q.layer_error(np.array([[3.0, 4.0]]), ref) == 0.0
    assert q.layer_error(np.array([[0.0, 4.0]]), ref) == pytest.approx(9.0 / 25.0, rel=0, abs=0)
