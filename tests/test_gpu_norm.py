"""GPU parity of the fold of 1/s into the RMS normalization in front of the
layer ("Move activation scale without changing the real linear map", para. 3:
fold the inverse factors into the preceding operation, with the same
compensation for every consumer).

  * sq_fold_norm_weight: bit-exact against the oracle.
  * sq_rmsnorm_quant_per_token: codes bit-exact (they do not depend on the
    token's RMS factor), padding zero, x_scale within one float ulp of the
    oracle's.  Both sides evaluate the scale in double from a sum of squares
    within K * 2^-53 of the exact one (the oracle's is exact) and round once
    to float, so they can differ only when that value lies that close to a
    float rounding boundary: by one ulp.
  * The chain h -> fused norm + quant -> product, with one s shared by the
    three projections that read the normalized activation, against the
    oracle (fp16 within 2^-10) and against the unquantized float64 layer.
"""
import numpy as np
import pytest

import workloads as W
from layout import padding_is_zero, unpack

pytestmark = pytest.mark.gpu

TOL = 2.0 ** -10
FLOOR = 2.0 ** -14
EPS = W.NORM_EPS


@pytest.fixture(scope="module")
def sq():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import w8a8_post_quantization_sq_amd as m
    m.lib()
    return m


@pytest.fixture(scope="module")
def dev():
    import torch
    return torch.device("cuda:0")


def T(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def H(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def scale_ulps(got, want):
    """Largest distance in float32 ulps (NaN must match NaN, zero must match zero)."""
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    fin = ~np.isnan(want)
    assert np.array_equal(got[fin] == 0, want[fin] == 0)
    d = np.abs(got[fin].view(np.int32).astype(np.int64) - want[fin].view(np.int32).astype(np.int64))
    return int(d.max()) if d.size else 0, int(np.count_nonzero(d))


def check_norm_quant(sq, dev, orc, h, g, eps, label, hv=None):
    M, K = h.shape
    xq, xs = sq.rmsnorm_quant(T(h, dev) if hv is None else hv, T(g, dev), eps)
    rq, rs = orc.rmsnorm_quant_per_token(h, g, eps)
    codes = H(xq)
    assert np.array_equal(unpack(codes, M, K), rq), label
    assert padding_is_zero(codes, M, K), label
    ulps, n = scale_ulps(H(xs), rs)
    print(f"[norm-quant] {label}: codes bit-exact, scales {M - n}/{M} bit-equal, "
          f"max {ulps} ulp", flush=True)
    assert ulps <= 1, label
    return xq, xs


def norm_factors(orc, inp, w, gamma, alpha):
    """s from the calibration tokens' normalized activations (float64
    normalization rounded to fp16, the activation the layer sees unfused)."""
    xc = orc.to_f16(orc.rmsnorm_fp64(inp.x_cal, gamma, EPS))
    s, inv, st = orc.smoothing_factors(orc.calibrate_absmax(xc), orc.row_absmax(w), alpha)
    assert st == 0
    return xc, s, inv


@pytest.mark.parametrize("K", [16, 64, 4096, 8192, 11008, 131056])
def test_fold_norm_weight_matches_oracle(sq, dev, orc, K):
    gamma = np.random.default_rng(K).uniform(-2, 2, K).astype(np.float16)
    inv = W.random_scales(K + 1, K, 1e-3, 40.0)
    g = H(sq.fold_norm_weight(T(gamma, dev), T(inv, dev)))
    want = orc.fold_norm_weight(gamma, inv)
    assert np.array_equal(g.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("name,m", [("tiny", None), ("qkv4096", None), ("decode8192", 1),
                                    ("decode8192", 4), ("decode8192", 16),
                                    ("prefill8192x3", None)])
def test_rmsnorm_quant_matches_oracle(sq, dev, orc, name, m):
    wl = W.WORKLOADS[name]
    inp = W.generate(wl, m=m)
    gamma = W.norm_weight(wl)
    _, _, inv = norm_factors(orc, inp, inp.w[:, :256], gamma, wl.alpha)
    g = orc.fold_norm_weight(gamma, inv)
    check_norm_quant(sq, dev, orc, inp.x, g, EPS, f"{name} M={inp.x.shape[0]} K={wl.K}")


@pytest.mark.parametrize("M,K,ld", [(1, 16, 16), (3, 48, 56), (37, 4096, 4096), (17, 2064, 2064),
                                    (9, 6144, 6144), (3, 7184, 7192), (33, 8192, 8200),
                                    (2, 8208, 8208), (64, 16384, 16384), (65, 8192, 8192),
                                    (100, 4096, 4104), (600, 11008, 11008), (520, 16384, 16392),
                                    (1001, 4096, 4104), (777, 6160, 6160), (2050, 8192, 8192),
                                    (300, 12288, 12288), (100, 9008, 9016), (900, 12288, 12296),
                                    (5, 32784, 32784), (1, 131056, 131056)])
def test_rmsnorm_quant_ragged_long_and_strided(sq, dev, orc, M, K, ld):
    h = W.random_f16(800 + K, M, ld, 3.0)
    g = W.random_scales(801 + K, K, 0.02, 4.0)
    hk = np.ascontiguousarray(h[:, :K])
    check_norm_quant(sq, dev, orc, hk, g, EPS, f"M={M} K={K} ld={ld}", hv=T(h, dev)[:, :K])


def test_rmsnorm_quant_degenerate_rows(sq, dev, orc):
    K = 64
    rng = np.random.default_rng(9)
    h = np.zeros((9, K), np.float16)
    h[0] = 0.25                                     # constant token
    h[1] = rng.standard_normal(K) * 1e-3            # mean square near eps
    h[2] = np.float16(2.0 ** -24) * np.arange(K)    # subnormals only
    h[3, 5] = np.nan
    h[4] = rng.standard_normal(K)
    h[4, 7] = -np.inf
    h[5] = 65504.0                                  # largest fp16 everywhere
    h[6, 11] = 3.0                                  # a single nonzero channel
    h[7] = rng.standard_normal(K) * 10              # ordinary
    # row 8 stays zero
    g = np.ones(K, np.float32)
    g[20] = 0.0                                     # a channel the fold zeroed
    for eps in (EPS, 0.0):
        _, xs = check_norm_quant(sq, dev, orc, h, g, eps, f"degenerate rows eps={eps}")
        s = H(xs)
        assert s[8] == 0.0 and np.isnan(s[3]) and np.isnan(s[4])


@pytest.mark.parametrize("M,K", [(5, 4096), (600, 4096), (300, 1040), (130, 16400)])
def test_rmsnorm_rows_whose_multiplier_overflows(sq, dev, orc, M, K):
    """A folded weight of 2^-120: rows whose maximum is below 127 / FLT_MAX
    take +-127 and 0, as in the plain quantizer."""
    from test_gpu_parity import overflow_mix
    h = overflow_mix(M, K, 960 + M)
    g = np.full(K, 2.0 ** -120, np.float32)
    check_norm_quant(sq, dev, orc, h, g, EPS, f"overflowing multipliers M={M} K={K}")


def test_rmsnorm_codes_are_the_quantizer_codes(sq, dev, orc):
    """The codes do not depend on the RMS factor: they equal the per-token
    quantizer's codes of h with the folded weight in place of 1/s."""
    wl = W.WORKLOADS["qkv4096"]
    inp = W.generate(wl)
    g = W.random_scales(5, wl.K, 0.01, 3.0)
    hg, gg = T(inp.x, dev), T(g, dev)
    xq1, _ = sq.rmsnorm_quant(hg, gg, EPS)
    xq2, _ = sq.quant(hg, gg)
    assert np.array_equal(H(xq1), H(xq2))


def test_norm_chain_three_consumers(sq, dev, orc):
    """One normalized activation read by three 8192 x 8192 projections: one s
    from all three (their weights folded side by side), gamma folded once, one
    fused normalization + quantization, one product."""
    wl = W.WORKLOADS["prefill8192x3"]
    inp = W.generate(wl)
    gamma = W.norm_weight(wl)
    K, M, N = wl.K, wl.M, wl.N
    print(f"[norm-chain] {wl.name} M={M} K={K} N={N}", flush=True)
    xc, s, inv = norm_factors(orc, inp, inp.w, gamma, wl.alpha)
    ax = sq.calibrate(T(xc, dev))
    f = sq.fold(T(inp.w, dev), ax, wl.alpha)
    assert np.array_equal(H(f.smooth).view(np.uint32), s.view(np.uint32))
    g = sq.fold_norm_weight(T(gamma, dev), f.inv_smooth)
    xq, xs = sq.rmsnorm_quant(T(inp.x, dev), g, EPS)
    y = H(sq.gemm(xq, xs, f.wq, f.w_scale, M, N, K))
    # the oracle's chain on sampled tokens
    rows = np.sort(np.concatenate([[0, M - 1],
                                   np.random.default_rng(21).choice(np.arange(1, M - 1), 14,
                                                                    replace=False)]))
    go = orc.fold_norm_weight(gamma, inv)
    rq, rs = orc.rmsnorm_quant_per_token(inp.x[rows], go, EPS)
    wq, wsc = orc.fold_quant_weights(inp.w, s)
    y64 = orc.dequant(orc.gemm_i32(rq, wq), rs, wsc)
    ref = y64.astype(np.float16).astype(np.float64)
    got = y[rows].astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    err = np.abs(got - ref) / np.maximum(np.abs(ref), FLOOR)
    print(f"[norm-chain] max rel err vs oracle {err.max():.3g}, "
          f"{np.mean(got == ref):.4f} bit-equal", flush=True)
    assert err.max() <= TOL
    # every consumer against the unquantized layer: normalized h times W_i
    xbar = orc.rmsnorm_fp64(inp.x[rows], gamma, EPS)
    n0 = 0
    for i, w_i in enumerate(inp.ws):
        n1 = n0 + w_i.shape[1]
        e = orc.rel_fro(got[:, n0:n1], xbar @ w_i.astype(np.float64))
        print(f"[norm-chain] consumer {i}: relative Frobenius error vs float64 {e:.3g}", flush=True)
        assert e < 0.02
        n0 = n1


def test_rmsnorm_quant_repeat_runs_are_bitwise_identical(sq, dev):
    wl = W.WORKLOADS["decode8192"]
    inp = W.generate(wl, m=16)
    g = T(W.random_scales(6, wl.K, 0.01, 3.0), dev)
    h = T(inp.x, dev)
    a = [sq.rmsnorm_quant(h, g, EPS) for _ in range(2)]
    assert np.array_equal(H(a[0][0]), H(a[1][0]))
    assert np.array_equal(H(a[0][1]).view(np.uint32), H(a[1][1]).view(np.uint32))
