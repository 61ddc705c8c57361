"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every stage is fed the oracle's own inputs (so a failure names its kernel),
then the whole chain runs on the GPU from the raw fp16 data.  Codes, scales,
statistics, factors and int32 sums must be bit-exact; fp16 outputs within
2^-10 relative (floor 2^-14) of the oracle's correctly rounded value.  The
workloads run at their real sizes in the launch configuration the benchmark
times; where the oracle's O(MNK) product would be slow, a seeded sample of
rows (always including the first and last token) is compared.

The library stores int8 codes in its packed operand order; the tests unpack
them with an independent numpy permutation (tests/layout.py) before
comparing, and check that the padding is zero.
"""
import numpy as np
import pytest

import workloads as W
from layout import pack, packed_bytes, padding_is_zero, unpack

pytestmark = pytest.mark.gpu

TOL = 2.0 ** -10
FLOOR = 2.0 ** -14


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


def bits_equal(a, b):
    a = np.asarray(a)
    b = np.asarray(b)
    if a.dtype.kind == "f":
        na, nb = np.isnan(a), np.isnan(b)
        if not np.array_equal(na, nb):
            return False
        return np.array_equal(a[~na].view(np.uint32 if a.dtype == np.float32 else np.uint16),
                              b[~nb].view(np.uint32 if b.dtype == np.float32 else np.uint16))
    return np.array_equal(a, b)


def assert_f16_close(y_gpu, y64_ref):
    ref = np.asarray(y64_ref, np.float64).astype(np.float16).astype(np.float64)
    g = np.asarray(y_gpu).astype(np.float64)
    assert np.array_equal(np.isnan(g), np.isnan(ref))
    fin = np.isfinite(ref)
    assert np.array_equal(g[~fin & ~np.isnan(ref)], ref[~fin & ~np.isnan(ref)])
    err = np.abs(g[fin] - ref[fin]) / np.maximum(np.abs(ref[fin]), FLOOR)
    assert err.size == 0 or err.max() <= TOL, f"max rel err {err.max():.3g}"
    return err


def gemm_i32_threads(orc, xq, wq, threads=8):
    """The oracle's int32 product, its token rows split into blocks that run
    on host threads (the C call releases the interpreter lock); each block is
    the oracle's own computation, so the result is the oracle's."""
    from concurrent.futures import ThreadPoolExecutor
    M = xq.shape[0]
    step = max(1, (M + threads - 1) // threads)
    blocks = [(r, min(M, r + step)) for r in range(0, M, step)]
    with ThreadPoolExecutor(len(blocks)) as ex:
        parts = list(ex.map(lambda b: orc.gemm_i32(np.ascontiguousarray(xq[b[0]:b[1]]), wq),
                            blocks))
    return np.concatenate(parts, axis=0)


def tile_rows(M, tile=256, wave_rows=32, seed=0):
    """Token rows that touch every tile row of the product's 256-token tiles:
    the first and last row of each tile (so both sides of every tile boundary,
    255/256, ..., and M - 1), and one more per tile inside the 32-row slice of
    wave t % 8 (tile t), at a seeded offset, so that across tiles every wave
    position of the workgroup is compared.  All N columns of each row are
    compared, which covers every tile column.  Up to 64 tokens (the decode
    kernels, no token tiles) every row."""
    if M <= 64:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    rows = []
    for t in range((M + tile - 1) // tile):
        lo, hi = t * tile, min(M, (t + 1) * tile) - 1
        w = t % (tile // wave_rows)
        mid = min(hi, lo + w * wave_rows + int(rng.integers(0, wave_rows)))
        rows += [lo, mid, hi]
    return np.unique(np.asarray(rows, np.int64))


ALL = ["tiny", "qkv4096", "down11008", "decode8192", "prefill8192x3"]


def wl_inputs(name, m=None):
    wl = W.WORKLOADS[name]
    return wl, W.generate(wl, m=m)


# ---- A1 calibration ----------------------------------------------------------------

@pytest.mark.parametrize("name", ALL)
def test_calibrate_matches_oracle(sq, dev, orc, name):
    wl, inp = wl_inputs(name, m=16 if name != "tiny" else None)
    print(f"[calibrate] {name} T={inp.x_cal.shape[0]} K={wl.K}", flush=True)
    ax = sq.calibrate(T(inp.x_cal, dev))
    assert bits_equal(H(ax), orc.calibrate_absmax(inp.x_cal))
    # streamed in two uneven batches
    half = inp.x_cal.shape[0] // 3 + 1
    ax2 = sq.calibrate(T(inp.x_cal[:half], dev))
    sq.calibrate(T(inp.x_cal[half:], dev), ax2)
    assert bits_equal(H(ax2), orc.calibrate_absmax(inp.x_cal))


@pytest.mark.parametrize("T_,K,ld", [(1, 16, 16), (37, 48, 48), (5, 80, 96), (300, 528, 536),
                                    # wide rows (257 and 313 channel groups) and a ragged one
                                    (200, 16400, 16408), (30, 20000, 20000), (513, 4112, 4120)])
def test_calibrate_ragged_and_strided(sq, dev, orc, T_, K, ld):
    x = W.random_f16(100 + K, T_, ld, scale=4.0)
    xv = T(x, dev)[:, :K]
    ax = sq.calibrate(xv)
    assert bits_equal(H(ax), orc.calibrate_absmax(np.ascontiguousarray(x[:, :K])))


@pytest.mark.parametrize("T_", [1025, 3000])
def test_calibrate_sliced_and_negative_zero(sq, dev, orc, T_):
    """More tokens than one workgroup takes (slices combined with atomics), a
    ragged last slice, K not a multiple of 64, a row stride; and accumulation
    onto -0.0 entries, which count as zero in both launch forms."""
    import torch
    K, ld = 208, 224
    x = W.random_f16(900 + T_, T_, ld, scale=3.0)
    xv = T(x, dev)[:, :K]
    ax = sq.calibrate(xv)
    assert bits_equal(H(ax), orc.calibrate_absmax(np.ascontiguousarray(x[:, :K])))
    for t in (T_, 100):
        buf = torch.full((K,), -0.0, device=dev)
        sq.sq_calibrate_absmax(xv[:t], buf, accumulate=True)
        assert bits_equal(H(buf), orc.calibrate_absmax(np.ascontiguousarray(x[:t, :K])))


def test_calibrate_nonfinite_and_empty(sq, dev, orc):
    import torch
    x = W.random_f16(7, 64, 64)
    x[3, 5] = np.nan
    x[60, 9] = -np.inf
    ax = sq.calibrate(T(x, dev))
    ref = orc.calibrate_absmax(x)
    assert bits_equal(np.isnan(H(ax)), np.isnan(ref)) and np.isinf(H(ax)[9])
    assert bits_equal(H(ax)[~np.isnan(ref)], ref[~np.isnan(ref)])
    # T = 0: zeros, or unchanged when accumulating
    buf = torch.full((64,), 3.0, device=dev)
    sq.sq_calibrate_absmax(T(x, dev)[:0], buf, accumulate=True)
    assert np.all(H(buf) == 3.0)
    sq.sq_calibrate_absmax(T(x, dev)[:0], buf, accumulate=False)
    assert np.all(H(buf) == 0.0)


# ---- A2 + A3 fold ----------------------------------------------------------------------

FOLD_CASES = [("tiny", 0.5), ("tiny", 0.0), ("tiny", 1.0), ("qkv4096", 0.5), ("qkv4096", 0.25),
              ("qkv4096", 1.0), ("down11008", 0.5), ("down11008", 0.8), ("decode8192", 0.5),
              ("prefill8192x3", 0.5)]


@pytest.mark.parametrize("name,alpha", FOLD_CASES)
def test_fold_matches_oracle(sq, dev, orc, name, alpha):
    wl, inp = wl_inputs(name, m=16 if name != "tiny" else None)
    print(f"[fold] {name} alpha={alpha} K={wl.K} N={wl.N}", flush=True)
    ax = orc.calibrate_absmax(inp.x_cal)
    w = inp.w
    f = sq.fold(T(w, dev), T(ax, dev), alpha)
    s, inv, st = orc.smoothing_factors(ax, orc.row_absmax(w), alpha)
    assert st == 0
    assert bits_equal(H(f.smooth), s)
    assert bits_equal(H(f.inv_smooth), inv)
    wq, wsc = orc.fold_quant_weights(w, s)
    assert bits_equal(H(f.w_scale), wsc)
    g = H(f.wq)
    assert np.array_equal(unpack(g, wl.N, wl.K), wq)
    assert padding_is_zero(g, wl.N, wl.K)


@pytest.mark.parametrize("alpha", [0.5, 0.25, 0.75, 0.8])
def test_smoothing_factors_random_statistics(sq, dev, orc, alpha):
    """s and 1/s for 131056 channels of random positive statistics, bit for bit
    against the oracle.  The kernel forms s_j in double (square roots at
    alpha = 1/2, the device's pow otherwise) and the oracle with the host's
    pow; both are within about one double ulp of the exact value, so the
    rounded floats agree unless that value lies within ~2^-52 of a float
    rounding boundary: this sample checks it on many more channels than the
    workloads have.  ax is a float drawn log-uniformly over [2^-24, 2^16), aw
    every kind of positive finite fp16 magnitude (subnormals included), held
    in a one-column W of row stride 8."""
    import torch
    K = 131056
    rng = np.random.default_rng(2000 + int(alpha * 100))
    ax = np.exp2(rng.uniform(-24.0, 16.0, K)).astype(np.float32)
    bits = rng.integers(1, 0x7C00, K).astype(np.uint16)          # +subnormal .. 65504
    sign = rng.integers(0, 2, K).astype(np.uint16) << 15
    w = np.zeros((K, 8), np.float16)
    w[:, 0] = (bits | sign).view(np.float16)
    aw = np.abs(w[:, 0].astype(np.float32))
    ref_s, ref_inv, st = orc.smoothing_factors(ax, aw, alpha)
    assert st == 0
    s_, inv_ = sq.smoothing_factors(T(w, dev)[:, :1], T(ax, dev), alpha)
    gs, gi = H(s_), H(inv_)
    nbad = int(np.sum(gs.view(np.uint32) != ref_s.view(np.uint32)))
    print(f"[factors] alpha={alpha}: {K - nbad}/{K} bit-equal", flush=True)
    assert bits_equal(gs, ref_s) and bits_equal(gi, ref_inv)


def test_fold_given_factors_and_consumer_slices(sq, dev, orc):
    """One smoothed X feeding three projections: the fold of the concatenated
    weights equals three folds with the shared factors (smooth_in)."""
    K = 256
    ws = [W.random_f16(200 + i, K, n, 0.015) for i, n in enumerate((96, 40, 136))]
    wcat = np.concatenate(ws, axis=1)
    ax = orc.calibrate_absmax(W.random_f16(210, 64, K, 5.0))
    fcat = sq.fold(T(wcat, dev), T(ax, dev), 0.5)
    wq_cat = unpack(H(fcat.wq), wcat.shape[1], K)
    ws_cat = H(fcat.w_scale)
    off = 0
    for w in ws:
        f1 = sq.fold(T(w, dev), None, 0.5, smooth_in=fcat.smooth)
        n = w.shape[1]
        assert np.array_equal(unpack(H(f1.wq), n, K), wq_cat[off:off + n])
        assert bits_equal(H(f1.w_scale), ws_cat[off:off + n])
        assert bits_equal(H(f1.smooth), H(fcat.smooth))
        q1, s1 = orc.fold_quant_weights(w, H(fcat.smooth))
        assert np.array_equal(unpack(H(f1.wq), n, K), q1)
        off += n


@pytest.mark.parametrize("K,N,ldw", [(16, 1, 8), (48, 13, 16), (272, 100, 104), (528, 64, 64),
                                     (1040, 520, 520), (272, 4093, 4096), (64, 4097, 4104)])
def test_fold_ragged_and_strided(sq, dev, orc, K, N, ldw):
    w = W.random_f16(300 + N, K, ldw, 0.05)
    ax = orc.calibrate_absmax(W.random_f16(301, 20, K, 3.0))
    f = sq.fold(T(w, dev)[:, :N], T(ax, dev), 0.5)
    wc = np.ascontiguousarray(w[:, :N])
    s, inv, _ = orc.smoothing_factors(ax, orc.row_absmax(wc), 0.5)
    wq, wsc = orc.fold_quant_weights(wc, s)
    assert bits_equal(H(f.smooth), s)
    g = H(f.wq)
    assert np.array_equal(unpack(g, N, K), wq) and bits_equal(H(f.w_scale), wsc)
    assert padding_is_zero(g, N, K)


def test_fold_sequence_reuses_scratch(sq, dev, orc):
    """Folds of different widths in a row (one pass over W up to 4096 output
    channels, two beyond): the column-maxima scratch is reused, grown and
    cleared between them, and every fold still matches the oracle."""
    for i, (K, N) in enumerate([(272, 520), (272, 96), (1040, 1000), (64, 4200), (272, 3000),
                                (272, 3000)]):
        w = W.random_f16(1300 + i, K, N, 0.05)
        ax = orc.calibrate_absmax(W.random_f16(1400 + i, 24, K, 3.0))
        f = sq.fold(T(w, dev), T(ax, dev), 0.5)
        s_, _, _ = orc.smoothing_factors(ax, orc.row_absmax(w), 0.5)
        wq, wsc = orc.fold_quant_weights(w, s_)
        assert np.array_equal(unpack(H(f.wq), N, K), wq), (K, N)
        assert bits_equal(H(f.w_scale), wsc), (K, N)


def test_fold_degenerate_channels(sq, dev, orc):
    """Dead activation channels and all-zero weight rows take s = 1; an
    all-zero output column gets scale 0 and codes 0."""
    K, N = 64, 48
    w = W.random_f16(400, K, N, 0.02)
    w[5, :] = 0
    w[:, 7] = 0
    ax = orc.calibrate_absmax(W.random_f16(401, 16, K, 2.0))
    ax[9] = 0
    f = sq.fold(T(w, dev), T(ax, dev), 0.5)
    s, inv, _ = orc.smoothing_factors(ax, orc.row_absmax(w), 0.5)
    assert H(f.smooth)[5] == 1.0 and H(f.smooth)[9] == 1.0
    wq, wsc = orc.fold_quant_weights(w, s)
    g = unpack(H(f.wq), N, K)
    assert np.array_equal(g, wq) and bits_equal(H(f.w_scale), wsc)
    assert H(f.w_scale)[7] == 0 and np.all(g[7] == 0)


def test_fold_data_errors_report_status(sq, dev, orc):
    """Bad statistics or factors come back as data errors after the queued
    fold has run on them (outputs unspecified; the stream stays usable)."""
    import torch
    K, N = 64, 32
    w = W.random_f16(500, K, N, 0.02)
    ax = orc.calibrate_absmax(W.random_f16(501, 8, K))

    def run(w_, ax_, alpha=0.5, sin=None):
        f = sq.Folded(torch.empty(K, device=dev), torch.empty(K, device=dev),
                      torch.full((packed_bytes(N, K),), 55, dtype=torch.int8, device=dev),
                      torch.empty(N, device=dev), K, N)
        with pytest.raises(sq.SqError) as ei:
            sq.sq_smooth_fold_weights(T(w_, dev), None if ax_ is None else T(ax_, dev), alpha,
                                      None if sin is None else T(sin, dev), f.smooth,
                                      f.inv_smooth, f.wq, f.w_scale)
        torch.cuda.synchronize()
        return ei.value.status

    a = ax.copy(); a[3] = np.nan
    assert run(w, a) == sq.SQ_ERR_NONFINITE
    a = ax.copy(); a[3] = np.inf
    assert run(w, a) == sq.SQ_ERR_NONFINITE
    a = ax.copy(); a[3] = -1.0
    assert run(w, a) == sq.SQ_ERR_NONFINITE
    w2 = w.copy(); w2[4, 6] = np.inf
    assert run(w2, ax) == sq.SQ_ERR_NONFINITE
    w2 = w.copy(); w2[4, 6] = np.nan
    assert run(w2, ax) == sq.SQ_ERR_NONFINITE
    a = ax.copy(); a[3] = 3e38
    assert run(w, a, alpha=1.0) == sq.SQ_ERR_RANGE        # 1/s subnormal
    sin = np.ones(K, np.float32); sin[2] = 0.0
    assert run(w, None, sin=sin) == sq.SQ_ERR_RANGE
    sin = np.ones(K, np.float32); sin[2] = -2.0
    assert run(w, None, sin=sin) == sq.SQ_ERR_NONFINITE
    f = sq.fold(T(w, dev), T(ax, dev), 0.5)
    s_, _, _ = orc.smoothing_factors(ax, orc.row_absmax(w), 0.5)
    wq, wsc = orc.fold_quant_weights(w, s_)
    assert np.array_equal(unpack(H(f.wq), N, K), wq) and bits_equal(H(f.w_scale), wsc)


# ---- A4 per-token quantization --------------------------------------------------------

@pytest.mark.parametrize("name", ALL)
def test_quant_matches_oracle(sq, dev, orc, name):
    wl, inp = wl_inputs(name)
    print(f"[quant] {name} M={inp.x.shape[0]} K={wl.K}", flush=True)
    ax = orc.calibrate_absmax(inp.x_cal)
    _, inv, _ = orc.smoothing_factors(ax, orc.row_absmax(inp.ws[0][:, :64]), wl.alpha)
    xq, xs = sq.quant(T(inp.x, dev), T(inv, dev))
    rq, rs = orc.quant_act_per_token(inp.x, inv)
    assert bits_equal(H(xs), rs)
    g = H(xq)
    assert np.array_equal(unpack(g, inp.x.shape[0], wl.K), rq)
    assert padding_is_zero(g, inp.x.shape[0], wl.K)


# up to 64 tokens and K <= 16384 the one-token-per-workgroup form runs (one or
# two chunks per lane); beyond 64 tokens the row-group form (2 rows per
# workgroup up to 512 tokens, 4 beyond; 2 waves per row up to K = 8192; up to
# 12288, 3 waves (8 waves of 3 chunks at most 512 tokens); 4 up to 16384), and
# past K = 16384 the 8-row streaming form
@pytest.mark.parametrize("M,K,ld", [(1, 16, 16), (3, 48, 56), (17, 2064, 2064), (2, 4112, 4128),
                                    (4, 11008, 11024), (64, 16384, 16384), (33, 8192, 8192),
                                    (65, 4096, 4096), (64, 16400, 16400),
                                    (70, 16, 16), (100, 4096, 4104), (513, 1040, 1040),
                                    (300, 11008, 11024), (520, 8208, 8208), (600, 16384, 16392),
                                    (130, 16400, 16400),
                                    # above 512 tokens and K <= 8192: the 4-row column form, whole and
                                    # ragged chunk columns, M not a multiple of 4 or 16, strided rows
                                    (530, 2048, 2056), (1001, 4096, 4104), (777, 3088, 3088),
                                    (2050, 8176, 8192), (600, 8192, 8192), (515, 16, 16),
                                    # 8193..12288 channels: ragged and exact cover, both group shapes
                                    (700, 11008, 11024), (513, 9008, 9008), (600, 12288, 12288),
                                    (200, 12288, 12296), (90, 8208, 8208),
                                    (5, 32784, 32784), (2, 40000, 40000), (1, 131056, 131056)])
def test_quant_ragged_long_and_strided(sq, dev, orc, M, K, ld):
    x = W.random_f16(600 + K, M, ld, 2.0)
    inv = W.random_scales(601, K, 0.05, 3.0)
    xq, xs = sq.quant(T(x, dev)[:, :K], T(inv, dev))
    rq, rs = orc.quant_act_per_token(np.ascontiguousarray(x[:, :K]), inv)
    g = H(xq)
    assert bits_equal(H(xs), rs) and np.array_equal(unpack(g, M, K), rq)
    assert padding_is_zero(g, M, K)


def test_quant_ties_and_degenerate_rows(sq, dev, orc):
    row = np.array([127, 2.5, 3.5, -2.5, 0.5, 1.5, -0.5, 126.5,
                    -126.5, 5.5, -5.5, 0.25, 7.5, -7.5, 64.5, 0], np.float16)
    x = np.zeros((5, 16), np.float16)
    x[0] = row
    x[2] = row
    x[2, 3] = np.nan
    x[3] = row
    x[3, 0] = np.inf
    x[4] = -row
    ones = np.ones(16, np.float32)
    xq, xs = sq.quant(T(x, dev), T(ones, dev))
    rq, rs = orc.quant_act_per_token(x, ones)
    g = unpack(H(xq), 5, 16)
    assert bits_equal(H(xs), rs) and np.array_equal(g, rq)
    assert g[0].tolist() == [127, 2, 4, -2, 0, 2, 0, 126, -126, 6, -6, 0, 8, -8, 64, 0]
    assert H(xs)[1] == 0 and np.isnan(H(xs)[2]) and np.isnan(H(xs)[3])


def overflow_mix(M, K, seed):
    """fp16 rows for a 1/s of 2^-120: even rows have every magnitude in
    [2^-6, 2^-2] or zero, so their scaled maximum is at most 2^-122 and the
    float multiplier 127 / a overflows; odd rows reach 2^4, a finite
    multiplier.  Every scaled value is a normal float or zero; every seventh
    channel is zero, some others negative zero."""
    rng = np.random.default_rng(seed)
    mag = 2.0 ** rng.uniform(-6.0, -2.0, size=(M, K))
    mag[1::2] *= 64.0
    x = (mag * rng.choice([-1.0, 1.0], size=(M, K))).astype(np.float16)
    x[:, ::7] = 0.0
    x[1::4, 3::5] = -0.0
    return x


# every quantizer form: one token per workgroup (5, 40), row groups with and
# without whole-row chunks (600 x 4096, 70 x 1024 / 300 x 1040, 520 x 8208),
# and the 8-row streaming form past K = 16384 (130 x 16400)
@pytest.mark.parametrize("M,K", [(5, 64), (40, 8192), (600, 4096), (70, 1024), (300, 1040),
                                 (520, 8208), (130, 16400)])
def test_quant_rows_whose_multiplier_overflows(sq, dev, orc, M, K):
    """A caller's tiny 1/s: rows whose maximum is below 127 / FLT_MAX take
    +-127 for nonzero values and 0 for zeros, as the oracle defines them."""
    x = overflow_mix(M, K, 900 + M)
    inv = np.full(K, 2.0 ** -120, np.float32)
    xq, xs = sq.quant(T(x, dev), T(inv, dev))
    rq, rs = orc.quant_act_per_token(x, inv)
    g = H(xq)
    assert bits_equal(H(xs), rs) and np.array_equal(unpack(g, M, K), rq)
    assert padding_is_zero(g, M, K)
    ev = rq[0::2]
    assert np.all(np.isin(ev, [-127, 0, 127])) and (ev == 0).any() and (ev == 127).any()


def test_fold_columns_whose_multiplier_overflows(sq, dev, orc):
    """The fold with a caller's factors of 2^-120 (the smallest magnitudes the
    factor checks accept are normal floats): even output channels' maxima
    fall below 127 / FLT_MAX."""
    K, N = 256, 200
    w = np.ascontiguousarray(overflow_mix(N, K, 950).T)
    s = np.full(K, 2.0 ** -120, np.float32)
    f = sq.fold(T(w, dev), T(np.ones(K, np.float32), dev), 0.5, smooth_in=T(s, dev))
    rq, rs = orc.fold_quant_weights(w, s)
    assert bits_equal(H(f.w_scale), rs)
    assert np.array_equal(unpack(H(f.wq), N, K), rq)
    assert np.all(np.isin(rq[0::2], [-127, 0, 127])) and (rq[0::2] == 0).any()


# ---- A5 + A6 the product -----------------------------------------------------------------

# token counts 1..64 run the decode kernels (1, 2, 3 or 4 activation row blocks;
# non-temporal weight loads up to 2 of them; at 9..32 tokens with 512 or more
# channel blocks, 2, 4 or 7 blocks per workgroup, also with a partial last
# workgroup); 65 and up the multi-block kernel over 64-token groups while the
# 256 x 128 tiles would number at most 64, beyond that the tile kernels
GEMM_SHAPES = [(1, 1, 16), (3, 5, 48), (17, 100, 80), (40, 100, 320), (49, 1000, 1088),
               (9, 64, 4096), (25, 33, 256), (32, 48, 1024),
               (16, 28672, 128), (9, 28672, 64), (24, 8192, 64), (32, 12304, 64), (20, 8200, 64),
               # 7 blocks per workgroup of 8 waves over more than one batch round, one and
               # two row blocks, a ragged last window
               (16, 28672, 2112), (32, 28672, 2112), (25, 28672, 1040),
               (64, 70, 4096), (65, 33, 64), (100, 200, 64), (128, 128, 4096),
               # mid-size batches (at most 64 tiles of 256 x 128): 64-token groups of the
               # multi-block kernel, 2 and 4 channel blocks, ragged tokens and channels
               (512, 4096, 1024), (200, 1000, 4160), (1000, 128, 256), (320, 2048, 512),
               (65, 4096, 2048),
               (130, 129, 1040), (256, 384, 2048), (1, 28672, 128), (16, 300, 8192), (513, 77, 112),
               # 256 x 128 tiles (65..256 of them): ragged tokens, channels and k windows
               (300, 8200, 1040), (1100, 1950, 208), (600, 4000, 80), (2100, 1030, 64),
               # the switch: 64 tiles (multi-block kernel) and 65 (tile kernel)
               (256, 8192, 64), (256, 8320, 64),
               # 256 x 256 tiles (their rounds of 256 CUs beat the 256 x 128 ones'): ragged M,
               # N (a partial row block) and K, and a full-width one
               (4000, 4040, 80), (4096, 8192, 64)]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_i32_bit_exact(sq, dev, orc, M, N, K):
    xq = W.random_i8(700 + M, M, K, -128, 127)
    wq = W.random_i8(701 + N, N, K, -128, 127)
    acc = sq.gemm(T(pack(xq), dev), None, T(pack(wq), dev), None, M, N, K, out_kind=sq.SQ_OUT_I32)
    assert np.array_equal(H(acc), orc.gemm_i32(xq, wq))


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_f16_epilogue(sq, dev, orc, M, N, K):
    xq = W.random_i8(800 + M, M, K)
    wq = W.random_i8(801 + N, N, K)
    xs = W.random_scales(802, M, 1e-3, 2e-2)
    ws = W.random_scales(803, N, 1e-3, 2e-2)
    y = sq.gemm(T(pack(xq), dev), T(xs, dev), T(pack(wq), dev), T(ws, dev), M, N, K)
    assert_f16_close(H(y), orc.dequant(orc.gemm_i32(xq, wq), xs, ws))


def test_gemm_extreme_sums_and_strided_output(sq, dev, orc):
    import torch
    K = 131056
    xq = np.full((2, K), 127, np.int8)
    xq[1] = -128
    wq = np.full((3, K), -127, np.int8)
    wq[1] = 127
    wq[2] = -128
    acc = sq.gemm(T(pack(xq), dev), None, T(pack(wq), dev), None, 2, 3, K, out_kind=sq.SQ_OUT_I32)
    assert np.array_equal(H(acc), orc.gemm_i32(xq, wq))
    # output rows with a stride larger than N
    xq = W.random_i8(900, 40, 64)
    wq = W.random_i8(901, 24, 64)
    xs = W.random_scales(902, 40)
    ws = W.random_scales(903, 24)
    big = torch.full((40, 32), 7.0, dtype=torch.float16, device=dev)
    sq.sq_w8a8_gemm(T(pack(xq), dev), T(xs, dev), T(pack(wq), dev), T(ws, dev), big[:, :24], 64)
    out = H(big)
    assert np.all(out[:, 24:] == 7.0)
    assert_f16_close(out[:, :24], orc.dequant(orc.gemm_i32(xq, wq), xs, ws))


def test_gemm_mid_path_at_max_k(sq, dev, orc):
    """65 tokens (the multi-block kernel over 64-token groups, two groups) at
    the largest K the library takes: window offsets up to 2047 KiB per row
    block, int32 sums near their bound."""
    M, N, K = 65, 40, 131056
    xq = W.random_i8(920, M, K, -128, 127)
    wq = W.random_i8(921, N, K, -128, 127)
    acc = sq.gemm(T(pack(xq), dev), None, T(pack(wq), dev), None, M, N, K, out_kind=sq.SQ_OUT_I32)
    assert np.array_equal(H(acc), orc.gemm_i32(xq, wq))
    xs = W.random_scales(922, M, 1e-6, 1e-5)
    ws = W.random_scales(923, N, 1e-6, 1e-5)
    y = sq.gemm(T(pack(xq), dev), T(xs, dev), T(pack(wq), dev), T(ws, dev), M, N, K)
    assert_f16_close(H(y), orc.dequant(orc.gemm_i32(xq, wq), xs, ws))


def test_gemm_nan_row_propagates(sq, dev, orc):
    xq = W.random_i8(910, 4, 64)
    wq = W.random_i8(911, 8, 64)
    xs = W.random_scales(912, 4)
    xs[2] = np.nan
    ws = W.random_scales(913, 8)
    y = H(sq.gemm(T(pack(xq), dev), T(xs, dev), T(pack(wq), dev), T(ws, dev), 4, 8, 64))
    assert np.isnan(y[2]).all() and np.isfinite(np.delete(y, 2, axis=0)).all()


# ---- the whole chain ------------------------------------------------------------------------

# (workload, alpha, tokens served or None for the workload's own count).  The
# decode workload is also served at 1 and 4 tokens: its first 1 or 4 tokens
# against the same 8192 x 28672 folded weights, as the benchmark times them.
# Rows compared: every row up to 64 tokens; beyond, tile_rows (every 256-token
# tile row, both sides of every tile boundary, every wave position).
E2E = [("tiny", 0.5, None), ("qkv4096", 0.5, None), ("down11008", 0.5, None),
       ("down11008", 0.8, None), ("decode8192", 0.5, 1), ("decode8192", 0.5, 4),
       ("decode8192", 0.5, None), ("prefill8192x3", 0.5, None)]


@pytest.mark.parametrize("name,alpha,m", E2E)
def test_end_to_end(sq, dev, orc, name, alpha, m):
    wl, inp = wl_inputs(name)
    x = inp.x if m is None else np.ascontiguousarray(inp.x[:m])
    M = x.shape[0]
    print(f"[e2e] {name} alpha={alpha} M={M} K={wl.K} N={wl.N}", flush=True)
    xg = T(x, dev)
    ax = sq.calibrate(T(inp.x_cal, dev))
    f = sq.fold(T(inp.w, dev), ax, alpha)
    xq, xs = sq.quant(xg, f.inv_smooth)
    y = sq.gemm(xq, xs, f.wq, f.w_scale, M, wl.N, wl.K)
    acc = sq.gemm(xq, xs, f.wq, f.w_scale, M, wl.N, wl.K, out_kind=sq.SQ_OUT_I32)
    rows = tile_rows(M, seed=17)
    print(f"[e2e] {name}: comparing {len(rows)} of {M} token rows", flush=True)
    ref = orc.smoothed_linear(x, inp.x_cal, inp.w, alpha, rows=rows)
    assert ref.status == 0
    assert bits_equal(H(ax), ref.ax)
    assert bits_equal(H(f.smooth), ref.s) and bits_equal(H(f.inv_smooth), ref.inv_s)
    assert bits_equal(H(f.w_scale), ref.w_scale)
    assert np.array_equal(unpack(H(f.wq), wl.N, wl.K), ref.wq)
    assert bits_equal(H(xs), ref.x_scale)
    assert np.array_equal(unpack(H(xq), M, wl.K), ref.xq)
    accg = H(acc)[rows]
    assert np.array_equal(accg, ref.acc)
    err = assert_f16_close(H(y)[rows], ref.y64)
    print(f"[e2e] {name}: max rel err {err.max():.3g}, "
          f"{np.mean(H(y)[rows].astype(np.float64) == ref.y16.astype(np.float64)):.4f} bit-equal",
          flush=True)


def test_repeat_runs_are_bitwise_identical(sq, dev, orc):
    wl, inp = wl_inputs("qkv4096")
    ax1 = H(sq.calibrate(T(inp.x_cal, dev)))
    ax2 = H(sq.calibrate(T(inp.x_cal, dev)))
    assert bits_equal(ax1, ax2)
    f = sq.fold(T(inp.w, dev), T(ax1, dev), 0.5)
    xq, xs = sq.quant(T(inp.x, dev), f.inv_smooth)
    y1 = H(sq.gemm(xq, xs, f.wq, f.w_scale, wl.M, wl.N, wl.K))
    y2 = H(sq.gemm(xq, xs, f.wq, f.w_scale, wl.M, wl.N, wl.K))
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))


# ---- layout helpers -------------------------------------------------------------------------

@pytest.mark.parametrize("rows,K,ld", [(1, 16, 16), (17, 80, 96), (64, 4096, 4096), (33, 11008, 11024)])
def test_pack_unpack_helpers(sq, dev, rows, K, ld):
    import torch
    codes = W.random_i8(1000 + rows, rows, ld, -128, 127)
    src = T(codes, dev)[:, :K]
    packed = sq.pack_i8(src)
    ref = pack(np.ascontiguousarray(codes[:, :K]))
    assert np.array_equal(H(packed)[:ref.size], ref)
    back = torch.full((rows, ld), 9, dtype=torch.int8, device=dev)
    sq.sq_unpack_i8(packed, back[:, :K])
    out = H(back)
    assert np.array_equal(out[:, :K], codes[:, :K]) and np.all(out[:, K:] == 9)


def test_gemm_wide_tile_path_strided_output(sq, dev, orc):
    """The 256 x 256 tile kernel (4000 x 4040: 256 wide tiles in one round
    against 512 narrow ones in two) with output rows of stride 4049 starting 3
    elements into the buffer, so the 16-byte row stores are off and every
    output takes the element path; and with an aligned stride."""
    import torch
    M, N, K = 4000, 4040, 64
    xq = W.random_i8(1200, M, K)
    wq = W.random_i8(1201, N, K)
    xs = W.random_scales(1202, M)
    ws = W.random_scales(1203, N)
    ref = orc.dequant(orc.gemm_i32(xq, wq), xs, ws)
    for ldy, off in ((4049, 3), (4048, 8)):
        big = torch.full((M * ldy + 64,), 5.0, dtype=torch.float16, device=dev)
        view = big[off:off + M * ldy].view(M, ldy)[:, :N]
        sq.sq_w8a8_gemm(T(pack(xq), dev), T(xs, dev), T(pack(wq), dev), T(ws, dev), view, K)
        out = H(big)
        assert np.all(out[:off] == 5.0) and np.all(out[off + M * ldy:] == 5.0)
        out = out[off:off + M * ldy].reshape(M, ldy)
        assert np.all(out[:, N:] == 5.0)
        assert_f16_close(out[:, :N], ref)


@pytest.mark.parametrize("M,N,K", [(4000, 4040, 1040), (4096, 4096, 2064)])
def test_gemm_wide_tile_path_deep_k_full_output(sq, dev, orc, M, N, K):
    """The 256 x 256 tile kernel over more k windows than its 8-deep LDS ring
    holds (17 and 33 windows, the last one ragged), so the ring wraps and the
    steady-state waits run: every int32 sum and every fp16 output against
    the oracle, ragged tiles included (4000 x 4040)."""
    print(f"[gemm wide] {M}x{N}x{K}", flush=True)
    xq = W.random_i8(1300 + K, M, K, -128, 127)
    wq = W.random_i8(1301 + K, N, K, -128, 127)
    ref = gemm_i32_threads(orc, xq, wq)
    px, pw = T(pack(xq), dev), T(pack(wq), dev)
    acc = sq.gemm(px, None, pw, None, M, N, K, out_kind=sq.SQ_OUT_I32)
    assert np.array_equal(H(acc), ref)
    xs = W.random_scales(1302, M, 1e-5, 1e-4)
    ws = W.random_scales(1303, N, 1e-5, 1e-4)
    y = sq.gemm(px, T(xs, dev), pw, T(ws, dev), M, N, K)
    assert_f16_close(H(y), orc.dequant(ref, xs, ws))


@pytest.mark.parametrize("M,N,ldy,off", [(100, 72, 80, 0), (300, 130, 136, 8), (257, 64, 72, 4),
                                         (300, 8200, 8208, 8), (2100, 1030, 1040, 4)])
def test_gemm_large_m_strided_and_offset_output(sq, dev, orc, M, N, ldy, off):
    """Token counts above 64, on the multi-block kernel over 64-token groups
    (the first three) and on the 256 x 128 tile kernel (65 and 81 tiles), with
    output rows of stride ldy >= N, starting `off` elements into the buffer
    (8- or 16-byte aligned or not)."""
    import torch
    K = 192
    xq = W.random_i8(1100 + M, M, K)
    wq = W.random_i8(1101 + N, N, K)
    xs = W.random_scales(1102, M)
    ws = W.random_scales(1103, N)
    big = torch.full((M * ldy + 64,), 5.0, dtype=torch.float16, device=dev)
    view = big[off:off + M * ldy].view(M, ldy)[:, :N]
    sq.sq_w8a8_gemm(T(pack(xq), dev), T(xs, dev), T(pack(wq), dev), T(ws, dev), view, K)
    out = H(big)[off:off + M * ldy].reshape(M, ldy)
    assert_f16_close(out[:, :N], orc.dequant(orc.gemm_i32(xq, wq), xs, ws))
    assert np.all(out[:, N:] == 5.0) and np.all(H(big)[:off] == 5.0)
