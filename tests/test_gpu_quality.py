"""The alpha sweep on the GPU path: every quality measure computed from the
library's outputs (factors, codes, scales, fp16 layer output) must equal the
oracle's (oracle/quality.py) for the same inputs, for S = I and for alpha in
{0, .25, .5, .75, .8, 1}, with held-out and in-sample calibration.

The factors, codes and scales are bit-exact, so the weight and activation
measures are equal to the last bit; the layer error compares fp16 outputs
that agree to 2^-10 per element, which bounds how far the summed measure may
move (see the assertion).
The sweep's table is printed (run pytest with -s to see it).
"""
import numpy as np
import pytest

import workloads as W
from layout import unpack

pytestmark = pytest.mark.gpu

ALPHAS = [None, 0.0, 0.25, 0.5, 0.75, 0.8, 1.0]
MEASURES = ["layer_error", "weight_recon_error", "act_difficulty", "weight_difficulty",
            "static_clip_fraction"]


@pytest.fixture(scope="module")
def sq():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import w8a8_post_quantization_sq_amd as m
    m.lib()
    return m


def T(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def H(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def gpu_measures(sq, q, orc, x, x_cal, w, stat, alpha, rows, ref):
    """One sweep point on the GPU: calibrate on `stat`, fold, quantize the
    sampled rows, product in fp16; the measures from what the GPU returned."""
    import torch
    dev = torch.device("cuda:0")
    K, N = w.shape
    wt = T(w, dev)
    if alpha is None:
        f = sq.fold(wt, None, 0.0, smooth_in=torch.ones(K, device=dev))
    else:
        f = sq.fold(wt, sq.calibrate(T(stat, dev)), alpha)
    xr = x[rows]
    xq, xs = sq.quant(T(xr, dev), f.inv_smooth)
    y = sq.gemm(xq, xs, f.wq, f.w_scale, len(rows), N, K)
    s, inv = H(f.smooth), H(f.inv_smooth)
    wq = unpack(H(f.wq), N, K)
    return {
        "layer_error": q.layer_error(H(y).astype(np.float64), ref),
        "weight_recon_error": q.weight_recon_error(w, s, wq, H(f.w_scale)),
        "act_difficulty": q.activation_difficulty(x, inv),
        "weight_difficulty": q.weight_difficulty(w, s),
        "static_clip_fraction": q.static_clip_fraction(x, x_cal, inv),
    }


@pytest.mark.parametrize("name,nrows", [("tiny", None), ("qkv4096", 16), ("down11008", 12)])
def test_alpha_sweep_matches_oracle(sq, orc, name, nrows):
    from oracle import quality as q
    wl = W.WORKLOADS[name]
    inp = W.generate(wl)
    x, x_cal, w = inp.x, inp.x_cal, inp.w
    M = x.shape[0]
    if nrows is None:
        rows = np.arange(M)
    else:   # seeded sample, always with the first and last token and the outlier tokens
        rng = np.random.default_rng(77)
        extra = np.zeros(0, np.int64) if inp.outlier_tokens is None else \
            np.asarray(inp.outlier_tokens[:4], np.int64)
        rows = np.unique(np.concatenate([np.array([0, M - 1], np.int64), extra,
                                         rng.choice(np.arange(1, M - 1), nrows, replace=False)]))
    ref_table = q.sweep(x, x_cal, w, ALPHAS, rows=rows)
    ref = orc.matmul_fp64(x[rows], w)
    print(f"\n[alpha sweep] {name}: {len(rows)} token rows for the layer error", flush=True)
    print(f"{'alpha/calibration':>20} " + " ".join(f"{m:>21}" for m in MEASURES), flush=True)
    for alpha in ALPHAS:
        for tag, stat in (("held_out", x_cal), ("in_sample", x)):
            key = f"{'I' if alpha is None else alpha}/{tag}"
            got = gpu_measures(sq, q, orc, x, x_cal, w, stat, alpha, rows, ref)
            want = ref_table[key]
            print(f"{key:>20} " + " ".join(f"{got[m]:21.6e}" for m in MEASURES), flush=True)
            for m in MEASURES[1:]:
                assert got[m] == want[m], (key, m, got[m], want[m])
            # fp16 outputs within 2^-10 of the oracle's (a few 1-ulp steps are
            # allowed): with a = y_gpu - ref, b = y_oracle - ref,
            # | |a|^2 - |b|^2 | <= |a - b| |a + b| <= 2^-10 |y| (2 |b| + 2^-10 |y|),
            # and |y| ~ |ref|, so relative to |ref|^2 the error measure moves by
            # at most 2^-10 (2 sqrt(err) + 2^-10)
            tol = 2.0 ** -10 * (2.0 * np.sqrt(want["layer_error"]) + 2.0 ** -10) * 1.01
            assert abs(got["layer_error"] - want["layer_error"]) <= tol, key
