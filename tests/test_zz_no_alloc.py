"""The allocation-free fold (sq_smooth_fold_weights_noalloc) through the C ABI
against the allocating fold (sq_smooth_fold_weights) on the same inputs: s,
1/s, the packed codes and the scales bit for bit, on two calls in a row, the
second with a smaller input (the static scratch keeps the first call's column
maxima and status, which the second must not see); data errors come back
with the same status; a width beyond the scratch is refused.
"""
import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import w8a8_post_quantization_sq_amd as sq
    return torch, sq, sq.lib(), torch.device("cuda:0")


def _fold_both(env, w, ax, alpha=0.5, smooth_in=None):
    """(allocating, allocation-free) results: status, s, 1/s, codes, scales."""
    torch, sq, L, dev = env
    K, N = w.shape
    wt = torch.from_numpy(w).to(dev)
    axt = None if ax is None else torch.from_numpy(ax).to(dev)
    sit = None if smooth_in is None else torch.from_numpy(smooth_in).to(dev)
    hs = torch.cuda.current_stream(dev).cuda_stream
    outs = []
    for fn in (L.sq_smooth_fold_weights, L.sq_smooth_fold_weights_noalloc):
        s = torch.full((K,), -7.0, device=dev)
        inv = torch.full((K,), -7.0, device=dev)
        wq = torch.full((sq.packed_bytes(N, K),), 99, dtype=torch.int8, device=dev)
        ws = torch.full((N,), -7.0, device=dev)
        st = fn(wt.data_ptr(), K, N, N, None if axt is None else axt.data_ptr(), float(alpha),
                None if sit is None else sit.data_ptr(), s.data_ptr(), inv.data_ptr(),
                wq.data_ptr(), ws.data_ptr(), hs)
        torch.cuda.synchronize()
        outs.append((st, s.cpu().numpy(), inv.cpu().numpy(), wq.cpu().numpy(),
                     ws.cpu().numpy()))
    return outs


def _same(a, b):
    return all(np.array_equal(x.view(np.uint8), y.view(np.uint8)) for x, y in zip(a[1:], b[1:]))


@pytest.mark.parametrize("first,second", [((1040, 3000), (272, 520)), ((4096, 4096), (64, 48))])
def test_noalloc_fold_matches_the_fold_twice(env, first, second):
    for i, (K, N) in enumerate((first, second)):
        print(f"[noalloc] call {i + 1}: K={K} N={N}", flush=True)
        w = W.random_f16(2100 + K + N, K, N, 0.05)
        ax = np.abs(W.random_f16(2200 + K, 32, K, 4.0).astype(np.float32)).max(axis=0)
        ax[3] = 0.0                                   # a dead channel: s = 1
        a, b = _fold_both(env, w, ax)
        assert a[0] == 0 and b[0] == 0
        assert _same(a, b)


def test_noalloc_fold_workload_and_given_factors(env):
    """The q/k/v-style workload's weights, then a smaller fold with given
    factors (the multi-consumer form)."""
    wl = W.WORKLOADS["qkv4096"]
    inp = W.generate(wl, m=16)
    ax = np.abs(inp.x_cal.astype(np.float32)).max(axis=0)
    a, b = _fold_both(env, inp.w, ax, wl.alpha)
    assert a[0] == 0 and b[0] == 0 and _same(a, b)
    sin = a[1][:1024].copy()
    w2 = np.ascontiguousarray(inp.w[:1024, :200])
    a, b = _fold_both(env, w2, None, smooth_in=sin)
    assert a[0] == 0 and b[0] == 0 and _same(a, b)


def test_noalloc_fold_data_errors_then_a_clean_call(env):
    """NaN and out-of-range statistics give the fold's statuses; the status
    word is cleared, so the next clean call returns SQ_OK."""
    torch, sq, L, dev = env
    K, N = 64, 40
    w = W.random_f16(2300, K, N, 0.02)
    ax = np.abs(W.random_f16(2301, 8, K).astype(np.float32)).max(axis=0)
    bad = ax.copy()
    bad[5] = np.nan
    a, b = _fold_both(env, w, bad)
    assert a[0] == sq.SQ_ERR_NONFINITE and b[0] == sq.SQ_ERR_NONFINITE
    big = ax.copy()
    big[7] = 3e38
    a, b = _fold_both(env, w, big, alpha=1.0)
    assert a[0] == sq.SQ_ERR_RANGE and b[0] == sq.SQ_ERR_RANGE
    a, b = _fold_both(env, w, ax)
    assert a[0] == 0 and b[0] == 0 and _same(a, b)


def test_noalloc_fold_refuses_a_width_beyond_its_scratch(env):
    torch, sq, L, dev = env
    K, N = 16, sq.SQ_NOALLOC_MAX_N + 8
    w = torch.zeros((K, N), dtype=torch.float16, device=dev)
    ax = torch.ones(K, device=dev)
    s = torch.empty(K, device=dev)
    inv = torch.empty(K, device=dev)
    wq = torch.zeros(sq.packed_bytes(N, K), dtype=torch.int8, device=dev)
    ws = torch.zeros(N, device=dev)
    st = L.sq_smooth_fold_weights_noalloc(w.data_ptr(), K, N, N, ax.data_ptr(), 0.5, None,
                                          s.data_ptr(), inv.data_ptr(), wq.data_ptr(),
                                          ws.data_ptr(), torch.cuda.current_stream(dev).cuda_stream)
    assert st == sq.SQ_ERR_SHAPE
