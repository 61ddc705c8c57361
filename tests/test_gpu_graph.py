"""The serving calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

A serving loop that cannot afford a host launch per kernel records the layer
once and replays it.  The serving calls (per-token quantization, the fused
normalization + quantization, the 4-bit rotated quantization and both
products) launch kernels only: no allocation, no memset, no host wait.  Each
case records the calls on static buffers, then replays the graph several
times with new inputs copied into those buffers, with eager work on the same
stream between the replays, and requires every replay to equal the eager
calls on the same input bit for bit (codes, scales and the fp16 or int32
output).  The first replay of the 8-bit layer is also compared with the
oracle on sampled token rows.
"""
import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu

REPLAYS = 3


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


def same_bits(a, b):
    a, b = np.asarray(a), np.asarray(b)
    if a.dtype.kind == "f":
        u = np.uint32 if a.dtype == np.float32 else np.uint16
        return np.array_equal(a.view(u), b.view(u))
    return np.array_equal(a, b)


def capture(fn):
    """fn() recorded in a graph on a side stream, after one eager warm-up
    there (the pattern torch asks for before capture)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def inputs(seed, M, K, N):
    x = [W.random_f16(seed + r, M, K) for r in range(REPLAYS)]
    x_cal = W.random_f16(seed + 100, 64, K)
    w = W.random_f16(seed + 200, K, N, 0.02)
    return x, x_cal, w


@pytest.mark.parametrize("M,K,N", [(2048, 4096, 4096), (300, 1040, 520), (1, 8192, 4096),
                                   (16, 8192, 3584), (5, 4096, 1000)])
def test_layer_graph_replays_equal_eager(sq, dev, orc, M, K, N):
    """Quantization + W8A8 product (fp16 out) recorded once, replayed on new
    tokens; 2048 tokens take the tile kernel, 300 the multi-block kernel over
    64-token groups, 1 token the one-token decode kernel, 5-16 tokens the
    multi-block decode kernel."""
    import torch
    from test_gpu_parity import assert_f16_close, tile_rows
    print(f"[graph] layer M={M} K={K} N={N}", flush=True)
    xs_np, x_cal, w = inputs(7000 + M, M, K, N)
    f = sq.fold(T(w, dev), sq.calibrate(T(x_cal, dev)), 0.5)
    x = torch.empty((M, K), dtype=torch.float16, device=dev)
    x.copy_(T(xs_np[0], dev))
    xq = torch.empty(sq.packed_bytes(M, K), dtype=torch.int8, device=dev)
    xsc = torch.empty(M, dtype=torch.float32, device=dev)
    y = torch.empty((M, N), dtype=torch.float16, device=dev)

    def layer():
        sq.sq_quant_act_per_token(x, f.inv_smooth, xq, xsc)
        sq.sq_w8a8_gemm(xq, xsc, f.wq, f.w_scale, y, K)

    g = capture(layer)
    for r in range(REPLAYS):
        xr = T(xs_np[r], dev)
        x.copy_(xr)
        g.replay()
        got = (H(xq), H(xsc), H(y))
        # eager calls on the same tokens, plus unrelated work on the stream
        eq, es = sq.quant(xr, f.inv_smooth)
        ey = sq.gemm(eq, es, f.wq, f.w_scale, M, N, K)
        _ = (xr.float() * 2.0).sum()
        assert same_bits(got[0], H(eq)), f"replay {r}: codes differ"
        assert same_bits(got[1], H(es)), f"replay {r}: scales differ"
        assert same_bits(got[2], H(ey)), f"replay {r}: output differs"
        if r == 0 and M * N * K <= 2048 * 4096 * 4096:
            rows = tile_rows(M, seed=3)
            ref = orc.smoothed_linear(xs_np[0], x_cal, w, 0.5, rows=rows)
            assert ref.status == 0
            assert_f16_close(got[2][rows], ref.y64)


def test_allocating_layer_in_a_graph(sq, dev):
    """smoothed_linear, whose intermediate codes and output come from the
    allocator, recorded in a graph (the graph's own memory pool): each replay
    rewrites the same output tensor, equal to the eager layer."""
    import torch
    M, K, N = 512, 2048, 1536
    xs_np, x_cal, w = inputs(7100, M, K, N)
    f = sq.fold(T(w, dev), sq.calibrate(T(x_cal, dev)), 0.5)
    x = T(xs_np[0], dev)
    out = {}

    def layer():
        out["y"] = sq.smoothed_linear(x, f)

    g = capture(layer)
    for r in range(REPLAYS):
        xr = T(xs_np[r], dev)
        x.copy_(xr)
        g.replay()
        got = H(out["y"])
        assert same_bits(got, H(sq.smoothed_linear(xr, f))), f"replay {r}"


def test_int32_product_graph(sq, dev):
    """The raw int32 sums through a graph, both product families."""
    import torch
    for M, K, N in [(700, 2112, 640), (3, 8192, 2048)]:
        print(f"[graph] int32 M={M} K={K} N={N}", flush=True)
        codes = [W.random_i8(7200 + r, M, K) for r in range(REPLAYS)]
        wq = sq.pack_i8(T(W.random_i8(7300, N, K), dev))
        xq = torch.empty(sq.packed_bytes(M, K), dtype=torch.int8, device=dev)
        acc = torch.empty((M, N), dtype=torch.int32, device=dev)

        def prod():
            sq.sq_w8a8_gemm(xq, None, wq, None, acc, K, out_kind=sq.SQ_OUT_I32)

        g = capture(prod)
        for r in range(REPLAYS):
            packed = sq.pack_i8(T(codes[r], dev))
            xq.copy_(packed)
            g.replay()
            got = H(acc)
            ref = np.asarray(codes[r], np.int64) @ H(sq.unpack_i8(wq, N, K)).astype(np.int64).T
            assert np.array_equal(got, ref.astype(np.int32)), f"replay {r}"


@pytest.mark.parametrize("M,K", [(2048, 4096), (16, 8192)])
def test_norm_layer_graph(sq, dev, M, K):
    """RMS normalization with 1/s folded into its weight, then the product."""
    import torch
    N = 1024
    hs_np, x_cal, w = inputs(7400 + M, M, K, N)
    gamma = W.random_f16(7500, 1, K)[0]
    f = sq.fold(T(w, dev), sq.calibrate(T(x_cal, dev)), 0.5)
    gf = sq.fold_norm_weight(T(gamma, dev), f.inv_smooth)
    h = T(hs_np[0], dev)
    xq = torch.empty(sq.packed_bytes(M, K), dtype=torch.int8, device=dev)
    xsc = torch.empty(M, dtype=torch.float32, device=dev)
    y = torch.empty((M, N), dtype=torch.float16, device=dev)

    def layer():
        sq.sq_rmsnorm_quant_per_token(h, gf, 1e-5, xq, xsc)
        sq.sq_w8a8_gemm(xq, xsc, f.wq, f.w_scale, y, K)

    g = capture(layer)
    for r in range(REPLAYS):
        hr = T(hs_np[r], dev)
        h.copy_(hr)
        g.replay()
        got = (H(xq), H(xsc), H(y))
        eq, es = sq.rmsnorm_quant(hr, gf, 1e-5)
        ey = sq.gemm(eq, es, f.wq, f.w_scale, M, N, K)
        assert same_bits(got[0], H(eq)) and same_bits(got[1], H(es)), f"replay {r}"
        assert same_bits(got[2], H(ey)), f"replay {r}"


@pytest.mark.parametrize("M,K,rotate", [(2048, 4096, 1), (1, 8192, 1), (64, 2048, 0)])
def test_w4a4_layer_graph(sq, dev, M, K, rotate):
    """Smooth Rotation at 4 bits: rotated 4-bit tokens, then the product with
    packed 4-bit weights."""
    import torch
    N = 1024
    xs_np, x_cal, w = inputs(7600 + M, M, K, N)
    wd = T(w, dev)
    s, inv = sq.smoothing_factors(wd, sq.calibrate(T(x_cal, dev)), 0.5)
    wq4, ws = sq.fold4(wd, s, bool(rotate))
    x = T(xs_np[0], dev)
    xq = torch.empty(sq.packed_bytes(M, K), dtype=torch.int8, device=dev)
    xsc = torch.empty(M, dtype=torch.float32, device=dev)
    y = torch.empty((M, N), dtype=torch.float16, device=dev)

    def layer():
        sq.sq_a4_quant_per_token(x, inv, bool(rotate), xq, xsc)
        sq.sq_w4_gemm(xq, xsc, wq4, ws, y, K)

    g = capture(layer)
    for r in range(REPLAYS):
        xr = T(xs_np[r], dev)
        x.copy_(xr)
        g.replay()
        got = (H(xq), H(xsc), H(y))
        eq, es = sq.quant4(xr, inv, bool(rotate))
        ey = sq.gemm4(eq, es, wq4, ws, M, N, K)
        assert same_bits(got[0], H(eq)) and same_bits(got[1], H(es)), f"replay {r}"
        assert same_bits(got[2], H(ey)), f"replay {r}"
