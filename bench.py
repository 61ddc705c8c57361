#!/usr/bin/env python3
"""Benchmark of the SmoothQuant-smoothed W8A8 linear layer on one MI355X.

One step is one pass of every stage of the layer over one batch of synthetic
input, each through the C ABI on one HIP stream:
  A1 sq_calibrate_absmax     per-channel max |X| over the 512 calibration tokens
  A2+A3 sq_smooth_fold_weights  smoothing factors, fold into W, int8 per channel
  A4 sq_quant_act_per_token  per-token int8 quantization of the batch X
  A5+A6 sq_w8a8_gemm         int8 matrix-core product + fp16 epilogue
The default workload is the LLaMA-7B q/k/v-style layer: X fp16 2048 x 4096
(1% of channels x U(50, 100)), W fp16 4096 x 4096 ~ N(0, 0.02^2), alpha 0.5,
calibration on a separate 512-token draw.

Printed: one JSON line with the whole-step throughput (2MNK per step / wall
time), the product kernel against the int8 matrix-core roofline (its duration
from HIP events around it on the library's stream, on every 10th timed step),
the per-stage GPU times from a separate pass with events between the stages,
the serving-time layer (A4 + A5/A6, the two calls a deployed layer makes per
batch), and, outside the step: the product at the other large-token
configurations (down_proj 2048 x 11008 -> 4096, prefill 8192 x 8192 -> 3 x 8192),
the decode-size layer (M = 1, 4 and 16 tokens
against an 8192 x 28672 layer, the metric's M <= 16 half, as GB/s of its
weights), the fused RMS-norm + quantization that replaces A4 when 1/s is
folded into the normalization in front of the layer, the rotated 4-bit
quantizer of Smooth Rotation against the unrotated one, the matrix cores'
and HBM's attainable rates measured on this GPU (a matrix-instruction loop
with the product's register pattern on the workload's codes, a 1 GiB
streaming read) beside the published peaks, and the CPU oracle timed on a
bounded sample as a baseline.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0     # MI355X dense int8 matrix-core peak, 5.0 POP/s
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, 8 TB/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_qkv4096.txt")
GEMM_SRC = os.path.join(ROOT, "w8a8_post_quantization_sq_amd", "csrc", "k_gemm.hip")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash(path):
    """Hash of a source file's code: comments and whitespace do not count, so
    the recorded counters stay valid across comment-only edits."""
    import re
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    text = re.sub(r"\s+", "", text)
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def read_traffic(workload):
    """HBM bytes per product launch from the committed rocprofv3 counter
    summary, or None when it is missing, for another workload, or was taken
    on a different version of the product kernel."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("workload") != workload or kv.get("k_gemm_sha256_16") != source_hash(GEMM_SRC):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(inp, wl, budget_s):
    """The CPU oracle, as it stands, on a bounded sample of the same step:
    A1-A3 in full, then A4-A6 on blocks of 64 tokens until the time budget is
    spent; the step time is scaled to the whole batch."""
    import numpy as np
    import oracle
    t0 = time.perf_counter()
    ax = oracle.calibrate_absmax(inp.x_cal)
    s, inv, st = oracle.smoothing_factors(ax, oracle.row_absmax(inp.w), wl.alpha)
    wq, wsc = oracle.fold_quant_weights(inp.w, s)
    t_off = time.perf_counter() - t0
    rows = 0
    t1 = time.perf_counter()
    while rows < wl.M:
        r1 = min(wl.M, rows + 64)
        oracle.layer_block(np.ascontiguousarray(inp.x[rows:r1]), inv, wq, wsc)
        rows = r1
        if time.perf_counter() - t1 > budget_s:
            break
    t_layer = time.perf_counter() - t1
    t_step = t_off + t_layer * (wl.M / rows)
    ops = 2.0 * wl.M * wl.N * wl.K
    return {
        "value": ops / t_step / 1e12, "unit": "TOP/s", "cores": 1, "kind": "oracle",
        "sample": (f"single-threaded C oracle: calibration, factors and fold in full "
                   f"({t_off:.2f} s), quantization + int32 product + dequantization on the "
                   f"first {rows} of {wl.M} tokens ({t_layer:.2f} s), scaled to the batch: "
                   f"{t_step:.1f} s per step"),
    }


def prefill_leg(torch, workloads, sq, L, dev, stream, hs, launches):
    """The metric's M >= 2048 half beyond the step's workload: the product at
    the down_proj-style (2048 x 11008 -> 4096, alpha 0.5) and the large-prefill
    (8192 x 8192 -> 3 x 8192, one smoothed X for the three projections)
    configurations, on their own calibrated, folded and quantized codes (the
    matrix cores' power, and so their clock, depends on the codes), each as
    `launches` launches between one event pair; and the per-token quantizer of
    the same batches, `launches` launches likewise (HBM-bound: 2MK bytes of X,
    MK of codes, 4M of scales)."""
    out = {"peak": PEAK_INT8_TOPS, "unit": "TOP/s"}
    for name in ("down11008", "prefill8192x3"):
        wl = workloads.WORKLOADS[name]
        inp = workloads.generate(wl)
        M, K, N = wl.M, wl.K, wl.N
        x = torch.from_numpy(inp.x).to(dev)
        xcal = torch.from_numpy(inp.x_cal).to(dev)
        w = torch.from_numpy(inp.w).to(dev)
        del inp
        ax = torch.empty(K, dtype=torch.float32, device=dev)
        s = torch.empty(K, dtype=torch.float32, device=dev)
        inv = torch.empty(K, dtype=torch.float32, device=dev)
        wq = torch.empty(sq.packed_bytes(N, K), dtype=torch.int8, device=dev)
        wsc = torch.empty(N, dtype=torch.float32, device=dev)
        xq = torch.empty(sq.packed_bytes(M, K), dtype=torch.int8, device=dev)
        xsc = torch.empty(M, dtype=torch.float32, device=dev)
        y = torch.empty((M, N), dtype=torch.float16, device=dev)
        st = L.sq_calibrate_absmax(xcal.data_ptr(), xcal.shape[0], K, K, ax.data_ptr(), 0, hs)
        st |= L.sq_smooth_fold_weights(w.data_ptr(), K, N, N, ax.data_ptr(), float(wl.alpha), None,
                                       s.data_ptr(), inv.data_ptr(), wq.data_ptr(), wsc.data_ptr(),
                                       hs)
        st |= L.sq_quant_act_per_token(x.data_ptr(), M, K, K, inv.data_ptr(), xq.data_ptr(),
                                       xsc.data_ptr(), hs)
        if st:
            raise RuntimeError(f"{name}: preparing the product failed")
        del w, xcal

        def quant():
            return L.sq_quant_act_per_token(x.data_ptr(), M, K, K, inv.data_ptr(), xq.data_ptr(),
                                            xsc.data_ptr(), hs)
        for _ in range(3):
            if quant():
                raise RuntimeError(f"{name}: quantizer failed")
        q0, q1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        q0.record(stream)
        for _ in range(launches):
            quant()
        q1.record(stream)
        torch.cuda.synchronize()
        q_us = q0.elapsed_time(q1) * 1e3 / launches
        q_gbs = (3.0 * M * K + 4.0 * M) / (q_us * 1e-6) / 1e9
        del x

        def run():
            return L.sq_w8a8_gemm(xq.data_ptr(), xsc.data_ptr(), wq.data_ptr(), wsc.data_ptr(), M,
                                  N, K, y.data_ptr(), N, sq.SQ_OUT_F16, hs)
        for _ in range(3):
            if run():
                raise RuntimeError(f"{name}: product failed")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(launches):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / launches
        tops = 2.0 * M * N * K / (us * 1e-6) / 1e12
        out[name] = {"M": M, "K": K, "N": N, "us": round(us, 2), "tops": round(tops, 1),
                     "frac": round(tops / PEAK_INT8_TOPS, 4),
                     "quant_us": round(q_us, 2), "quant_gbs": round(q_gbs, 1),
                     "quant_frac_hbm": round(q_gbs / PEAK_HBM_GBS, 4)}
        log(f"product {name}: {us:.1f} us, {tops:.0f} TOP/s; quantizer {q_us:.1f} us, "
            f"{q_gbs:.0f} GB/s")
        del xq, wq, y
    return out


def decode_leg(torch, workloads, sq, L, dev, stream, hs, launches):
    """The serving-time layer at decode sizes, the metric's M <= 16 half: the
    decode8192 workload (K 8192, N 28672) folded once, its codes copied 4 times
    (940 MB, beyond the 256 MB Infinity Cache) and the copies taken in turn, so
    every product streams its weights from HBM.  Per token count, the product
    alone and quantization + product (M = 1, 4, 16), each as `launches`
    launches between one event pair; GB/s = the weights' bytes / time."""
    wl = workloads.WORKLOADS["decode8192"]
    inp = workloads.generate(wl)
    K, N = wl.K, wl.N
    w = torch.from_numpy(inp.w).to(dev)
    ax = torch.empty(K, dtype=torch.float32, device=dev)
    s = torch.empty(K, dtype=torch.float32, device=dev)
    inv = torch.empty(K, dtype=torch.float32, device=dev)
    wsc = torch.empty(N, dtype=torch.float32, device=dev)
    wq0 = torch.empty(sq.packed_bytes(N, K), dtype=torch.int8, device=dev)
    xcal = torch.from_numpy(inp.x_cal).to(dev)
    st = L.sq_calibrate_absmax(xcal.data_ptr(), xcal.shape[0], K, K, ax.data_ptr(), 0, hs)
    st |= L.sq_smooth_fold_weights(w.data_ptr(), K, N, N, ax.data_ptr(), float(wl.alpha), None,
                                   s.data_ptr(), inv.data_ptr(), wq0.data_ptr(), wsc.data_ptr(), hs)
    if st:
        raise RuntimeError("decode fold failed")
    del w
    copies = [wq0] + [wq0.clone() for _ in range(3)]
    out = {"workload": "decode8192: K 8192, N 28672, 4 weight copies taken in turn",
           "weight_bytes": N * K, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    for m in (1, 4, 16):
        x = torch.from_numpy(inp.x[:m].copy()).to(dev)
        xq = torch.empty(sq.packed_bytes(m, K), dtype=torch.int8, device=dev)
        xs = torch.empty(m, dtype=torch.float32, device=dev)
        y = torch.empty((m, N), dtype=torch.float16, device=dev)

        def run(i, with_quant):
            r = 0
            if with_quant:
                r |= L.sq_quant_act_per_token(x.data_ptr(), m, K, K, inv.data_ptr(), xq.data_ptr(),
                                              xs.data_ptr(), hs)
            r |= L.sq_w8a8_gemm(xq.data_ptr(), xs.data_ptr(), copies[i % 4].data_ptr(),
                                wsc.data_ptr(), m, N, K, y.data_ptr(), N, sq.SQ_OUT_F16, hs)
            return r
        res = {}
        for with_quant in (True, False, True, False):
            for i in range(8):
                if run(i, with_quant):
                    raise RuntimeError("decode layer call failed")
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(launches):
                run(i, with_quant)
            e1.record(stream)
            torch.cuda.synchronize()
            res[with_quant] = e0.elapsed_time(e1) * 1e3 / launches
        gb_layer = N * K / (res[True] * 1e-6) / 1e9
        gb_gemm = N * K / (res[False] * 1e-6) / 1e9
        out[f"M{m}"] = {"layer_us": round(res[True], 2), "gemm_us": round(res[False], 2),
                        "layer_gbs": round(gb_layer, 1), "gemm_gbs": round(gb_gemm, 1),
                        "layer_frac": round(gb_layer / PEAK_HBM_GBS, 4),
                        "gemm_frac": round(gb_gemm / PEAK_HBM_GBS, 4)}
        log(f"decode M={m}: layer {res[True]:.2f} us, product {res[False]:.2f} us")

    # The same layer as Smooth Rotation at 4 bits: factors, Hadamard-rotated
    # 4-bit weights packed two per byte (half the bytes), rotated 4-bit tokens.
    w = torch.from_numpy(inp.w).to(dev)
    work = torch.empty(sq.sq_w4_workspace_bytes(K, N), dtype=torch.uint8, device=dev)
    w4 = torch.empty(sq.packed4_bytes(N, K), dtype=torch.uint8, device=dev)
    ws4 = torch.empty(N, dtype=torch.float32, device=dev)
    st = L.sq_smoothing_factors(w.data_ptr(), K, N, N, ax.data_ptr(), float(wl.alpha),
                                s.data_ptr(), inv.data_ptr(), hs)
    st |= L.sq_w4_fold_weights(w.data_ptr(), K, N, N, s.data_ptr(), 1, w4.data_ptr(),
                               ws4.data_ptr(), work.data_ptr(), hs)
    torch.cuda.synchronize()
    if st:
        raise RuntimeError("4-bit decode fold failed")
    del w, work
    copies4 = [w4] + [w4.clone() for _ in range(3)]
    w4a4 = {"what": "Smooth Rotation W4A4: rotated 4-bit tokens (sq_a4_quant_per_token, rotate=1) + "
                    "product with 4-bit weights (sq_w4_gemm)", "weight_bytes": N * K // 2}
    for m in (1, 16):
        x = torch.from_numpy(inp.x[:m].copy()).to(dev)
        xq = torch.empty(sq.packed_bytes(m, K), dtype=torch.int8, device=dev)
        xs = torch.empty(m, dtype=torch.float32, device=dev)
        y = torch.empty((m, N), dtype=torch.float16, device=dev)

        def run4(i, with_quant):
            r = 0
            if with_quant:
                r |= L.sq_a4_quant_per_token(x.data_ptr(), m, K, K, inv.data_ptr(), 1,
                                             xq.data_ptr(), xs.data_ptr(), hs)
            r |= L.sq_w4_gemm(xq.data_ptr(), xs.data_ptr(), copies4[i % 4].data_ptr(),
                              ws4.data_ptr(), m, N, K, y.data_ptr(), N, sq.SQ_OUT_F16, hs)
            return r
        res = {}
        for with_quant in (True, False, True, False):
            for i in range(8):
                if run4(i, with_quant):
                    raise RuntimeError("4-bit decode layer call failed")
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(launches):
                run4(i, with_quant)
            e1.record(stream)
            torch.cuda.synchronize()
            res[with_quant] = e0.elapsed_time(e1) * 1e3 / launches
        gb = N * K // 2 / (res[True] * 1e-6) / 1e9
        w4a4[f"M{m}"] = {"layer_us": round(res[True], 2), "gemm_us": round(res[False], 2),
                         "layer_gbs": round(gb, 1), "layer_frac": round(gb / PEAK_HBM_GBS, 4)}
        log(f"decode W4A4 M={m}: layer {res[True]:.2f} us, product {res[False]:.2f} us")
    out["w4a4"] = w4a4
    return out


def attainable_leg(torch, sq, dev, stream, hs, wq, xq):
    """Measured ceilings on this GPU, reported beside the published peaks
    (libsq_probe.so): the int8 matrix cores' sustained rate with the product
    kernel's register pattern (one workgroup of 8 waves per CU, 16 MFMAs per
    k-step into 16 accumulators) on the workload's own weight and activation
    codes, and a streaming read of 1 GiB (beyond the 256 MB Infinity Cache)."""
    P = sq.probe_lib()
    a = wq.view(-1)[:65536]
    b = xq.view(-1)[:16384]
    a = a.repeat((65536 + a.numel() - 1) // a.numel())[:65536].contiguous()
    b = b.repeat((16384 + b.numel() - 1) // b.numel())[:16384].contiguous()
    blocks, iters, reps = 256, 2000, 5
    out = torch.empty(blocks * 512, dtype=torch.int32, device=dev)
    if P.sqp_mfma_rate(a.data_ptr(), b.data_ptr(), 50, blocks, out.data_ptr(), hs):
        raise RuntimeError("sqp_mfma_rate failed")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        P.sqp_mfma_rate(a.data_ptr(), b.data_ptr(), iters, blocks, out.data_ptr(), hs)
    e1.record(stream)
    torch.cuda.synchronize()
    ops = blocks * 8 * iters * 16 * (2 * 16 * 16 * 64) * reps
    mfma_tops = ops / (e0.elapsed_time(e1) * 1e-3) / 1e12
    nbytes, rblocks = 1 << 30, 8192
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    rout = torch.empty(rblocks * 256, dtype=torch.int32, device=dev)
    if P.sqp_stream_read(buf.data_ptr(), nbytes, rblocks, rout.data_ptr(), hs):
        raise RuntimeError("sqp_stream_read failed")
    e0.record(stream)
    for _ in range(reps):
        P.sqp_stream_read(buf.data_ptr(), nbytes, rblocks, rout.data_ptr(), hs)
    e1.record(stream)
    torch.cuda.synchronize()
    read_gbs = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf
    log(f"attainable: matrix cores {mfma_tops:.0f} TOP/s on the workload's codes, "
        f"streaming read {read_gbs:.0f} GB/s")
    return {"what": "measured on this GPU (libsq_probe.so): int8 MFMA rate with the product's "
                    "register pattern on the workload's codes, 2 waves per SIMD; streaming "
                    "read of 1 GiB with 16-byte non-temporal loads",
            "mfma_int8_tops": round(mfma_tops, 1), "hbm_read_gbs": round(read_gbs, 1)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="qkv4096",
                    help="qkv4096 | down11008 | prefill8192x3 | tiny")
    ap.add_argument("--alpha", type=float, default=None)
    ap.add_argument("--event-every", type=int, default=10,
                    help="bracket the product kernel with HIP events on every n-th timed step")
    ap.add_argument("--stage-steps", type=int, default=20,
                    help="steps of the separate, untimed pass with an event between stages")
    ap.add_argument("--layer-launches", type=int, default=100,
                    help="quant + product pairs of the serving-time layer timed back to back "
                         "between one event pair (0: take the stage pass's two stages)")
    ap.add_argument("--norm-launches", type=int, default=100,
                    help="launches of the fused RMS-norm + quantization (and of the plain "
                         "quantizer) timed between one pair of events (0: skip)")
    ap.add_argument("--rot-launches", type=int, default=100,
                    help="launches of the rotated 4-bit quantizer (and of the unrotated one) "
                         "timed between one pair of events (0: skip)")
    ap.add_argument("--decode-launches", type=int, default=40,
                    help="launches per token count of the decode layer (decode8192: K 8192, "
                         "N 28672, M 1, 4 and 16), timed over 4 rotated weight copies (0: skip)")
    ap.add_argument("--prefill-launches", type=int, default=10,
                    help="launches of the product at the other large-token configurations "
                         "(down11008, prefill8192x3), on their folded codes (0: skip)")
    ap.add_argument("--attainable", type=int, default=1,
                    help="measure the matrix cores' and HBM's attainable rates on this GPU "
                         "(libsq_probe.so) and report them beside the published peaks (0: skip)")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle layer work in the CPU baseline (0: skip)")
    ap.add_argument("--copy-kernel", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run 3 plain device copies of MIB MiB "
                         "(the reference for calibrating rocprofv3's FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the library runs on one GPU; a sharded multi-GPU path is not "
              "implemented (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    import w8a8_post_quantization_sq_amd as sq

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    L = sq.lib()     # raises if the HIP library is not built: there is no fallback
    dev = torch.device("cuda:0")
    if args.copy_kernel > 0:
        n = args.copy_kernel << 20
        a = torch.ones(n // 4, dtype=torch.int32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_kernel_bytes": n, "launches": 3}), flush=True)
        return
    wl = workloads.WORKLOADS[args.workload]
    if args.alpha is not None:
        wl = wl.with_alpha(args.alpha)
    M, K, N, T = wl.M, wl.K, wl.N, wl.T_cal or wl.M
    log(f"workload {wl.name}: M={M} K={K} N={N} T_cal={T} alpha={wl.alpha}")
    inp = workloads.generate(wl)

    # inputs resident in HBM before the timed region
    x = torch.from_numpy(inp.x).to(dev)
    xcal = torch.from_numpy(inp.x_cal).to(dev)
    w = torch.from_numpy(inp.w).to(dev)
    ax = torch.empty(K, dtype=torch.float32, device=dev)
    s = torch.empty(K, dtype=torch.float32, device=dev)
    inv = torch.empty(K, dtype=torch.float32, device=dev)
    wq = torch.empty(sq.packed_bytes(N, K), dtype=torch.int8, device=dev)   # packed codes
    wsc = torch.empty(N, dtype=torch.float32, device=dev)
    xq = torch.empty(sq.packed_bytes(M, K), dtype=torch.int8, device=dev)
    xsc = torch.empty(M, dtype=torch.float32, device=dev)
    y = torch.empty((M, N), dtype=torch.float16, device=dev)
    stream = torch.cuda.current_stream(dev)
    hs = stream.cuda_stream
    p = {k: t.data_ptr() for k, t in dict(x=x, xcal=xcal, w=w, ax=ax, s=s, inv=inv, wq=wq,
                                            wsc=wsc, xq=xq, xsc=xsc, y=y).items()}
    alpha = float(wl.alpha)

    def step(ev=None, gemm_ev=None):
        # each call goes straight through the C ABI with the tensors' device pointers
        if ev: ev[0].record(stream)
        st = L.sq_calibrate_absmax(p["xcal"], T, K, K, p["ax"], 0, hs)
        if ev: ev[1].record(stream)
        st |= L.sq_smooth_fold_weights(p["w"], K, N, N, p["ax"], alpha, None, p["s"], p["inv"],
                                       p["wq"], p["wsc"], hs)
        if ev: ev[2].record(stream)
        st |= L.sq_quant_act_per_token(p["x"], M, K, K, p["inv"], p["xq"], p["xsc"], hs)
        if ev: ev[3].record(stream)
        if gemm_ev: gemm_ev[0].record(stream)
        st |= L.sq_w8a8_gemm(p["xq"], p["xsc"], p["wq"], p["wsc"], M, N, K, p["y"], N,
                             sq.SQ_OUT_F16, hs)
        if gemm_ev: gemm_ev[1].record(stream)
        if ev: ev[4].record(stream)
        if st:
            raise RuntimeError(f"library call failed: status bits {st}")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    # Timed region: the only events in it bracket the product kernel, on every
    # --event-every-th step (each event record adds ~3 us of its own to the
    # device timeline, so bracketing every step would inflate the step time).
    every = max(1, args.event_every)
    gemm_events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
                   for _ in range(0, args.steps, every)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(gemm_ev=gemm_events[i // every] if i % every == 0 else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"timed {args.steps} steps in {wall:.3f} s")
    gemm_samples = sorted(a.elapsed_time(b) for a, b in gemm_events)
    gemm_ms = sum(gemm_samples) / len(gemm_samples)

    def pct(q):
        return gemm_samples[min(len(gemm_samples) - 1, int(q * len(gemm_samples)))] * 1e3

    # Per-stage breakdown, from a separate pass with an event between stages
    # (those events lengthen these steps a little; the headline is not taken here).
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)]
              for _ in range(args.stage_steps)]
    for i in range(args.stage_steps):
        step(ev=events[i])
    torch.cuda.synchronize()
    names = ["calibrate", "fold", "quant", "gemm"]
    per = {n: 0.0 for n in names}
    for ev in events:
        for j, n in enumerate(names):
            per[n] += ev[j].elapsed_time(ev[j + 1])
    per = {n: v / max(1, args.stage_steps) for n, v in per.items()}    # ms per call

    # The serving-time layer as a deployed model runs it (the weights folded
    # offline): quantization + product, --layer-launches pairs back to back on
    # the stream between one event pair, on the step's folded weights.
    layer_ms = per["quant"] + per["gemm"]
    layer_how = "stage pass (events between the calls)"
    if args.layer_launches > 0:
        def layer_pair():
            st = L.sq_quant_act_per_token(p["x"], M, K, K, p["inv"], p["xq"], p["xsc"], hs)
            st |= L.sq_w8a8_gemm(p["xq"], p["xsc"], p["wq"], p["wsc"], M, N, K, p["y"], N,
                                 sq.SQ_OUT_F16, hs)
            if st:
                raise RuntimeError("layer launch failed")
        for _ in range(5):
            layer_pair()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.layer_launches):
            layer_pair()
        e1.record(stream)
        torch.cuda.synchronize()
        layer_ms = e0.elapsed_time(e1) / args.layer_launches
        layer_how = f"{args.layer_launches} quant + product pairs back to back, one event pair"

    # The normalization in front of the layer with 1/s folded into its weight:
    # the fused RMS-norm + quantization against the plain quantizer on the
    # same batch, each timed as a run of launches between one event pair
    # (the per-launch average includes the gaps between launches).
    norm = None
    if args.norm_launches > 0:
        gamma = torch.from_numpy(workloads.norm_weight(wl)).to(dev)
        g = torch.empty(K, dtype=torch.float32, device=dev)
        if L.sq_fold_norm_weight(gamma.data_ptr(), K, p["inv"], g.data_ptr(), hs):
            raise RuntimeError("sq_fold_norm_weight failed")
        eps = workloads.NORM_EPS

        def run(fused):
            if fused:
                return L.sq_rmsnorm_quant_per_token(p["x"], M, K, K, g.data_ptr(), eps, p["xq"],
                                                    p["xsc"], hs)
            return L.sq_quant_act_per_token(p["x"], M, K, K, p["inv"], p["xq"], p["xsc"], hs)

        us = {}
        for fused in (False, True, False, True):     # second round is the one kept
            for _ in range(10):
                run(fused)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(args.norm_launches):
                if run(fused):
                    raise RuntimeError("quantizer call failed")
            e1.record(stream)
            torch.cuda.synchronize()
            us[fused] = e0.elapsed_time(e1) * 1e3 / args.norm_launches
        nbytes = 2 * M * K + M * K + 4 * M + 4 * K
        gbs = nbytes / (us[True] * 1e-6) / 1e9
        norm = {"what": "RMS norm with 1/s folded into its weight, fused with per-token quant "
                        "(sq_rmsnorm_quant_per_token; replaces a separate norm pass)",
                "us": round(us[True], 3), "plain_quant_us": round(us[False], 3),
                "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4),
                "per_launch": f"2MK (h) + MK (codes) + 4M + 4K = {nbytes} bytes",
                "saved_bytes_per_batch": 4 * M * K}
        log(f"fused norm + quant {us[True]:.2f} us, plain quant {us[False]:.2f} us")

    # Smooth Rotation at 4 bits (outside the step): the per-token quantizer
    # with the Hadamard transform against the same quantizer without it, on
    # the same batch and factors; the product takes their codes unchanged.
    rot = None
    if args.rot_launches > 0 and K & (K - 1) == 0 and K <= 8192:
        us = {}
        for rotate in (0, 1, 0, 1):                  # second round is the one kept
            def run4():
                return L.sq_a4_quant_per_token(p["x"], M, K, K, p["inv"], rotate, p["xq"],
                                               p["xsc"], hs)
            for _ in range(10):
                run4()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(args.rot_launches):
                if run4():
                    raise RuntimeError("4-bit quantizer call failed")
            e1.record(stream)
            torch.cuda.synchronize()
            us[rotate] = e0.elapsed_time(e1) * 1e3 / args.rot_launches
        nbytes = 2 * M * K + M * K + 4 * M + 4 * K
        gbs = nbytes / (us[1] * 1e-6) / 1e9
        rot = {"what": "Smooth Rotation 4-bit per-token quantizer: x/s, fast Walsh-Hadamard "
                       "transform, 4-bit codes (sq_a4_quant_per_token, rotate=1)",
               "us": round(us[1], 3), "unrotated_us": round(us[0], 3),
               "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
               "frac": round(gbs / PEAK_HBM_GBS, 4),
               "per_launch": f"2MK (x) + MK (codes, one per byte) + 4M + 4K = {nbytes} bytes",
               "transform_flops": int(M * K * (K.bit_length() - 1))}
        log(f"rotated 4-bit quant {us[1]:.2f} us, unrotated {us[0]:.2f} us")

    prefill = None
    if args.prefill_launches > 0:
        prefill = prefill_leg(torch, workloads, sq, L, dev, stream, hs, args.prefill_launches)

    decode = None
    if args.decode_launches > 0:
        decode = decode_leg(torch, workloads, sq, L, dev, stream, hs, args.decode_launches)

    ops = 2.0 * M * N * K
    ms_step = wall * 1e3 / args.steps
    gemm_tops = ops / (gemm_ms * 1e-3) / 1e12
    layer_tops = ops / (layer_ms * 1e-3) / 1e12 if layer_ms > 0 else 0.0
    traffic = read_traffic(wl.name)
    # algorithmic HBM bytes of the runtime layer per batch (int8 weights and
    # scales, fp16 X in, 1/s, fp16 Y out)
    layer_bytes = K * N + 4 * N + 2 * M * K + 4 * K + 2 * M * N

    out = {
        "metric": "W8A8 smoothed-linear TOPS (M>=2048) & GB/s (M<=16), % of MI355X roofline",
        "value": round(ops * args.steps / wall / 1e12, 3),
        "unit": "TOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic (seeded, outlier structure of the workload; no trained weights)",
        "config": {"workload": f"{wl.name}: {wl.description}", "M": M, "K": K, "N": N,
                   "alpha": wl.alpha, "calibration_tokens": T, "seed": wl.seed,
                   "step": "calibrate + smooth/fold + per-token quant + W8A8 GEMM"},
        "stage_ms": {n: round(v, 4) for n, v in per.items()},
        "layer": {"what": "serving-time layer: per-token quant + W8A8 GEMM (weights folded offline)",
                  "how": layer_how, "ms": round(layer_ms, 4), "tops": round(layer_tops, 2),
                  "frac_int8_peak": round(layer_tops / PEAK_INT8_TOPS, 4),
                  "hbm_gbs_algorithmic": round(layer_bytes / (layer_ms * 1e-3) / 1e9, 1)
                  if layer_ms > 0 else 0.0},
        "roofline": {"kernel": "k_gemm_w8a8 (sq_w8a8_gemm)", "bound": "mfma",
                     "achieved": round(gemm_tops, 2), "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                     "frac": round(gemm_tops / PEAK_INT8_TOPS, 4), "traffic": traffic,
                     "launch_us": {"mean": round(gemm_ms * 1e3, 2), "p10": round(pct(0.1), 2),
                                   "p50": round(pct(0.5), 2), "p90": round(pct(0.9), 2),
                                   "samples": len(gemm_samples)},
                     "per_launch": f"2*M*N*K = {ops:.4g} int8 ops per launch"},
        "prefill": prefill,
        "decode": decode,
        "norm_fold": norm,
        "rotation_w4": rot,
        "cpu_baseline": None,
    }
    if args.attainable:
        att = attainable_leg(torch, sq, dev, stream, hs, wq, xq)
        att["product_frac_of_mfma"] = round(gemm_tops / att["mfma_int8_tops"], 4)
        if decode:
            att["decode_layer_frac_of_read"] = {
                k: round(v["layer_gbs"] / att["hbm_read_gbs"], 4)
                for k, v in decode.items() if k in ("M1", "M4", "M16")}
        out["attainable"] = att
    if args.cpu_budget > 0:
        log("timing the CPU oracle baseline")
        out["cpu_baseline"] = cpu_baseline(inp, wl, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
