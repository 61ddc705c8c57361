"""Python binding of the MI355X SmoothQuant-smoothed W8A8 linear layer.

A thin ctypes layer over the C ABI in include/sq.h (libsq.so, built in-tree
by ``build.py``).  It only marshals torch tensors into device pointers,
strides and the current HIP stream; every step of the layer runs in the
library's gfx950 kernels.  There is no CPU fallback: without the built
library, or without a GPU, the calls raise.

Same-name calls (caller-allocated outputs, as in the C ABI):
    sq_calibrate_absmax, sq_smooth_fold_weights, sq_smooth_fold_weights_noalloc,
    sq_quant_act_per_token,
    sq_w8a8_gemm, sq_packed_bytes, sq_pack_i8, sq_unpack_i8,
    sq_fold_norm_weight, sq_rmsnorm_quant_per_token, sq_smoothing_factors,
    sq_w4_workspace_bytes, sq_w4_fold_weights, sq_a4_quant_per_token,
    sq_packed4_bytes, sq_w4_gemm
Allocating helpers built on them:
    calibrate, fold, quant, gemm, smoothed_linear, pack_i8, unpack_i8,
    fold_norm_weight, rmsnorm_quant, smoothing_factors, fold4, quant4, gemm4

The int8 codes (xq, wq) travel as flat int8 tensors in the packed operand
order the C ABI documents (16-row x 64-byte fragments of 1 KiB); their sizes
are packed_bytes(rows, K).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsq.so")

SQ_NOALLOC_MAX_N = 131072
SQ_OK = 0
SQ_ERR_NULL = 1
SQ_ERR_SHAPE = 2
SQ_ERR_ALIGN = 3
SQ_ERR_ALPHA = 4
SQ_ERR_NONFINITE = 5
SQ_ERR_RANGE = 6
SQ_ERR_HIP = 7
SQ_ERR_KIND = 8
SQ_ERR_EPS = 9
SQ_OUT_F16 = 0
SQ_OUT_I32 = 1
SQ_MAX_K = 131056

EXPORTS = ("sq_status_str", "sq_version", "sq_packed_bytes", "sq_calibrate_absmax",
           "sq_smooth_fold_weights", "sq_quant_act_per_token", "sq_w8a8_gemm", "sq_pack_i8",
           "sq_unpack_i8", "sq_fold_norm_weight", "sq_rmsnorm_quant_per_token",
           "sq_smoothing_factors", "sq_w4_workspace_bytes", "sq_w4_fold_weights",
           "sq_a4_quant_per_token", "sq_packed4_bytes", "sq_w4_gemm",
           "sq_smooth_fold_weights_noalloc")

_LIB = None


class SqError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = int(status)
        super().__init__(f"{call}: {status_str(status)}")


def lib() -> ctypes.CDLL:
    """The loaded libsq.so.  Raises if it has not been built: there is no fallback."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m w8a8_post_quantization_sq_amd.build` "
                              "or __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, f32, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
        L.sq_status_str.restype = ctypes.c_char_p
        L.sq_status_str.argtypes = [ci]
        L.sq_version.restype = ci
        L.sq_version.argtypes = []
        L.sq_calibrate_absmax.restype = ci
        L.sq_calibrate_absmax.argtypes = [vp, i64, i64, i64, vp, ci, vp]
        L.sq_smooth_fold_weights.restype = ci
        L.sq_smooth_fold_weights.argtypes = [vp, i64, i64, i64, vp, f32, vp, vp, vp, vp, vp, vp]
        L.sq_smooth_fold_weights_noalloc.restype = ci
        L.sq_smooth_fold_weights_noalloc.argtypes = [vp, i64, i64, i64, vp, f32, vp, vp, vp, vp,
                                                     vp, vp]
        L.sq_quant_act_per_token.restype = ci
        L.sq_quant_act_per_token.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp]
        L.sq_w8a8_gemm.restype = ci
        L.sq_w8a8_gemm.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, i64, ci, vp]
        L.sq_packed_bytes.restype = i64
        L.sq_packed_bytes.argtypes = [i64, i64]
        L.sq_pack_i8.restype = ci
        L.sq_pack_i8.argtypes = [vp, i64, i64, i64, vp, vp]
        L.sq_unpack_i8.restype = ci
        L.sq_unpack_i8.argtypes = [vp, i64, i64, vp, i64, vp]
        L.sq_fold_norm_weight.restype = ci
        L.sq_fold_norm_weight.argtypes = [vp, i64, vp, vp, vp]
        L.sq_rmsnorm_quant_per_token.restype = ci
        L.sq_rmsnorm_quant_per_token.argtypes = [vp, i64, i64, i64, vp, f32, vp, vp, vp]
        L.sq_smoothing_factors.restype = ci
        L.sq_smoothing_factors.argtypes = [vp, i64, i64, i64, vp, f32, vp, vp, vp]
        L.sq_w4_workspace_bytes.restype = i64
        L.sq_w4_workspace_bytes.argtypes = [i64, i64]
        L.sq_w4_fold_weights.restype = ci
        L.sq_w4_fold_weights.argtypes = [vp, i64, i64, i64, vp, ci, vp, vp, vp, vp]
        L.sq_packed4_bytes.restype = i64
        L.sq_packed4_bytes.argtypes = [i64, i64]
        L.sq_w4_gemm.restype = ci
        L.sq_w4_gemm.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, i64, ci, vp]
        L.sq_a4_quant_per_token.restype = ci
        L.sq_a4_quant_per_token.argtypes = [vp, i64, i64, i64, vp, ci, vp, vp, vp]
        _LIB = L
    return _LIB


PROBE_PATH = os.path.join(HERE, "libsq_probe.so")
PROBE_EXPORTS = ("sqp_mfma_rate", "sqp_stream_read", "sqp_wall_clock_khz", "sqp_clock_watch")
_PROBE = None


def probe_lib() -> ctypes.CDLL:
    """libsq_probe.so, the benchmark's measured ceilings (include/sq_probe.h):
    not part of the layer.  Raises if it has not been built."""
    global _PROBE
    if _PROBE is None:
        if not os.path.exists(PROBE_PATH):
            raise ImportError(f"{PROBE_PATH} is missing: build it with "
                              "`python -m w8a8_post_quantization_sq_amd.build`")
        P = ctypes.CDLL(PROBE_PATH)
        vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        P.sqp_mfma_rate.restype = ci
        P.sqp_mfma_rate.argtypes = [vp, vp, ci, ci, vp, vp]
        P.sqp_stream_read.restype = ci
        P.sqp_stream_read.argtypes = [vp, i64, ci, vp, vp]
        P.sqp_wall_clock_khz.restype = ci
        P.sqp_wall_clock_khz.argtypes = [ctypes.POINTER(ci)]
        P.sqp_clock_watch.restype = ci
        P.sqp_clock_watch.argtypes = [ctypes.c_uint64, ctypes.c_uint64, vp, vp]
        _PROBE = P
    return _PROBE


def status_str(status: int) -> str:
    return lib().sq_status_str(int(status)).decode()


def packed_bytes(rows: int, K: int) -> int:
    """Bytes of a packed int8 operand of `rows` rows of K codes."""
    return int(lib().sq_packed_bytes(int(rows), int(K)))


def packed4_bytes(rows: int, K: int) -> int:
    """Bytes of a packed 4-bit operand of `rows` rows of K codes."""
    return int(lib().sq_packed4_bytes(int(rows), int(K)))


def _check(st: int, call: str) -> None:
    if st != SQ_OK:
        raise SqError(st, call)


# ---- marshalling helpers ------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _torch_stream(stream, device):
    """The torch stream object of `stream`: the current stream of `device` for
    None, a raw hipStream_t handle (int) wrapped as an external stream."""
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream(device)
    if hasattr(stream, "cuda_stream"):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def _stream(stream, device) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _need(t, dtype, name, ndim=None, numel=None):
    """dtype, rank, a contiguous last dimension and, for vectors, at least
    `numel` entries (the kernels index them up to that count).  The device is
    checked afterwards, for all of a call's tensors at once (_on_one_gpu)."""
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got {t.dim()}")
    if t.dim() >= 1 and t.stride(-1) != 1 and t.numel() > 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name}: expected at least {numel} entries, got {t.numel()}")
    return t


def _on_one_gpu(**tensors):
    """Every given tensor (None entries skipped) is a GPU tensor, all on one device."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name}: expected a GPU tensor (there is no CPU path)")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name}: on {t.device}, the call's other tensors on {dev}")


def _ld(t) -> int:
    return int(t.stride(0)) if t.dim() == 2 and t.shape[0] > 1 else int(t.shape[-1])


# ---- the four calls, same names as the C ABI -----------------------------------
#
# Each wrapper checks dtypes, ranks and sizes first (every vector needs as many
# entries as the kernels index), then that all its tensors sit on one GPU, and
# only then calls the library, which checks the rest (alignment, strides,
# limits) before it launches anything.

def sq_calibrate_absmax(x_cal, act_absmax, accumulate: bool = False, stream=None) -> None:
    """act_absmax[j] (float32 [K]) := max_t |x_cal[t][j]| (with accumulate: also
    over its previous contents).  x_cal: float16 [T][K]."""
    torch = _torch()
    _need(x_cal, torch.float16, "x_cal", 2)
    T, K = x_cal.shape
    _need(act_absmax, torch.float32, "act_absmax", 1, K)
    _on_one_gpu(x_cal=x_cal, act_absmax=act_absmax)
    _check(lib().sq_calibrate_absmax(_ptr(x_cal), T, K, _ld(x_cal), _ptr(act_absmax),
                                     1 if accumulate else 0, _stream(stream, x_cal.device)),
           "sq_calibrate_absmax")


def _need_packed(t, rows, K, name):
    torch = _torch()
    _need(t, torch.int8, name, 1)
    if not t.is_contiguous() or t.numel() < packed_bytes(rows, K):
        raise ValueError(f"{name}: expected a contiguous int8 buffer of "
                         f"{packed_bytes(rows, K)} bytes (packed {rows} x {K} codes)")


def sq_smooth_fold_weights(w, act_absmax, alpha: float, smooth_in, smooth_out, inv_smooth_out,
                           wq, w_scale, stream=None) -> None:
    """Smoothing factors and the offline fold.  w: float16 [K][N] (input x
    output channels); wq: packed int8 buffer of packed_bytes(N, K); w_scale:
    float32 [N]; smooth_out, inv_smooth_out: float32 [K]; smooth_in: None or
    float32 [K]."""
    torch = _torch()
    _need(w, torch.float16, "w", 2)
    K, N = w.shape
    _need(smooth_out, torch.float32, "smooth_out", 1, K)
    _need(inv_smooth_out, torch.float32, "inv_smooth_out", 1, K)
    _need(w_scale, torch.float32, "w_scale", 1, N)
    if act_absmax is not None:
        _need(act_absmax, torch.float32, "act_absmax", 1, K)
    if smooth_in is not None:
        _need(smooth_in, torch.float32, "smooth_in", 1, K)
    _need_packed(wq, N, K, "wq")
    _on_one_gpu(w=w, act_absmax=act_absmax, smooth_in=smooth_in, smooth_out=smooth_out,
                inv_smooth_out=inv_smooth_out, wq=wq, w_scale=w_scale)
    _check(lib().sq_smooth_fold_weights(_ptr(w), K, N, _ld(w), _ptr(act_absmax), float(alpha),
                                        _ptr(smooth_in), _ptr(smooth_out), _ptr(inv_smooth_out),
                                        _ptr(wq), _ptr(w_scale), _stream(stream, w.device)),
           "sq_smooth_fold_weights")


def sq_smooth_fold_weights_noalloc(w, act_absmax, alpha: float, smooth_in, smooth_out,
                                   inv_smooth_out, wq, w_scale, stream=None) -> None:
    """sq_smooth_fold_weights without any allocation in the library (scratch in
    its static per-device array; N <= SQ_NOALLOC_MAX_N); same arguments."""
    torch = _torch()
    _need(w, torch.float16, "w", 2)
    K, N = w.shape
    _need(smooth_out, torch.float32, "smooth_out", 1, K)
    _need(inv_smooth_out, torch.float32, "inv_smooth_out", 1, K)
    _need(w_scale, torch.float32, "w_scale", 1, N)
    if act_absmax is not None:
        _need(act_absmax, torch.float32, "act_absmax", 1, K)
    if smooth_in is not None:
        _need(smooth_in, torch.float32, "smooth_in", 1, K)
    _need_packed(wq, N, K, "wq")
    _on_one_gpu(w=w, act_absmax=act_absmax, smooth_in=smooth_in, smooth_out=smooth_out,
                inv_smooth_out=inv_smooth_out, wq=wq, w_scale=w_scale)
    _check(lib().sq_smooth_fold_weights_noalloc(
        _ptr(w), K, N, _ld(w), _ptr(act_absmax), float(alpha), _ptr(smooth_in), _ptr(smooth_out),
        _ptr(inv_smooth_out), _ptr(wq), _ptr(w_scale), _stream(stream, w.device)),
        "sq_smooth_fold_weights_noalloc")


def sq_quant_act_per_token(x, inv_smooth, xq, x_scale, stream=None) -> None:
    """xq (packed int8, packed_bytes(M, K)) and x_scale (float32 [M]) of
    x (float16 [M][K]) times inv_smooth."""
    torch = _torch()
    _need(x, torch.float16, "x", 2)
    M, K = x.shape
    _need(inv_smooth, torch.float32, "inv_smooth", 1, K)
    _need(x_scale, torch.float32, "x_scale", 1, M)
    _need_packed(xq, M, K, "xq")
    _on_one_gpu(x=x, inv_smooth=inv_smooth, xq=xq, x_scale=x_scale)
    _check(lib().sq_quant_act_per_token(_ptr(x), M, K, _ld(x), _ptr(inv_smooth), _ptr(xq),
                                        _ptr(x_scale), _stream(stream, x.device)),
           "sq_quant_act_per_token")


def _gemm_operands(xq, x_scale, w_scale, y, out_kind):
    torch = _torch()
    if out_kind == SQ_OUT_F16:
        _need(y, torch.float16, "y", 2)
        M, N = y.shape
        if x_scale is None or w_scale is None:
            raise ValueError("x_scale and w_scale are needed for fp16 output")
        _need(x_scale, torch.float32, "x_scale", 1, M)
        _need(w_scale, torch.float32, "w_scale", 1, N)
    else:
        _need(y, torch.int32, "y", 2)
        M, N = y.shape
        for t, name, n in ((x_scale, "x_scale", M), (w_scale, "w_scale", N)):
            if t is not None:          # unused by the raw sums, but checked if given
                _need(t, torch.float32, name, 1, n)
    return M, N


def sq_w8a8_gemm(xq, x_scale, wq, w_scale, y, K: int, out_kind: int = SQ_OUT_F16,
                 stream=None) -> None:
    """y [M][N] (float16, or int32 raw sums) from packed xq (M tokens) and
    packed wq (N channels) of K codes each."""
    M, N = _gemm_operands(xq, x_scale, w_scale, y, out_kind)
    _need_packed(xq, M, K, "xq")
    _need_packed(wq, N, K, "wq")
    _on_one_gpu(xq=xq, x_scale=x_scale, wq=wq, w_scale=w_scale, y=y)
    _check(lib().sq_w8a8_gemm(_ptr(xq), _ptr(x_scale), _ptr(wq), _ptr(w_scale), M, N, int(K),
                              _ptr(y), _ld(y), int(out_kind), _stream(stream, xq.device)),
           "sq_w8a8_gemm")


def sq_fold_norm_weight(gamma, inv_smooth, gamma_out, stream=None) -> None:
    """gamma_out (float32 [K]) = float(gamma) * inv_smooth: the RMS
    normalization's weight gamma (float16 [K]) with 1/s folded in."""
    torch = _torch()
    _need(gamma, torch.float16, "gamma", 1)
    K = gamma.shape[0]
    _need(inv_smooth, torch.float32, "inv_smooth", 1, K)
    _need(gamma_out, torch.float32, "gamma_out", 1, K)
    _on_one_gpu(gamma=gamma, inv_smooth=inv_smooth, gamma_out=gamma_out)
    _check(lib().sq_fold_norm_weight(_ptr(gamma), K, _ptr(inv_smooth), _ptr(gamma_out),
                                     _stream(stream, gamma.device)), "sq_fold_norm_weight")


def sq_rmsnorm_quant_per_token(h, gamma_folded, eps: float, xq, x_scale, stream=None) -> None:
    """xq (packed int8, packed_bytes(M, K)) and x_scale (float32 [M]) of the
    RMS-normalized hidden state h (float16 [M][K]) with the folded weight."""
    torch = _torch()
    _need(h, torch.float16, "h", 2)
    M, K = h.shape
    _need(gamma_folded, torch.float32, "gamma_folded", 1, K)
    _need(x_scale, torch.float32, "x_scale", 1, M)
    _need_packed(xq, M, K, "xq")
    _on_one_gpu(h=h, gamma_folded=gamma_folded, xq=xq, x_scale=x_scale)
    _check(lib().sq_rmsnorm_quant_per_token(_ptr(h), M, K, _ld(h), _ptr(gamma_folded),
                                            float(eps), _ptr(xq), _ptr(x_scale),
                                            _stream(stream, h.device)),
           "sq_rmsnorm_quant_per_token")


def sq_smoothing_factors(w, act_absmax, alpha: float, smooth_out, inv_smooth_out,
                         stream=None) -> None:
    """s and 1/s (float32 [K]) from the statistics and w (float16 [K][N])."""
    torch = _torch()
    _need(w, torch.float16, "w", 2)
    K, N = w.shape
    _need(act_absmax, torch.float32, "act_absmax", 1, K)
    _need(smooth_out, torch.float32, "smooth_out", 1, K)
    _need(inv_smooth_out, torch.float32, "inv_smooth_out", 1, K)
    _on_one_gpu(w=w, act_absmax=act_absmax, smooth_out=smooth_out,
                inv_smooth_out=inv_smooth_out)
    _check(lib().sq_smoothing_factors(_ptr(w), K, N, _ld(w), _ptr(act_absmax), float(alpha),
                                      _ptr(smooth_out), _ptr(inv_smooth_out),
                                      _stream(stream, w.device)), "sq_smoothing_factors")


def sq_w4_workspace_bytes(K: int, N: int) -> int:
    return int(lib().sq_w4_workspace_bytes(int(K), int(N)))


def _need_packed4(t, rows, K, name):
    torch = _torch()
    _need(t, torch.uint8, name, 1)
    if not t.is_contiguous() or t.numel() < packed4_bytes(rows, K):
        raise ValueError(f"{name}: expected a contiguous uint8 buffer of "
                         f"{packed4_bytes(rows, K)} bytes (packed 4-bit {rows} x {K} codes)")


def sq_w4_fold_weights(w, smooth, rotate: bool, wq4, w_scale, workspace, stream=None) -> None:
    """4-bit codes (packed two per byte, uint8) and scales of H (s W) per
    output channel, or of s W with rotate False; workspace: a device buffer of
    sq_w4_workspace_bytes(K, N) bytes."""
    torch = _torch()
    _need(w, torch.float16, "w", 2)
    K, N = w.shape
    _need(smooth, torch.float32, "smooth", 1, K)
    _need(w_scale, torch.float32, "w_scale", 1, N)
    _need_packed4(wq4, N, K, "wq4")
    if not workspace.is_contiguous() or \
            workspace.numel() * workspace.element_size() < sq_w4_workspace_bytes(K, N):
        raise ValueError("workspace: expected a contiguous buffer of "
                         "sq_w4_workspace_bytes(K, N) bytes")
    _on_one_gpu(w=w, smooth=smooth, wq4=wq4, w_scale=w_scale, workspace=workspace)
    _check(lib().sq_w4_fold_weights(_ptr(w), K, N, _ld(w), _ptr(smooth), 1 if rotate else 0,
                                    _ptr(wq4), _ptr(w_scale), _ptr(workspace),
                                    _stream(stream, w.device)), "sq_w4_fold_weights")


def sq_w4_gemm(xq, x_scale, wq4, w_scale, y, K: int, out_kind: int = SQ_OUT_F16,
               stream=None) -> None:
    """y [M][N] from packed int8 xq (M tokens) and packed 4-bit wq4 (N
    channels) of K codes each."""
    M, N = _gemm_operands(xq, x_scale, w_scale, y, out_kind)
    _need_packed(xq, M, K, "xq")
    _need_packed4(wq4, N, K, "wq4")
    _on_one_gpu(xq=xq, x_scale=x_scale, wq4=wq4, w_scale=w_scale, y=y)
    _check(lib().sq_w4_gemm(_ptr(xq), _ptr(x_scale), _ptr(wq4), _ptr(w_scale), M, N, int(K),
                            _ptr(y), _ld(y), int(out_kind), _stream(stream, xq.device)),
           "sq_w4_gemm")


def sq_a4_quant_per_token(x, inv_smooth, rotate: bool, xq, x_scale, stream=None) -> None:
    """4-bit per-token codes (packed int8) and scales of (x / s) H, or of
    x / s with rotate False."""
    torch = _torch()
    _need(x, torch.float16, "x", 2)
    M, K = x.shape
    _need(inv_smooth, torch.float32, "inv_smooth", 1, K)
    _need(x_scale, torch.float32, "x_scale", 1, M)
    _need_packed(xq, M, K, "xq")
    _on_one_gpu(x=x, inv_smooth=inv_smooth, xq=xq, x_scale=x_scale)
    _check(lib().sq_a4_quant_per_token(_ptr(x), M, K, _ld(x), _ptr(inv_smooth),
                                       1 if rotate else 0, _ptr(xq), _ptr(x_scale),
                                       _stream(stream, x.device)), "sq_a4_quant_per_token")


def sq_pack_i8(src, dst, stream=None) -> None:
    """Row-major int8 codes src [rows][K] -> packed dst (padding zeroed)."""
    torch = _torch()
    _need(src, torch.int8, "src", 2)
    rows, K = src.shape
    _need_packed(dst, rows, K, "dst")
    _on_one_gpu(src=src, dst=dst)
    _check(lib().sq_pack_i8(_ptr(src), rows, K, _ld(src), _ptr(dst), _stream(stream, src.device)),
           "sq_pack_i8")


def sq_unpack_i8(src, dst, stream=None) -> None:
    """Packed src -> row-major int8 codes dst [rows][K]."""
    torch = _torch()
    _need(dst, torch.int8, "dst", 2)
    rows, K = dst.shape
    _need_packed(src, rows, K, "src")
    _on_one_gpu(src=src, dst=dst)
    _check(lib().sq_unpack_i8(_ptr(src), rows, K, _ptr(dst), _ld(dst), _stream(stream, dst.device)),
           "sq_unpack_i8")


# ---- allocating helpers ---------------------------------------------------------

@dataclass
class Folded:
    """The exported representation of one smoothed, quantized linear layer."""
    smooth: "object"       # float32 [K]  s
    inv_smooth: "object"   # float32 [K]  1/s
    wq: "object"           # packed int8 codes of the N x K folded weights
    w_scale: "object"      # float32 [N]
    K: int = 0
    N: int = 0


def _alloc_stream(stream, device):
    """Torch stream on which a helper allocates its outputs and temporaries:
    the stream the library call runs on, so that the caching allocator hands a
    freed block to later work on that stream only (stream-ordered reuse) and
    never to another stream while a kernel may still read it."""
    return _torch_stream(stream, device)


def calibrate(x_cal, act_absmax=None, stream=None):
    torch = _torch()
    st = _alloc_stream(stream, x_cal.device)
    out = act_absmax
    if out is None:
        with torch.cuda.stream(st):
            out = torch.empty(x_cal.shape[1], dtype=torch.float32, device=x_cal.device)
    sq_calibrate_absmax(x_cal, out, accumulate=act_absmax is not None, stream=st)
    return out


def fold(w, act_absmax, alpha: float, smooth_in=None, stream=None) -> Folded:
    torch = _torch()
    K, N = w.shape
    dev = w.device
    st = _alloc_stream(stream, dev)
    with torch.cuda.stream(st):
        f = Folded(torch.empty(K, dtype=torch.float32, device=dev),
                   torch.empty(K, dtype=torch.float32, device=dev),
                   torch.empty(packed_bytes(N, K), dtype=torch.int8, device=dev),
                   torch.empty(N, dtype=torch.float32, device=dev), K, N)
    sq_smooth_fold_weights(w, act_absmax, alpha, smooth_in, f.smooth, f.inv_smooth, f.wq,
                           f.w_scale, stream=st)
    return f


def quant(x, inv_smooth, stream=None):
    """Returns (packed xq, x_scale)."""
    torch = _torch()
    M, K = x.shape
    st = _alloc_stream(stream, x.device)
    with torch.cuda.stream(st):
        xq = torch.empty(packed_bytes(M, K), dtype=torch.int8, device=x.device)
        xs = torch.empty(M, dtype=torch.float32, device=x.device)
    sq_quant_act_per_token(x, inv_smooth, xq, xs, stream=st)
    return xq, xs


def gemm(xq, x_scale, wq, w_scale, M: int, N: int, K: int, out_kind: int = SQ_OUT_F16,
         stream=None):
    torch = _torch()
    dt = torch.float16 if out_kind == SQ_OUT_F16 else torch.int32
    st = _alloc_stream(stream, xq.device)
    with torch.cuda.stream(st):
        y = torch.empty((M, N), dtype=dt, device=xq.device)
    sq_w8a8_gemm(xq, x_scale, wq, w_scale, y, K, out_kind, stream=st)
    return y


def fold_norm_weight(gamma, inv_smooth, stream=None):
    """Returns gamma / s as float32 [K]."""
    torch = _torch()
    st = _alloc_stream(stream, gamma.device)
    with torch.cuda.stream(st):
        out = torch.empty(gamma.shape[0], dtype=torch.float32, device=gamma.device)
    sq_fold_norm_weight(gamma, inv_smooth, out, stream=st)
    return out


def rmsnorm_quant(h, gamma_folded, eps: float, stream=None):
    """Returns (packed xq, x_scale) of the normalized, smoothed hidden state."""
    torch = _torch()
    M, K = h.shape
    st = _alloc_stream(stream, h.device)
    with torch.cuda.stream(st):
        xq = torch.empty(packed_bytes(M, K), dtype=torch.int8, device=h.device)
        xs = torch.empty(M, dtype=torch.float32, device=h.device)
    sq_rmsnorm_quant_per_token(h, gamma_folded, eps, xq, xs, stream=st)
    return xq, xs


def smoothing_factors(w, act_absmax, alpha: float, stream=None):
    """Returns (s, 1/s) as float32 [K]."""
    torch = _torch()
    K = w.shape[0]
    st = _alloc_stream(stream, w.device)
    with torch.cuda.stream(st):
        s = torch.empty(K, dtype=torch.float32, device=w.device)
        inv = torch.empty(K, dtype=torch.float32, device=w.device)
    sq_smoothing_factors(w, act_absmax, alpha, s, inv, stream=st)
    return s, inv


def fold4(w, smooth, rotate: bool, stream=None):
    """Returns (packed 4-bit codes of the N output channels (uint8), w_scale).
    The workspace is allocated on the call's stream, so its block is reused
    only by later work on that stream once the call's kernels are queued."""
    torch = _torch()
    K, N = w.shape
    st = _alloc_stream(stream, w.device)
    with torch.cuda.stream(st):
        wq = torch.empty(packed4_bytes(N, K), dtype=torch.uint8, device=w.device)
        ws = torch.empty(N, dtype=torch.float32, device=w.device)
        work = torch.empty(max(16, sq_w4_workspace_bytes(K, N)), dtype=torch.uint8,
                           device=w.device)
    sq_w4_fold_weights(w, smooth, rotate, wq, ws, work, stream=st)
    return wq, ws


def gemm4(xq, x_scale, wq4, w_scale, M: int, N: int, K: int, out_kind: int = SQ_OUT_F16,
          stream=None):
    torch = _torch()
    dt = torch.float16 if out_kind == SQ_OUT_F16 else torch.int32
    st = _alloc_stream(stream, xq.device)
    with torch.cuda.stream(st):
        y = torch.empty((M, N), dtype=dt, device=xq.device)
    sq_w4_gemm(xq, x_scale, wq4, w_scale, y, K, out_kind, stream=st)
    return y


def quant4(x, inv_smooth, rotate: bool, stream=None):
    """Returns (packed 4-bit codes of the M tokens, x_scale)."""
    torch = _torch()
    M, K = x.shape
    st = _alloc_stream(stream, x.device)
    with torch.cuda.stream(st):
        xq = torch.empty(packed_bytes(M, K), dtype=torch.int8, device=x.device)
        xs = torch.empty(M, dtype=torch.float32, device=x.device)
    sq_a4_quant_per_token(x, inv_smooth, rotate, xq, xs, stream=st)
    return xq, xs


def pack_i8(codes, stream=None):
    torch = _torch()
    rows, K = codes.shape
    st = _alloc_stream(stream, codes.device)
    with torch.cuda.stream(st):
        dst = torch.empty(packed_bytes(rows, K), dtype=torch.int8, device=codes.device)
    sq_pack_i8(codes, dst, stream=st)
    return dst


def unpack_i8(packed, rows: int, K: int, stream=None):
    torch = _torch()
    st = _alloc_stream(stream, packed.device)
    with torch.cuda.stream(st):
        dst = torch.empty((rows, K), dtype=torch.int8, device=packed.device)
    sq_unpack_i8(packed, dst, stream=st)
    return dst


def smoothed_linear(x, folded: Folded, stream=None):
    """Serving-time layer: per-token quantization of x, then the W8A8 product.
    The intermediate codes and scales are allocated on the call's stream and
    dropped after the product is queued there; the allocator reuses their
    blocks only for later work on the same stream."""
    st = _alloc_stream(stream, x.device)
    xq, xs = quant(x, folded.inv_smooth, stream=st)
    return gemm(xq, xs, folded.wq, folded.w_scale, x.shape[0], folded.N, folded.K, stream=st)
