// C ABI of the smoothed W8A8 linear layer: argument checks, then launches on
// the caller's stream.  Every check runs before the first HIP call, so a call
// rejected for its arguments has no side effects.  The only host-side data
// work is the fold's check of the smoothing factors it has just computed,
// which overlaps the rest of the fold on the device.  The fold keeps a little
// state per (thread, device): a host buffer for the factors and a device
// scratch for the column maxima.  Its allocation-free variant uses the
// library's static per-device array instead and checks the factors on the
// device.
#include <math.h>
#include <stdint.h>

#include <vector>

#include "sq.h"
#include "sq_internal.h"

#define SQ_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;   // M, N, T < 2^31

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

inline sq_status hip_status(hipError_t e) { return e == hipSuccess ? SQ_OK : SQ_ERR_HIP; }

// K: 16 <= K <= SQ_MAX_K, K % 16 == 0 (int8 rows are whole 16-byte chunks).
inline bool k_ok(int64_t K) { return K >= 16 && K <= SQ_MAX_K && (K % 16) == 0; }

// Per (thread, device) state of the fold, made on first use and kept until
// the process ends:
//   host, host_dev  a pinned, host-coherent buffer of K floats that the
//                   factor kernel writes s into directly (no copy kernel);
//   ready           marks the end of that kernel on the caller's stream;
//   amax            device scratch of N floats: the column maxima, which the
//                   code kernel turns into w_scale;
//   last            the stream of the previous fold: a fold on another stream
//                   first waits (on the host) until the device is idle, as the
//                   old stream's kernels may still use amax.  (An event per
//                   fold for this costs more on the device than the rare wait.)
// A thread's calls wait for `ready` before returning, so the next call may
// reuse the host buffer.
struct Staging {
    float *host = nullptr;
    float *host_dev = nullptr;
    int64_t cap = 0;
    float *amax = nullptr;
    int64_t amax_cap = 0;
    hipEvent_t ready = nullptr;
    hipStream_t last = nullptr;
    bool used = false;
};

// Makes (or grows) the state of the stream's device; the buffers are
// allocated with that device current.
hipError_t staging_for(hipStream_t st, int64_t K, int64_t N, Staging **out) {
    static thread_local std::vector<Staging> per_device;
    int cur = 0, dev = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    dev = cur;
    if (st) {
        e = hipStreamGetDevice(st, &dev);
        if (e != hipSuccess) return e;
    }
    if (dev < 0) return hipErrorInvalidDevice;
    if ((int)per_device.size() <= dev) per_device.resize((size_t)dev + 1);
    Staging &g = per_device[(size_t)dev];
    const bool switch_dev = dev != cur;
    if (switch_dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    if (!g.ready) {
        hipEvent_t ev = nullptr;
        e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
        if (e == hipSuccess) g.ready = ev;
    }
    if (e == hipSuccess && g.cap < K) {
        if (g.host) e = hipHostFree(g.host);
        g.host = g.host_dev = nullptr;
        g.cap = 0;
        void *p = nullptr, *pd = nullptr;
        if (e == hipSuccess) e = hipHostMalloc(&p, (size_t)K * sizeof(float), hipHostMallocCoherent);
        if (e == hipSuccess) e = hipHostGetDevicePointer(&pd, p, 0);
        if (e == hipSuccess) {
            g.host = static_cast<float *>(p);
            g.host_dev = static_cast<float *>(pd);
            g.cap = K;
        }
    }
    // a fold on another stream than this thread's previous one: wait until the
    // device is done with the scratch (the old stream may be gone, so the
    // wait is for the whole device; this is the rare case)
    if (e == hipSuccess && g.used && g.last != st) e = hipDeviceSynchronize();
    if (e == hipSuccess && g.amax_cap < N) {
        // (hipFree waits for the device, so a previous fold is done with it)
        if (g.amax) e = hipFree(g.amax);
        g.amax = nullptr;
        g.amax_cap = 0;
        void *p = nullptr;
        if (e == hipSuccess) e = hipMalloc(&p, (size_t)N * sizeof(float));
        if (e == hipSuccess) {
            g.amax = static_cast<float *>(p);
            g.amax_cap = N;
        }
    }
    if (switch_dev) {
        const hipError_t e2 = hipSetDevice(cur);
        if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    *out = &g;
    return hipSuccess;
}

// The fold's check of the factors it wrote to the host buffer.  1/s is the
// IEEE float quotient on both sides, so the host recomputes it for the range
// check instead of copying it back.
sq_status check_factors(const float *host, int64_t K) {
    bool nonfinite = false, range = false;
    for (int64_t j = 0; j < K; ++j) {
        const float sj = host[j];
        if (isnan(sj)) nonfinite = true;
        else if (!isnormal(sj) || !isnormal(1.0f / sj) || sj < 0.0f) range = true;
    }
    if (nonfinite) return SQ_ERR_NONFINITE;
    if (range) return SQ_ERR_RANGE;
    return SQ_OK;
}

}  // namespace

SQ_API const char *sq_status_str(int status) {
    switch (status) {
        case SQ_OK: return "SQ_OK";
        case SQ_ERR_NULL: return "SQ_ERR_NULL: a required pointer is NULL";
        case SQ_ERR_SHAPE: return "SQ_ERR_SHAPE: a size or stride is out of range";
        case SQ_ERR_ALIGN: return "SQ_ERR_ALIGN: a pointer or stride breaks the 16-byte alignment rules";
        case SQ_ERR_ALPHA: return "SQ_ERR_ALPHA: alpha must lie in [0, 1]";
        case SQ_ERR_NONFINITE: return "SQ_ERR_NONFINITE: a statistic or factor is NaN, infinite or negative";
        case SQ_ERR_RANGE: return "SQ_ERR_RANGE: a factor or its reciprocal is zero, infinite or subnormal";
        case SQ_ERR_HIP: return "SQ_ERR_HIP: the HIP runtime reported an error";
        case SQ_ERR_KIND: return "SQ_ERR_KIND: unknown out_kind";
        case SQ_ERR_EPS: return "SQ_ERR_EPS: eps must be finite and >= 0";
        default: return "unknown sq_status";
    }
}

SQ_API int sq_version(void) { return 10500; }

SQ_API int64_t sq_packed_bytes(int64_t rows, int64_t K) {
    if (rows < 0 || rows >= kMaxDim || !k_ok(K)) return 0;
    return ((rows + 15) / 16) * ((K + 63) / 64) * 1024;
}

SQ_API sq_status sq_calibrate_absmax(const void *x_cal_f16, int64_t T, int64_t K, int64_t ldx,
                                     float *act_absmax, int accumulate, void *stream) {
    if (!act_absmax || (T > 0 && !x_cal_f16)) return SQ_ERR_NULL;
    if (T < 0 || T >= kMaxDim || !k_ok(K) || ldx < K) return SQ_ERR_SHAPE;
    if (!aligned16(act_absmax) || (x_cal_f16 && !aligned16(x_cal_f16)) || (ldx % 8) != 0)
        return SQ_ERR_ALIGN;
    return hip_status(sq::launch_calib_absmax(static_cast<const uint16_t *>(x_cal_f16), T, K, ldx,
                                              act_absmax, accumulate != 0, as_stream(stream)));
}

// The fold's argument checks, shared by both fold entry points.
static sq_status fold_args(const void *w_f16, int64_t K, int64_t N, int64_t ldw,
                           const float *act_absmax, float alpha, const float *smooth_in,
                           const float *smooth_out, const float *inv_smooth_out, const int8_t *wq,
                           const float *w_scale) {
    if (!smooth_out || !inv_smooth_out || (!smooth_in && !act_absmax)) return SQ_ERR_NULL;
    if (N > 0 && (!w_f16 || !wq || !w_scale)) return SQ_ERR_NULL;
    if (N < 0 || N >= kMaxDim || !k_ok(K) || (N > 0 && ldw < N)) return SQ_ERR_SHAPE;
    if (!aligned16(smooth_out) || !aligned16(inv_smooth_out) ||
        (act_absmax && !aligned16(act_absmax)) || (smooth_in && !aligned16(smooth_in)))
        return SQ_ERR_ALIGN;
    if (N > 0 && (!aligned16(w_f16) || !aligned16(wq) || !aligned16(w_scale) || (ldw % 8) != 0))
        return SQ_ERR_ALIGN;
    if (!smooth_in && !(alpha >= 0.0f && alpha <= 1.0f)) return SQ_ERR_ALPHA;
    return SQ_OK;
}

SQ_API sq_status sq_smooth_fold_weights(const void *w_f16, int64_t K, int64_t N, int64_t ldw,
                                        const float *act_absmax, float alpha,
                                        const float *smooth_in, float *smooth_out,
                                        float *inv_smooth_out, int8_t *wq, float *w_scale,
                                        void *stream) {
    const sq_status a = fold_args(w_f16, K, N, ldw, act_absmax, alpha, smooth_in, smooth_out,
                                  inv_smooth_out, wq, w_scale);
    if (a != SQ_OK) return a;

    const hipStream_t st = as_stream(stream);
    const uint16_t *w = static_cast<const uint16_t *>(w_f16);
    Staging *g = nullptr;
    hipError_t e = staging_for(st, K, N, &g);
    if (e != hipSuccess) return SQ_ERR_HIP;
    // Everything is queued before the one wait: the factor kernel writes s
    // straight to the host buffer, and the column maxima and the codes follow
    // on the stream while the host waits for it.  With N == 0 no row is read
    // (aw = 0).
    e = sq::launch_row_smooth(w, K, N, ldw, act_absmax, smooth_in, alpha, smooth_out,
                              inv_smooth_out, g->host_dev, g->amax, nullptr, st);
    if (e == hipSuccess) e = hipEventRecord(g->ready, st);
    if (e != hipSuccess) return SQ_ERR_HIP;
    if (N > 0) {
        e = sq::launch_fold_colabsmax(w, K, N, ldw, smooth_out, g->amax, st);
        if (e == hipSuccess)
            e = sq::launch_fold_quant(w, K, N, ldw, smooth_out, g->amax, wq, w_scale, st);
    }
    g->last = st;
    g->used = true;
    const hipError_t ew = hipEventSynchronize(g->ready);
    if (e != hipSuccess || ew != hipSuccess) return SQ_ERR_HIP;

    return check_factors(g->host, K);
}

// The same fold without allocating: column maxima and the factors' status in
// the library's per-device scratch array, the check of the factors done on
// the device, one 4-byte copy of the status to the host and one wait for the
// stream at the end.  No hipMalloc, hipHostMalloc, hipFree or event.
SQ_API sq_status sq_smooth_fold_weights_noalloc(const void *w_f16, int64_t K, int64_t N,
                                                int64_t ldw, const float *act_absmax, float alpha,
                                                const float *smooth_in, float *smooth_out,
                                                float *inv_smooth_out, int8_t *wq,
                                                float *w_scale, void *stream) {
    const sq_status a = fold_args(w_f16, K, N, ldw, act_absmax, alpha, smooth_in, smooth_out,
                                  inv_smooth_out, wq, w_scale);
    if (a != SQ_OK) return a;
    if (N > SQ_NOALLOC_MAX_N) return SQ_ERR_SHAPE;

    const hipStream_t st = as_stream(stream);
    int dev = 0;
    hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
    float *amax = nullptr;
    uint32_t *status = nullptr;
    if (e == hipSuccess) e = sq::noalloc_scratch(dev, &amax, &status);
    if (e != hipSuccess) return SQ_ERR_HIP;
    const uint16_t *w = static_cast<const uint16_t *>(w_f16);
    // the status word keeps the previous call's value: clear it (a fill
    // kernel; the factor kernel clears the column maxima itself)
    e = sq::launch_fill_f32(reinterpret_cast<float *>(status), 1, 0.0f, st);
    if (e == hipSuccess)
        e = sq::launch_row_smooth(w, K, N, ldw, act_absmax, smooth_in, alpha, smooth_out,
                                  inv_smooth_out, nullptr, amax, status, st);
    uint32_t host_status = 0;
    if (e == hipSuccess)
        e = hipMemcpyAsync(&host_status, status, sizeof(host_status), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess && N > 0) {
        e = sq::launch_fold_colabsmax(w, K, N, ldw, smooth_out, amax, st);
        if (e == hipSuccess)
            e = sq::launch_fold_quant(w, K, N, ldw, smooth_out, amax, wq, w_scale, st);
    }
    // wait for the status copy (and the rest of the fold) even after a failed
    // launch, so host_status is never written after this frame is gone
    const hipError_t ew = hipStreamSynchronize(st);
    if (e != hipSuccess || ew != hipSuccess) return SQ_ERR_HIP;
    if (host_status & 1u) return SQ_ERR_NONFINITE;
    if (host_status & 2u) return SQ_ERR_RANGE;
    return SQ_OK;
}

SQ_API sq_status sq_smoothing_factors(const void *w_f16, int64_t K, int64_t N, int64_t ldw,
                                      const float *act_absmax, float alpha, float *smooth_out,
                                      float *inv_smooth_out, void *stream) {
    if (!smooth_out || !inv_smooth_out || !act_absmax || (N > 0 && !w_f16)) return SQ_ERR_NULL;
    if (N < 0 || N >= kMaxDim || !k_ok(K) || (N > 0 && ldw < N)) return SQ_ERR_SHAPE;
    if (!aligned16(smooth_out) || !aligned16(inv_smooth_out) || !aligned16(act_absmax))
        return SQ_ERR_ALIGN;
    if (N > 0 && (!aligned16(w_f16) || (ldw % 8) != 0)) return SQ_ERR_ALIGN;
    if (!(alpha >= 0.0f && alpha <= 1.0f)) return SQ_ERR_ALPHA;
    const hipStream_t st = as_stream(stream);
    Staging *g = nullptr;
    if (staging_for(st, K, 0, &g) != hipSuccess) return SQ_ERR_HIP;
    hipError_t e = sq::launch_row_smooth(static_cast<const uint16_t *>(w_f16), K, N, ldw,
                                         act_absmax, nullptr, alpha, smooth_out, inv_smooth_out,
                                         g->host_dev, nullptr, nullptr, st);
    if (e == hipSuccess) e = hipEventRecord(g->ready, st);
    g->last = st;
    g->used = true;
    if (e != hipSuccess) {
        (void)hipStreamSynchronize(st);
        return SQ_ERR_HIP;
    }
    if (hipEventSynchronize(g->ready) != hipSuccess) return SQ_ERR_HIP;
    return check_factors(g->host, K);
}

SQ_API int64_t sq_packed4_bytes(int64_t rows, int64_t K) {
    if (rows < 0 || rows >= kMaxDim || !k_ok(K)) return 0;
    return ((rows + 15) / 16) * ((K + 63) / 64) * 512;
}

SQ_API int64_t sq_w4_workspace_bytes(int64_t K, int64_t N) {
    if (N < 0 || N >= kMaxDim || !k_ok(K)) return 0;
    return 2 * K * N + sq_packed_bytes(N, K);
}

// K for the 4-bit calls: a whole number of 16-code rows up to the register-
// resident kernels' 8192, and a power of two when rotated (Sylvester matrix).
static bool k4_ok(int64_t K, int rotate) {
    if (!k_ok(K) || K > 8192) return false;
    return !rotate || (K & (K - 1)) == 0;
}

SQ_API sq_status sq_a4_quant_per_token(const void *x_f16, int64_t M, int64_t K, int64_t ldx,
                                       const float *inv_smooth, int rotate, int8_t *xq,
                                       float *x_scale, void *stream) {
    if (!inv_smooth || (M > 0 && (!x_f16 || !xq || !x_scale))) return SQ_ERR_NULL;
    if (M < 0 || M >= kMaxDim || !k4_ok(K, rotate) || ldx < K) return SQ_ERR_SHAPE;
    if (!aligned16(inv_smooth) || (ldx % 8) != 0) return SQ_ERR_ALIGN;
    if (M > 0 && (!aligned16(x_f16) || !aligned16(xq) || !aligned16(x_scale))) return SQ_ERR_ALIGN;
    return hip_status(sq::launch_quant4_rows(static_cast<const uint16_t *>(x_f16), M, K, ldx,
                                             inv_smooth, rotate != 0, 1.0f, xq, x_scale,
                                             as_stream(stream)));
}

SQ_API sq_status sq_w4_fold_weights(const void *w_f16, int64_t K, int64_t N, int64_t ldw,
                                    const float *smooth, int rotate, uint8_t *wq4, float *w_scale,
                                    void *workspace, void *stream) {
    uint8_t *wq = wq4;
    if (!smooth || (N > 0 && (!w_f16 || !wq || !w_scale || !workspace))) return SQ_ERR_NULL;
    if (N < 0 || N >= kMaxDim || !k4_ok(K, rotate) || (N > 0 && ldw < N)) return SQ_ERR_SHAPE;
    if (!aligned16(smooth)) return SQ_ERR_ALIGN;
    if (N > 0 && (!aligned16(w_f16) || !aligned16(wq) || !aligned16(w_scale) ||
                  !aligned16(workspace) || (ldw % 8) != 0))
        return SQ_ERR_ALIGN;
    return hip_status(sq::launch_fold4(static_cast<const uint16_t *>(w_f16), K, N, ldw, smooth,
                                       rotate != 0, wq, w_scale,
                                       static_cast<uint8_t *>(workspace), as_stream(stream)));
}

SQ_API sq_status sq_w4_gemm(const int8_t *xq, const float *x_scale, const uint8_t *wq4,
                            const float *w_scale, int64_t M, int64_t N, int64_t K, void *y,
                            int64_t ldy, int out_kind, void *stream) {
    if (out_kind != SQ_OUT_F16 && out_kind != SQ_OUT_I32) return SQ_ERR_KIND;
    const bool work = M > 0 && N > 0;
    if (work && (!xq || !wq4 || !y)) return SQ_ERR_NULL;
    if (work && out_kind == SQ_OUT_F16 && (!x_scale || !w_scale)) return SQ_ERR_NULL;
    if (M < 0 || N < 0 || M >= kMaxDim || N >= kMaxDim || !k_ok(K)) return SQ_ERR_SHAPE;
    if (work && ldy < N) return SQ_ERR_SHAPE;
    if (work && ((M + 255) / 256) * ((N + 127) / 128) >= kMaxDim) return SQ_ERR_SHAPE;
    if (work) {
        if (!aligned16(xq) || !aligned16(wq4)) return SQ_ERR_ALIGN;
        if (out_kind == SQ_OUT_F16 && (!aligned16(x_scale) || !aligned16(w_scale))) return SQ_ERR_ALIGN;
        if (((uintptr_t)y % (out_kind == SQ_OUT_F16 ? 2u : 4u)) != 0) return SQ_ERR_ALIGN;
    }
    if (!work) return SQ_OK;
    return hip_status(sq::launch_gemm_w4(xq, x_scale, wq4, w_scale, M, N, K, y, ldy, out_kind,
                                         as_stream(stream)));
}

SQ_API sq_status sq_quant_act_per_token(const void *x_f16, int64_t M, int64_t K, int64_t ldx,
                                        const float *inv_smooth, int8_t *xq, float *x_scale,
                                        void *stream) {
    if (!inv_smooth || (M > 0 && (!x_f16 || !xq || !x_scale))) return SQ_ERR_NULL;
    if (M < 0 || M >= kMaxDim || !k_ok(K) || ldx < K) return SQ_ERR_SHAPE;
    if (!aligned16(inv_smooth) || (ldx % 8) != 0) return SQ_ERR_ALIGN;
    if (M > 0 && (!aligned16(x_f16) || !aligned16(xq) || !aligned16(x_scale))) return SQ_ERR_ALIGN;
    return hip_status(sq::launch_quant_act(static_cast<const uint16_t *>(x_f16), M, K, ldx,
                                           inv_smooth, xq, x_scale, as_stream(stream)));
}

SQ_API sq_status sq_fold_norm_weight(const void *gamma_f16, int64_t K, const float *inv_smooth,
                                     float *gamma_out, void *stream) {
    if (!gamma_f16 || !inv_smooth || !gamma_out) return SQ_ERR_NULL;
    if (!k_ok(K)) return SQ_ERR_SHAPE;
    if (!aligned16(gamma_f16) || !aligned16(inv_smooth) || !aligned16(gamma_out)) return SQ_ERR_ALIGN;
    return hip_status(sq::launch_fold_norm_weight(static_cast<const uint16_t *>(gamma_f16), K,
                                                  inv_smooth, gamma_out, as_stream(stream)));
}

SQ_API sq_status sq_rmsnorm_quant_per_token(const void *h_f16, int64_t M, int64_t K, int64_t ldh,
                                            const float *gamma_folded, float eps, int8_t *xq,
                                            float *x_scale, void *stream) {
    if (!gamma_folded || (M > 0 && (!h_f16 || !xq || !x_scale))) return SQ_ERR_NULL;
    if (M < 0 || M >= kMaxDim || !k_ok(K) || ldh < K) return SQ_ERR_SHAPE;
    if (!(eps >= 0.0f) || !isfinite(eps)) return SQ_ERR_EPS;
    if (!aligned16(gamma_folded) || (ldh % 8) != 0) return SQ_ERR_ALIGN;
    if (M > 0 && (!aligned16(h_f16) || !aligned16(xq) || !aligned16(x_scale))) return SQ_ERR_ALIGN;
    return hip_status(sq::launch_rmsnorm_quant(static_cast<const uint16_t *>(h_f16), M, K, ldh,
                                               gamma_folded, eps, xq, x_scale, as_stream(stream)));
}

SQ_API sq_status sq_w8a8_gemm(const int8_t *xq, const float *x_scale, const int8_t *wq,
                              const float *w_scale, int64_t M, int64_t N, int64_t K, void *y,
                              int64_t ldy, int out_kind, void *stream) {
    if (out_kind != SQ_OUT_F16 && out_kind != SQ_OUT_I32) return SQ_ERR_KIND;
    const bool work = M > 0 && N > 0;
    if (work && (!xq || !wq || !y)) return SQ_ERR_NULL;
    if (work && out_kind == SQ_OUT_F16 && (!x_scale || !w_scale)) return SQ_ERR_NULL;
    if (M < 0 || N < 0 || M >= kMaxDim || N >= kMaxDim || !k_ok(K)) return SQ_ERR_SHAPE;
    if (work && ldy < N) return SQ_ERR_SHAPE;
    // one workgroup per 256 x 128 output tile: the tile count must fit a 1-D grid
    if (work && ((M + 255) / 256) * ((N + 127) / 128) >= kMaxDim) return SQ_ERR_SHAPE;
    if (work) {
        if (!aligned16(xq) || !aligned16(wq)) return SQ_ERR_ALIGN;
        if (out_kind == SQ_OUT_F16 && (!aligned16(x_scale) || !aligned16(w_scale))) return SQ_ERR_ALIGN;
        // y needs only its element alignment; any ldy >= N works
        if (((uintptr_t)y % (out_kind == SQ_OUT_F16 ? 2u : 4u)) != 0) return SQ_ERR_ALIGN;
    }
    if (!work) return SQ_OK;
    return hip_status(sq::launch_gemm(xq, x_scale, wq, w_scale, M, N, K, y, ldy, out_kind,
                                      as_stream(stream)));
}

SQ_API sq_status sq_pack_i8(const int8_t *src, int64_t rows, int64_t K, int64_t ld, int8_t *dst,
                            void *stream) {
    if (rows > 0 && (!src || !dst)) return SQ_ERR_NULL;
    if (rows < 0 || rows >= kMaxDim || !k_ok(K) || ld < K) return SQ_ERR_SHAPE;
    if (rows > 0 && (!aligned16(src) || !aligned16(dst) || (ld % 16) != 0)) return SQ_ERR_ALIGN;
    if (rows == 0) return SQ_OK;
    return hip_status(sq::launch_pack_i8(src, rows, K, ld, dst, as_stream(stream)));
}

SQ_API sq_status sq_unpack_i8(const int8_t *src, int64_t rows, int64_t K, int8_t *dst, int64_t ld,
                              void *stream) {
    if (rows > 0 && (!src || !dst)) return SQ_ERR_NULL;
    if (rows < 0 || rows >= kMaxDim || !k_ok(K) || ld < K) return SQ_ERR_SHAPE;
    if (rows > 0 && (!aligned16(src) || !aligned16(dst) || (ld % 16) != 0)) return SQ_ERR_ALIGN;
    if (rows == 0) return SQ_OK;
    return hip_status(sq::launch_unpack_i8(src, rows, K, dst, ld, as_stream(stream)));
}
