// Calibration statistics: per-input-channel max |X| over calibration tokens.
//
// The smoothing factor divides by each activation channel's maximum magnitude
// (Pith review of arXiv 2506.01967, key machinery, Eq. 4), estimated on a
// small calibration set (SmoothQuant glossary entry, calibration data).
//
// Layout: X fp16 [T][ldx], K channels.  A workgroup covers 64 channels (8
// lanes x 8 fp16, one 16-byte load per lane, a 128-byte row segment per 8
// lanes), so one wave load spans 8 tokens and the workgroup 32; every lane
// keeps CB_U loads in flight before it reduces them.
// Maxima are taken on the magnitude bits of the fp16 values (sign cleared),
// which order exactly like the magnitudes and put NaN above +inf, so a NaN
// anywhere in a column survives.
//
// Two launch forms:
//   owner   (T <= CB_OWNER_T): one workgroup per 64 channels takes every
//           token and writes the maximum itself (combined with the previous
//           contents when accumulating): no atomics and no separate clear.
//   sliced  (larger T): workgroups take slices of 512 tokens and combine
//           with one atomicMax per channel on the float bit pattern, which is
//           monotone for non-negative floats (and again puts NaN on top);
//           the buffer is cleared first, or, when accumulating, its -0.0
//           entries are made +0.0 so the unsigned order holds.
// max is order-free, so neither form depends on the slice count or the order
// the atomics land in.
#include "sq_device.h"

namespace sq {

constexpr int CB_COLS = 64;      // channels per workgroup
constexpr int CB_U = 16;         // loads in flight per lane
constexpr int CB_ROUND = 32 * CB_U;   // tokens per workgroup round (512)
constexpr int64_t CB_OWNER_T = 1024;

__global__ void __launch_bounds__(256) k_fill_f32(float *__restrict__ p, int64_t n, float v) {
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = v;
}

hipError_t launch_fill_f32(float *p, int64_t n, float v, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    k_fill_f32<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st>>>(p, n, v);
    return hipGetLastError();
}

// -0.0 -> +0.0 (every other value, NaN included, unchanged)
__global__ void __launch_bounds__(256) k_canon_zero(float *__restrict__ p, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n && __float_as_uint(p[i]) == 0x80000000u) p[i] = 0.0f;
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

template <bool OWNER>
__global__ void __launch_bounds__(256)
k_calib_absmax(const uint16_t *__restrict__ x, int64_t T, int64_t K, int64_t ldx,
               int64_t rows_per_block, int accumulate, float *__restrict__ ax) {
    __shared__ uint32_t red[4][CB_COLS];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t c0 = (int64_t)blockIdx.x * CB_COLS + (lane & 7) * 8;
    const int sub = wave * 8 + (lane >> 3);          // token within a group of 32
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
    const int64_t r1 = r0 + rows_per_block < T ? r0 + rows_per_block : T;
    uint32_t m[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) m[i] = 0;
    if (c0 < K) {   // K % 16 == 0, so c0 < K means all 8 channels exist
        for (int64_t rb = r0 + sub; rb < r1; rb += CB_ROUND) {
            uint4 v[CB_U];
#pragma unroll
            for (int u = 0; u < CB_U; ++u) {
                const int64_t r = rb + 32 * u;
                v[u] = r < r1 ? *reinterpret_cast<const uint4 *>(x + r * ldx + c0)
                              : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < CB_U; ++u) {
                const uint32_t q[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    m[2 * i] = umax(m[2 * i], q[i] & 0x7fffu);
                    m[2 * i + 1] = umax(m[2 * i + 1], (q[i] >> 16) & 0x7fffu);
                }
            }
        }
    }
    // the 8 lanes of one channel octet in a wave: lanes l, l+8, ..., l+56
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        m[i] = umax(m[i], (uint32_t)__shfl_xor((int)m[i], 8, 64));
        m[i] = umax(m[i], (uint32_t)__shfl_xor((int)m[i], 16, 64));
        m[i] = umax(m[i], (uint32_t)__shfl_xor((int)m[i], 32, 64));
    }
    if (lane < 8) {
#pragma unroll
        for (int i = 0; i < 8; ++i) red[wave][lane * 8 + i] = m[i];
    }
    __syncthreads();
    if (threadIdx.x < CB_COLS) {
        const int c = threadIdx.x;
        const uint32_t b = umax(umax(red[0][c], red[1][c]), umax(red[2][c], red[3][c]));
        const int64_t col = (int64_t)blockIdx.x * CB_COLS + c;
        if (col < K) {
            uint32_t f = __float_as_uint(h2f(b));   // NaN stays NaN, 0x7c00 becomes +inf
            if (OWNER) {
                if (accumulate) {
                    uint32_t p = __float_as_uint(ax[col]);
                    if (p == 0x80000000u) p = 0;    // -0.0 counts as 0
                    f = umax(f, p);                 // a NaN (either sign) stays on top
                }
                ax[col] = __uint_as_float(f);
            } else if (r1 > r0) {
                atomicMax(reinterpret_cast<unsigned int *>(ax + col), f);
            }
        }
    }
}

hipError_t launch_calib_absmax(const uint16_t *x, int64_t T, int64_t K, int64_t ldx, float *ax,
                               int accumulate, hipStream_t st) {
    if (T <= 0) return accumulate ? hipSuccess : launch_fill_f32(ax, K, 0.0f, st);
    const unsigned col_blocks = (unsigned)((K + CB_COLS - 1) / CB_COLS);
    if (T <= CB_OWNER_T) {
        k_calib_absmax<true><<<dim3(col_blocks, 1), dim3(256), 0, st>>>(x, T, K, ldx, T,
                                                                          accumulate, ax);
        return hipGetLastError();
    }
    if (accumulate) {
        k_canon_zero<<<dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st>>>(ax, K);
    } else {
        k_fill_f32<<<dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st>>>(ax, K, 0.0f);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // about 2048 workgroups at most: slices of whole rounds
    const int64_t rounds = (T + CB_ROUND - 1) / CB_ROUND;
    int64_t want = 2048 / (int64_t)col_blocks;
    if (want < 1) want = 1;
    const int64_t rows = CB_ROUND * ((rounds + want - 1) / want);
    const int64_t row_blocks = (T + rows - 1) / rows;
    k_calib_absmax<false><<<dim3(col_blocks, (unsigned)row_blocks), dim3(256), 0, st>>>(
        x, T, K, ldx, rows, accumulate, ax);
    return hipGetLastError();
}

}  // namespace sq
