// Offline fold of the smoothing factors into W and per-output-channel int8
// quantization of the result.
//
// Row j of W (input channel j) is multiplied by s_j, compensating the division
// of activation channel j by s_j, so (X S^-1)(S W) = X W ("Move activation
// scale without changing the real linear map", para. 1); the transform runs
// offline, before serving ("Quantization", learn-kernels.com, para. 2).
// s_j = max|X_j|^alpha / max|W_j|^(1-alpha) (Pith review of arXiv 2506.01967,
// key machinery, Eq. 4 at alpha = 1/2).
//
// Kernels, in launch order:
//   k_row_absmax      aw_j = max_n |W[j][n]|              (one wave per row)
//   k_smooth_factors  s_j, 1/s_j in float; zeroes w_scale (one lane per channel)
//   -- the host checks s and 1/s here --
//   k_fold_colabsmax  amax_n = max_j |float(W[j][n]) * s_j|  (into w_scale, atomics)
//   k_fold_quant      Wq[n][j] = clamp(rint((W*s) * (127/amax_n)), +-127), transposed
//                     through LDS and written as packed 16 x 64-byte fragments
//                     (the operand order of the int8 matrix instruction), with
//                     the padding rows and windows written as zero
//   k_fold_finalize   w_scale[n] = amax_n / 127
#include <math.h>

#include "sq_device.h"

namespace sq {

// ---- aw_j = max_n |W[j][n]| --------------------------------------------------

__global__ void __launch_bounds__(256)
k_row_absmax(const uint16_t *__restrict__ w, int64_t K, int64_t N, int64_t ldw,
             float *__restrict__ aw) {
    const int lane = threadIdx.x & 63;
    const int64_t j = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (j >= K) return;
    const uint16_t *row = w + j * ldw;
    uint32_t m = 0;
    for (int64_t c = (int64_t)lane * 8; c < N; c += 512) {
        if (c + 8 <= N) {
            const uint4 v = *reinterpret_cast<const uint4 *>(row + c);
            const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t lo = q[i] & 0x7fffu, hi = (q[i] >> 16) & 0x7fffu;
                m = m > lo ? m : lo;
                m = m > hi ? m : hi;
            }
        } else {
            for (int64_t e = c; e < N; ++e) {
                const uint32_t b = row[e] & 0x7fffu;
                m = m > b ? m : b;
            }
        }
    }
    m = wave_max_u32(m);
    if (lane == 0) aw[j] = h2f(m);   // NaN bits stay NaN, 0x7c00 becomes +inf
}

hipError_t launch_row_absmax(const uint16_t *w, int64_t K, int64_t N, int64_t ldw, float *aw,
                             hipStream_t st) {
    k_row_absmax<<<dim3((unsigned)((K + 3) / 4)), dim3(256), 0, st>>>(w, K, N, ldw, aw);
    return hipGetLastError();
}

// ---- smoothing factors ---------------------------------------------------------

// On entry aw_inv holds aw; on exit it holds 1/s.  A statistic that is NaN,
// infinite or negative (or such a given factor) yields s = NaN, which the host
// reports as non-finite; range problems (s or 1/s zero, infinite, subnormal)
// are left for the host to see.  The division is IEEE-correct in float.
__global__ void __launch_bounds__(256)
k_smooth_factors(const float *__restrict__ ax, const float *__restrict__ smooth_in,
                 float *__restrict__ aw_inv, double alpha, int64_t K, float *__restrict__ s_out,
                 float *__restrict__ w_scale, int64_t N) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < K) {
        const float aw = aw_inv[i];
        float s;
        if (!isfinite(aw)) {
            s = __builtin_nanf("");
        } else if (smooth_in) {
            const float v = smooth_in[i];
            s = (isfinite(v) && v >= 0.0f) ? v : __builtin_nanf("");
        } else {
            const float a = ax[i];
            if (!isfinite(a) || a < 0.0f)
                s = __builtin_nanf("");
            else if (a == 0.0f || aw == 0.0f)
                s = 1.0f;   // dead channel or zero row: the plainest positive factor
            else
                s = (float)(pow((double)a, alpha) / pow((double)aw, 1.0 - alpha));
        }
        s_out[i] = s;
        aw_inv[i] = 1.0f / s;
    }
    if (i < N) w_scale[i] = 0.0f;
}

hipError_t launch_smooth_factors(const float *ax, const float *smooth_in, float *aw_in_inv_out,
                                 float alpha, int64_t K, float *s_out, float *w_scale_zero,
                                 int64_t N, hipStream_t st) {
    const int64_t n = K > N ? K : N;
    k_smooth_factors<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st>>>(
        ax, smooth_in, aw_in_inv_out, (double)alpha, K, s_out, w_scale_zero, N);
    return hipGetLastError();
}

// ---- amax_n = max_j |float(W[j][n]) * s_j| ---------------------------------------

// Same layout as the calibration kernel: 512 columns per workgroup, 8 per lane,
// waves stride over a slice of rows, LDS combine, one atomicMax per column on
// the (non-negative) float bits.  W has already been checked finite.
__global__ void __launch_bounds__(256)
k_fold_colabsmax(const uint16_t *__restrict__ w, int64_t K, int64_t N, int64_t ldw,
                 const float *__restrict__ s, int rows_per_block, float *__restrict__ amax) {
    __shared__ uint32_t red[4][512];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t c0 = (int64_t)blockIdx.x * 512 + lane * 8;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
    const int64_t r1 = r0 + rows_per_block < K ? r0 + rows_per_block : K;
    float m[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) m[i] = 0.0f;
    if (c0 < N) {
        for (int64_t r = r0 + wave; r < r1; r += 4) {
            const float sj = s[r];
            const uint16_t *row = w + r * ldw + c0;
            if (c0 + 8 <= N) {
                const uint4 v = *reinterpret_cast<const uint4 *>(row);
                const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    m[2 * i] = fmaxf(m[2 * i], fabsf(h2f(q[i] & 0xffffu) * sj));
                    m[2 * i + 1] = fmaxf(m[2 * i + 1], fabsf(h2f(q[i] >> 16) * sj));
                }
            } else {
                for (int i = 0; i < 8 && c0 + i < N; ++i)
                    m[i] = fmaxf(m[i], fabsf(h2f(row[i]) * sj));
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) red[wave][lane * 8 + i] = __float_as_uint(m[i]);
    __syncthreads();
    for (int c = threadIdx.x; c < 512; c += 256) {
        uint32_t b = red[0][c];
        b = b > red[1][c] ? b : red[1][c];
        b = b > red[2][c] ? b : red[2][c];
        b = b > red[3][c] ? b : red[3][c];
        const int64_t col = (int64_t)blockIdx.x * 512 + c;
        if (col < N && r1 > r0) atomicMax(reinterpret_cast<unsigned int *>(amax + col), b);
    }
}

hipError_t launch_fold_colabsmax(const uint16_t *w, int64_t K, int64_t N, int64_t ldw,
                                 const float *s, float *amax, hipStream_t st) {
    const int64_t col_blocks = (N + 511) / 512;
    int64_t want = 2048 / col_blocks;
    if (want < 1) want = 1;
    int64_t rows = (K + want - 1) / want;
    if (rows < 8) rows = 8;
    const int64_t row_blocks = (K + rows - 1) / rows;
    k_fold_colabsmax<<<dim3((unsigned)col_blocks, (unsigned)row_blocks), dim3(256), 0, st>>>(
        w, K, N, ldw, s, (int)rows, amax);
    return hipGetLastError();
}

// ---- quantize and transpose ---------------------------------------------------------

// Tile: 64 output channels x 256 input channels.  A work item is 4 consecutive
// rows j x 8 consecutive columns n (four 16-byte loads); each of its 8 columns
// yields 4 consecutive codes of one Wq row, packed into a 32-bit LDS store.
// The tile then leaves as 4 x 4 packed fragments of 1 KiB (16 channels x 64
// input channels each), one 16-byte store per lane.  Out-of-range channels and
// input channels hold zero codes, so the padding of the packed buffer is zero.
constexpr int FQ_TN = 64;
constexpr int FQ_TK = 256;
constexpr int FQ_LDS = FQ_TK + 16;   // row pitch in bytes; breaks power-of-two strides

__global__ void __launch_bounds__(256)
k_fold_quant(const uint16_t *__restrict__ w, int64_t K, int64_t N, int64_t ldw,
             const float *__restrict__ s, const float *__restrict__ amax,
             int8_t *__restrict__ wq) {
    __shared__ __align__(16) uint8_t tile[FQ_TN * FQ_LDS];
    const int64_t n0 = (int64_t)blockIdx.x * FQ_TN;
    const int64_t k0 = (int64_t)blockIdx.y * FQ_TK;
    // 64 row-quads x 8 column-octets = 512 work items, 2 per thread
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int item = threadIdx.x + it * 256;
        const int oct = item & 7;          // column octet within the tile
        const int quad = item >> 3;        // row quad within the tile
        const int64_t n = n0 + oct * 8;
        const int64_t j = k0 + quad * 4;
        uint32_t packed[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) packed[c] = 0;
        float r[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float a = (n + c < N) ? amax[n + c] : 0.0f;
            r[c] = a > 0.0f ? 127.0f / a : 0.0f;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t jj = j + q;
            if (jj >= K) break;
            const float sj = s[jj];
            float v[8];
            const uint16_t *row = w + jj * ldw + n;
            if (n + 8 <= N) {
                const uint4 raw = *reinterpret_cast<const uint4 *>(row);
                const uint32_t h[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[2 * i] = h2f(h[i] & 0xffffu);
                    v[2 * i + 1] = h2f(h[i] >> 16);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = (n + i < N) ? h2f(row[i]) : 0.0f;
            }
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const float wt = v[c] * sj;                 // W~ = W * s_j (float)
                float qf = __builtin_rintf(wt * r[c]);      // round half to even
                qf = fminf(fmaxf(qf, -127.0f), 127.0f);
                packed[c] |= ((uint32_t)(int)qf & 0xffu) << (8 * q);
            }
        }
#pragma unroll
        for (int c = 0; c < 8; ++c)
            *reinterpret_cast<uint32_t *>(tile + (oct * 8 + c) * FQ_LDS + quad * 4) = packed[c];
    }
    __syncthreads();
    // 16 fragments x 64 lanes of 16 bytes = 1024 chunks, 4 per thread
    const int64_t KW = (K + 63) >> 6;
    const int64_t RB = (N + 15) >> 4;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int item = threadIdx.x + it * 256;
        const int l = item & 63;
        const int f = item >> 6;             // fragment: 4 channel blocks x 4 windows
        const int rbl = f >> 2, kwl = f & 3;
        const int64_t rb = (n0 >> 4) + rbl;
        const int64_t kw = (k0 >> 6) + kwl;
        const int rn = rbl * 16 + (l & 15);
        const int kk = kwl * 64 + (l >> 4) * 16;
        if (rb < RB && kw < KW)
            *reinterpret_cast<uint4 *>(wq + ((rb * KW + kw) << 10) + l * 16) =
                *reinterpret_cast<const uint4 *>(tile + rn * FQ_LDS + kk);
    }
}

hipError_t launch_fold_quant(const uint16_t *w, int64_t K, int64_t N, int64_t ldw, const float *s,
                             const float *amax, int8_t *wq, hipStream_t st) {
    const dim3 grid((unsigned)((N + FQ_TN - 1) / FQ_TN), (unsigned)((K + FQ_TK - 1) / FQ_TK));
    k_fold_quant<<<grid, dim3(256), 0, st>>>(w, K, N, ldw, s, amax, wq);
    return hipGetLastError();
}

// ---- w_scale[n] = amax_n / 127 -----------------------------------------------------

__global__ void __launch_bounds__(256) k_fold_finalize(float *__restrict__ w_scale, int64_t N) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < N) w_scale[i] = w_scale[i] / 127.0f;
}

hipError_t launch_fold_finalize(float *w_scale, int64_t N, hipStream_t st) {
    if (N <= 0) return hipSuccess;
    k_fold_finalize<<<dim3((unsigned)((N + 255) / 256)), dim3(256), 0, st>>>(w_scale, N);
    return hipGetLastError();
}

}  // namespace sq
