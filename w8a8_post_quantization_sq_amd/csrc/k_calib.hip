// Calibration statistics: per-input-channel max |X| over calibration tokens.
//
// The smoothing factor divides by each activation channel's maximum magnitude
// (Pith review of arXiv 2506.01967, key machinery, Eq. 4), estimated on a
// small calibration set (SmoothQuant glossary entry, calibration data).
//
// Layout: X fp16 [T][ldx], K channels.  One workgroup covers 512 channels
// (64 lanes x 8 fp16 = one 16-byte load per lane, a fully coalesced 1 KiB row
// segment per wave) over a slice of tokens; its 4 waves take every 4th token.
// Maxima are taken on the magnitude bits of the fp16 values (sign cleared),
// which order exactly like the magnitudes and put NaN above +inf, so a NaN
// anywhere in a column survives.  Slices combine with one atomicMax per
// channel on the float bit pattern, which is monotone for non-negative floats
// (and again puts NaN on top); max is order-free, so the result does not
// depend on the slice count or the order the atomics land in.
#include "sq_device.h"

namespace sq {

__global__ void __launch_bounds__(256) k_fill_f32(float *__restrict__ p, int64_t n, float v) {
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = v;
}

hipError_t launch_fill_f32(float *p, int64_t n, float v, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    k_fill_f32<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st>>>(p, n, v);
    return hipGetLastError();
}

__global__ void __launch_bounds__(256)
k_calib_absmax(const uint16_t *__restrict__ x, int64_t T, int64_t K, int64_t ldx,
               int rows_per_block, float *__restrict__ ax) {
    __shared__ uint32_t red[4][512];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t c0 = (int64_t)blockIdx.x * 512 + lane * 8;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
    const int64_t r1 = r0 + rows_per_block < T ? r0 + rows_per_block : T;
    uint32_t m[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) m[i] = 0;
    if (c0 < K) {   // K % 16 == 0, so c0 < K means all 8 channels exist
        for (int64_t r = r0 + wave; r < r1; r += 4) {
            const uint4 v = *reinterpret_cast<const uint4 *>(x + r * ldx + c0);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t lo = w[i] & 0x7fffu, hi = (w[i] >> 16) & 0x7fffu;
                m[2 * i] = m[2 * i] > lo ? m[2 * i] : lo;
                m[2 * i + 1] = m[2 * i + 1] > hi ? m[2 * i + 1] : hi;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) red[wave][lane * 8 + i] = m[i];
    __syncthreads();
    for (int c = threadIdx.x; c < 512; c += 256) {
        uint32_t b = red[0][c];
        b = b > red[1][c] ? b : red[1][c];
        b = b > red[2][c] ? b : red[2][c];
        b = b > red[3][c] ? b : red[3][c];
        const int64_t col = (int64_t)blockIdx.x * 512 + c;
        if (col < K && r1 > r0)
            atomicMax(reinterpret_cast<unsigned int *>(ax + col), __float_as_uint(h2f(b)));
    }
}

hipError_t launch_calib_absmax(const uint16_t *x, int64_t T, int64_t K, int64_t ldx, float *ax,
                               hipStream_t st) {
    if (T <= 0) return hipSuccess;
    const int64_t col_blocks = (K + 511) / 512;
    // about 1024 workgroups in total, at least 8 tokens (2 per wave) each
    int64_t want = 1024 / col_blocks;
    if (want < 1) want = 1;
    int64_t rows = (T + want - 1) / want;
    if (rows < 8) rows = 8;
    const int64_t row_blocks = (T + rows - 1) / rows;
    k_calib_absmax<<<dim3((unsigned)col_blocks, (unsigned)row_blocks), dim3(256), 0, st>>>(
        x, T, K, ldx, (int)rows, ax);
    return hipGetLastError();
}

}  // namespace sq
