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
//   k_row_smooth      aw_j = max_n |W[j][n]| (four rows per wave), then s_j and
//                     1/s_j in float, s also into a host buffer (the host checks
//                     s and 1/s while the rest runs); zeroes the amax scratch
//   k_fold_colabsmax  amax_n = max_j |float(W[j][n]) * s_j|  (atomics)
//   k_fold_quant      Wq[n][j] = clamp(rint((W*s) * (127/amax_n)), +-127), transposed
//                     through LDS and written as packed 16 x 64-byte fragments
//                     (the operand order of the int8 matrix instruction), with
//                     the padding rows and windows written as zero; and
//                     w_scale[n] = amax_n / 127
#include <math.h>

#include <mutex>
#include <vector>

#include "sq.h"
#include "sq_device.h"

namespace sq {

// ---- aw_j = max_n |W[j][n]|, then s_j and 1/s_j ---------------------------------------

// One single-wave workgroup per RS_ROWS rows; for each row a lane keeps RS_U
// 16-byte loads (of 8 columns each, 512 columns apart) in flight, RS_ROWS x
// RS_U in all, before reducing them.  Maxima are taken on the fp16 magnitude
// bits, which order like the magnitudes and put NaN above +inf.  Lanes
// 0..RS_ROWS-1 then form the factors of the wave's rows side by side: a
// statistic that is NaN, infinite or negative (or such a given factor) yields
// s = NaN; range problems (s or 1/s zero, infinite, subnormal) are left as
// they come.  The host checks both, on the copy of s the kernel writes into a
// host buffer.  The workgroups also clear the column maxima's accumulator.
constexpr int RS_ROWS = 4;
constexpr int RS_U = 4;

// a^alpha / aw^(1 - alpha) in double, a and aw positive finite.  The general
// power is long code that each wave runs once at its very end (measured: ~3.5
// us added to the kernel), so the exponents with a short exact form take it:
// alpha = 1/2 gives sqrt(a) / sqrt(aw) (the square-root form of the factor),
// alpha = 1 gives a / 1 and alpha = 0 gives 1 / aw (x^0 = 1 and x^1 = x are
// exact in pow).  The square roots and the power agree to about the last bit
// of a double, which the rounding to float absorbs.
__device__ __forceinline__ double pow_ratio(float a, float aw, double alpha) {
    if (alpha == 0.5) return sqrt((double)a) / sqrt((double)aw);
    if (alpha == 1.0) return (double)a;
    if (alpha == 0.0) return 1.0 / (double)aw;
    return pow((double)a, alpha) / pow((double)aw, 1.0 - alpha);
}

__global__ void __launch_bounds__(64)
k_row_smooth(const uint16_t *__restrict__ w, int64_t K, int64_t N, int64_t ldw,
             const float *__restrict__ ax, const float *__restrict__ smooth_in, double alpha,
             float *__restrict__ s_out, float *__restrict__ inv_out, float *__restrict__ s_host,
             float *__restrict__ amax, uint32_t *__restrict__ status) {
    if (amax)   // (the factors alone need no column maxima)
        for (int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x; i < N; i += (int64_t)gridDim.x * 64)
            amax[i] = 0.0f;
    const int lane = threadIdx.x;
    const int64_t j0 = (int64_t)blockIdx.x * RS_ROWS;
    const int64_t nfull = N & ~(int64_t)7;          // columns in whole octets
    uint32_t m[RS_ROWS];
#pragma unroll
    for (int r = 0; r < RS_ROWS; ++r) m[r] = 0;
    for (int64_t base = (int64_t)lane * 8; base < nfull; base += RS_U * 512) {
        uint4 v[RS_ROWS][RS_U];
#pragma unroll
        for (int r = 0; r < RS_ROWS; ++r) {
#pragma unroll
            for (int u = 0; u < RS_U; ++u) {
                const int64_t c = base + (int64_t)u * 512;
                v[r][u] = (j0 + r < K && c < nfull)
                              ? *reinterpret_cast<const uint4 *>(w + (j0 + r) * ldw + c)
                              : make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int r = 0; r < RS_ROWS; ++r) {
#pragma unroll
            for (int u = 0; u < RS_U; ++u) {
                const uint32_t q[4] = {v[r][u].x, v[r][u].y, v[r][u].z, v[r][u].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t lo = q[i] & 0x7fffu, hi = (q[i] >> 16) & 0x7fffu;
                    m[r] = m[r] > lo ? m[r] : lo;
                    m[r] = m[r] > hi ? m[r] : hi;
                }
            }
        }
    }
    // the last < 8 columns of each row: lane r takes row r
    if (lane < RS_ROWS && j0 + lane < K) {
        for (int64_t e = nfull; e < N; ++e) {
#pragma unroll
            for (int r = 0; r < RS_ROWS; ++r) {
                if (r == lane) {
                    const uint32_t b = w[(j0 + r) * ldw + e] & 0x7fffu;
                    m[r] = m[r] > b ? m[r] : b;
                }
            }
        }
    }
    uint32_t mine = 0;   // lane r ends with row r's maximum
#pragma unroll
    for (int r = 0; r < RS_ROWS; ++r) {
        const uint32_t t = wave_max_u32(m[r]);
        if (lane == r) mine = t;
    }
    const int64_t j = j0 + lane;
    if (lane >= RS_ROWS || j >= K) return;
    const float aw = h2f(mine);   // NaN bits stay NaN, 0x7c00 becomes +inf
    float s;
    if (!isfinite(aw)) {
        s = __builtin_nanf("");
    } else if (smooth_in) {
        const float v = smooth_in[j];
        s = (isfinite(v) && v >= 0.0f) ? v : __builtin_nanf("");
    } else {
        const float a = ax[j];
        if (!isfinite(a) || a < 0.0f)
            s = __builtin_nanf("");
        else if (a == 0.0f || aw == 0.0f)
            s = 1.0f;   // dead channel or zero row: the plainest positive factor
        else
            s = (float)(pow_ratio(a, aw, alpha));
    }
    const float inv = 1.0f / s;   // IEEE-correct float division
    s_out[j] = s;
    inv_out[j] = inv;
    if (s_host) s_host[j] = s;   // for the host's check, without a copy kernel
    if (status) {
        // the same check on the device: bit 0 a NaN factor (a bad statistic
        // or given factor), bit 1 a factor or reciprocal that is zero,
        // infinite, subnormal or negative
        const uint32_t bad = __builtin_isnan(s) ? 1u
                             : (!__builtin_isnormal(s) || !__builtin_isnormal(inv) || s < 0.0f) ? 2u
                                                                                                : 0u;
        if (bad) atomicOr(status, bad);
    }
}

hipError_t launch_row_smooth(const uint16_t *w, int64_t K, int64_t N, int64_t ldw,
                             const float *ax, const float *smooth_in, float alpha, float *s_out,
                             float *inv_out, float *s_host, float *amax, uint32_t *status,
                             hipStream_t st) {
    k_row_smooth<<<dim3((unsigned)((K + RS_ROWS - 1) / RS_ROWS)), dim3(64), 0, st>>>(
        w, K, N, ldw, ax, smooth_in, (double)alpha, s_out, inv_out, s_host, amax, status);
    return hipGetLastError();
}

// ---- amax_n = max_j |float(W[j][n]) * s_j| ---------------------------------------

// A workgroup covers 128 columns (16 lanes x 8, a 256-byte row segment) over a
// slice of rows; a wave load spans 4 rows, and each lane keeps CA_U loads
// (16 rows apart) in flight before reducing them.  The 16 row phases combine
// through shuffles and LDS, then one atomicMax per column on the (non-negative)
// float bits.  With factors that the host will reject, the values are
// meaningless but every access stays in bounds.
constexpr int CA_COLS = 128;
constexpr int CA_U = 8;
constexpr int CA_ROUND = 16 * CA_U;   // rows per workgroup round

__global__ void __launch_bounds__(256)
k_fold_colabsmax(const uint16_t *__restrict__ w, int64_t K, int64_t N, int64_t ldw,
                 const float *__restrict__ s, int64_t rows_per_block, float *__restrict__ amax) {
    __shared__ float red[4][CA_COLS];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t c0 = (int64_t)blockIdx.x * CA_COLS + (lane & 15) * 8;
    const int sub = wave * 4 + (lane >> 4);          // row phase 0..15
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
    const int64_t r1 = r0 + rows_per_block < K ? r0 + rows_per_block : K;
    const bool full = c0 + 8 <= N;
    const int tail = full ? 0 : (c0 < N ? (int)(N - c0) : 0);   // columns of a partial octet
    float m[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) m[i] = 0.0f;
    for (int64_t rb = r0 + sub; rb < r1; rb += CA_ROUND) {
        uint4 v[CA_U];
        float sj[CA_U];
#pragma unroll
        for (int u = 0; u < CA_U; ++u) {
            const int64_t r = rb + 16 * u;
            const bool ok = r < r1;
            v[u] = (ok && full) ? *reinterpret_cast<const uint4 *>(w + r * ldw + c0)
                                : make_uint4(0, 0, 0, 0);
            sj[u] = ok ? s[r] : 0.0f;
        }
        if (tail) {   // the octet that N cuts: element loads, zeros past N
#pragma unroll
            for (int u = 0; u < CA_U; ++u) {
                const int64_t r = rb + 16 * u;
                uint32_t h[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                if (r < r1)
                    for (int i = 0; i < tail; ++i) h[i] = w[r * ldw + c0 + i];
                v[u] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                                  h[6] | (h[7] << 16));
            }
        }
#pragma unroll
        for (int u = 0; u < CA_U; ++u) {
            const uint32_t q[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                m[2 * i] = fmaxf(m[2 * i], fabsf(h2f(q[i] & 0xffffu) * sj[u]));
                m[2 * i + 1] = fmaxf(m[2 * i + 1], fabsf(h2f(q[i] >> 16) * sj[u]));
            }
        }
    }
    // lanes l, l+16, l+32, l+48 hold the same columns
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        m[i] = fmaxf(m[i], __shfl_xor(m[i], 16, 64));
        m[i] = fmaxf(m[i], __shfl_xor(m[i], 32, 64));
    }
    if (lane < 16) {
#pragma unroll
        for (int i = 0; i < 8; ++i) red[wave][lane * 8 + i] = m[i];
    }
    __syncthreads();
    if (threadIdx.x < CA_COLS) {
        const int c = threadIdx.x;
        const float b = fmaxf(fmaxf(red[0][c], red[1][c]), fmaxf(red[2][c], red[3][c]));
        const int64_t col = (int64_t)blockIdx.x * CA_COLS + c;
        if (col < N && r1 > r0)
            atomicMax(reinterpret_cast<unsigned int *>(amax + col), __float_as_uint(b));
    }
}

hipError_t launch_fold_colabsmax(const uint16_t *w, int64_t K, int64_t N, int64_t ldw,
                                 const float *s, float *amax, hipStream_t st) {
    const int64_t col_blocks = (N + CA_COLS - 1) / CA_COLS;
    // about 512 workgroups: slices of whole rounds
    const int64_t rounds = (K + CA_ROUND - 1) / CA_ROUND;
    int64_t want = 512 / col_blocks;
    if (want < 1) want = 1;
    const int64_t rows = CA_ROUND * ((rounds + want - 1) / want);
    const int64_t row_blocks = (K + rows - 1) / rows;
    k_fold_colabsmax<<<dim3((unsigned)col_blocks, (unsigned)row_blocks), dim3(256), 0, st>>>(
        w, K, N, ldw, s, rows, amax);
    return hipGetLastError();
}

// ---- quantize and transpose ---------------------------------------------------------

// Tile: 64 output channels x 256 input channels.  A work item is 4 consecutive
// rows j x 8 consecutive columns n (four 16-byte loads); each of its 8 columns
// yields 4 consecutive codes of one Wq row, packed into a 32-bit LDS store.
// Each thread issues the loads of both its items before it converts any.  The
// quotients 127 / amax_n are formed once per column and passed by shuffles.
// The tile then leaves as 4 x 4 packed fragments of 1 KiB (16 channels x 64
// input channels each), one 16-byte store per lane.  Out-of-range channels and
// input channels hold zero codes, so the padding of the packed buffer is zero.
//
// LDS holds the tile as 64 rows (channels) of 16 chunks of 16 bytes (4 input
// channels per word).  The chunk index is XOR-swizzled with bits of the row,
// so the 32-bit stores (8 rows x 8 words per wave) and the 16-byte reads (16
// rows of one chunk column per 16 lanes) both spread over the banks.
constexpr int FQ_TN = 64;
constexpr int FQ_TK = 256;

__device__ __forceinline__ int fq_word(int row, int word) {   // word: 4-byte column 0..63
    const int swz = (((row ^ (row >> 3)) & 7) << 1) | ((row >> 3) & 1);
    return row * (FQ_TK / 4) + ((((word >> 2) ^ swz) << 2) | (word & 3));
}

__global__ void __launch_bounds__(256)
k_fold_quant(const uint16_t *__restrict__ w, int64_t K, int64_t N, int64_t ldw,
             const float *__restrict__ s, const float *__restrict__ amax,
             int8_t *__restrict__ wq, float *__restrict__ w_scale) {
    __shared__ __align__(16) uint32_t tile[FQ_TN * FQ_TK / 4];
    const int64_t n0 = (int64_t)blockIdx.x * FQ_TN;
    const int64_t k0 = (int64_t)blockIdx.y * FQ_TK;
    // 64 row-quads x 8 column-octets = 512 work items, 2 per thread; both
    // items of a thread share its column octet (threadIdx.x % 8)
    const int lane = threadIdx.x & 63;
    const int oct = threadIdx.x & 7;       // column octet within the tile
    const int64_t n = n0 + oct * 8;
    const bool full = n + 8 <= N;
    uint4 raw[2][4];
    float sj[2][4];
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int64_t j = k0 + ((threadIdx.x + it * 256) >> 3) * 4;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const bool ok = j + q < K;
            raw[it][q] = (ok && full) ? *reinterpret_cast<const uint4 *>(w + (j + q) * ldw + n)
                                      : make_uint4(0, 0, 0, 0);
            sj[it][q] = ok ? s[j + q] : 0.0f;
        }
    }
    // 127 / amax: lane l divides for tile column l, and each lane picks up
    // the 8 quotients of its octet from the lanes that made them
    const float al = n0 + lane < N ? amax[n0 + lane] : 0.0f;
    const float rl = al > 0.0f ? 127.0f / al : 0.0f;
    // the first tile row of each column block also writes the scales
    if (blockIdx.y == 0 && threadIdx.x < 64 && n0 + lane < N) w_scale[n0 + lane] = al / 127.0f;
    float r[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) r[c] = __shfl(rl, oct * 8 + c, 64);
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int quad = (threadIdx.x + it * 256) >> 3;   // row quad within the tile
        const int64_t j = k0 + quad * 4;
        if (n < N && n + 8 > N) {   // the octet that N cuts: element loads, zeros past N
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t h[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                if (j + q < K)
                    for (int i = 0; n + i < N; ++i) h[i] = w[(j + q) * ldw + n + i];
                raw[it][q] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16),
                                        h[4] | (h[5] << 16), h[6] | (h[7] << 16));
            }
        }
        uint32_t packed[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) packed[c] = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t hq[4] = {raw[it][q].x, raw[it][q].y, raw[it][q].z, raw[it][q].w};
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const float v = h2f(c & 1 ? hq[c >> 1] >> 16 : hq[c >> 1] & 0xffffu);
                const float wt = v * sj[it][q];             // W~ = W * s_j (float)
                float qf = __builtin_rintf(wt * r[c]);      // round half to even
                qf = fminf(fmaxf(qf, -127.0f), 127.0f);
                // a zero value's code is 0, also where 127 / amax overflowed
                // (a column maximum below 127 / FLT_MAX makes wt * r NaN there)
                const uint32_t b = wt == 0.0f ? 0u : ((uint32_t)(int)qf & 0xffu);
                packed[c] |= b << (8 * q);
            }
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) tile[fq_word(oct * 8 + c, quad)] = packed[c];
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
        const int word = kwl * 16 + (l >> 4) * 4;     // first of 4 words (16 codes)
        // plain stores: where the product follows the fold, it finds the
        // codes in the caches
        if (rb < RB && kw < KW)
            *reinterpret_cast<v4i *>(wq + ((rb * KW + kw) << 10) + l * 16) =
                *reinterpret_cast<const v4i *>(tile + fq_word(rn, word));
    }
}

hipError_t launch_fold_quant(const uint16_t *w, int64_t K, int64_t N, int64_t ldw, const float *s,
                             const float *amax, int8_t *wq, float *w_scale, hipStream_t st) {
    const dim3 grid((unsigned)((N + FQ_TN - 1) / FQ_TN), (unsigned)((K + FQ_TK - 1) / FQ_TK));
    k_fold_quant<<<grid, dim3(256), 0, st>>>(w, K, N, ldw, s, amax, wq, w_scale);
    return hipGetLastError();
}

// ---- the fold's scratch for callers that cannot allocate ------------------------------
//
// sq_smooth_fold_weights_noalloc takes its column maxima (N floats) and its
// status word from this file-scope device array instead of the per-(thread,
// device) buffers the allocating fold makes.  Each GPU holds its own copy
// from the library's load until the process ends.  In host code `scratch` is
// only a stand-in for the symbol: its device address on a device comes from
// hipGetSymbolAddress with that device current, once per device, and only
// that address is ever passed to kernels or copies.
constexpr int64_t NOALLOC_WORDS = (int64_t)SQ_NOALLOC_MAX_N + 64;   // maxima, then the status
static __device__ __align__(256) uint32_t scratch[NOALLOC_WORDS];

hipError_t noalloc_scratch(int dev, float **amax, uint32_t **status) {
    static std::mutex mu;
    static std::vector<void *> addr;     // per device, found once
    std::lock_guard<std::mutex> lock(mu);
    if (dev < 0) return hipErrorInvalidDevice;
    if ((int)addr.size() <= dev) addr.resize((size_t)dev + 1, nullptr);
    if (!addr[(size_t)dev]) {
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[(size_t)dev] = p;
    }
    *amax = static_cast<float *>(addr[(size_t)dev]);
    *status = static_cast<uint32_t *>(addr[(size_t)dev]) + SQ_NOALLOC_MAX_N;
    return hipSuccess;
}

}  // namespace sq
