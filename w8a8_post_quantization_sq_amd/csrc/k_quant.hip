// Per-token dynamic activation quantization with the smoothing division fused in.
//
// Instead of a separate runtime kernel that divides X by s ("Move activation
// scale without changing the real linear map", para. 3, on avoiding an extra
// scaling kernel), the quantizer multiplies each fp16 activation by 1/s_j on
// its way in, then quantizes the token symmetrically to int8 ([-127, 127],
// round half to even) with one float scale per token:
//   xt = float(x) * inv_s[j];  a = max_j |xt|;  scale = a / 127;
//   q  = clamp(rint(xt * (127 / a)), -127, 127)
// The two divisions are IEEE-correct float divisions (the compiler's default,
// no fast-math) and each product one correctly rounded float operation (x *
// inv_s as a mixed-precision fma with a +0 addend, x * r a multiply), and
// rint is taken by a float addition whose rounding is exactly it (quant8),
// so the codes are the ones the plain definition gives.
//
// The same kernels also serve the normalization in front of the layer with
// 1/s folded into its weight (the fold into the preceding operation that the
// same paragraph allows): x is then the hidden state h, inv_s the folded
// weight g = gamma / s, and the token's root-mean-square factor
//   rstd = 1 / sqrt(sum_j h_j^2 / K + eps)
// enters the scale only, scale = float(a * rstd / 127) in double: the codes of
// rstd * h * g are those of h * g, since a positive per-token factor scales
// the token's maximum alike.  Each lane sums the squares of its fp16 values,
// which are exact in float (11-bit significands), in double; the row's sum is
// reduced in double too, so it is within K * 2^-53 of the exact sum and the
// scale within one float rounding of the exact-sum value.
//
// With QMAX = 7 the same kernels quantize to 4 bits symmetrically ([-7, 7],
// scale = a / 7), the unrotated 4-bit quantizer of the Smooth Rotation
// comparison.
//
// The codes are written in the packed operand order of the int8 matrix
// instruction (16-row x 64-byte fragments of 1 KiB, lane order quarter-major,
// row-minor), so 16 consecutive codes of a row are one 16-byte piece and the
// pieces of 16 consecutive rows for one quarter of a 64-code window are
// contiguous.  X is read from HBM once (the second pass hits L2).
#include <type_traits>

#include "sq_device.h"

namespace sq {

// One 8-channel chunk: the raw fp16 values and their 1/s factors, loaded
// together; scale8 then forms x * inv_s and folds the magnitudes into a
// running maximum.
// Callers issue the loads of all their chunks before scaling any, so the
// loads are in flight together (a load followed at once by its use makes
// the compiler wait for each one in turn).
struct Chunk {
    uint4 raw;
    float4 s0, s1;
};

__device__ __forceinline__ Chunk load8(const uint16_t *__restrict__ x,
                                       const float *__restrict__ inv_s, int64_t c) {
    Chunk ch;
    ch.raw = *reinterpret_cast<const uint4 *>(x + c);
    ch.s0 = *reinterpret_cast<const float4 *>(inv_s + c);
    ch.s1 = *reinterpret_cast<const float4 *>(inv_s + c + 4);
    return ch;
}

// x * inv_s for the 8 values of a chunk, each as fma(float(x), inv_s, +0):
// the compiler makes it one v_fma_mix_f32, which widens the fp16 operand
// inside the instruction.  The +0 addend changes no product except the sign
// of a zero (-0 becomes +0), which neither the codes nor |x * inv_s| see.
// With NORM, also adds the chunk's squares (exact in float) to ss in double.
template <bool NORM = false>
__device__ __forceinline__ void scale8(const Chunk &ch, float v[8], AbsMax &am,
                                       double *ss = nullptr) {
    const float sv[8] = {ch.s0.x, ch.s0.y, ch.s0.z, ch.s0.w, ch.s1.x, ch.s1.y, ch.s1.z, ch.s1.w};
    const uint32_t h[4] = {ch.raw.x, ch.raw.y, ch.raw.z, ch.raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = h2f(h[i] & 0xffffu), hi = h2f(h[i] >> 16);
        if (NORM) {
            *ss += (double)__builtin_fmaf(lo, lo, 0.0f);
            *ss += (double)__builtin_fmaf(hi, hi, 0.0f);
        }
        v[2 * i] = __builtin_fmaf(lo, sv[2 * i], 0.0f);
        v[2 * i + 1] = __builtin_fmaf(hi, sv[2 * i + 1], 0.0f);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) am.add(v[i]);
}

// Codes of 8 values, clamp(rint(v * r), -QMAX, QMAX), zero codes for a row
// with zero set.  For a finite multiplier r: for |y| <= 2^22 the float sum
// y + 1.5 * 2^23 lies in [2^23, 2^24), where the floats are exactly the
// integers, so its one rounding (to nearest, ties to even) is rint(y), and
// the low byte of its bits is rint(y) mod 256, the two's-complement code.
// The clamp cannot act: r = QMAX / a is a correctly rounded quotient and
// every |v| <= a, so |v * r| <= QMAX (1 + 2^-24) and rint gives at most QMAX.
// v_perm_b32 gathers the low bytes: selector bytes 0..3 pick bytes of its
// second operand, 4..7 of its first, 0x0c a zero byte.
// OVERFLOW: the form for a row whose r overflowed (a maximum below
// QMAX / FLT_MAX): v * r is +-inf, which the clamp takes to +-QMAX, for
// v != 0, and a zero value's code is 0 (the code 0 * r has for every
// finite r).
template <int QMAX, bool OVERFLOW = false>
__device__ __forceinline__ uint2 quant8(const float v[8], float r, bool zero) {
#pragma clang fp contract(off)
    uint32_t b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (OVERFLOW) {
            b[i] = v[i] > 0.0f ? (uint32_t)QMAX : (v[i] < 0.0f ? (uint32_t)(256 - QMAX) : 0u);
        } else {
            const float y = v[i] * r;
            b[i] = __float_as_uint(y + 12582912.0f);
        }
    }
    const uint32_t lo = __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u) |
                        __builtin_amdgcn_perm(b[3], b[2], 0x04000c0cu);
    const uint32_t hi = __builtin_amdgcn_perm(b[5], b[4], 0x0c0c0400u) |
                        __builtin_amdgcn_perm(b[7], b[6], 0x04000c0cu);
    return zero ? make_uint2(0u, 0u) : make_uint2(lo, hi);
}

// A double moved between lanes by one DPP control (both halves; a lane whose
// source is outside its row of 16 reads +0).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
    const uint64_t b = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xf, 0xf, false);
    const uint32_t hi =
        (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xf, 0xf, false);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum over a 64-lane wavefront (every lane active), returned to every lane,
// in one fixed order: row shifts by 1, 2, 4 and 8 leave each row's sum in the
// row's last lane, and the four row sums are added in row order.
__device__ __forceinline__ double wave_sum_f64(double v) {
    v += dpp_f64<0x111>(v);    // row_shr:1
    v += dpp_f64<0x112>(v);    // row_shr:2
    v += dpp_f64<0x114>(v);    // row_shr:4
    v += dpp_f64<0x118>(v);    // row_shr:8
    auto lane_val = [](double x, int l) {
        const uint64_t b = __builtin_bit_cast(uint64_t, x);
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
        return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
    };
    return ((lane_val(v, 15) + lane_val(v, 31)) + lane_val(v, 47)) + lane_val(v, 63);
}

// Turns the row maximum into (scale, multiplier, all-zero-codes flag).
template <int QMAX>
__device__ __forceinline__ void row_params(uint32_t abits, float &scale, float &r, bool &zero) {
    if (abits >= 0x7f800000u) {          // a non-finite scaled value in the row
        scale = __builtin_nanf("");
        r = 0.0f;
        zero = true;
    } else if (abits == 0u) {
        scale = 0.0f;
        r = 0.0f;
        zero = true;
    } else {
        const float a = __uint_as_float(abits);
        scale = a / (float)QMAX;
        r = (float)QMAX / a;
        zero = false;
    }
}

// The normalized row's scale from its maximum and its sum of squares ss
// (non-finite and zero maxima as in row_params).
__device__ __forceinline__ float norm_scale(uint32_t abits, double ss, int64_t K, double eps) {
    if (abits >= 0x7f800000u) return __builtin_nanf("");
    if (abits == 0u) return 0.0f;
    const double rstd = 1.0 / sqrt(ss / (double)K + eps);
    return (float)((double)__uint_as_float(abits) * rstd / 127.0);
}

// Row-group kernel: a workgroup of 8 waves owns 8 consecutive token rows
// (half a packed row block).
//   pass 1: wave w streams row m0 + w once from HBM (16-byte loads) and
//           reduces max |x * inv_s| across the wave (DPP); lane 0 stores the
//           scale and keeps (multiplier, zero-row flag) in LDS;
//   pass 2: the rows are now in L2; lane p of the group makes one 16-code piece
//           (row p % 8, quarter (p / 8) % 4, window p / 32), so consecutive
//           lanes write consecutive 16-byte pieces of a fragment quarter: a
//           wave stores 8 contiguous runs of 128 bytes.
// Rows past M and chunks past K are padding and get zero codes.
constexpr int QR = 8;   // rows per workgroup

template <bool NORM, int QMAX>
__global__ void __launch_bounds__(512)
k_quant_rows(const uint16_t *__restrict__ x, int64_t M, int64_t K, int64_t ldx,
             const float *__restrict__ inv_s, double eps, int8_t *__restrict__ xq,
             float *__restrict__ x_scale) {
    __shared__ float s_r[QR];
    __shared__ int s_zero[QR];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t m0 = (int64_t)blockIdx.x * QR;
    const int64_t KW = (K + 63) >> 6;
    {
        const int64_t m = m0 + wave;
        AbsMax am;
        double ss = 0.0;
        if (m < M) {
            const uint16_t *row = x + m * ldx;
            // 4 chunks per lane in flight at a time (the loop is latency-bound otherwise)
            for (int64_t c0 = (int64_t)lane * 8; c0 < K; c0 += 4 * 512) {
                Chunk ch[4];
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (c0 + u * 512 < K) ch[u] = load8(row, inv_s, c0 + u * 512);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    float v[8];
                    if (c0 + u * 512 < K) scale8<NORM>(ch[u], v, am, &ss);
                }
            }
        }
        const uint32_t amax = wave_max_u32(am.bits());
        if (NORM) ss = wave_sum_f64(ss);
        float scale, r;
        bool zero;
        row_params<QMAX>(amax, scale, r, zero);
        if (NORM) scale = norm_scale(amax, ss, K, eps);
        if (lane == 0) {
            if (m < M) x_scale[m] = scale;
            s_r[wave] = r;
            s_zero[wave] = (m < M && !zero) ? 0 : 1;
        }
    }
    __syncthreads();
    const int64_t rb = m0 >> 4;                 // packed row block
    const int half = (int)(m0 & 15);            // 0 or 8: which half of it
    const int64_t pieces = (int64_t)QR * 4 * KW;
    int8_t *base = xq + ((rb * KW) << 10);
    // a lane's row is fixed (512 is a multiple of 8), so its multiplier is too
    const int r = threadIdx.x & 7;
    const float rr = s_r[r];
    const bool skip = s_zero[r] != 0;
    const uint16_t *row = x + (m0 + r) * ldx;
    for (int64_t p0 = threadIdx.x; p0 < pieces; p0 += 4 * 512) {
        float v[4][16];
        AbsMax dummy;
        Chunk ch[4][2];
#pragma unroll
        for (int u = 0; u < 4; ++u) {   // all loads of 4 pieces first
            const int64_t p = p0 + u * 512;
            const int64_t k = (p >> 5) * 64 + ((p >> 3) & 3) * 16;
            if (!skip && p < pieces && k < K) {
                ch[u][0] = load8(row, inv_s, k);
                ch[u][1] = load8(row, inv_s, k + 8);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t p = p0 + u * 512;
            const int64_t k = (p >> 5) * 64 + ((p >> 3) & 3) * 16;
            if (!skip && p < pieces && k < K) {
                scale8(ch[u][0], &v[u][0], dummy);
                scale8(ch[u][1], &v[u][8], dummy);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t p = p0 + u * 512;
            if (p >= pieces) break;
            const int q = (int)((p >> 3) & 3);
            const int64_t kw = p >> 5;
            const int64_t k = kw * 64 + q * 16;
            uint4 out = make_uint4(0u, 0u, 0u, 0u);
            if (!skip && k < K) {
                uint2 a, b;
                if (finite_r(rr)) {
                    a = quant8<QMAX>(&v[u][0], rr, false);
                    b = quant8<QMAX>(&v[u][8], rr, false);
                } else {
                    a = quant8<QMAX, true>(&v[u][0], rr, false);
                    b = quant8<QMAX, true>(&v[u][8], rr, false);
                }
                out = make_uint4(a.x, a.y, b.x, b.y);
            }
            // piece (window kw, quarter q, row half + r) of the packed row block
            *reinterpret_cast<uint4 *>(base + ((kw * 64 + q * 16 + half + r) << 4)) = out;
        }
    }
}

// Register-resident variant for K <= 16384: RG rows per workgroup, WPR waves
// per row (RG * WPR <= 16).  Every lane loads all its chunks of its row at
// once (the only HBM read of X), keeps x * inv_s in registers through the row
// reduction (a DPP wave reduction, then the WPR waves of a row through LDS),
// quantizes, and writes its codes into an LDS copy of the RG rows; the group
// then leaves LDS as packed 16-byte pieces, consecutive lanes on consecutive
// rows (runs of RG * 16 bytes).  Workgroups of 512 threads let two share a CU
// at up to 128 registers a lane, so one group's loads overlap another's
// reduction and stores.
template <int CPL, bool NORM, int QMAX, int RG, int WPR, bool FULL>
__global__ void __launch_bounds__(RG * WPR * 64)
k_quant_rows_reg(const uint16_t *__restrict__ x, int64_t M, int64_t K, int64_t ldx,
                 const float *__restrict__ inv_s, double eps, int8_t *__restrict__ xq,
                 float *__restrict__ x_scale) {
    static_assert(RG * WPR <= 16 && (RG == 2 || RG == 4 || RG == 8), "group shape");
    extern __shared__ __align__(16) int8_t codes[];     // [RG][KW * 64]
    __shared__ uint32_t s_max[16];
    __shared__ double s_ss[16];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = wave / WPR;                            // row of the group
    const int h = wave % WPR;                            // which of the row's chunk phases
    const int64_t m0 = (int64_t)blockIdx.x * RG;
    const int64_t m = m0 + r;
    const int64_t KW = (K + 63) >> 6;
    const int64_t pitch = KW * 64;
    const bool real = m < M;
    const uint16_t *row = x + (real ? m : 0) * ldx;
    float v[CPL][8];
    AbsMax am;
    double ss = 0.0;
    // Every load of the row first; with the sum of squares at 8 chunks per
    // lane that needs more than the 128 registers a lane has here, so there
    // the loads go in two rounds of 4.
    constexpr int ROUND = (NORM && CPL == 8) ? 4 : CPL;
#pragma unroll
    for (int c0 = 0; c0 < CPL; c0 += ROUND) {
        Chunk ch[ROUND];
#pragma unroll
        for (int c = 0; c < ROUND; ++c) {
            const int64_t k = ((int64_t)((c0 + c) * WPR + h) * 64 + lane) * 8;
            if (FULL || (real && k < K)) ch[c] = load8(row, inv_s, k);
        }
#pragma unroll
        for (int c = 0; c < ROUND; ++c) {
            const int64_t k = ((int64_t)((c0 + c) * WPR + h) * 64 + lane) * 8;
            if (FULL || (real && k < K)) scale8<NORM>(ch[c], v[c0 + c], am, &ss);
        }
    }
    const uint32_t amax = wave_max_u32(am.bits());
    if (NORM) ss = wave_sum_f64(ss);
    if (lane == 0) {
        s_max[wave] = amax;
        if (NORM) s_ss[wave] = ss;
    }
    __syncthreads();
    uint32_t arow = 0;
#pragma unroll
    for (int i = 0; i < WPR; ++i) {
        const uint32_t t = s_max[r * WPR + i];
        arow = arow > t ? arow : t;
    }
    float scale, rr;
    bool zero;
    row_params<QMAX>(arow, scale, rr, zero);
    if (!NORM && real && h == 0 && lane == 0) x_scale[m] = scale;
    zero = zero || !real;
    auto put = [&](auto overflow) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int64_t k = ((int64_t)(c * WPR + h) * 64 + lane) * 8;
            if (FULL || k < pitch)   // codes past K (padding) are zero
                *reinterpret_cast<uint2 *>(codes + r * pitch + k) =
                    (FULL || k < K) ? quant8<QMAX, decltype(overflow)::value>(v[c], rr, zero)
                                    : make_uint2(0u, 0u);
        }
    };
    if (finite_r(rr)) put(std::false_type{});
    else put(std::true_type{});
    // the normalized scale once the row's values are no longer held (the
    // row's partial sums added in wave order)
    if (NORM && real && h == 0 && lane == 0) {
        double t = 0.0;
#pragma unroll
        for (int i = 0; i < WPR; ++i) t += s_ss[r * WPR + i];
        x_scale[m] = norm_scale(arow, t, K, eps);
    }
    __syncthreads();
    const int64_t rb = m0 >> 4;
    const int first = (int)(m0 & 15);                    // the group's first row in its block
    int8_t *base = xq + ((rb * KW) << 10);
    const int64_t pieces = (int64_t)RG * 4 * KW;
    for (int64_t p = threadIdx.x; p < pieces; p += RG * WPR * 64) {
        const int pr = (int)(p % RG);
        const int q = (int)((p / RG) & 3);
        const int64_t kw = p / (RG * 4);
        // plain stores: the product reads the codes next, and finds them in
        // the caches (non-temporal stores sent them to HBM, which cost the
        // product ~2 us at 2048 x 4096)
        *reinterpret_cast<v4i *>(base + ((kw * 64 + q * 16 + first + pr) << 4)) =
            *reinterpret_cast<const v4i *>(codes + pr * pitch + kw * 64 + q * 16);
    }
}

// Decode-size batches (M <= 64): one token per workgroup of 1024 threads, one
// (K <= 8192) or two chunks of 8 channels per lane, so a token's loads all go
// out at once over 16 waves and each reduction is one DPP wave reduction plus one
// LDS round (every thread folds the 16 wave results in the same order, so the
// double sum of squares is the same everywhere).  Each lane writes its 8 codes
// straight into the packed layout (half of a 16-byte piece); rows of the last
// 16-row block past M get zero codes.
template <int CPL, bool NORM, int QMAX>
__global__ void __launch_bounds__(1024)
k_quant_row1(const uint16_t *__restrict__ x, int64_t M, int64_t K, int64_t ldx,
             const float *__restrict__ inv_s, double eps, int8_t *__restrict__ xq,
             float *__restrict__ x_scale) {
    __shared__ uint32_t s_max[16];
    __shared__ double s_ss[16];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t m = blockIdx.x;
    const bool real = m < M;
    const uint16_t *row = x + (real ? m : 0) * ldx;
    float v[CPL][8];
    AbsMax am;
    double ss = 0.0;
    Chunk ch[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int64_t k = ((int64_t)c * 1024 + threadIdx.x) * 8;
        if (real && k < K) ch[c] = load8(row, inv_s, k);
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int64_t k = ((int64_t)c * 1024 + threadIdx.x) * 8;
        if (real && k < K) scale8<NORM>(ch[c], v[c], am, &ss);
    }
    const uint32_t amax = wave_max_u32(am.bits());
    if (NORM) ss = wave_sum_f64(ss);
    if (lane == 0) {
        s_max[wave] = amax;
        if (NORM) s_ss[wave] = ss;
    }
    __syncthreads();
    uint32_t a = 0;
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
        a = a > s_max[w] ? a : s_max[w];
        if (NORM) t += s_ss[w];
    }
    float scale, r;
    bool zero;
    row_params<QMAX>(a, scale, r, zero);
    if (NORM) scale = norm_scale(a, t, K, eps);
    if (real && threadIdx.x == 0) x_scale[m] = scale;
    zero = zero || !real;
    const int64_t KW = (K + 63) >> 6;
    int8_t *base = xq + (((m >> 4) * KW) << 10) + (m & 15) * 16;
    auto put = [&](auto overflow) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int64_t k = ((int64_t)c * 1024 + threadIdx.x) * 8;
            if (k < KW * 64) {   // codes past K (padding) are zero
                const uint2 q = (k < K) ? quant8<QMAX, decltype(overflow)::value>(v[c], r, zero)
                                        : make_uint2(0u, 0u);
                *reinterpret_cast<uint2 *>(base + ((k >> 6) << 10) + (((k >> 4) & 3) << 8) +
                                           (k & 15)) = q;
            }
        }
    };
    if (finite_r(r)) put(std::false_type{});
    else put(std::true_type{});
}

template <bool NORM, int QMAX>
hipError_t launch_rows(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, const float *inv_s,
                       double eps, int8_t *xq, float *x_scale, hipStream_t st) {
    if (M <= 0) return hipSuccess;
    if (M <= 64 && K <= 16384) {   // decode sizes: one token per workgroup
        const dim3 g((unsigned)((M + 15) / 16 * 16));
        if (K <= 8192)
            k_quant_row1<1, NORM, QMAX><<<g, dim3(1024), 0, st>>>(x, M, K, ldx, inv_s, eps, xq, x_scale);
        else
            k_quant_row1<2, NORM, QMAX><<<g, dim3(1024), 0, st>>>(x, M, K, ldx, inv_s, eps, xq, x_scale);
        return hipGetLastError();
    }
    // every row of the padded row blocks: 4 rows per workgroup, or 2 where
    // that leaves too few workgroups for the CUs; 2 waves per row up to 8192
    // channels; up to 12288, 3 waves of 8 chunks (a quarter fewer idle lanes
    // than 4 waves at K = 11008), or on small batches 8 waves of 3 chunks;
    // 4 waves up to 16384
    const int64_t blocks = (M + 15) / 16;
    const int64_t KW = (K + 63) / 64;
    // FULL: the lanes' chunks cover K exactly (no chunk past the row's end)
#define SQ_QR(C, RG, WPR)                                                                        \
    do {                                                                                         \
        const dim3 g_((unsigned)(blocks * (16 / RG))), b_(RG * WPR * 64);                         \
        const size_t lds_ = (size_t)RG * KW * 64;                                                \
        if (K == (int64_t)(C) * (WPR) * 512)                                                     \
            k_quant_rows_reg<C, NORM, QMAX, RG, WPR, true><<<g_, b_, lds_, st>>>(                 \
                x, M, K, ldx, inv_s, eps, xq, x_scale);                                          \
        else                                                                                     \
            k_quant_rows_reg<C, NORM, QMAX, RG, WPR, false><<<g_, b_, lds_, st>>>(                \
                x, M, K, ldx, inv_s, eps, xq, x_scale);                                          \
    } while (0)
    if (K <= 8192) {
        const int64_t cpl = (K + 1023) / 1024;    // chunks of 8 per lane
        if (M > 512) {
            if (cpl <= 1) SQ_QR(1, 4, 2);
            else if (cpl <= 2) SQ_QR(2, 4, 2);
            else if (cpl <= 4) SQ_QR(4, 4, 2);
            else SQ_QR(8, 4, 2);
        } else {
            if (cpl <= 1) SQ_QR(1, 2, 2);
            else if (cpl <= 2) SQ_QR(2, 2, 2);
            else if (cpl <= 4) SQ_QR(4, 2, 2);
            else SQ_QR(8, 2, 2);
        }
    } else if (K <= 12288) {
        if (M > 512) SQ_QR(8, 4, 3);
        else SQ_QR(3, 2, 8);
    } else if (K <= 16384) {
        if (M > 512) SQ_QR(8, 4, 4);
        else SQ_QR(8, 2, 4);
    } else {
        k_quant_rows<NORM, QMAX><<<dim3((unsigned)(blocks * 2)), dim3(512), 0, st>>>(
            x, M, K, ldx, inv_s, eps, xq, x_scale);
    }
#undef SQ_QR
    return hipGetLastError();
}

hipError_t launch_quant_act(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                            const float *inv_s, int8_t *xq, float *x_scale, hipStream_t st) {
    return launch_rows<false, 127>(x, M, K, ldx, inv_s, 0.0, xq, x_scale, st);
}

hipError_t launch_rmsnorm_quant(const uint16_t *h, int64_t M, int64_t K, int64_t ldh,
                                const float *g, float eps, int8_t *xq, float *x_scale,
                                hipStream_t st) {
    return launch_rows<true, 127>(h, M, K, ldh, g, (double)eps, xq, x_scale, st);
}

hipError_t launch_quant4_plain(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                               const float *mult, int8_t *q, float *scale, hipStream_t st) {
    return launch_rows<false, 7>(x, M, K, ldx, mult, 0.0, q, scale, st);
}

// g[j] = float(gamma[j]) * inv_s[j], 8 channels per thread (K % 16 == 0).
__global__ void __launch_bounds__(256)
k_fold_norm_weight(const uint16_t *__restrict__ gamma, int64_t K, const float *__restrict__ inv_s,
                   float *__restrict__ g) {
    const int64_t c = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (c >= K) return;
    const uint4 raw = *reinterpret_cast<const uint4 *>(gamma + c);
    const float4 s0 = *reinterpret_cast<const float4 *>(inv_s + c);
    const float4 s1 = *reinterpret_cast<const float4 *>(inv_s + c + 4);
    float4 o0, o1;
    o0.x = h2f(raw.x & 0xffffu) * s0.x;
    o0.y = h2f(raw.x >> 16) * s0.y;
    o0.z = h2f(raw.y & 0xffffu) * s0.z;
    o0.w = h2f(raw.y >> 16) * s0.w;
    o1.x = h2f(raw.z & 0xffffu) * s1.x;
    o1.y = h2f(raw.z >> 16) * s1.y;
    o1.z = h2f(raw.w & 0xffffu) * s1.z;
    o1.w = h2f(raw.w >> 16) * s1.w;
    *reinterpret_cast<float4 *>(g + c) = o0;
    *reinterpret_cast<float4 *>(g + c + 4) = o1;
}

hipError_t launch_fold_norm_weight(const uint16_t *gamma, int64_t K, const float *inv_s, float *g,
                                   hipStream_t st) {
    const int64_t threads = K / 8;
    k_fold_norm_weight<<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st>>>(gamma, K,
                                                                                      inv_s, g);
    return hipGetLastError();
}

}  // namespace sq
