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
// no fast-math), the products single float multiplies, so the codes are the
// ones the plain definition gives.
//
// One 256-thread workgroup per token row.  Each lane owns CPT chunks of 8
// channels (a 16-byte fp16 load, two 16-byte loads of inv_s, an 8-byte int8
// store); the scaled row stays in registers between the absmax reduction
// (wave shuffles, then 4 waves through LDS) and the quantization, so X is read
// from HBM exactly once.  Rows longer than 256 * 8 * 16 channels take a
// streaming variant that reads the row twice.
//
// The codes are written in the packed operand order of the int8 matrix
// instruction (16-row x 64-byte fragments of 1 KiB): 8 consecutive codes of a
// row are 8 contiguous bytes there.  The grid covers the padded rows and
// windows too, writing their codes as zero.
#include "sq_device.h"

namespace sq {

__device__ __forceinline__ void load8(const uint16_t *__restrict__ x, const float *__restrict__ inv_s,
                                      int64_t c, float v[8], uint32_t &amax) {
    const uint4 raw = *reinterpret_cast<const uint4 *>(x + c);
    const float4 s0 = *reinterpret_cast<const float4 *>(inv_s + c);
    const float4 s1 = *reinterpret_cast<const float4 *>(inv_s + c + 4);
    const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    const uint32_t h[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = h2f(h[i] & 0xffffu) * sv[2 * i];
        v[2 * i + 1] = h2f(h[i] >> 16) * sv[2 * i + 1];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        // magnitude bits order like magnitudes; NaN sits above +inf
        const uint32_t b = __float_as_uint(v[i]) & 0x7fffffffu;
        amax = amax > b ? amax : b;
    }
}

// Byte offset of codes (m, k .. k + 7), k % 8 == 0, in the packed layout.
__device__ __forceinline__ int64_t packed_off(int64_t m, int64_t k, int64_t KW) {
    return (((m >> 4) * KW + (k >> 6)) << 10) + (((k >> 4) & 3) << 8) + ((m & 15) << 4) + (k & 15);
}

__device__ __forceinline__ uint2 quant8(const float v[8], float r, bool zero) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float q = __builtin_rintf(v[i] * r);
        q = fminf(fmaxf(q, -127.0f), 127.0f);
        const uint32_t b = zero ? 0u : ((uint32_t)(int)q & 0xffu);
        if (i < 4) lo |= b << (8 * i);
        else hi |= b << (8 * (i - 4));
    }
    return make_uint2(lo, hi);
}

// Reduces the per-lane magnitude maxima of one row to the whole workgroup.
__device__ __forceinline__ uint32_t block_max_256(uint32_t v) {
    __shared__ uint32_t part[4];
    v = wave_max_u32(v);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
    __syncthreads();
    uint32_t a = part[0];
    a = a > part[1] ? a : part[1];
    a = a > part[2] ? a : part[2];
    a = a > part[3] ? a : part[3];
    return a;
}

// Turns the row maximum into (scale, multiplier, all-zero-codes flag).
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
        scale = a / 127.0f;
        r = 127.0f / a;
        zero = false;
    }
}

// Block m < M quantizes token m; blocks M .. 16 * ceil(M / 16) - 1 write the
// zero codes of the padding rows.  Chunks at k >= K are padding too.
template <int CPT>
__global__ void __launch_bounds__(256)
k_quant_act(const uint16_t *__restrict__ x, int64_t M, int64_t K, int64_t ldx,
            const float *__restrict__ inv_s, int8_t *__restrict__ xq,
            float *__restrict__ x_scale) {
    const int64_t m = blockIdx.x;
    const int64_t nch = K >> 3;
    const int64_t KW = (K + 63) >> 6;
    const int64_t nch_pad = KW << 3;
    const bool real = m < M;
    const uint16_t *row = x + (real ? m : 0) * ldx;
    float v[CPT][8];
    uint32_t amax = 0;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const int64_t ch = threadIdx.x + c * 256;
        if (real && ch < nch) load8(row, inv_s, ch * 8, v[c], amax);
    }
    float scale, r;
    bool zero;
    row_params(block_max_256(amax), scale, r, zero);
    if (real && threadIdx.x == 0) x_scale[m] = scale;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const int64_t ch = threadIdx.x + c * 256;
        if (ch < nch_pad)
            *reinterpret_cast<uint2 *>(xq + packed_off(m, ch * 8, KW)) =
                (real && ch < nch) ? quant8(v[c], r, zero) : make_uint2(0u, 0u);
    }
}

// Long rows: first pass for the maximum, second pass (from cache) for the codes.
__global__ void __launch_bounds__(256)
k_quant_act_stream(const uint16_t *__restrict__ x, int64_t M, int64_t K, int64_t ldx,
                   const float *__restrict__ inv_s, int8_t *__restrict__ xq,
                   float *__restrict__ x_scale) {
    const int64_t m = blockIdx.x;
    const int64_t nch = K >> 3;
    const int64_t KW = (K + 63) >> 6;
    const int64_t nch_pad = KW << 3;
    const bool real = m < M;
    const uint16_t *row = x + (real ? m : 0) * ldx;
    uint32_t amax = 0;
    float v[8];
    if (real)
        for (int64_t ch = threadIdx.x; ch < nch; ch += 256) load8(row, inv_s, ch * 8, v, amax);
    float scale, r;
    bool zero;
    row_params(block_max_256(amax), scale, r, zero);
    if (real && threadIdx.x == 0) x_scale[m] = scale;
    for (int64_t ch = threadIdx.x; ch < nch_pad; ch += 256) {
        uint2 q = make_uint2(0u, 0u);
        if (real && ch < nch) {
            uint32_t dummy = 0;
            load8(row, inv_s, ch * 8, v, dummy);
            q = quant8(v, r, zero);
        }
        *reinterpret_cast<uint2 *>(xq + packed_off(m, ch * 8, KW)) = q;
    }
}

hipError_t launch_quant_act(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                            const float *inv_s, int8_t *xq, float *x_scale, hipStream_t st) {
    if (M <= 0) return hipSuccess;
    const int64_t nch_pad = ((K + 63) / 64) * 8;
    const int64_t cpt = (nch_pad + 255) / 256;
    const dim3 grid((unsigned)((M + 15) / 16 * 16)), block(256);
#define SQ_Q(C) k_quant_act<C><<<grid, block, 0, st>>>(x, M, K, ldx, inv_s, xq, x_scale)
    if (cpt <= 1) SQ_Q(1);
    else if (cpt <= 2) SQ_Q(2);
    else if (cpt <= 3) SQ_Q(3);
    else if (cpt <= 4) SQ_Q(4);
    else if (cpt <= 6) SQ_Q(6);
    else if (cpt <= 8) SQ_Q(8);
    else if (cpt <= 12) SQ_Q(12);
    else if (cpt <= 16) SQ_Q(16);
    else k_quant_act_stream<<<grid, block, 0, st>>>(x, M, K, ldx, inv_s, xq, x_scale);
#undef SQ_Q
    return hipGetLastError();
}

}  // namespace sq
