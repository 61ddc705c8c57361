// 4-bit symmetric quantization of rows, optionally after the Hadamard rotation
// of Smooth Rotation (Pith review of arXiv 2506.01967, key machinery: scale the
// channels, then multiply activations and weights by the same Hadamard matrix;
// core discovery: 4-bit symmetric round-to-nearest on both).
//
// Per row of M rows (fp16 x, row stride ldx) with a per-channel float factor
// `mult` (1/s for activations, s for the rows of W transposed); the rotation
// off, the 7-level form of the 8-bit per-token quantizer does the same without
// the transform:
//   v[j]     = float(x[j]) * mult[j]
//   v        = v H           (rotation on: the unnormalized Sylvester matrix,
//                             H[i][j] = (-1)^popcount(i & j), K a power of two)
//   a        = max_j |v[j]|,  q[j] = clamp(rint(v[j] * (7 / a)), -7, 7)
//   scale    = (a / 7) * post (post a power of two, so the product is exact)
// The two factors 1/sqrt(K) of the orthonormal rotation multiply to 1/K, which
// the weight side passes as `post`.  A zero row gets scale 0, a row with a
// non-finite value scale NaN, both with zero codes.
//
// The transform is the fast one, with its stages in the order h = 1, 2, 4, ...,
// K/2 and every butterfly (a + b, a - b) in float, a being the element at the
// lower index.  Up to K = 2048 (k_quant4_rows) each stage only changes where
// the two operands live:
//   element k = (u * 64 + lane) * 8 + e  of a row held by one wave, so
//   h = 1, 2, 4    (bits 0-2: e)     pair within a lane's 8-element chunk,
//   h = 8 .. 256   (bits 3-8: lane)  pair across lanes (a shuffle),
//   h = 512 ..     (bits 9+:  u)     pair across a lane's chunks.
// So every value is the same float that the plain in-order transform gives.
//
// Codes leave as int8 in the packed operand order of the int8 matrix
// instruction (the 4-bit values widened to bytes), through an LDS copy of the
// workgroup's 8 rows, as the 8-bit quantizer writes them.
#include "sq_device.h"

namespace sq {

constexpr int R4 = 8;   // rows per workgroup, one wave each

template <int U>
__global__ void __launch_bounds__(512)
k_quant4_rows(const uint16_t *__restrict__ x, int64_t M, int64_t K, int64_t ldx,
              const float *__restrict__ mult, float post, int8_t *__restrict__ q,
              float *__restrict__ scale) {
    extern __shared__ __align__(16) int8_t codes[];     // [8][KW * 64]
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;                   // the row of the group
    const int64_t m0 = (int64_t)blockIdx.x * R4;
    const int64_t m = m0 + wave;
    const int64_t KW = (K + 63) >> 6;
    const int64_t pitch = KW * 64;
    const bool real = m < M;
    const uint16_t *row = x + (real ? m : 0) * ldx;

    float v[U][8];
    // loads in rounds of 4 chunks (16 bytes of x and 32 of factors each)
#pragma unroll
    for (int u0 = 0; u0 < U; u0 += 4) {
        uint4 raw[4];
        float4 f0[4], f1[4];
#pragma unroll
        for (int i = 0; i < 4 && u0 + i < U; ++i) {
            const int64_t k = ((int64_t)(u0 + i) * 64 + lane) * 8;
            if (real && k < K) {
                raw[i] = *reinterpret_cast<const uint4 *>(row + k);
                f0[i] = *reinterpret_cast<const float4 *>(mult + k);
                f1[i] = *reinterpret_cast<const float4 *>(mult + k + 4);
            } else {
                raw[i] = make_uint4(0u, 0u, 0u, 0u);
                f0[i] = f1[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
#pragma unroll
        for (int i = 0; i < 4 && u0 + i < U; ++i) {
            const uint32_t h[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
            const float f[8] = {f0[i].x, f0[i].y, f0[i].z, f0[i].w,
                                f1[i].x, f1[i].y, f1[i].z, f1[i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[u0 + i][2 * e] = h2f(h[e] & 0xffffu) * f[2 * e];
                v[u0 + i][2 * e + 1] = h2f(h[e] >> 16) * f[2 * e + 1];
            }
        }
    }

    {
        // h = 1, 2, 4: inside each chunk
#pragma unroll
        for (int hb = 1; hb < 8; hb <<= 1) {
            if (hb >= K) break;
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if ((e & hb) == 0) {
                        const float a = v[u][e], b = v[u][e + hb];
                        v[u][e] = a + b;
                        v[u][e + hb] = a - b;
                    }
        }
        // h = 8 .. 256: lane bit t pairs lane l with l ^ (1 << t); the lower
        // lane keeps a + b, the upper one a - b
#pragma unroll
        for (int t = 0; t < 6; ++t) {
            if ((8 << t) >= K) break;
            const bool upper = (lane >> t) & 1;
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float p = __shfl_xor(v[u][e], 1 << t, 64);
                    v[u][e] = upper ? p - v[u][e] : v[u][e] + p;
                }
        }
        // h = 512 ..: between chunks u and u + 2^t (U = K / 512 here)
#pragma unroll
        for (int hu = 1; hu < U; hu <<= 1)
#pragma unroll
            for (int u = 0; u < U; ++u)
                if ((u & hu) == 0)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float a = v[u][e], b = v[u + hu][e];
                        v[u][e] = a + b;
                        v[u + hu][e] = a - b;
                    }
    }

    // row maximum on the magnitude bits (NaN above +inf); elements past K are 0
    uint32_t amax = 0;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t b = __float_as_uint(v[u][e]) & 0x7fffffffu;
            amax = amax > b ? amax : b;
        }
    amax = wave_max_u32(amax);
    float r = 0.0f;
    bool zero = true;
    if (amax >= 0x7f800000u) {
        if (real && lane == 0) scale[m] = __builtin_nanf("");
    } else if (amax == 0u) {
        if (real && lane == 0) scale[m] = 0.0f;
    } else {
        const float a = __uint_as_float(amax);
        r = 7.0f / a;
        zero = false;
        if (real && lane == 0) scale[m] = (a / 7.0f) * post;
    }
    zero = zero || !real;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t k = ((int64_t)u * 64 + lane) * 8;
        if (k < pitch) {
            uint32_t lo = 0, hi = 0;
            if (!zero && k < K) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    // (a zero value's code is 0 also where r overflowed)
                    float c = __builtin_rintf(v[u][e] * r);
                    c = fminf(fmaxf(c, -7.0f), 7.0f);
                    const uint32_t b = v[u][e] == 0.0f ? 0u : (uint32_t)(int)c & 0xffu;
                    if (e < 4) lo |= b << (8 * e);
                    else hi |= b << (8 * (e - 4));
                }
            }
            *reinterpret_cast<uint2 *>(codes + wave * pitch + k) = make_uint2(lo, hi);
        }
    }
    __syncthreads();
    const int64_t rb = m0 >> 4;
    const int half = (int)(m0 & 15);
    int8_t *base = q + ((rb * KW) << 10);
    const int64_t pieces = (int64_t)R4 * 4 * KW;
    for (int64_t p = threadIdx.x; p < pieces; p += 512) {
        const int pr = (int)(p & 7);
        const int qq = (int)((p >> 3) & 3);
        const int64_t kw = p >> 5;
        // plain stores: the product reads the codes next
        *reinterpret_cast<v4i *>(base + ((kw * 64 + qq * 16 + half + pr) << 4)) =
            *reinterpret_cast<const v4i *>(codes + pr * pitch + kw * 64 + qq * 16);
    }
}

// Wide rows, K = 64 * V (4096 or 8192), one wave per row, 4 rows per group.
// Lane l holds the contiguous elements l*V .. l*V + V - 1, so the stages
// h = 1 .. V/2 (the low log2(V) index bits) run in its registers; one
// transpose through LDS then gives lane l' the elements h*V + l' + 64 j
// (h = 0..63, j < V/64), the six high index bits in registers for the stages
// h = V .. K/2.  No butterfly crosses lanes.  The transpose area, 64 rows of
// 64 floats padded to 68 per wave (writes and reads free of bank conflicts),
// is the wave's own, so the transpose needs no workgroup barrier (a wave-level
// ordering of its lanes' accesses suffices); it is reused for the wave's
// codes, and one barrier before the packed stores takes all 4 rows.
//
// The inputs arrive in line order.  Loaded straight into that lane layout, a
// load whose 64 lanes each read 16 bytes of another 128-byte line costs the
// vector memory path a tag lookup per lane: at K = 4096 a wave issued 24 such
// loads (its row and its factors), and they, not HBM, held each wave up for
// about half its time.  Here 8 consecutive lanes read one line, and the data
// passes through the transpose areas (before the transposes need them) into
// lane order: the group's one copy of the factors (16 or 32 KiB) and each
// wave's row, 8 KiB at a time.  Both copies place 16-byte chunk c at slot
// c ^ ((c >> S) & 15) (S = log2 of the lane's chunks: 3 for the row, 4 or 5
// for the factors), so the line-order writes and the lane-order reads alike
// touch 16 different 16-byte bank groups per 16 lanes (8 per 8); a barrier
// publishes the factors and another frees the areas for the transposes.
constexpr int RT = 4;     // rows per workgroup
constexpr int TP = 68;    // padded floats per transpose row

__device__ __forceinline__ int swz(int c, int s) { return c ^ ((c >> s) & 15); }

template <int V>
__global__ void __launch_bounds__(64 * RT)
k_quant4_rot_t(const uint16_t *__restrict__ x, int64_t M, int64_t K, int64_t ldx,
               const float *__restrict__ mult, float post, int8_t *__restrict__ q,
               float *__restrict__ scale) {
    static_assert(V == 64 || V == 128, "K = 4096 or 8192");
    extern __shared__ __align__(16) float tr_all[];     // [RT][64][TP]
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t m0 = (int64_t)blockIdx.x * RT;
    const int64_t m = m0 + wave;
    const bool real = m < M;
    const uint16_t *row = x + (real ? m : 0) * ldx;
    float *tr = tr_all + wave * 64 * TP;

    float v[V];
    // 16-byte chunks in line order.  The factors (the same for the 4 rows)
    // are loaded by the whole group, chunk c = 256 i + thread (elements
    // 4c .. 4c + 3), into the first halves of the areas (chunk slot s at
    // area s >> 9, offset 16 (s & 511)); each wave's row, 64 elements of
    // every lane at a time, into the second half of its own area (offset
    // 9216): lane l of load t takes chunk (V/8) (8 t + l / 8) + 8 h + l % 8
    // (8 elements; h the half), 8 consecutive lanes one line.
    constexpr int XOFF = 9216 / 4;                    // floats
    constexpr int SF = V == 64 ? 4 : 5;               // log2 of the lane's factor chunks
    static_assert(64 * TP * 4 - 9216 >= 8192 && 9216 * RT >= V * 64 * 4, "staging fits");
    // The row first: it comes from HBM.  At K = 4096 a row past M reads row 0
    // (its codes are zeroed and its scale not written below), so no load is
    // predicated (9.64 -> 9.44 us at 2048 x 4096, 29.7 -> 27.8 at 8192 x 4096);
    // at K = 8192 the unpredicated form scheduled the second half's loads late
    // (18.6 -> 25.8 us at 2048 x 8192), so there rows past M load nothing.
    uint4 raw[V / 64][8];
#pragma unroll
    for (int h = 0; h < V / 64; ++h)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int c = V == 64 ? t * 64 + lane       // (the same chunk, written plainly)
                                  : (t * 8 + (lane >> 3)) * (V / 8) + 8 * h + (lane & 7);
            raw[h][t] = (V == 64 || real) ? *reinterpret_cast<const uint4 *>(row + c * 8)
                                          : make_uint4(0u, 0u, 0u, 0u);
        }
    float4 fl[V / 16];
#pragma unroll
    for (int i = 0; i < V / 16; ++i)
        fl[i] = *reinterpret_cast<const float4 *>(mult + (i * 256 + (int)threadIdx.x) * 4);
    auto fslot = [&](int c) {
        const int sl = swz(c, SF);
        return reinterpret_cast<float4 *>(tr_all + (sl >> 9) * 64 * TP) + (sl & 511);
    };
#pragma unroll
    for (int i = 0; i < V / 16; ++i) *fslot(i * 256 + (int)threadIdx.x) = fl[i];
    uint4 *xs = reinterpret_cast<uint4 *>(tr + XOFF);
#pragma unroll
    for (int h = 0; h < V / 64; ++h) {
        if (h > 0) wave_lds_exchange();               // the last half's reads are done
#pragma unroll
        for (int t = 0; t < 8; ++t) xs[swz(t * 64 + lane, 3)] = raw[h][t];
        if (h == 0) __syncthreads();                  // the group's factors (and the row)
        else wave_lds_exchange();
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint4 r4 = xs[swz(lane * 8 + j, 3)];   // elements V lane + 64 h + 8 j ..
            const int c = lane * (V / 4) + 16 * h + 2 * j;   // and their factors
            const float4 f0 = *fslot(c), f1 = *fslot(c + 1);
            const uint32_t hw[4] = {r4.x, r4.y, r4.z, r4.w};
            const float f[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
            float *vv = v + 64 * h + 8 * j;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                vv[2 * e] = __builtin_fmaf(h2f(hw[e] & 0xffffu), f[2 * e], 0.0f);
                vv[2 * e + 1] = __builtin_fmaf(h2f(hw[e] >> 16), f[2 * e + 1], 0.0f);
            }
        }
    }
    // the transposes below write over the factors and rows
    __syncthreads();
    // stages h = 1 .. V/2: inside the lane's segment
#pragma unroll
    for (int hb = 1; hb < V; hb <<= 1)
#pragma unroll
        for (int r = 0; r < V; ++r)
            if ((r & hb) == 0) {
                const float a = v[r], b = v[r + hb];
                v[r] = a + b;
                v[r + hb] = a - b;
            }
    // transpose, one block of 64 segment positions at a time: lane l writes
    // its positions 64 j .. 64 j + 63 as transpose row l; lane l' reads column
    // l', i.e. element h*V + l' + 64 j for h = 0..63, into v[64 j + h]
#pragma unroll
    for (int j = 0; j < V / 64; ++j) {
#pragma unroll
        for (int r4 = 0; r4 < 64; r4 += 4)
            *reinterpret_cast<float4 *>(tr + lane * TP + r4) =
                make_float4(v[64 * j + r4], v[64 * j + r4 + 1], v[64 * j + r4 + 2],
                            v[64 * j + r4 + 3]);
        // the area is this wave's own: the exchange between its lanes needs
        // no workgroup barrier, only the ordering of the wave's own accesses
        wave_lds_exchange();
#pragma unroll
        for (int h = 0; h < 64; ++h) v[64 * j + h] = tr[h * TP + lane];
        // the next block's writes (or the codes below) reuse the area
        wave_lds_exchange();
    }
    // stages h = V .. K/2: the six high index bits, now the register index h
#pragma unroll
    for (int j = 0; j < V / 64; ++j)
#pragma unroll
        for (int hb = 1; hb < 64; hb <<= 1)
#pragma unroll
            for (int h = 0; h < 64; ++h)
                if ((h & hb) == 0) {
                    const float a = v[64 * j + h], b = v[64 * j + h + hb];
                    v[64 * j + h] = a + b;
                    v[64 * j + h + hb] = a - b;
                }

    AbsMax am;
#pragma unroll
    for (int i = 0; i < V; ++i) am.add(v[i]);
    const uint32_t amax = wave_max_u32(am.bits());
    float r = 0.0f;
    bool zero = true;
    if (amax >= 0x7f800000u) {
        if (real && lane == 0) scale[m] = __builtin_nanf("");
    } else if (amax == 0u) {
        if (real && lane == 0) scale[m] = 0.0f;
    } else {
        const float a = __uint_as_float(amax);
        r = 7.0f / a;
        zero = false;
        if (real && lane == 0) scale[m] = (a / 7.0f) * post;
    }
    zero = zero || !real;
    // codes into the wave's (now free) transpose area, row-major (17 KiB >= K)
    int8_t *codes = reinterpret_cast<int8_t *>(tr);
    if (zero) {
#pragma unroll
        for (int j = 0; j < V / 64; ++j)
#pragma unroll
            for (int h = 0; h < 64; ++h) codes[h * V + 64 * j + lane] = 0;
    } else if (finite_r(r)) {
        // |v r| <= 7 (1 + 2^-23)^2 < 7.5: no clamp needed.  rint by one
        // float add: y + 1.5 * 2^23 lies in [2^23, 2^24), where the floats are
        // the integers, so its rounding (ties to even) is rint(y) and the low
        // byte of its bits, which the byte store takes, is the code
#pragma clang fp contract(off)
#pragma unroll
        for (int j = 0; j < V / 64; ++j)
#pragma unroll
            for (int h = 0; h < 64; ++h) {
                const float y = v[64 * j + h] * r;
                codes[h * V + 64 * j + lane] = (int8_t)__float_as_uint(y + 12582912.0f);
            }
    } else {
        // r overflowed (a maximum below 7 / FLT_MAX): v r is +-inf, clamped to
        // +-7, and a zero value's code is 0
#pragma unroll
        for (int j = 0; j < V / 64; ++j)
#pragma unroll
            for (int h = 0; h < 64; ++h) {
                const float x = v[64 * j + h];
                codes[h * V + 64 * j + lane] = (int8_t)(x > 0.0f ? 7 : (x < 0.0f ? -7 : 0));
            }
    }
    __syncthreads();
    const int64_t KW = K >> 6;
    const int64_t rb = m0 >> 4;
    const int quarter = (int)(m0 & 15);          // 0, 4, 8 or 12
    int8_t *base = q + ((rb * KW) << 10);
    const int8_t *cb = reinterpret_cast<const int8_t *>(tr_all);
    const int64_t pieces = (int64_t)RT * 4 * KW;
    for (int64_t p = threadIdx.x; p < pieces; p += 256) {
        const int pr = (int)(p & 3);
        const int qq = (int)((p >> 2) & 3);
        const int64_t kw = p >> 4;
        // plain stores: the product reads the codes next
        *reinterpret_cast<v4i *>(base + ((kw * 64 + qq * 16 + quarter + pr) << 4)) =
            *reinterpret_cast<const v4i *>(cb + pr * (64 * TP * 4) + kw * 64 + qq * 16);
    }
}

// Decode-size batches (M <= 64) with K = 4096 or 8192: one token per workgroup
// of K / 8 threads (8 or 16 waves), each holding one chunk of 8 consecutive
// elements, k = tid * 8 + e.  Stages h = 1, 2, 4 in registers, h = 8 .. 256
// across the lanes of a wave (shuffles), then one LDS transpose: thread p <
// 512 takes the elements p + 512 w of every wave w, so the wave bits are its
// register index for the stages h = 512 .. K/2.  Same stage order and
// butterflies as everywhere else.  The codes go to LDS in element order and
// leave as packed 16-byte pieces.
template <int WAVES>
__global__ void __launch_bounds__(64 * WAVES)
k_quant4_rot_row1(const uint16_t *__restrict__ x, int64_t M, int64_t ldx,
                  const float *__restrict__ mult, float post, int8_t *__restrict__ q,
                  float *__restrict__ scale) {
    constexpr int K = 512 * WAVES;
    __shared__ __align__(16) float tr[K];
    __shared__ __align__(16) int8_t codes[K];
    __shared__ uint32_t s_max[WAVES];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t m = blockIdx.x;
    const bool real = m < M;
    const uint16_t *row = x + (real ? m : 0) * ldx;
    float v[8];
    {
        uint4 raw = make_uint4(0u, 0u, 0u, 0u);
        float4 f0 = make_float4(0.f, 0.f, 0.f, 0.f), f1 = f0;
        if (real) {
            raw = *reinterpret_cast<const uint4 *>(row + tid * 8);
            f0 = *reinterpret_cast<const float4 *>(mult + tid * 8);
            f1 = *reinterpret_cast<const float4 *>(mult + tid * 8 + 4);
        }
        const uint32_t h[4] = {raw.x, raw.y, raw.z, raw.w};
        const float f[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[2 * e] = h2f(h[e] & 0xffffu) * f[2 * e];
            v[2 * e + 1] = h2f(h[e] >> 16) * f[2 * e + 1];
        }
    }
#pragma unroll
    for (int hb = 1; hb < 8; hb <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if ((e & hb) == 0) {
                const float a = v[e], b = v[e + hb];
                v[e] = a + b;
                v[e + hb] = a - b;
            }
#pragma unroll
    for (int t = 0; t < 6; ++t) {
        const bool upper = (lane >> t) & 1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float p = __shfl_xor(v[e], 1 << t, 64);
            v[e] = upper ? p - v[e] : v[e] + p;
        }
    }
    *reinterpret_cast<float4 *>(&tr[tid * 8]) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4 *>(&tr[tid * 8 + 4]) = make_float4(v[4], v[5], v[6], v[7]);
    __syncthreads();
    // thread p < 512: the elements p + 512 w, w = 0 .. WAVES-1 (the wave bits)
    float u[WAVES];
    uint32_t amax = 0;
    if (tid < 512) {
#pragma unroll
        for (int w = 0; w < WAVES; ++w) u[w] = tr[tid + 512 * w];
#pragma unroll
        for (int hb = 1; hb < WAVES; hb <<= 1)
#pragma unroll
            for (int w = 0; w < WAVES; ++w)
                if ((w & hb) == 0) {
                    const float a = u[w], b = u[w + hb];
                    u[w] = a + b;
                    u[w + hb] = a - b;
                }
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            const uint32_t b = __float_as_uint(u[w]) & 0x7fffffffu;
            amax = amax > b ? amax : b;
        }
    }
    amax = wave_max_u32(amax);
    if (lane == 0) s_max[wave] = amax;
    __syncthreads();
    uint32_t a = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) a = a > s_max[w] ? a : s_max[w];
    float r = 0.0f;
    bool zero = true;
    if (a >= 0x7f800000u) {
        if (real && tid == 0) scale[m] = __builtin_nanf("");
    } else if (a == 0u) {
        if (real && tid == 0) scale[m] = 0.0f;
    } else {
        const float af = __uint_as_float(a);
        r = 7.0f / af;
        zero = false;
        if (real && tid == 0) scale[m] = (af / 7.0f) * post;
    }
    zero = zero || !real;
    if (tid < 512) {
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            float c = __builtin_rintf(u[w] * r);
            c = fminf(fmaxf(c, -7.0f), 7.0f);
            // (a zero value's code is 0 also where r overflowed)
            codes[tid + 512 * w] = (zero || u[w] == 0.0f) ? (int8_t)0 : (int8_t)(int)c;
        }
    }
    __syncthreads();
    // K / 16 pieces of 16 codes: piece j (k = 16 j ..) to window j / 4, quarter j % 4
    constexpr int KW = K / 64;
    int8_t *base = q + (((m >> 4) * KW) << 10) + (m & 15) * 16;
    for (int j = tid; j < K / 16; j += 64 * WAVES)
        *reinterpret_cast<v4i *>(base + ((j >> 2) << 10) + ((j & 3) << 8)) =
            *reinterpret_cast<const v4i *>(&codes[j * 16]);
}

hipError_t launch_quant4_rows(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                              const float *mult, int rotate, float post, int8_t *q, float *scale,
                              hipStream_t st) {
    if (M <= 0) return hipSuccess;
    // unrotated: the per-token quantizer at 7 levels (post is 1 there)
    if (!rotate) return launch_quant4_plain(x, M, K, ldx, mult, q, scale, st);
    if (M <= 64 && (K == 4096 || K == 8192)) {   // decode sizes: one token per workgroup
        const dim3 g((unsigned)((M + 15) / 16 * 16));   // every row of the padded blocks
        if (K == 4096) k_quant4_rot_row1<8><<<g, dim3(512), 0, st>>>(x, M, ldx, mult, post, q, scale);
        else k_quant4_rot_row1<16><<<g, dim3(1024), 0, st>>>(x, M, ldx, mult, post, q, scale);
        return hipGetLastError();
    }
    if (K == 4096 || K == 8192) {
        const dim3 g((unsigned)((M + 15) / 16 * 4)), b(256);   // every row of the padded blocks
        const size_t lds = (size_t)RT * 64 * TP * sizeof(float);
        if (K == 4096) k_quant4_rot_t<64><<<g, b, lds, st>>>(x, M, K, ldx, mult, post, q, scale);
        else k_quant4_rot_t<128><<<g, b, lds, st>>>(x, M, K, ldx, mult, post, q, scale);
        return hipGetLastError();
    }
    const int64_t groups = (M + 15) / 16 * 2;       // every row of the padded row blocks
    const int64_t chunks = (K + 511) / 512;          // chunks of 8 per lane
    const size_t lds = (size_t)R4 * ((K + 63) / 64) * 64;
    const dim3 g((unsigned)groups), b(512);
#define SQ_Q4(U_) k_quant4_rows<U_><<<g, b, lds, st>>>(x, M, K, ldx, mult, post, q, scale)
    if (chunks <= 1) SQ_Q4(1);
    else if (chunks <= 2) SQ_Q4(2);
    else SQ_Q4(4);                                   // K <= 2048 (wider rows above)
#undef SQ_Q4
    return hipGetLastError();
}

// W fp16 [K][ldw] -> W^T fp16 [N][K]: 64 x 64 tiles through LDS.
__global__ void __launch_bounds__(256)
k_transpose_f16(const uint16_t *__restrict__ w, int64_t K, int64_t N, int64_t ldw,
                uint16_t *__restrict__ wt) {
    __shared__ uint16_t tile[64][66];
    const int64_t n0 = (int64_t)blockIdx.x * 64, k0 = (int64_t)blockIdx.y * 64;
    const int c = threadIdx.x & 63, r0 = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < 16; ++i) {   // consecutive lanes on consecutive columns
        const int r = r0 + 4 * i;
        const int64_t k = k0 + r, n = n0 + c;
        tile[r][c] = (k < K && n < N) ? w[k * ldw + n] : (uint16_t)0;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {    // 16 bytes (8 consecutive k) of one output row each
        const int idx = threadIdx.x + 256 * i;
        const int nn = idx >> 3, kc = (idx & 7) * 8;
        const int64_t n = n0 + nn, k = k0 + kc;
        if (n < N && k < K) {
            uint32_t p[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                p[j] = (uint32_t)tile[kc + 2 * j][nn] | ((uint32_t)tile[kc + 2 * j + 1][nn] << 16);
            *reinterpret_cast<uint4 *>(wt + n * K + k) = make_uint4(p[0], p[1], p[2], p[3]);
        }
    }
}

hipError_t launch_fold4(const uint16_t *w, int64_t K, int64_t N, int64_t ldw, const float *s,
                        int rotate, uint8_t *wq4, float *w_scale, uint8_t *work, hipStream_t st) {
    if (N <= 0) return hipSuccess;
    // workspace: W^T (N x K fp16), then the codes one per byte (packed int8 order)
    uint16_t *wt = reinterpret_cast<uint16_t *>(work);
    int8_t *q8 = reinterpret_cast<int8_t *>(work + 2 * K * N);
    k_transpose_f16<<<dim3((unsigned)((N + 63) / 64), (unsigned)((K + 63) / 64)), dim3(256), 0,
                      st>>>(w, K, N, ldw, wt);
    hipError_t e = hipGetLastError();
    // with the rotation the weight scale carries the 1/K of the two transforms
    if (e == hipSuccess)
        e = launch_quant4_rows(wt, N, K, K, s, rotate, rotate ? 1.0f / (float)K : 1.0f, q8,
                               w_scale, st);
    if (e == hipSuccess) e = launch_pack4_from8(q8, N, K, wq4, st);
    return e;
}

}  // namespace sq
