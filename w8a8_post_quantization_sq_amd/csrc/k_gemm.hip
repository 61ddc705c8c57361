// The W8A8 product on CDNA4 int8 matrix cores with a fused dequantizing epilogue.
//
//   acc[m][n] = sum_j xq[m][j] * wq[n][j]        (exact int32)
//   y[m][n]   = fp16_rne((float(acc) * x_scale[m]) * w_scale[n])
//
// Both operands are int8, so the product runs on the int8 matrix cores
// ("Quantization", learn-kernels.com, para. 2: with both operands quantized
// the product itself runs at low precision, beyond the saving in bytes).
//
// Instruction: v_mfma_i32_16x16x64_i8.  Lane l supplies 16 bytes of row
// (l % 16) of the A block and of column (l % 16) of the B block, quarter l / 16
// of the 64-deep k window; the accumulator of lane l holds column l % 16,
// rows 4 * (l / 16) + r, r = 0..3.  Both operands arrive packed in exactly
// this order (each 16-row x 64-byte fragment is 1 KiB, lane l's 16 bytes at
// l * 16), so every fragment load is one contiguous 1 KiB run, and the packed
// padding is zero, so ragged M, N and K need no masks in the main loop.
//
// Operand roles: A = weight fragment (16 output channels n), B = activation
// fragment (16 tokens m); each lane ends with one token and four consecutive
// channels: one x_scale, a 16-byte w_scale load and an 8-byte fp16 store per
// 16 x 16 block.
//
// k_gemm_tile (M > 64): output tile 256 tokens x 128 channels per workgroup
// of 8 waves, two per SIMD, so one wave's products cover the other's waits;
// wave w owns tokens [32w, 32w + 32) and all 128 channels.
//   - activation fragments are private to a wave and go straight from global
//     memory into a register ring, 3 k-steps ahead;
//   - the 8 KiB weight slice of a k-step is shared by the 8 waves: loaded
//     straight into a ring of 8 LDS buffers, 4 steps ahead (4-bit weights:
//     staged through registers and widened into a ring of 4), in lane order,
//     so reads are conflict-free;
//   - the loop is software-pipelined: while the matrix cores work on step t,
//     each wave already reads step t+1's weight fragments from LDS (one
//     fragment after the 2 products that used its register) and issues the
//     step's global loads, spread over its products; one barrier per step,
//     and no LDS wait sits in front of the first product of a step;
//   - workgroups are numbered so that the 32 tiles one XCD (and its L2) runs
//     form a 4 x 8 block of the tile grid, which shares activation and weight
//     rows.
// k_gemm_wide (M > 64, where enough 256 x 256 tiles fill the CUs, 8-bit
// weights): the same loop with 256 channels per workgroup, so a CU moves a
// third fewer operand bytes per product.
// k_gemm_skinny (M <= 64, decode): one workgroup per 16 output channels; its
// 4 waves split the k windows, stream the weight fragments (the dominant HBM
// traffic) with 8 1 KiB loads in flight each (non-temporal for up to 32
// tokens), and combine their partial sums through LDS.  Activation lanes of
// token rows past M load nothing.  k_gemm_skinny_cb takes 2, 4 or 7 channel
// blocks per workgroup (4-bit weights, and 8-bit ones at 9 to 32 tokens).
//
// With W4 the weights are 4-bit codes, two per byte (the Smooth Rotation
// variant's W4A4): each 16 x 64 fragment is 512 bytes in the same lane order,
// a lane's 8 bytes holding its 16 codes as two's-complement nibbles (byte j
// of each 4-byte half: code j in the low nibble, code j + 4 in the high one).
// They are widened to the int8 operand in registers (unpack4), so the matrix
// instruction, the sums and the epilogue are the 8-bit ones; the decode kernel
// streams half the bytes, the tile kernel widens while staging into LDS.
#include <type_traits>

#include "sq_device.h"
#include "sq.h"

namespace sq {

constexpr uint32_t OOB = 0x80000000u;        // an offset past any buffer extent used here
constexpr uint32_t OOB_BASE = 0x40000000u;   // row base past the buffer (sums stay < 2^31)
constexpr uint32_t OOB_WIN = 0x40000000u;    // window offset past the buffer

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    const int32_t n = bytes > 0x7fffffff ? 0x7fffffff : (int32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}

// 16-byte buffer load; offsets at or past the buffer's extent read as zero.
__device__ __forceinline__ v4i bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// 8-byte buffer load; offsets at or past the buffer's extent read as zero.
__device__ __forceinline__ uint2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    return make_uint2((uint32_t)v[0], (uint32_t)v[1]);
}

// Four two's-complement nibbles (one per byte, high nibbles clear) to four
// int8: with t = n ^ 8 = code + 8 in [0, 15], (t + 0x78) ^ 0x80 is t - 8 mod
// 256 in every byte, and t + 0x78 <= 0x87 never carries into the next byte.
__device__ __forceinline__ int sext4(uint32_t n) {
    return (int)(((n ^ 0x08080808u) + 0x78787878u) ^ 0x80808080u);
}

// A lane's 8 bytes of 4-bit codes to its 16-byte int8 operand.
__device__ __forceinline__ v4i unpack4(uint2 p) {
    constexpr uint32_t LO = 0x0F0F0F0Fu;
    return v4i{sext4(p.x & LO), sext4((p.x >> 4) & LO), sext4(p.y & LO), sext4((p.y >> 4) & LO)};
}

// 16 bytes per lane from a buffer straight into LDS (buffer_load_dwordx4 ...
// lds): lane l's bytes land at lds + 16 l, lds wave-uniform (it goes to M0);
// lanes past the buffer's extent write zeros.  The load counts in vmcnt like
// any other.  The builtin exists only for the device target: the host pass,
// which emits the kernels' launch stubs, would drop every template instance
// that names it, so only the device pass sees it.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, int8_t *lds, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, voff,
                                             0, 0, 0);
#endif
}

__device__ __forceinline__ v4i mfma(const v4i &a, const v4i &b, const v4i &c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// XCD-aware tile order.  Workgroup b runs on XCD b % 8.  Tile ids are dealt
// out so that XCD x receives a contiguous run of ids, and ids are laid out in
// groups of 4 tile rows (m) walked column-major, so a run of 32 ids is a
// 4 x 8 block of tiles.
__device__ __forceinline__ void tile_of(int b, int tiles_m, int tiles_n, int &tm, int &tn) {
    const int total = tiles_m * tiles_n;
    int t = b;
    if ((total & 7) == 0) t = (b & 7) * (total >> 3) + (b >> 3);
    constexpr int G = 4;
    const int per_group = G * tiles_n;
    const int g = t / per_group;
    const int first_m = g * G;
    const int gm = (tiles_m - first_m) < G ? (tiles_m - first_m) : G;
    const int r = t - g * per_group;
    tm = first_m + r % gm;
    tn = r / gm;
}

// Dequantizes and stores the four outputs (m, n .. n + 3) a lane holds.
template <bool F16OUT>
__device__ __forceinline__ void store4(void *Y, int64_t ldy, bool vec_ok, int m, int n, int M,
                                       int N, const v4i &acc, float xsm,
                                       const float *__restrict__ ws) {
    if (m >= M || n >= N) return;
    if (F16OUT) {
        uint16_t *row = reinterpret_cast<uint16_t *>(Y) + (int64_t)m * ldy;
        if (vec_ok && n + 3 < N) {
            const float4 w4 = *reinterpret_cast<const float4 *>(ws + n);
            const uint32_t lo = (uint32_t)f2h_bits(((float)acc[0] * xsm) * w4.x) |
                                ((uint32_t)f2h_bits(((float)acc[1] * xsm) * w4.y) << 16);
            const uint32_t hi = (uint32_t)f2h_bits(((float)acc[2] * xsm) * w4.z) |
                                ((uint32_t)f2h_bits(((float)acc[3] * xsm) * w4.w) << 16);
            *reinterpret_cast<uint2 *>(row + n) = make_uint2(lo, hi);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (n + r < N) row[n + r] = f2h_bits(((float)acc[r] * xsm) * ws[n + r]);
        }
    } else {
        int32_t *row = reinterpret_cast<int32_t *>(Y) + (int64_t)m * ldy;
        if (vec_ok && n + 3 < N) {
            *reinterpret_cast<v4i *>(row + n) = acc;
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (n + r < N) row[n + r] = acc[r];
        }
    }
}

// ---- large token counts --------------------------------------------------------------

constexpr int T_BM = 256;            // tokens per tile (16 row blocks, 2 per wave)
constexpr int T_BN = 128;            // channels per tile (8 row blocks)
constexpr int T_FRAG = 1024;         // bytes per packed fragment
constexpr int T_SLICE = 8 * T_FRAG;  // weight bytes per k-step
constexpr int T_WAVES = 8;

template <bool F16OUT, bool W4>
__global__ void __launch_bounds__(64 * T_WAVES)
k_gemm_tile(const int8_t *__restrict__ X, const int8_t *__restrict__ W,
            const float *__restrict__ xs, const float *__restrict__ ws, int M, int N, int K,
            void *__restrict__ Y, int64_t ldy, int tiles_m, int tiles_n, int vec_ok) {
    // LDS: the ring of weight slices during the k loop (8 with 8-bit weights,
    // 4 with 4-bit ones), then 8 wave tiles of the epilogue
    constexpr int EPI_PITCH = 128 * 2 + 16;            // bytes per row of 128 fp16, padded
    constexpr int EPI_WAVE = 32 * EPI_PITCH;            // 32 rows per wave
    constexpr int RING = W4 ? 4 : 8;
    constexpr int LDS_BYTES =
        (RING * T_SLICE > T_WAVES * EPI_WAVE) ? RING * T_SLICE : T_WAVES * EPI_WAVE;
    __shared__ __align__(16) int8_t lds_raw[LDS_BYTES];
    int8_t (*ldsw)[T_SLICE] = reinterpret_cast<int8_t (*)[T_SLICE]>(lds_raw);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * T_BM;
    const int n0 = tn * T_BN;
    const int KW = (K + 63) >> 6;
    const int rbx = (M + 15) >> 4, rbw = (N + 15) >> 4;    // row blocks in the buffers
    const int nbx = min(16, rbx - (m0 >> 4));               // ... present in this tile
    const int nbw = min(8, rbw - (n0 >> 4));
    const __amdgpu_buffer_rsrc_t rx =
        make_rsrc(X + (int64_t)(m0 >> 4) * KW * T_FRAG, (int64_t)nbx * KW * T_FRAG);
    constexpr int WF = W4 ? T_FRAG / 2 : T_FRAG;           // weight bytes per fragment
    const __amdgpu_buffer_rsrc_t rw =
        make_rsrc(W + (int64_t)(n0 >> 4) * KW * WF, (int64_t)nbw * KW * WF);

    // the epilogue's scales are loaded now and wait in registers
    float xsv[2];
    float4 wsv[8];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int m = m0 + wave * 32 + i * 16 + (lane & 15);
        xsv[i] = (F16OUT && m < M) ? xs[m] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int n = n0 + j * 16 + (lane >> 4) * 4;
        wsv[j] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (F16OUT) {
            if (n + 3 < N) {
                // one 16-byte load: ws is 16-byte aligned and n a multiple of 4
                wsv[j] = *reinterpret_cast<const float4 *>(ws + n);
            } else {
                if (n < N) wsv[j].x = ws[n];
                if (n + 1 < N) wsv[j].y = ws[n + 1];
                if (n + 2 < N) wsv[j].z = ws[n + 2];
            }
        }
    }

    // activation fragments: this wave's row blocks 2w and 2w + 1
    uint32_t xbase[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int b = wave * 2 + i;
        xbase[i] = b < nbx ? (uint32_t)(b * KW * T_FRAG + lane * 16) : OOB_BASE;
    }
    // weight slice: 512 chunks of 16 bytes (8 with W4), one per thread; chunk
    // tid = fragment tid / 64, lane tid % 64
    uint32_t wbase;
    {
        const int b = tid >> 6;
        wbase = b < nbw ? (uint32_t)(b * KW * WF + (tid & 63) * (WF / 64)) : OOB_BASE;
    }
    // Offset of k window t (uniform): windows past the last one get OOB_WIN, so
    // every lane's base + offset falls past the buffer and reads zero.  Bases
    // are < 2^25 or OOB_BASE, offsets < 2^21 or OOB_WIN, so sums never wrap.
    auto win = [&](int t) -> uint32_t { return t < KW ? (uint32_t)t * T_FRAG : OOB_WIN; };
    auto winw = [&](int t) -> uint32_t { return t < KW ? (uint32_t)t * WF : OOB_WIN; };

    v4i acc[2][8];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    v4i xr[4][2];    // activation ring: steps t .. t+3
    v4i wf[8];       // weight fragments of the current step
    auto load_x = [&](int slot, int t) {
        const uint32_t wo = win(t);
#pragma unroll
        for (int i = 0; i < 2; ++i) xr[slot][i] = bload(rx, xbase[i] + wo);
    };

    if constexpr (!W4) {
        // 8-bit weights go straight from global memory into the LDS ring (slice t
        // in buffer t & 7), 4 steps ahead of their use: no register staging and
        // no LDS store, and 3 steps between a slice's load and its first reader,
        // enough for weights that come from HBM.  Wave w loads fragment w of the
        // slice (its lanes' 16 bytes land in lane order, as the readers expect).
        int8_t *ring = lds_raw;
        auto dma_w = [&](int t) {
            lds_load16(rw, ring + (t & 7) * T_SLICE + wave * T_FRAG, wbase + winw(t));
        };
        // Prologue: slices 0..3 and activation steps 0..2, interleaved (slice s,
        // then step s's two fragments), then every load of it waited for:
        // all four slices are in LDS before the loop, which is what the loop's
        // one wait per step assumes for steps 0 and 1.  (A wait for slices 0
        // and 1 only is what __syncthreads' own release fence turns into a
        // full wait anyway, and a barrier without that fence lets the
        // compiler sink the activation loads below it.)
#pragma unroll
        for (int s = 0; s < 3; ++s) {
            __builtin_amdgcn_sched_barrier(0);
            dma_w(s);
            load_x(s, s);
        }
        __builtin_amdgcn_sched_barrier(0);
        dma_w(3);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0x0F70);        // vmcnt(0): slices 0..3 have landed
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 8; ++j)
            wf[j] = *reinterpret_cast<const v4i *>(ring + j * T_FRAG + lane * 16);

        const int nsteps = (KW + 3) & ~3;
        for (int t0 = 0; t0 < nsteps; t0 += 4) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int t = t0 + u;
                const int8_t *nb = ring + ((t + 1) & 7) * T_SLICE;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
#pragma unroll
                    for (int i = 0; i < 2; ++i) acc[i][j] = mfma(wf[j], xr[u][i], acc[i][j]);
                    wf[j] = *reinterpret_cast<const v4i *>(nb + j * T_FRAG + lane * 16);
                    // the step's three global loads (weight slice t+4 into its
                    // buffer, then the two activation fragments of t+3) spread
                    // over its products, each pinned in place: issued together at
                    // the top of the step, the two waves of a SIMD queued all their
                    // loads at once and then waited on the address path with no
                    // products to issue
                    if (j == 1) {
                        __builtin_amdgcn_sched_barrier(0);
                        dma_w(t + 4);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    if (j == 4) {
                        __builtin_amdgcn_sched_barrier(0);
                        xr[(u + 3) & 3][0] = bload(rx, xbase[0] + win(t + 3));
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    if (j == 7) {
                        __builtin_amdgcn_sched_barrier(0);
                        xr[(u + 3) & 3][1] = bload(rx, xbase[1] + win(t + 3));
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                // Slice t+2, read from the next step on, was loaded at step t-2;
                // 8 loads were issued after it (2 in its step, 3 in each later
                // one), and memory loads complete in order, so vmcnt(8) means it
                // has landed in this wave's part of the buffer; the barrier then
                // publishes every wave's part.  Slices 2 and 3 (steps 0 and 1)
                // landed in the prologue.  The same wait on every step matters:
                // a different wait for the first steps made the compiler peel
                // the first 4 steps and sink their activation loads past the
                // loop's exit test, leaving fewer than 8 loads behind slices 4
                // and 5.  The buffer a step loads into (slice t+4: buffer
                // (t-4) & 7) was last read in step t-5.
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_waitcnt(0x0F78);    // vmcnt(8)
                __builtin_amdgcn_s_barrier();
                // keep each step's products inside the step: hoisting them above
                // the barrier would put them right behind the LDS reads they use
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // the slices loaded past the last step still land in LDS, which the
        // epilogue reuses: wait for them
        __builtin_amdgcn_s_waitcnt(0x0F70);            // vmcnt(0)
    } else {
        // 4-bit weights: staged through registers (the packed 8 bytes of slices
        // t+2 and t+3), widened on their way into a ring of 4 LDS buffers
        uint2 wst[2];
        auto load_w = [&](int slot, int t) { wst[slot] = bload8(rw, wbase + winw(t)); };
        auto store_w = [&](int slot, int buf) {
            *reinterpret_cast<v4i *>(&ldsw[buf][tid * 16]) = unpack4(wst[slot]);
        };
        // prologue: weight slices 0 and 1 in LDS, slice 2 staged, activations 0..2 in flight
#pragma unroll
        for (int s = 0; s < 3; ++s) load_x(s, s);
        load_w(0, 0);
        load_w(1, 1);
        store_w(0, 0);
        store_w(1, 1);
        load_w(0, 2);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 8; ++j)
            wf[j] = *reinterpret_cast<const v4i *>(&ldsw[0][j * T_FRAG + lane * 16]);

        const int nsteps = (KW + 3) & ~3;
        for (int t0 = 0; t0 < nsteps; t0 += 4) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int t = t0 + u;
                const int nb = (u + 1) & 3;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
#pragma unroll
                    for (int i = 0; i < 2; ++i) acc[i][j] = mfma(wf[j], xr[u][i], acc[i][j]);
                    wf[j] = *reinterpret_cast<const v4i *>(&ldsw[nb][j * T_FRAG + lane * 16]);
                    // The step's three global loads (weight slice t+3, then the two
                    // activation fragments of t+3) and the LDS store of slice t+2
                    // are spread over its products, each pinned in place: issued
                    // together at the top of the step, the two waves of a SIMD
                    // queued all their loads at once and then waited on the
                    // address path with no products to issue.  The slice stored
                    // here was loaded a step earlier, so its wait leaves the later
                    // loads in flight.
                    if (j == 1) {
                        __builtin_amdgcn_sched_barrier(0);
                        load_w((u + 1) & 1, t + 3);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    if (j == 4) {
                        __builtin_amdgcn_sched_barrier(0);
                        xr[(u + 3) & 3][0] = bload(rx, xbase[0] + win(t + 3));
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    if (j == 5) {
                        __builtin_amdgcn_sched_barrier(0);
                        store_w(u & 1, (u + 2) & 3);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    if (j == 6) {
                        __builtin_amdgcn_sched_barrier(0);
                        xr[(u + 3) & 3][1] = bload(rx, xbase[1] + win(t + 3));
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                // Before the barrier only the store must be complete: LDS
                // operations of a wave complete in order, so at most the 2 later
                // fragment reads (6 and 7) may still be in flight (they read slice
                // t+1, which nobody overwrites before two more barriers).
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_waitcnt(0xc07f | (2 << 8));   // lgkmcnt(2)
                __builtin_amdgcn_s_barrier();
                // keep each step's products inside the step: hoisting them above
                // the barrier would put them right behind the LDS reads they use
                __builtin_amdgcn_sched_barrier(0);
            }
        }

    }

    // epilogue.  fp16 output goes through LDS (the weight buffers are free
    // now): each wave converts its 32 x 128 block into a padded LDS tile and
    // writes it back as rows of 256 contiguous bytes, 16 bytes per lane.
    if (F16OUT && (vec_ok & 2)) {
        constexpr int PITCH = EPI_PITCH;
        int8_t *tile = lds_raw + wave * EPI_WAVE;     // this wave's 8.5 KiB
        __syncthreads();                              // every wave is done with the slices
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const v4i &a = acc[i][j];
                const uint32_t lo = (uint32_t)f2h_bits(((float)a[0] * xsv[i]) * wsv[j].x) |
                                    ((uint32_t)f2h_bits(((float)a[1] * xsv[i]) * wsv[j].y) << 16);
                const uint32_t hi = (uint32_t)f2h_bits(((float)a[2] * xsv[i]) * wsv[j].z) |
                                    ((uint32_t)f2h_bits(((float)a[3] * xsv[i]) * wsv[j].w) << 16);
                *reinterpret_cast<uint2 *>(tile + (i * 16 + (lane & 15)) * PITCH +
                                           (j * 16 + (lane >> 4) * 4) * 2) = make_uint2(lo, hi);
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);           // lgkmcnt(0): this wave's LDS writes done
        wave_lds_exchange();                          // lanes read what other lanes wrote
        // 32 rows x 16 chunks of 16 bytes, 8 per lane; 4 rows per instruction
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int r = c * 4 + (lane >> 4);
            const int m = m0 + wave * 32 + r;
            const int n = n0 + (lane & 15) * 8;
            const uint4 v = *reinterpret_cast<const uint4 *>(tile + r * PITCH + (lane & 15) * 16);
            if (m < M) {
                uint16_t *dst = reinterpret_cast<uint16_t *>(Y) + (int64_t)m * ldy + n;
                if (n + 7 < N) {
                    // non-temporal: the output is not read again here
                    const v4i vv = {(int)v.x, (int)v.y, (int)v.z, (int)v.w};
                    __builtin_nontemporal_store(vv, reinterpret_cast<v4i *>(dst));
                } else {
                    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (n + e < N) dst[e] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
                }
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int m = m0 + wave * 32 + i * 16 + (lane & 15);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                store4<F16OUT>(Y, ldy, (vec_ok & 1) != 0, m, n0 + j * 16 + (lane >> 4) * 4, M, N,
                               acc[i][j], xsv[i], ws);
        }
    }
}

// ---- small token counts (decode) ---------------------------------------------------------

constexpr int S_UNROLL = 8;   // k windows in flight per wave (twice that with 4-bit weights,
                              // so a lane keeps the same 128 bytes of weights in flight)

template <int MB, bool F16OUT>
__global__ void __launch_bounds__(256)
k_gemm_skinny(const int8_t *__restrict__ X, const int8_t *__restrict__ W,
              const float *__restrict__ xs, const float *__restrict__ ws, int M, int N, int K,
              void *__restrict__ Y, int64_t ldy, int vec_ok) {
    __shared__ __align__(16) v4i part[3][MB][64];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nb = blockIdx.x;                   // 16-channel block
    const int KW = (K + 63) >> 6;
    const int rbx = (M + 15) >> 4;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(X, (int64_t)rbx * KW * T_FRAG);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(W + (int64_t)nb * KW * T_FRAG, (int64_t)KW * T_FRAG);
    // Up to 2 row blocks, lanes of token rows past M (zero padding) load no
    // activations: at M = 1, 15 of 16 lanes.  (With more row blocks this
    // kernel keeps its registers low instead, which measured faster.)
    bool xrow[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b) xrow[b] = MB > 2 || b * 16 + (lane & 15) < M;

    v4i acc[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b) acc[b] = v4i{0, 0, 0, 0};
    // wave w takes windows w, w + 4, w + 8, ...: the 4 waves stream adjacent KiB
    for (int t0 = wave; t0 < KW; t0 += 4 * S_UNROLL) {
        v4i wf[S_UNROLL], xf[S_UNROLL][MB];
#pragma unroll
        for (int u = 0; u < S_UNROLL; ++u) {
            const int t = t0 + 4 * u;
            // The weights are read exactly once.  Up to 32 tokens, non-temporal
            // global loads stream them faster than buffer loads; with 64 tokens
            // (4 activation fragments per window) the buffer loads measure faster.
            if constexpr (MB <= 2)
                wf[u] = t < KW ? __builtin_nontemporal_load(reinterpret_cast<const v4i *>(
                                     W + ((int64_t)nb * KW + t) * T_FRAG + lane * 16))
                               : v4i{0, 0, 0, 0};
            else
                wf[u] = bload(rw, t < KW ? (uint32_t)(t * T_FRAG + lane * 16) : OOB);
#pragma unroll
            for (int b = 0; b < MB; ++b)
                xf[u][b] = bload(rx, (t < KW && b < rbx && xrow[b])
                                         ? (uint32_t)((b * KW + t) * T_FRAG + lane * 16) : OOB);
        }
#pragma unroll
        for (int u = 0; u < S_UNROLL; ++u)
#pragma unroll
            for (int b = 0; b < MB; ++b) acc[b] = mfma(wf[u], xf[u][b], acc[b]);
    }
    if (wave > 0) {
#pragma unroll
        for (int b = 0; b < MB; ++b) part[wave - 1][b][lane] = acc[b];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int b = 0; b < MB; ++b) {
#pragma unroll
        for (int w = 0; w < 3; ++w) {
            const v4i p = part[w][b][lane];
            acc[b][0] += p[0];
            acc[b][1] += p[1];
            acc[b][2] += p[2];
            acc[b][3] += p[3];
        }
        const int m = b * 16 + (lane & 15);
        const float xsm = (F16OUT && m < M) ? xs[m] : 0.0f;
        store4<F16OUT>(Y, ldy, (vec_ok & 1) != 0, m, nb * 16 + (lane >> 4) * 4, M, N, acc[b], xsm, ws);
    }
}

// Decode with CB channel blocks per workgroup: each activation fragment a
// wave loads feeds CB weight fragments, which divides the activations' share
// of the L2 traffic by CB (it matters with 16 or more real token rows, and
// always with 4-bit weights, whose 512-byte fragments would otherwise be
// outweighed by the activations); a window batch's loads stay ahead of its
// products, and 4-bit codes are widened just before the matrix instruction.
// NW waves per workgroup take interleaved k windows; with 7 blocks (one
// workgroup per CU) 8 waves of half the batch each keep two waves on every
// SIMD, so one wave's products overlap another's loads.  blockIdx.y picks the
// workgroup's MB row blocks of tokens (one group at decode sizes; 64-token
// groups for the mid-size batches below).
template <int MB, bool F16OUT, bool W4, int CB, int NW = 4>
__global__ void __launch_bounds__(64 * NW)
k_gemm_skinny_cb(const int8_t *__restrict__ X, const int8_t *__restrict__ W,
              const float *__restrict__ xs, const float *__restrict__ ws, int M, int N, int K,
              void *__restrict__ Y, int64_t ldy, int vec_ok) {
    static_assert(NW == 4 || NW == 8, "waves per workgroup");
    __shared__ __align__(16) v4i part[NW - 1][CB][MB][64];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nb0 = blockIdx.x * CB;             // first 16-channel block
    const int m0 = blockIdx.y * MB * 16;         // first token of this workgroup's rows
    const int KW = (K + 63) >> 6;
    const int rbx = min(MB, ((M + 15) >> 4) - (m0 >> 4));   // row blocks present
    const int rbw = (N + 15) >> 4;
    const int ncb = rbw - nb0 < CB ? rbw - nb0 : CB;   // blocks present
    const __amdgpu_buffer_rsrc_t rx =
        make_rsrc(X + (int64_t)(m0 >> 4) * KW * T_FRAG, (int64_t)rbx * KW * T_FRAG);
    constexpr int WF = W4 ? T_FRAG / 2 : T_FRAG;           // weight bytes per fragment
    const __amdgpu_buffer_rsrc_t rw =
        make_rsrc(W + (int64_t)nb0 * KW * WF, (int64_t)ncb * KW * WF);
    // A lane feeds token row 16 b + lane % 16 of each activation fragment:
    // rows past M are zero padding, so those lanes load nothing (at M = 1,
    // 15 of 16 lanes), which keeps the activations' L2 traffic to the real rows.
    bool xrow[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b) xrow[b] = m0 + b * 16 + (lane & 15) < M;

    v4i acc[CB][MB];
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
        for (int b = 0; b < MB; ++b) acc[c][b] = v4i{0, 0, 0, 0};
    // wave w takes windows w, w + NW, w + 2 NW, ...: the waves stream adjacent
    // KiB; a batch is SU windows, so a workgroup keeps the same bytes in flight
    // for either wave count
    constexpr int SU = (MB >= 3 ? S_UNROLL / 2 : S_UNROLL) * 4 / NW;
    for (int t0 = wave; t0 < KW; t0 += NW * SU) {
        v4i xf[SU][MB], wf[SU][CB];
        uint2 wp[SU][CB];   // 4-bit: the packed codes as loaded
#pragma unroll
        for (int u = 0; u < SU; ++u) {
            const int t = t0 + NW * u;
            // the weights are read exactly once (non-temporal up to 32 tokens)
#pragma unroll
            for (int c = 0; c < CB; ++c) {
                const bool in = t < KW && c < ncb;
                const int64_t goff = ((int64_t)(nb0 + c) * KW + t) * WF;
                const uint32_t boff = in ? (uint32_t)((c * KW + t) * WF) : OOB;
                if constexpr (W4) {
                    if constexpr (MB <= 2) {
                        typedef unsigned int v2u __attribute__((ext_vector_type(2)));
                        const v2u p = in ? __builtin_nontemporal_load(
                                               reinterpret_cast<const v2u *>(W + goff + lane * 8))
                                         : v2u{0u, 0u};
                        wp[u][c] = make_uint2(p[0], p[1]);
                    } else {
                        wp[u][c] = bload8(rw, boff == OOB ? OOB : boff + lane * 8);
                    }
                } else if constexpr (MB <= 2) {
                    wf[u][c] = in ? __builtin_nontemporal_load(
                                        reinterpret_cast<const v4i *>(W + goff + lane * 16))
                                  : v4i{0, 0, 0, 0};
                } else {
                    wf[u][c] = bload(rw, boff == OOB ? OOB : boff + lane * 16);
                }
            }
#pragma unroll
            for (int b = 0; b < MB; ++b)
                xf[u][b] = bload(rx, (t < KW && b < rbx && xrow[b])
                                         ? (uint32_t)((b * KW + t) * T_FRAG + lane * 16) : OOB);
        }
        // all of the batch's loads stay ahead of its products
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < SU; ++u) {
#pragma unroll
            for (int c = 0; c < CB; ++c) {
                if constexpr (W4) wf[u][c] = unpack4(wp[u][c]);
#pragma unroll
                for (int b = 0; b < MB; ++b) acc[c][b] = mfma(wf[u][c], xf[u][b], acc[c][b]);
            }
        }
    }
    if (wave > 0) {
#pragma unroll
        for (int c = 0; c < CB; ++c)
#pragma unroll
            for (int b = 0; b < MB; ++b) part[wave - 1][c][b][lane] = acc[c][b];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int c = 0; c < CB; ++c) {
#pragma unroll
        for (int b = 0; b < MB; ++b) {
#pragma unroll
            for (int w = 0; w < NW - 1; ++w) {
                const v4i p = part[w][c][b][lane];
                acc[c][b][0] += p[0];
                acc[c][b][1] += p[1];
                acc[c][b][2] += p[2];
                acc[c][b][3] += p[3];
            }
            if (c >= ncb) continue;
            const int m = m0 + b * 16 + (lane & 15);
            const float xsm = (F16OUT && m < M) ? xs[m] : 0.0f;
            store4<F16OUT>(Y, ldy, (vec_ok & 1) != 0, m, (nb0 + c) * 16 + (lane >> 4) * 4, M, N,
                           acc[c][b], xsm, ws);
        }
    }
}

// Channel blocks per decode workgroup.  8-bit weights: one (k_gemm_skinny) up
// to 8 tokens, where the activation loads are mostly skipped, and from 3 row
// blocks on, where its low register count measured best; at 9..32 tokens the
// one of 2, 4, 7 whose workgroup count fills whole rounds of the 256 CUs best
// (N = 28672: 7, one workgroup per CU), as long as at least 512 blocks exist.
// 4-bit weights: 2 at one row block, 4 beyond (measured).
inline int decode_blocks(bool w4, int M, int64_t nblk) {
    if (w4) return M <= 16 ? 2 : 4;
    if (M <= 8 || M > 32 || nblk < 512) return 1;
    int best = 2;
    double best_waste = 2.0;
    for (int cb : {2, 4, 7}) {
        const int64_t wg = (nblk + cb - 1) / cb;
        const double waste = (double)((wg + 255) / 256 * 256) / (double)wg;
        if (waste < best_waste - 1e-9) {
            best = cb;
            best_waste = waste;
        }
    }
    return best;
}

template <int MB, bool F16OUT, bool W4>
void launch_skinny(int cb, dim3 grid, hipStream_t st, const int8_t *xq, const int8_t *wq,
                   const float *x_scale, const float *w_scale, int m, int n, int k, void *y,
                   int64_t ldy, int vec_ok) {
    const dim3 b(256);
    if constexpr (!W4) {
        if (cb == 1 || MB > 2) {
            k_gemm_skinny<MB, F16OUT><<<grid, b, 0, st>>>(xq, wq, x_scale, w_scale, m, n, k, y,
                                                          ldy, vec_ok);
            return;
        }
    }
    if constexpr (W4 || MB <= 2) {
        if (cb == 2)
            k_gemm_skinny_cb<MB, F16OUT, W4, 2><<<grid, b, 0, st>>>(xq, wq, x_scale, w_scale, m, n,
                                                                   k, y, ldy, vec_ok);
        else if (cb == 4)
            k_gemm_skinny_cb<MB, F16OUT, W4, 4><<<grid, b, 0, st>>>(xq, wq, x_scale, w_scale, m, n,
                                                                   k, y, ldy, vec_ok);
        else if constexpr (!W4)   // 8 waves (measured: 37.7-38.0 vs 38.3-38.9 us at 16 tokens)
            k_gemm_skinny_cb<MB, F16OUT, W4, 7, 8><<<grid, dim3(512), 0, st>>>(
                xq, wq, x_scale, w_scale, m, n, k, y, ldy, vec_ok);
    }
}

// ---- wide tiles: 256 tokens x 256 channels ---------------------------------------------

constexpr int W_BN = 256;             // channels per tile (16 row blocks)
constexpr int W_SLICE = 16 * T_FRAG;  // weight bytes per k-step

// Like k_gemm_tile with twice the channels per workgroup: wave w owns tokens
// [32w, 32w + 32) x 256 channels (32 accumulators of 16 x 16).  The 16 KiB
// weight slice of a k-step goes straight into an 8-deep LDS ring, 4 steps
// ahead (wave w loads fragments w and w + 8).  Weight fragments are read from
// LDS one half-step ahead of their products through a ring of 8 registers:
// after the products of fragment j, fragment j + 8 of this step (j < 8) or
// fragment j - 8 of the next step (j >= 8).  Per k-step a CU moves 32 KiB of
// operands for 2 x the products of the 256 x 128 tile (24 KiB).
template <bool F16OUT>
__global__ void __launch_bounds__(64 * T_WAVES)
k_gemm_wide(const int8_t *__restrict__ X, const int8_t *__restrict__ W,
            const float *__restrict__ xs, const float *__restrict__ ws, int M, int N, int K,
            void *__restrict__ Y, int64_t ldy, int tiles_m, int tiles_n, int vec_ok) {
    constexpr int EPI_PITCH = W_BN * 2 + 16;           // bytes per row of 256 fp16, padded
    constexpr int EPI_WAVE = 32 * EPI_PITCH;            // 32 rows per wave
    constexpr int LDS_BYTES =
        (8 * W_SLICE > T_WAVES * EPI_WAVE) ? 8 * W_SLICE : T_WAVES * EPI_WAVE;
    __shared__ __align__(16) int8_t lds_raw[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * T_BM;
    const int n0 = tn * W_BN;
    const int KW = (K + 63) >> 6;
    const int rbx = (M + 15) >> 4, rbw = (N + 15) >> 4;
    const int nbx = min(16, rbx - (m0 >> 4));
    const int nbw = min(16, rbw - (n0 >> 4));
    const __amdgpu_buffer_rsrc_t rx =
        make_rsrc(X + (int64_t)(m0 >> 4) * KW * T_FRAG, (int64_t)nbx * KW * T_FRAG);
    const __amdgpu_buffer_rsrc_t rw =
        make_rsrc(W + (int64_t)(n0 >> 4) * KW * T_FRAG, (int64_t)nbw * KW * T_FRAG);

    float xsv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int m = m0 + wave * 32 + i * 16 + (lane & 15);
        xsv[i] = (F16OUT && m < M) ? xs[m] : 0.0f;
    }
    uint32_t xbase[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int b = wave * 2 + i;
        xbase[i] = b < nbx ? (uint32_t)(b * KW * T_FRAG + lane * 16) : OOB_BASE;
    }
    uint32_t wbase[2];   // this wave's two fragments of every slice: w and w + 8
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int b = wave + 8 * h;
        wbase[h] = b < nbw ? (uint32_t)(b * KW * T_FRAG + lane * 16) : OOB_BASE;
    }
    auto win = [&](int t) -> uint32_t { return t < KW ? (uint32_t)t * T_FRAG : OOB_WIN; };

    v4i acc[2][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[i][j] = v4i{0, 0, 0, 0};
    v4i xr[4][2];
    v4i wf[8];
    int8_t *ring = lds_raw;
    auto dma_w = [&](int h, int t) {
        lds_load16(rw, ring + (t & 7) * W_SLICE + (wave + 8 * h) * T_FRAG, wbase[h] + win(t));
    };
    auto load_x = [&](int slot, int t) {
        const uint32_t wo = win(t);
#pragma unroll
        for (int i = 0; i < 2; ++i) xr[slot][i] = bload(rx, xbase[i] + wo);
    };
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        dma_w(0, s);
        dma_w(1, s);
    }
#pragma unroll
    for (int s = 0; s < 3; ++s) load_x(s, s);
    __builtin_amdgcn_s_waitcnt(0x0F73);        // vmcnt(3): slices 0..3 have landed
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) wf[j] = *reinterpret_cast<const v4i *>(ring + j * T_FRAG + lane * 16);

    const int nsteps = (KW + 3) & ~3;
    for (int t0 = 0; t0 < nsteps; t0 += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int t = t0 + u;
            const int8_t *cur = ring + (t & 7) * W_SLICE;
            const int8_t *nxt = ring + ((t + 1) & 7) * W_SLICE;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
#pragma unroll
                for (int i = 0; i < 2; ++i) acc[i][j] = mfma(wf[j & 7], xr[u][i], acc[i][j]);
                wf[j & 7] = *reinterpret_cast<const v4i *>(
                    (j < 8 ? cur + (j + 8) * T_FRAG : nxt + (j - 8) * T_FRAG) + lane * 16);
                // the step's four global loads (the two fragments of weight
                // slice t+4, then the two activation fragments of t+3) spread
                // over its products, each pinned in place
                if (j == 0) {
                    __builtin_amdgcn_sched_barrier(0);
                    dma_w(0, t + 4);
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (j == 4) {
                    __builtin_amdgcn_sched_barrier(0);
                    dma_w(1, t + 4);
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (j == 10) {
                    __builtin_amdgcn_sched_barrier(0);
                    xr[(u + 3) & 3][0] = bload(rx, xbase[0] + win(t + 3));
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (j == 14) {
                    __builtin_amdgcn_sched_barrier(0);
                    xr[(u + 3) & 3][1] = bload(rx, xbase[1] + win(t + 3));
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // Slice t+2, read from the next step on, was loaded at step t-2;
            // 10 loads were issued after its second fragment (2 in its step,
            // 4 in each later one), and loads complete in order, so vmcnt(10)
            // means it has landed; the barrier publishes every wave's part.
            // The buffer a step loads into (slice t+4: buffer (t-4) & 7) was
            // last read in step t-4.
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(0x0F7A);    // vmcnt(10)
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // the slices loaded past the last step still land in LDS, which the
    // epilogue reuses: wait for them
    __builtin_amdgcn_s_waitcnt(0x0F70);            // vmcnt(0)

    // epilogue as in k_gemm_tile, rows of 512 bytes; the weight scales are
    // loaded here (16 float4 per lane would not fit beside the loop)
    if (F16OUT && (vec_ok & 2)) {
        constexpr int PITCH = EPI_PITCH;
        int8_t *tile = lds_raw + wave * EPI_WAVE;     // this wave's 16.5 KiB
        __syncthreads();                              // every wave is done with the slices
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int n = n0 + j * 16 + (lane >> 4) * 4;
            float4 w4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (n + 3 < N) {
                w4 = *reinterpret_cast<const float4 *>(ws + n);
            } else {
                if (n < N) w4.x = ws[n];
                if (n + 1 < N) w4.y = ws[n + 1];
                if (n + 2 < N) w4.z = ws[n + 2];
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const v4i &a = acc[i][j];
                const uint32_t lo = (uint32_t)f2h_bits(((float)a[0] * xsv[i]) * w4.x) |
                                    ((uint32_t)f2h_bits(((float)a[1] * xsv[i]) * w4.y) << 16);
                const uint32_t hi = (uint32_t)f2h_bits(((float)a[2] * xsv[i]) * w4.z) |
                                    ((uint32_t)f2h_bits(((float)a[3] * xsv[i]) * w4.w) << 16);
                *reinterpret_cast<uint2 *>(tile + (i * 16 + (lane & 15)) * PITCH +
                                           (j * 16 + (lane >> 4) * 4) * 2) = make_uint2(lo, hi);
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);           // lgkmcnt(0): this wave's LDS writes done
        wave_lds_exchange();                          // lanes read what other lanes wrote
        // 32 rows x 32 chunks of 16 bytes, 16 per lane; 2 rows per instruction
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const int r = c * 2 + (lane >> 5);
            const int m = m0 + wave * 32 + r;
            const int n = n0 + (lane & 31) * 8;
            const uint4 v = *reinterpret_cast<const uint4 *>(tile + r * PITCH + (lane & 31) * 16);
            if (m < M) {
                uint16_t *dst = reinterpret_cast<uint16_t *>(Y) + (int64_t)m * ldy + n;
                if (n + 7 < N) {
                    const v4i vv = {(int)v.x, (int)v.y, (int)v.z, (int)v.w};
                    __builtin_nontemporal_store(vv, reinterpret_cast<v4i *>(dst));
                } else {
                    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (n + e < N) dst[e] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
                }
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int m = m0 + wave * 32 + i * 16 + (lane & 15);
#pragma unroll
            for (int j = 0; j < 16; ++j)
                store4<F16OUT>(Y, ldy, (vec_ok & 1) != 0, m, n0 + j * 16 + (lane >> 4) * 4, M, N,
                               acc[i][j], xsv[i], ws);
        }
    }
}

template <bool W4>
hipError_t launch_gemm_any(const int8_t *xq, const float *x_scale, const int8_t *wq,
                           const float *w_scale, int64_t M, int64_t N, int64_t K, void *y,
                           int64_t ldy, int out_kind, hipStream_t st) {
    if (M <= 0 || N <= 0) return hipSuccess;
    const bool f16 = out_kind == SQ_OUT_F16;
    // bit 0: stores of 4 elements (8-byte fp16 / 16-byte int32) line up with
    // every row; bit 1: 16-byte stores of 8 fp16 do
    const int elem = f16 ? 2 : 4;
    const int vec_ok = (((ldy % 4) == 0 && ((uintptr_t)y % (uintptr_t)(4 * elem)) == 0 &&
                         (!f16 || ((uintptr_t)w_scale % 16) == 0)) ? 1 : 0) |
                       ((f16 && (ldy % 8) == 0 && ((uintptr_t)y % 16) == 0) ? 2 : 0);
    const int m = (int)M, n = (int)N, k = (int)K;
    // Mid-size batches whose 256 x 128 tiles would occupy at most a quarter of
    // the 256 CUs (e.g. 65..512 tokens against 4096 channels): the multi-block
    // decode kernel over 64-token groups, each workgroup's 4 waves splitting K,
    // which spreads the same work over many more CUs (measured 21.6 -> 9.0 us
    // at 128 x 4096 x 4096, 49.8 -> 16.3 at 128 tokens, K 11008, N 4096; the
    // tiles win from about 96 of them on).  2 channel blocks per workgroup
    // while that keeps the workgroup count near one per CU, else 4.
    if (!W4 && M > 64 &&
        (int64_t)((m + T_BM - 1) / T_BM) * ((n + T_BN - 1) / T_BN) <= 64) {
        const int64_t nblk = (n + 15) / 16;
        const int64_t mt = (m + 63) / 64;
        const bool two = ((nblk + 1) / 2) * mt <= 256;
        const dim3 grid((unsigned)((nblk + (two ? 1 : 3)) / (two ? 2 : 4)), (unsigned)mt);
        if (f16) {
            if (two)
                k_gemm_skinny_cb<4, true, false, 2><<<grid, dim3(256), 0, st>>>(
                    xq, wq, x_scale, w_scale, m, n, k, y, ldy, vec_ok);
            else
                k_gemm_skinny_cb<4, true, false, 4><<<grid, dim3(256), 0, st>>>(
                    xq, wq, x_scale, w_scale, m, n, k, y, ldy, vec_ok);
        } else {
            if (two)
                k_gemm_skinny_cb<4, false, false, 2><<<grid, dim3(256), 0, st>>>(
                    xq, wq, x_scale, w_scale, m, n, k, y, ldy, vec_ok);
            else
                k_gemm_skinny_cb<4, false, false, 4><<<grid, dim3(256), 0, st>>>(
                    xq, wq, x_scale, w_scale, m, n, k, y, ldy, vec_ok);
        }
        return hipGetLastError();
    }
    if (M > 64) {
        const int tiles_m = (m + T_BM - 1) / T_BM;
        // 256 x 256 tiles (8-bit weights) where their rounds of 256 CUs cost
        // less: one takes ~1.8-1.9 times a 256 x 128 tile on a CU (measured
        // at 4096^3 and 8192 x 8192 -> 24576)
        const int64_t narrow = (int64_t)tiles_m * ((n + T_BN - 1) / T_BN);
        const int64_t wide = (int64_t)tiles_m * ((n + W_BN - 1) / W_BN);
        if (!W4 && 9 * ((wide + 255) / 256) < 5 * ((narrow + 255) / 256)) {
            const int tiles_n = (n + W_BN - 1) / W_BN;
            const dim3 grid((unsigned)(tiles_m * tiles_n));
            if (f16)
                k_gemm_wide<true><<<grid, dim3(64 * T_WAVES), 0, st>>>(
                    xq, wq, x_scale, w_scale, m, n, k, y, ldy, tiles_m, tiles_n, vec_ok);
            else
                k_gemm_wide<false><<<grid, dim3(64 * T_WAVES), 0, st>>>(
                    xq, wq, x_scale, w_scale, m, n, k, y, ldy, tiles_m, tiles_n, vec_ok);
            return hipGetLastError();
        }
        const int tiles_n = (n + T_BN - 1) / T_BN;
        const dim3 grid((unsigned)(tiles_m * tiles_n));
        if (f16)
            k_gemm_tile<true, W4><<<grid, dim3(64 * T_WAVES), 0, st>>>(
                xq, wq, x_scale, w_scale, m, n, k, y, ldy, tiles_m, tiles_n, vec_ok);
        else
            k_gemm_tile<false, W4><<<grid, dim3(64 * T_WAVES), 0, st>>>(
                xq, wq, x_scale, w_scale, m, n, k, y, ldy, tiles_m, tiles_n, vec_ok);
        return hipGetLastError();
    }
    const int64_t nblk = (n + 15) / 16;
    const int cb = decode_blocks(W4, m, nblk);
    const dim3 grid((unsigned)((nblk + cb - 1) / cb));
#define SQ_SK(MB)                                                                               \
    do {                                                                                        \
        if (f16) launch_skinny<MB, true, W4>(cb, grid, st, xq, wq, x_scale, w_scale, m, n, k, y, \
                                             ldy, vec_ok);                                      \
        else launch_skinny<MB, false, W4>(cb, grid, st, xq, wq, x_scale, w_scale, m, n, k, y,   \
                                          ldy, vec_ok);                                         \
    } while (0)
    const int64_t mb = (M + 15) / 16;
    if (mb == 1) SQ_SK(1);
    else if (mb == 2) SQ_SK(2);
    else if (mb == 3) SQ_SK(3);
    else SQ_SK(4);
#undef SQ_SK
    return hipGetLastError();
}

hipError_t launch_gemm(const int8_t *xq, const float *x_scale, const int8_t *wq,
                       const float *w_scale, int64_t M, int64_t N, int64_t K, void *y,
                       int64_t ldy, int out_kind, hipStream_t st) {
    return launch_gemm_any<false>(xq, x_scale, wq, w_scale, M, N, K, y, ldy, out_kind, st);
}

hipError_t launch_gemm_w4(const int8_t *xq, const float *x_scale, const uint8_t *wq4,
                          const float *w_scale, int64_t M, int64_t N, int64_t K, void *y,
                          int64_t ldy, int out_kind, hipStream_t st) {
    return launch_gemm_any<true>(xq, x_scale, reinterpret_cast<const int8_t *>(wq4), w_scale, M,
                                 N, K, y, ldy, out_kind, st);
}

}  // namespace sq
