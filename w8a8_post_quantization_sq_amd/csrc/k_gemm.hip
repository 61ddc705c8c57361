// The W8A8 product on CDNA4 int8 matrix cores with a fused dequantizing epilogue.
//
//   acc[m][n] = sum_j xq[m][j] * wq[n][j]        (exact int32)
//   y[m][n]   = fp16_rne((float(acc) * x_scale[m]) * w_scale[n])
//
// Both operands are int8, so the product runs on the low-precision matrix
// path ("Quantization", learn-kernels.com, para. 2: W8A8 lets the matrix
// multiply itself use faster low-precision hardware, not only save traffic).
//
// Both operands are K-contiguous (xq [M][K], wq [N][K]), which is the natural
// operand layout of v_mfma_i32_32x32x32_i8: lane l supplies 16 bytes of row
// (l % 32) of the A block and 16 bytes of column (l % 32) of the B block, the
// two lane halves covering the two 16-byte halves of the 32-deep k slice.
// The accumulator of lane l holds column l % 32 and rows
// 8 * (r / 4) + 4 * (l / 32) + r % 4, r = 0..15.  Integer sums do not depend
// on the order of the k terms, so any k permutation that A and B share gives
// the same exact result.
//
// Workgroup: 256 threads = 4 waves in a 2 x 2 grid, output tile BM x BN,
// k step 64 bytes.  Tiles of both operands pass through LDS, double-buffered
// (one barrier per k step); the next step's tiles are fetched into registers
// while the matrix cores work on the current one.  LDS rows are padded from
// 64 to 80 bytes so the 8 lanes of a 16-byte LDS read phase hit disjoint banks.
#include "sq_device.h"
#include "sq.h"

namespace sq {

constexpr int G_BK = 64;
constexpr int G_LDS_PITCH = G_BK + 16;

template <int BM, int BN, bool F16OUT>
__global__ void __launch_bounds__(256)
k_gemm_w8a8(const int8_t *__restrict__ A, const int8_t *__restrict__ B,
            const float *__restrict__ xs, const float *__restrict__ ws, int M, int N, int K,
            void *__restrict__ Y, int64_t ldy) {
    constexpr int WM = BM / 2, WN = BN / 2;      // wave tile
    constexpr int FM = WM / 32, FN = WN / 32;    // 32 x 32 blocks per wave
    constexpr int A_LD = BM * 4 / 256;           // 16-byte chunks per thread per k step
    constexpr int B_LD = BN * 4 / 256;
    static_assert(A_LD >= 1 && B_LD >= 1 && FM >= 1 && FN >= 1, "tile too small");
    __shared__ __align__(16) int8_t lds[2][(BM + BN) * G_LDS_PITCH];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int tiles_n = (N + BN - 1) / BN;
    const int m0 = (int)(blockIdx.x / tiles_n) * BM;
    const int n0 = (int)(blockIdx.x % tiles_n) * BN;

    v16i acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    v4i ra[A_LD], rb[B_LD];
    const v4i zero4 = {0, 0, 0, 0};
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_LD; ++i) {
            const int idx = tid + i * 256;
            const int row = idx >> 2, kk = k0 + (idx & 3) * 16;
            const int gm = m0 + row;
            ra[i] = (gm < M && kk < K)
                        ? *reinterpret_cast<const v4i *>(A + (int64_t)gm * K + kk)
                        : zero4;
        }
#pragma unroll
        for (int i = 0; i < B_LD; ++i) {
            const int idx = tid + i * 256;
            const int row = idx >> 2, kk = k0 + (idx & 3) * 16;
            const int gn = n0 + row;
            rb[i] = (gn < N && kk < K)
                        ? *reinterpret_cast<const v4i *>(B + (int64_t)gn * K + kk)
                        : zero4;
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_LD; ++i) {
            const int idx = tid + i * 256;
            *reinterpret_cast<v4i *>(&lds[buf][(idx >> 2) * G_LDS_PITCH + (idx & 3) * 16]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_LD; ++i) {
            const int idx = tid + i * 256;
            *reinterpret_cast<v4i *>(&lds[buf][(BM + (idx >> 2)) * G_LDS_PITCH + (idx & 3) * 16]) =
                rb[i];
        }
    };

    const int nk = (K + G_BK - 1) / G_BK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * G_BK);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int chunk = ks * 2 + (lane >> 5);
            v4i af[FM], bf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *reinterpret_cast<const v4i *>(
                    &lds[cur][(wm * WM + i * 32 + (lane & 31)) * G_LDS_PITCH + chunk * 16]);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bf[j] = *reinterpret_cast<const v4i *>(
                    &lds[cur][(BM + wn * WN + j * 32 + (lane & 31)) * G_LDS_PITCH + chunk * 16]);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) lstore(cur ^ 1);
        __syncthreads();
    }

    // epilogue: lane holds column (lane % 32) of each 32 x 32 block
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn * WN + j * 32 + (lane & 31);
        if (col >= N) continue;
        const float wsc = F16OUT ? ws[col] : 0.0f;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * WM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                if (row >= M) continue;
                if (F16OUT) {
                    const float y = ((float)acc[i][j][r] * xs[row]) * wsc;
                    reinterpret_cast<uint16_t *>(Y)[(int64_t)row * ldy + col] = f2h_bits(y);
                } else {
                    reinterpret_cast<int32_t *>(Y)[(int64_t)row * ldy + col] = acc[i][j][r];
                }
            }
        }
    }
}

hipError_t launch_gemm(const int8_t *xq, const float *x_scale, const int8_t *wq,
                       const float *w_scale, int64_t M, int64_t N, int64_t K, void *y,
                       int64_t ldy, int out_kind, hipStream_t st) {
    if (M <= 0 || N <= 0) return hipSuccess;
    constexpr int BM = 128, BN = 128;
    const dim3 grid((unsigned)(((N + BN - 1) / BN) * ((M + BM - 1) / BM)));
    if (out_kind == SQ_OUT_F16)
        k_gemm_w8a8<BM, BN, true><<<grid, dim3(256), 0, st>>>(xq, wq, x_scale, w_scale, (int)M,
                                                               (int)N, (int)K, y, ldy);
    else
        k_gemm_w8a8<BM, BN, false><<<grid, dim3(256), 0, st>>>(xq, wq, x_scale, w_scale, (int)M,
                                                                (int)N, (int)K, y, ldy);
    return hipGetLastError();
}

}  // namespace sq
