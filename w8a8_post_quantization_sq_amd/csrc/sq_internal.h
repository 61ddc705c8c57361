// Library-internal declarations shared by the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sq {

// ---- launchers (one per kernel family) -------------------------------------

hipError_t launch_fill_f32(float *p, int64_t n, float v, hipStream_t st);

// accumulate == 0: ax = the maximum (zeros for T == 0); else ax = max(ax, it)
hipError_t launch_calib_absmax(const uint16_t *x, int64_t T, int64_t K, int64_t ldx,
                               float *ax, int accumulate, hipStream_t st);

// aw_j = max_n |W[j][n]| -> s_out[j] = s_j (also into s_host when not NULL,
// a device-visible host buffer), inv_out[j] = 1/s_j; zeroes amax[0, N) when
// amax is not NULL; when status is not NULL, ORs into it 1 for a NaN factor
// and 2 for a factor or reciprocal that is not a positive normal float
hipError_t launch_row_smooth(const uint16_t *w, int64_t K, int64_t N, int64_t ldw,
                             const float *ax, const float *smooth_in, float alpha, float *s_out,
                             float *inv_out, float *s_host, float *amax, uint32_t *status,
                             hipStream_t st);

// device addresses, on device `dev`, of the allocation-free fold's scratch:
// SQ_NOALLOC_MAX_N floats of column maxima and one status word
hipError_t noalloc_scratch(int dev, float **amax, uint32_t **status);

// amax[n] = max(amax[n], max_j |float(W[j][n]) * s_j|)
hipError_t launch_fold_colabsmax(const uint16_t *w, int64_t K, int64_t N, int64_t ldw,
                                 const float *s, float *amax, hipStream_t st);

// packed codes of W * s against amax; w_scale[n] = amax[n] / 127
hipError_t launch_fold_quant(const uint16_t *w, int64_t K, int64_t N, int64_t ldw,
                             const float *s, const float *amax, int8_t *wq, float *w_scale,
                             hipStream_t st);

hipError_t launch_quant_act(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                            const float *inv_s, int8_t *xq, float *x_scale, hipStream_t st);

// the same quantizer on the hidden state h with the folded norm weight g:
// the scale takes the token's rstd = 1 / sqrt(sum h^2 / K + eps)
hipError_t launch_rmsnorm_quant(const uint16_t *h, int64_t M, int64_t K, int64_t ldh,
                                const float *g, float eps, int8_t *xq, float *x_scale,
                                hipStream_t st);

// g[j] = float(gamma[j]) * inv_s[j]
hipError_t launch_fold_norm_weight(const uint16_t *gamma, int64_t K, const float *inv_s, float *g,
                                   hipStream_t st);

// the per-token quantizer at 7 levels: 4-bit codes of x * mult, scale = max / 7
hipError_t launch_quant4_plain(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                               const float *mult, int8_t *q, float *scale, hipStream_t st);

// 4-bit quantization of rows (x * mult, rotated by the Sylvester Hadamard
// matrix when rotate != 0), codes packed as int8, scale = (max / 7) * post
hipError_t launch_quant4_rows(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                              const float *mult, int rotate, float post, int8_t *q, float *scale,
                              hipStream_t st);

// 4-bit weights: W transposed into the workspace (N x K fp16), its rows
// quantized with mult = s (and post = 1/K when rotated) into the workspace's
// second part (packed int8 order), then packed two codes per byte into wq4
hipError_t launch_fold4(const uint16_t *w, int64_t K, int64_t N, int64_t ldw, const float *s,
                        int rotate, uint8_t *wq4, float *w_scale, uint8_t *work, hipStream_t st);

// packed int8 codes in [-8, 7] -> packed 4-bit codes
hipError_t launch_pack4_from8(const int8_t *src, int64_t rows, int64_t K, uint8_t *dst,
                              hipStream_t st);

// the product with 4-bit weights (packed two per byte), widened to int8 in
// registers; everything else as launch_gemm
hipError_t launch_gemm_w4(const int8_t *xq, const float *x_scale, const uint8_t *wq4,
                          const float *w_scale, int64_t M, int64_t N, int64_t K, void *y,
                          int64_t ldy, int out_kind, hipStream_t st);

hipError_t launch_pack_i8(const int8_t *src, int64_t rows, int64_t K, int64_t ld, int8_t *dst,
                          hipStream_t st);

hipError_t launch_unpack_i8(const int8_t *src, int64_t rows, int64_t K, int8_t *dst, int64_t ld,
                            hipStream_t st);

hipError_t launch_gemm(const int8_t *xq, const float *x_scale, const int8_t *wq,
                       const float *w_scale, int64_t M, int64_t N, int64_t K, void *y,
                       int64_t ldy, int out_kind, hipStream_t st);

}  // namespace sq
