/*
 * sq.h -- C ABI of the MI355X (gfx950) SmoothQuant-smoothed W8A8 linear layer
 *
 *     Y = (X S^-1)(S W)
 *
 * X is tokens x input channels, W is input channels x output channels and S is
 * a positive diagonal over the input channels, so the product equals X W in
 * exact arithmetic ("Move activation scale without changing the real linear
 * map", para. 1).  The factors come from calibration statistics, the weights
 * are folded and quantized offline, and at serving time the activations are
 * quantized per token and multiplied on int8 matrix cores (SmoothQuant
 * glossary entry: W8A8, factors from calibration statistics; "Quantization",
 * learn-kernels.com, para. 2: both operands int8, transform applied offline).
 *
 * Conventions for every call:
 *   - All array arguments are caller-owned DEVICE pointers on the current HIP
 *     device (for instance a torch tensor's data_ptr()).  The library never
 *     allocates, frees or keeps them.
 *   - Matrices are row-major; "ld" arguments are row strides in elements.
 *   - fp16 data is IEEE binary16 passed as raw bits (const void*).
 *   - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *     Work is enqueued on that stream; only the calls that compute smoothing
 *     factors (the two folds and sq_smoothing_factors) wait, for s.
 *   - Every argument is checked before any HIP call or any write: a call that
 *     returns an argument error (SQ_ERR_NULL, _SHAPE, _ALIGN, _ALPHA, _KIND,
 *     _EPS) has no side effects.
 *   - Shape limits: sizes >= 0 (a zero token/output count is a no-op); K is a
 *     multiple of 16 with 16 <= K <= SQ_MAX_K, so that every int32 sum of K
 *     int8 products is exact; M, N, T < 2^31; ld >= the row length used.
 *   - Alignment: every input pointer 16-byte aligned and fp16 input strides
 *     multiples of 8 (whole 16-byte row chunks); the product's output y only
 *     needs its element alignment, with any stride ldy >= N.
 *   - Stateless and reentrant: calls on different streams may run
 *     concurrently; calls that write the same buffers must be ordered by the
 *     caller.
 *
 * Packed int8 operands.  The int8 codes of activations (xq) and folded
 * weights (wq) are stored in the operand order of the gfx950 int8 matrix
 * instruction (v_mfma_i32_16x16x64_i8), so that every 16-row x 64-byte
 * fragment is one contiguous, naturally aligned 1 KiB run:
 *   for a code matrix R[rows][K] (K % 16 == 0), KW = ceil(K / 64),
 *   element R[r][k] lives at byte
 *       ((r / 16) * KW + k / 64) * 1024 + ((k % 64) / 16) * 256 + (r % 16) * 16 + k % 16
 *   and the buffer holds sq_packed_bytes(rows, K) = ceil(rows / 16) * KW * 1024
 *   bytes.  Padding bytes (rows >= `rows` of the last row block, k >= K of the
 *   last window) must be zero; the library's producers write them as zero.
 * sq_pack_i8 / sq_unpack_i8 convert between this layout and row-major codes.
 *
 * Packed 4-bit weights (sq_w4_fold_weights, sq_w4_gemm) use the same fragment
 * order at half the size: codes in [-8, 7] as two's-complement nibbles, each
 * fragment 512 bytes, the lane chunk of 16 codes (k % 64 / 16 = quarter,
 * r % 16 = row, as above) 8 bytes at ((r / 16) * KW + k / 64) * 512 +
 * ((k % 64) / 16) * 128 + (r % 16) * 8; code i = k % 16 of the chunk in byte
 * (i % 4) + 4 * (i / 8), low nibble for i % 8 < 4, high nibble otherwise.
 * sq_packed4_bytes(rows, K) = ceil(rows / 16) * KW * 512 bytes; padding zero.
 */
#ifndef SQ_H
#define SQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SQ_OK = 0,
    SQ_ERR_NULL = 1,       /* a required pointer is NULL                          */
    SQ_ERR_SHAPE = 2,      /* a size or stride is out of range                    */
    SQ_ERR_ALIGN = 3,      /* a pointer or stride breaks the alignment rules      */
    SQ_ERR_ALPHA = 4,      /* alpha is not in [0, 1] (or is NaN)                  */
    SQ_ERR_NONFINITE = 5,  /* fold: a statistic or given factor is NaN, infinite
                              or negative                                        */
    SQ_ERR_RANGE = 6,      /* fold: a factor or its reciprocal is zero, infinite
                              or subnormal in float                              */
    SQ_ERR_HIP = 7,        /* the HIP runtime reported an error                   */
    SQ_ERR_KIND = 8,       /* unknown out_kind                                    */
    SQ_ERR_EPS = 9         /* eps is negative, NaN or infinite                    */
} sq_status;

/* Output kinds of sq_w8a8_gemm. */
enum {
    SQ_OUT_F16 = 0,        /* y fp16 = round_to_nearest_even((acc * x_scale[m]) * w_scale[n]) */
    SQ_OUT_I32 = 1         /* y int32 = acc, the raw integer sums                              */
};

/* Largest K: 131056 * 128 * 128 < 2^31, so int32 sums of any int8 codes are exact. */
#define SQ_MAX_K 131056

/* Bytes of a packed int8 operand with `rows` rows of K codes (0 when an
 * argument is out of range). */
int64_t sq_packed_bytes(int64_t rows, int64_t K);

/* Human-readable name of a status code (static string, never NULL). */
const char *sq_status_str(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int sq_version(void);

/*
 * Calibration statistics (offline).
 * The per-input-channel activation maximum max|X_j| that the smoothing factor
 * divides by (Pith review of arXiv 2506.01967, key machinery, Eq. 4), taken
 * over calibration tokens (SmoothQuant glossary: a small representative
 * dataset estimates the activation statistics).
 *
 *   x_cal       fp16 [T][ldx], T calibration tokens of K channels
 *   act_absmax  float [K], written: act_absmax[j] = max_t |x_cal[t][j]|;
 *               with accumulate != 0 the previous contents take part in the
 *               maximum (stream the calibration set batch by batch; the
 *               previous values must be >= 0 or NaN).  A NaN in a column makes
 *               its entry NaN, an infinity makes it +inf; sq_smooth_fold_weights
 *               rejects both.  T == 0 writes zeros (accumulate == 0) or leaves
 *               the buffer unchanged (accumulate != 0).
 * Asynchronous.
 */
sq_status sq_calibrate_absmax(const void *x_cal_f16, int64_t T, int64_t K, int64_t ldx,
                              float *act_absmax, int accumulate, void *stream);

/*
 * Smoothing factors and the offline fold of S into W (offline; waits for s).
 * s_j = act_absmax[j]^alpha / max_n|W[j][n]|^(1 - alpha), evaluated in double
 * and rounded once to float (alpha = 1/2 is the Pith review's
 * s_j = sqrt(max|X_j| / max|W_j|)); a channel whose activation or weight
 * statistic is 0 takes s_j = 1.  Row j of W (input channel j) is multiplied
 * by s_j, the compensation for dividing activation channel j by s_j ("Move
 * activation scale ...", para. 1); the result is quantized symmetrically per
 * output channel n to int8 with round-half-even:
 *   Wt[j][n]   = float(W[j][n]) * s_j
 *   w_scale[n] = max_j |Wt[j][n]| / 127
 *   wq[n][j]   = clamp(rint(Wt[j][n] * (127 / max_j|Wt[j][n]|)), -127, 127)
 * (an all-zero column gets scale 0 and codes 0; where 127 / max overflows, a
 * column maximum below 127 / FLT_MAX from a caller's tiny smooth_in, nonzero
 * values get +-127 and zeros 0).
 *
 *   w           fp16 [K][ldw], N output channels used per row
 *   act_absmax  float [K] from sq_calibrate_absmax; ignored when smooth_in != NULL
 *   alpha       migration strength in [0, 1]; ignored when smooth_in != NULL
 *   smooth_in   NULL, or float [K] of given factors (e.g. a factor vector shared
 *               by several consumers of one activation, "Move activation scale
 *               ...", para. 3); used as s as is
 *   smooth_out      float [K], written: s
 *   inv_smooth_out  float [K], written: 1.0f / s  (the input of
 *                   sq_quant_act_per_token)
 *   wq          int8, packed (sq_packed_bytes(N, K) bytes), written: the folded
 *               codes wq[n][j], padding zero
 *   w_scale     float [N], written
 * Several consumers of one activation: pass their weights side by side as one
 * K x (N1 + N2 + ...) matrix (ldw = total), so s uses the maximum over all of
 * them and each consumer's codes and scales are contiguous slices; or fold
 * each one with smooth_in set to the shared s.  Both give identical codes.
 *
 * The call queues all its work on the stream, then waits once, until s has
 * reached the host, and checks the statistics and factors there while the
 * rest of the fold runs on; on return the outputs are complete in stream order
 * (like the other calls).  Data errors: SQ_ERR_NONFINITE when a statistic (or
 * a smooth_in entry) is NaN, infinite or negative; SQ_ERR_RANGE when a factor
 * or its reciprocal is zero, infinite or subnormal.  On a data error all four
 * outputs hold unspecified values (the kernels stay in bounds whatever the
 * values).  Per (thread, device) the library keeps, from the first call on
 * and grown as needed, a pinned host buffer of 4*K bytes for this check, a
 * device scratch of 4*N bytes for the column maxima and an event; a call on
 * another stream than the same thread's previous call first waits until the
 * device is idle.
 */
sq_status sq_smooth_fold_weights(const void *w_f16, int64_t K, int64_t N, int64_t ldw,
                                 const float *act_absmax, float alpha, const float *smooth_in,
                                 float *smooth_out, float *inv_smooth_out,
                                 int8_t *wq, float *w_scale, void *stream);

/* Largest N that sq_smooth_fold_weights_noalloc takes: its column maxima live
 * in a fixed device array of SQ_NOALLOC_MAX_N floats (512 KiB) per GPU. */
#define SQ_NOALLOC_MAX_N 131072

/*
 * sq_smooth_fold_weights for callers that cannot allocate device or pinned
 * host memory (code under stream capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, outputs, argument checks and data
 * errors as sq_smooth_fold_weights; additionally SQ_ERR_SHAPE when
 * N > SQ_NOALLOC_MAX_N (nothing is launched).  The call allocates nothing:
 * the column maxima and a status word live in a file-scope device array of
 * the library (one per GPU, held until the process ends, its address looked
 * up once per device), the factors are checked on the device, and the call
 * copies 4 bytes of status to the host and waits for the whole stream before
 * it returns.  Every call on one GPU shares that array: calls that overlap on
 * one GPU (other threads or streams) race and must be serialized by the
 * caller.
 */
sq_status sq_smooth_fold_weights_noalloc(const void *w_f16, int64_t K, int64_t N, int64_t ldw,
                                         const float *act_absmax, float alpha,
                                         const float *smooth_in, float *smooth_out,
                                         float *inv_smooth_out, int8_t *wq, float *w_scale,
                                         void *stream);

/*
 * The smoothing factors alone, without the 8-bit fold: s and 1/s exactly as
 * sq_smooth_fold_weights computes them (same formula, same checks, same
 * per (thread, device) host buffer and one wait), for a caller that folds S
 * into W in another form (the 4-bit calls below).  N == 0 takes every weight
 * statistic as 0 (s_j = 1).  Data errors as in sq_smooth_fold_weights.
 */
sq_status sq_smoothing_factors(const void *w_f16, int64_t K, int64_t N, int64_t ldw,
                               const float *act_absmax, float alpha, float *smooth_out,
                               float *inv_smooth_out, void *stream);

/*
 * Per-token dynamic activation quantization with the 1/s scaling fused in,
 * instead of a separate runtime scaling kernel ("Move activation scale ...",
 * para. 3).  Per token m, in float:
 *   xt[j]      = float(x[m][j]) * inv_smooth[j]
 *   x_scale[m] = max_j |xt[j]| / 127
 *   xq[m][j]   = clamp(rint(xt[j] * (127 / max_j|xt[j]|)), -127, 127)
 * An all-zero row gets scale 0 and codes 0; a row with a non-finite xt gets
 * scale NaN and codes 0 (so its outputs are NaN).  A row whose maximum is
 * below 127 / FLT_MAX (possible only with a caller's 1/s far below the fold's
 * range) makes the float 127 / max infinite: its nonzero values get +-127 and
 * its zeros 0.
 *
 *   x           fp16 [M][ldx]
 *   inv_smooth  float [K] (inv_smooth_out of the fold)
 *   xq          int8, packed (sq_packed_bytes(M, K) bytes), written: the codes
 *               xq[m][j], padding zero
 *   x_scale     float [M], written
 * Asynchronous.
 */
sq_status sq_quant_act_per_token(const void *x_f16, int64_t M, int64_t K, int64_t ldx,
                                 const float *inv_smooth, int8_t *xq, float *x_scale,
                                 void *stream);

/*
 * The division by s folded into the RMS normalization in front of the layer
 * (offline part).  The inverse factors may be folded into the operation that
 * produces the activation instead of being applied at run time ("Move
 * activation scale ...", para. 3); for a root-mean-square normalization
 *   xbar[m][j] = h[m][j] * rstd_m * gamma[j],  rstd_m = 1 / sqrt(mean_j h[m][j]^2 + eps)
 * that means replacing its weight gamma by gamma / s:
 *   gamma_out[j] = float(gamma[j]) * inv_smooth[j]
 * Legal only when every consumer of the normalization's output is folded with
 * this same s (same paragraph): fold them together as one K x (N1 + N2 + ...)
 * matrix, or each with smooth_in = s.  A consumer that needs the unsmoothed
 * activation cannot read the folded normalization's output.
 *
 *   gamma       fp16 [K], the normalization weight
 *   inv_smooth  float [K] (inv_smooth_out of the fold)
 *   gamma_out   float [K], written
 * Asynchronous.
 */
sq_status sq_fold_norm_weight(const void *gamma_f16, int64_t K, const float *inv_smooth,
                              float *gamma_out, void *stream);

/*
 * RMS normalization with the folded weight and per-token int8 quantization in
 * one pass over the hidden state (serving time): the normalized activation
 * X S^-1 is never written to memory.  Per token m, in float:
 *   xt[j]      = float(h[m][j]) * gamma_folded[j]
 *   xq[m][j]   = clamp(rint(xt[j] * (127 / max_j|xt[j]|)), -127, 127)
 *   x_scale[m] = float(max_j|xt[j]| * rstd_m / 127), evaluated in double
 * with rstd_m from the sum of squares of the row (summed in double; every
 * square of an fp16 value is exact), so x_scale is within one float rounding
 * of its value for the exact sum.  The codes do not depend on rstd_m (a
 * positive per-token factor), so they are exactly sq_quant_act_per_token's
 * codes of h with inv_smooth = gamma_folded (the same rule for a row whose
 * float 127 / max overflows).  An all-zero row gets scale 0 and codes 0; a row
 * with a non-finite xt gets scale NaN and codes 0.
 *
 *   h             fp16 [M][ldh], the normalization's input (hidden state)
 *   gamma_folded  float [K] from sq_fold_norm_weight
 *   eps           the normalization's epsilon, finite and >= 0 (else SQ_ERR_EPS)
 *   xq            int8, packed (sq_packed_bytes(M, K) bytes), written, padding zero
 *   x_scale       float [M], written
 * The outputs go to sq_w8a8_gemm exactly as sq_quant_act_per_token's do.
 * Asynchronous.
 */
sq_status sq_rmsnorm_quant_per_token(const void *h_f16, int64_t M, int64_t K, int64_t ldh,
                                     const float *gamma_folded, float eps, int8_t *xq,
                                     float *x_scale, void *stream);

/*
 * Smooth Rotation at 4 bits (Pith review of arXiv 2506.01967: key machinery,
 * scale the channels and then multiply activations and weights by the same
 * Hadamard matrix; core discovery, 4-bit symmetric round-to-nearest on both).
 * The rotation R = H / sqrt(K) uses the Sylvester matrix
 * H[i][j] = (-1)^popcount(i & j), so (X S^-1 R)(R S W) = X W.  The calls apply
 * the unnormalized H by the fast transform in float (strides 1, 2, 4, ...,
 * K/2 in that order, each butterfly (a + b, a - b)), and the two factors
 * 1/sqrt(K) go into the weight scale as one exact 1/K.  With rotate == 0 the
 * same calls quantize to 4 bits without the transform (smoothing alone, or
 * S = I with smooth = ones: the other columns of the paper's comparison).
 * Activation codes are 4-bit values in [-7, 7] stored one per byte in the
 * packed int8 layout; weight codes two per byte in the packed 4-bit layout,
 * which sq_w4_gemm widens to int8 in registers (half the weight bytes).
 * Shapes: 16 <= K <= 8192, K % 16 == 0, and K a power of two when rotated
 * (SQ_ERR_SHAPE otherwise).
 */

/* Bytes of a packed 4-bit operand (0 when an argument is out of range). */
int64_t sq_packed4_bytes(int64_t rows, int64_t K);

/* Bytes of workspace sq_w4_fold_weights needs: 2 * K * N + sq_packed_bytes(N, K)
 * (0 when out of range). */
int64_t sq_w4_workspace_bytes(int64_t K, int64_t N);

/*
 * Offline: per output channel n, v = H (s * W[:, n]) (or s * W[:, n]), then
 *   w_scale[n] = (max_j |v_j| / 7) * (rotate ? 1/K : 1)
 *   wq[n][j]   = clamp(rint(v_j * (7 / max_j |v_j|)), -7, 7)
 * (products float(W) * s in float; a zero channel gets scale 0 and codes 0, a
 * non-finite value scale NaN and codes 0; where 7 / max overflows, nonzero
 * values get +-7 and zeros 0).
 *   w          fp16 [K][ldw]
 *   smooth     float [K] (s from sq_smoothing_factors, or ones for S = I)
 *   wq4        packed 4-bit, sq_packed4_bytes(N, K) bytes, written, padding zero
 *   w_scale    float [N], written
 *   workspace  device buffer of sq_w4_workspace_bytes(K, N) bytes, 16-byte
 *              aligned, caller-owned: W transposed, then the codes one per
 *              byte; its contents afterwards are unspecified
 * Asynchronous.
 */
sq_status sq_w4_fold_weights(const void *w_f16, int64_t K, int64_t N, int64_t ldw,
                             const float *smooth, int rotate, uint8_t *wq4, float *w_scale,
                             void *workspace, void *stream);

/*
 * Serving time: per token m, v = (float(x[m][j]) * inv_smooth[j]) H (or
 * without H), then
 *   x_scale[m] = max_j |v_j| / 7
 *   xq[m][j]   = clamp(rint(v_j * (7 / max_j |v_j|)), -7, 7)
 * (all-zero token: scale 0, codes 0; a non-finite value: scale NaN, codes 0;
 * where 7 / max overflows, a maximum of at most 2^-126, nonzero values get +-7
 * and zeros 0).
 *   x        fp16 [M][ldx]
 *   xq       packed int8, sq_packed_bytes(M, K) bytes, written, padding zero
 *   x_scale  float [M], written
 * Asynchronous.
 */
sq_status sq_a4_quant_per_token(const void *x_f16, int64_t M, int64_t K, int64_t ldx,
                                const float *inv_smooth, int rotate, int8_t *xq, float *x_scale,
                                void *stream);

/*
 * The product with 4-bit weights: as sq_w8a8_gemm, with wq4 in the packed
 * 4-bit layout (codes widened to int8 in registers before the int8 matrix
 * instruction, so the sums and the epilogue are exactly sq_w8a8_gemm's for
 * the same codes).  xq holds int8 codes (sq_a4_quant_per_token's 4-bit ones,
 * or any int8).  Asynchronous.
 */
sq_status sq_w4_gemm(const int8_t *xq, const float *x_scale, const uint8_t *wq4,
                     const float *w_scale, int64_t M, int64_t N, int64_t K, void *y,
                     int64_t ldy, int out_kind, void *stream);

/*
 * The W8A8 product on int8 matrix cores with a fused dequantizing epilogue
 * ("Quantization", learn-kernels.com, para. 2: both operands int8, run on the
 * low-precision hardware path):
 *   acc[m][n] = sum_j xq[m][j] * wq[n][j]        (exact int32)
 *   SQ_OUT_F16: y[m][n] = fp16_rne((float(acc) * x_scale[m]) * w_scale[n])
 *   SQ_OUT_I32: y[m][n] = acc                     (x_scale, w_scale may be NULL)
 *
 *   xq       int8 packed codes of M tokens (sq_quant_act_per_token's output)
 *   wq       int8 packed codes of N output channels (the fold's output)
 *   y        fp16 or int32 [M][ldy]
 * Asynchronous.
 */
sq_status sq_w8a8_gemm(const int8_t *xq, const float *x_scale, const int8_t *wq,
                       const float *w_scale, int64_t M, int64_t N, int64_t K,
                       void *y, int64_t ldy, int out_kind, void *stream);

/*
 * Layout helpers (not part of the layer's arithmetic): row-major int8 codes
 * src[rows][ld] -> packed dst (padding written as zero), and back.  For
 * callers that hold codes in row-major order.  Asynchronous.
 */
sq_status sq_pack_i8(const int8_t *src, int64_t rows, int64_t K, int64_t ld, int8_t *dst,
                     void *stream);
sq_status sq_unpack_i8(const int8_t *src, int64_t rows, int64_t K, int8_t *dst, int64_t ld,
                       void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SQ_H */
