/*
 * sq_oracle.c -- plain, slow CPU oracle for the SmoothQuant-smoothed W8A8
 * linear layer Y = (X S^-1)(S W).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library includes, links
 * or calls this file; only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark load it.  It shares no header, helper, table or
 * constant with the HIP path.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC.
 * No intrinsics, no vectorisation hints, rounding mode round-to-nearest-even.
 * On x86-64 every float operation below is a single IEEE-754 binary32
 * operation (SSE, no excess precision), so the op order written here is the
 * op order that is computed.
 *
 * Conventions (all row-major):
 *   X     fp16 bits [M][ldx]   tokens x input channels
 *   W     fp16 bits [K][ldw]   input channels x output channels
 *   Wq    int8      [N][K]     folded, quantized weights, K contiguous
 *   Xq    int8      [M][K]     quantized activations
 *   acc   int32     [M][N]
 *
 * Sources (pages the method is taken from):
 *   [P1] "Move activation scale without changing the real linear map"
 *        (study.greatitself.com, activation outliers and smoothing)
 *   [P2] SmoothQuant glossary entry (dataterminology.com)
 *   [P4] Pith review of arXiv 2506.01967 "Smooth Rotation"
 *   [P5] "Quantization" chapter (learn-kernels.com)
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes):
 *   - s_j = max|X_j|^alpha / max|W_j|^(1-alpha), evaluated in double and
 *     rounded once to float; alpha = 1/2 is [P4]'s key-machinery formula.
 *   - X is divided by s (multiplied by 1/s in float), row j of W (input
 *     channel j) is multiplied by s [P1 para. 1].
 *   - a zero statistic would make s zero or infinite, which [P1 para. 1]
 *     forbids; such a channel takes s = 1.
 *   - quantization is symmetric to [-127, 127] with round-half-even, per token
 *     for activations and per output channel for weights; scales are
 *     absmax/127 in float.
 *   - where the float multiplier 127/absmax overflows (a maximum below
 *     127/FLT_MAX), a zero value's code is 0 (code_of).
 *   - the int32 accumulator is exact for K < 133144.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ---- fp16 decoding ------------------------------------------------------ */

/* Exact value of an IEEE-754 binary16 bit pattern, as a float.  Every binary16
 * value is representable in binary32, so this conversion is exact. */
static float half_to_float(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);              /* zero and subnormals */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25);  /* 1.m * 2^(e-15) */
    return (float)(sign ? -v : v);
}

float oracle_half_to_float(uint16_t h) { return half_to_float(h); }

/* ---- A1: calibration statistics ---------------------------------------- */

/* ax[j] = max over the T calibration tokens of |X[t][j]|, the per-input-channel
 * activation maximum that the smoothing factor divides by ([P4] key machinery:
 * max|X_j|; [P2]: statistics from a small calibration set).  With accumulate,
 * the previous ax[j] takes part in the maximum, so batches can be streamed.
 * A NaN anywhere in a column (or in the previous ax[j]) makes ax[j] NaN. */
void oracle_calibrate_absmax(const uint16_t *x, int64_t T, int64_t K, int64_t ldx,
                             float *ax, int accumulate)
{
    for (int64_t j = 0; j < K; ++j) {
        float best = 0.0f;
        int nan = 0;
        if (accumulate) {
            if (isnan(ax[j])) nan = 1;
            else best = ax[j];
        }
        for (int64_t t = 0; t < T; ++t) {
            float v = half_to_float(x[t * ldx + j]);
            if (isnan(v)) { nan = 1; continue; }
            if (fabsf(v) > best) best = fabsf(v);
        }
        ax[j] = nan ? NAN : best;
    }
}

/* ---- A2: weight statistics and smoothing factors ----------------------- */

/* aw[j] = max over output channels n of |W[j][n]|: the maximum of weight row j,
 * i.e. of input channel j ([P4] key machinery: max|W_j|; W is in x out per
 * [P1 para. 1]).  NaN anywhere in the row gives NaN. */
void oracle_row_absmax(const uint16_t *w, int64_t K, int64_t N, int64_t ldw, float *aw)
{
    for (int64_t j = 0; j < K; ++j) {
        float best = 0.0f;
        int nan = 0;
        for (int64_t n = 0; n < N; ++n) {
            float v = half_to_float(w[j * ldw + n]);
            if (isnan(v)) { nan = 1; continue; }
            if (fabsf(v) > best) best = fabsf(v);
        }
        aw[j] = nan ? NAN : best;
    }
}

/* Smoothing factors.  [P4] key machinery gives s_j = sqrt(max|X_j| / max|W_j|)
 * (the paper's Eq. 4, strength 1/2); the general strength alpha weighs the two
 * statistics as max|X_j|^alpha / max|W_j|^(1-alpha), which is the same formula
 * at alpha = 1/2.  Evaluated in double, rounded once to float; inv_s is the
 * float reciprocal.  Returns 0 on success, 1 when a statistic is not finite
 * or negative, 2 when s or 1/s is not a finite normal float ([P1 para. 1]:
 * factors must be finite, nonzero and representable). */
int oracle_smoothing_factors(const float *ax, const float *aw, int64_t K, float alpha,
                             float *s, float *inv_s)
{
    const double a = (double)alpha;
    int status = 0;
    for (int64_t j = 0; j < K; ++j) {
        if (!isfinite(ax[j]) || !isfinite(aw[j]) || ax[j] < 0.0f || aw[j] < 0.0f) {
            s[j] = NAN;
            inv_s[j] = NAN;
            status = 1;
            continue;
        }
        float sj;
        if (ax[j] == 0.0f || aw[j] == 0.0f)
            sj = 1.0f;   /* dead channel or zero row: any positive s keeps Y; take 1 */
        else
            sj = (float)(pow((double)ax[j], a) / pow((double)aw[j], 1.0 - a));
        float ij = 1.0f / sj;
        s[j] = sj;
        inv_s[j] = ij;
        if (status == 0 && (!isnormal(sj) || !isnormal(ij)))
            status = 2;
    }
    return status;
}

/* ---- one code ------------------------------------------------------------ */

/* The code of a scaled value v with multiplier r = qmax / a (a the row's or
 * column's maximum |v|): clamp(rint(v * r), -qmax, qmax).  In float, r
 * overflows to infinity only for a maximum below qmax / FLT_MAX; then v * r
 * is +-inf for v != 0, which the clamp takes to +-qmax, and NaN for v == 0,
 * whose code is taken as 0, the code 0 * r has for every finite r. */
static int8_t code_of(float v, float r, float qmax)
{
    if (v == 0.0f) return 0;
    float q = rintf(v * r);
    if (q > qmax) q = qmax;
    if (q < -qmax) q = -qmax;
    return (int8_t)q;
}

/* ---- A3: fold S into W and quantize per output channel ------------------ */

/* Wt[j][n] = float(W[j][n]) * s[j]: row j of W takes the factor of input
 * channel j, which compensates X[:, j] / s[j] exactly in real arithmetic
 * ([P1 para. 1]; done offline before serving, [P5 para. 2]).
 * Per output channel n: amax = max_j |Wt[j][n]|, w_scale[n] = amax / 127,
 * r = 127 / amax, Wq[n][j] = clamp(rint(Wt[j][n] * r), -127, 127).
 * amax == 0 gives scale 0 and codes 0. */
void oracle_fold_quant_weights(const uint16_t *w, int64_t K, int64_t N, int64_t ldw,
                               const float *s, int8_t *wq, float *w_scale)
{
    for (int64_t n = 0; n < N; ++n) {
        float amax = 0.0f;
        for (int64_t j = 0; j < K; ++j) {
            float wt = half_to_float(w[j * ldw + n]) * s[j];
            if (fabsf(wt) > amax) amax = fabsf(wt);
        }
        if (amax == 0.0f) {
            w_scale[n] = 0.0f;
            for (int64_t j = 0; j < K; ++j) wq[n * K + j] = 0;
            continue;
        }
        float r = 127.0f / amax;
        w_scale[n] = amax / 127.0f;
        for (int64_t j = 0; j < K; ++j) {
            float wt = half_to_float(w[j * ldw + n]) * s[j];
            wq[n * K + j] = code_of(wt, r, 127.0f);
        }
    }
}

/* ---- A4: per-token dynamic activation quantization ---------------------- */

/* xt[m][j] = float(X[m][j]) * inv_s[j] -- the division by s applied where the
 * activation is quantized instead of in a separate scaling kernel ([P1 para.
 * 3]); xt stays in float.  Per token m: a = max_j |xt|, x_scale[m] = a / 127,
 * r = 127 / a, Xq[m][j] = clamp(rint(xt * r), -127, 127).  a == 0 gives scale
 * 0 and codes 0; a row holding a non-finite xt gets scale NaN and codes 0. */
void oracle_quant_act_per_token(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                                const float *inv_s, int8_t *xq, float *x_scale)
{
    for (int64_t m = 0; m < M; ++m) {
        float a = 0.0f;
        int bad = 0;
        for (int64_t j = 0; j < K; ++j) {
            float xt = half_to_float(x[m * ldx + j]) * inv_s[j];
            if (!isfinite(xt)) { bad = 1; continue; }
            if (fabsf(xt) > a) a = fabsf(xt);
        }
        if (bad || a == 0.0f) {
            x_scale[m] = bad ? NAN : 0.0f;
            for (int64_t j = 0; j < K; ++j) xq[m * K + j] = 0;
            continue;
        }
        float r = 127.0f / a;
        x_scale[m] = a / 127.0f;
        for (int64_t j = 0; j < K; ++j) {
            float xt = half_to_float(x[m * ldx + j]) * inv_s[j];
            xq[m * K + j] = code_of(xt, r, 127.0f);
        }
    }
}

/* ---- A5: integer matrix product ----------------------------------------- */

/* acc[m][n] = sum_j Xq[m][j] * Wq[n][j]: both operands int8 ([P2]: W8A8;
 * [P5 para. 2]: the product runs on low-precision hardware paths).  Summed in
 * int64 and stored as int32, which is exact whenever K * 127^2 < 2^31.
 * Returns the number of sums that did not fit int32 (0 for valid K). */
int64_t oracle_gemm_i32(const int8_t *xq, const int8_t *wq, int64_t M, int64_t N, int64_t K,
                        int32_t *acc)
{
    int64_t overflow = 0;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t t = 0;
            for (int64_t j = 0; j < K; ++j)
                t += (int64_t)xq[m * K + j] * (int64_t)wq[n * K + j];
            if (t > INT32_MAX || t < INT32_MIN) ++overflow;
            acc[m * N + n] = (int32_t)t;
        }
    }
    return overflow;
}

/* ---- A6: dequantization ------------------------------------------------- */

/* y[m][n] = acc[m][n] * x_scale[m] * w_scale[n], the value the two int8 codes
 * stand for.  Evaluated in double (relative error below 2^-52); the caller
 * rounds it once to the output precision. */
void oracle_dequant(const int32_t *acc, const float *x_scale, const float *w_scale,
                    int64_t M, int64_t N, double *y)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            y[m * N + n] = (double)acc[m * N + n] * (double)x_scale[m] * (double)w_scale[n];
}

/* The runtime layer (A4 + A5 + A6) on a block of tokens, for timing the
 * oracle as a CPU baseline.  Uses the functions above unchanged. */
void oracle_layer(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, const float *inv_s,
                  const int8_t *wq, const float *w_scale, int64_t N,
                  int8_t *xq_tmp, float *x_scale_tmp, int32_t *acc_tmp, double *y)
{
    oracle_quant_act_per_token(x, M, K, ldx, inv_s, xq_tmp, x_scale_tmp);
    oracle_gemm_i32(xq_tmp, wq, M, N, K, acc_tmp);
    oracle_dequant(acc_tmp, x_scale_tmp, w_scale, M, N, y);
}

/* ---- Next row: the division by s folded into the preceding RMS norm ----- */

/* The normalization in front of the layer, root-mean-square form (no mean
 * subtraction, no bias): for token m of the hidden state h,
 *     xbar[m][j] = h[m][j] * rstd_m * gamma[j],
 *     rstd_m     = 1 / sqrt((1/K) sum_j h[m][j]^2 + eps).
 * [P1 para. 3] allows the inverse factors to be folded into the operation that
 * precedes the layer, provided every consumer of its output receives the same
 * compensation.  Here that fold is gamma_j -> gamma_j / s_j, applied as the
 * float product g[j] = float(gamma[j]) * inv_s[j] (the same multiply by the
 * stored reciprocal that A4 uses). */
void oracle_fold_norm_weight(const uint16_t *gamma, int64_t K, const float *inv_s, float *g)
{
    for (int64_t j = 0; j < K; ++j)
        g[j] = half_to_float(gamma[j]) * inv_s[j];
}

/* sum_j h[j]^2 over K fp16 values, computed exactly and rounded once to
 * double.  |h| = i * 2^-24 for an integer i < 2^40 (i = m for subnormals,
 * (1024 + m) * 2^(e-1) otherwise), so h^2 = i^2 * 2^-48 and the sum is an
 * integer of at most 97 bits times 2^-48: it is summed in unsigned 128-bit
 * integers, converted to double (round to nearest even) and scaled by 2^-48
 * (exact).  A NaN element gives NaN, else an infinite one gives +inf. */
double oracle_row_sum_squares(const uint16_t *h, int64_t K)
{
    unsigned __int128 acc = 0;
    int nan = 0, inf = 0;
    for (int64_t j = 0; j < K; ++j) {
        int e = (h[j] >> 10) & 31;
        int m = h[j] & 1023;
        if (e == 31) {
            if (m) nan = 1;
            else inf = 1;
            continue;
        }
        uint64_t i = e ? (uint64_t)(m + 1024) << (e - 1) : (uint64_t)m;
        acc += (unsigned __int128)i * i;
    }
    if (nan) return NAN;
    if (inf) return INFINITY;
    return ldexp((double)acc, -48);
}

/* RMS normalization, the folded factors g = gamma / s and per-token int8
 * quantization in one step.  For token m:
 *     xt[j]      = float(h[m][j]) * g[j]            (float product)
 *     a          = max_j |xt[j]|
 *     Xq[m][j]   = clamp(rint(xt[j] * (127 / a)), -127, 127)
 *     x_scale[m] = float(a * rstd_m / 127)          (double, rounded once)
 * In exact arithmetic the codes of xbar / s = rstd_m * h * g do not depend on
 * the positive per-token factor rstd_m (it scales the token's maximum by the
 * same amount), so it enters the scale only.  rstd_m is taken in double from
 * the exact sum of squares.  a == 0 gives scale 0 and codes 0; a row holding
 * a non-finite xt gets scale NaN and codes 0 (as in A4). */
void oracle_rmsnorm_quant_per_token(const uint16_t *h, int64_t M, int64_t K, int64_t ldh,
                                    const float *g, float eps, int8_t *xq, float *x_scale)
{
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t *row = h + m * ldh;
        float a = 0.0f;
        int bad = 0;
        for (int64_t j = 0; j < K; ++j) {
            float xt = half_to_float(row[j]) * g[j];
            if (!isfinite(xt)) { bad = 1; continue; }
            if (fabsf(xt) > a) a = fabsf(xt);
        }
        if (bad || a == 0.0f) {
            x_scale[m] = bad ? NAN : 0.0f;
            for (int64_t j = 0; j < K; ++j) xq[m * K + j] = 0;
            continue;
        }
        double ms = oracle_row_sum_squares(row, K) / (double)K;
        double rstd = 1.0 / sqrt(ms + (double)eps);
        x_scale[m] = (float)((double)a * rstd / 127.0);
        float r = 127.0f / a;
        for (int64_t j = 0; j < K; ++j) {
            float xt = half_to_float(row[j]) * g[j];
            xq[m * K + j] = code_of(xt, r, 127.0f);
        }
    }
}

/* ---- Next row: Smooth Rotation, 4-bit ([P4]) ------------------------------ */

/* [P4] key machinery: after the diagonal scale, activations and weights are
 * multiplied by the same Hadamard matrix R with entries +-1/sqrt(d), which
 * leaves the product unchanged (R is orthogonal and symmetric), and both
 * tensors are quantized to 4 bits symmetrically with round-to-nearest ([P4]
 * core discovery).
 *
 * Rotation.  The Sylvester Hadamard matrix H_d, H[i][j] = (-1)^popcount(i & j)
 * for d a power of two, applied to a vector v as v H (its symmetric, so also
 * H v) by the fast Walsh-Hadamard transform: for h = 1, 2, 4, ..., d/2 in this
 * order, every pair (i, i + h) with (i & h) == 0 becomes (v_i + v_{i+h},
 * v_i - v_{i+h}).  In float, one IEEE add or subtract per butterfly.  The
 * transform is unnormalized (it computes v H, not v H / sqrt(d)): the two
 * factors 1/sqrt(d) of activation and weight multiply to 1/d, a power of two,
 * applied exactly in the weight scale below. */
void oracle_fwht_f32(float *v, int64_t d)
{
    for (int64_t h = 1; h < d; h <<= 1)
        for (int64_t i = 0; i < d; ++i)
            if ((i & h) == 0) {
                float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
}

/* 4-bit symmetric round-to-nearest quantization of rows, optionally rotated.
 * For each of the M rows of x (fp16, row stride ldx):
 *   v[j]     = float(x[m][j]) * mult[j]          (float product)
 *   v        = v H   if rotate                  (oracle_fwht_f32)
 *   a        = max_j |v[j]|
 *   q[m][j]  = clamp(rint(v[j] * (7 / a)), -7, 7)
 *   scale[m] = (a / 7) * post                    (post a power of two: exact)
 * a == 0 gives scale 0 and codes 0; a non-finite v gives scale NaN and codes
 * 0.  Activations use mult = 1/s and post = 1 (one row per token); weights
 * use the rows of W transposed (one per output channel), mult = s and
 * post = 1/d when rotated (1 otherwise). */
void oracle_quant4_rows(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                        const float *mult, int rotate, float post, int8_t *q, float *scale,
                        float *work /* K floats */)
{
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t j = 0; j < K; ++j)
            work[j] = half_to_float(x[m * ldx + j]) * mult[j];
        if (rotate)
            oracle_fwht_f32(work, K);
        float a = 0.0f;
        int bad = 0;
        for (int64_t j = 0; j < K; ++j) {
            if (!isfinite(work[j])) { bad = 1; continue; }
            if (fabsf(work[j]) > a) a = fabsf(work[j]);
        }
        if (bad || a == 0.0f) {
            scale[m] = bad ? NAN : 0.0f;
            for (int64_t j = 0; j < K; ++j) q[m * K + j] = 0;
            continue;
        }
        float r = 7.0f / a;
        scale[m] = (a / 7.0f) * post;
        for (int64_t j = 0; j < K; ++j) {
            q[m * K + j] = code_of(work[j], r, 7.0f);
        }
    }
}
