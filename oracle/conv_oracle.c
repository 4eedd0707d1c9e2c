/*
 * conv_oracle.c -- the CPU oracle for 2D convolution forward (fprop).
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests, the smoke check and the bench's
 * CPU-baseline leg may load this file's library.  The GPU library never links,
 * includes or calls it, and this file includes nothing from the GPU library.
 *
 * Every function here is the plain definition of what it computes, written as
 * nested loops with no blocking, fusion or reordering:
 *
 *   acc[n][k][p][q] = sum_{c<C} sum_{r<R} sum_{s<S}
 *                        X(n, c, p*sh - ph + r*dh, q*sw - pw + s*dw) * w[k][c][r][s]
 *
 * with X(.) = x inside [0,H) x [0,W) and 0 outside (zero padding).  This is
 * cross-correlation: the filter is not flipped.  Sources:
 *   - "Kimi-K2.6 l1_p80" POPCORNBENCH transcript (an agent writing a conv2d
 *     kernel), first turn: the output-size formula with padding, dilation and
 *     stride; the reference loop over (ic, kh, kw) with ih = oh*stride -
 *     pad + kh*dil; the weight layout [C_out][C_in][kH][kW].
 *   - "[QST] How to optimize cutlass int8 fprop2d kernel with NCxHWx
 *     interleaved layout" (CUTLASS issue 2996), section "CUTLASS Kernel
 *     Configuration": int8 operands, int32 accumulator, fp32 alpha-only
 *     scaling, clamp to int8 (LinearCombinationClamp, OnlyAlphaScaling);
 *     the NCxHWx<32> activation/output and CxRSKx<32> filter layouts.
 *
 * Precision: the int8 path multiplies and sums in int64 (exact), then applies
 * the epilogue y = clamp(rint(fl32(fl32(acc) * alpha)), -128, 127).  The fp32
 * path forms each product exactly in double and sums in double in (c, r, s)
 * order, then rounds once to float.  OpenMP (when nthreads > 1) only splits
 * the outer (n, k) loop; every output's summation order is unchanged.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -fopenmp -ffp-contract=off -lm.
 */
#include <fenv.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_SHAPE 1
#define ORACLE_ERR_RANGE 2    /* an int8 accumulator does not fit in int32 */
#define ORACLE_ERR_ROUNDING 3 /* the FPU is not in round-to-nearest mode  */

/* Output extent along one dimension:
 *   out = floor((in + 2*pad - dil*(k-1) - 1) / stride) + 1,
 * as derived in the first turn of the "Kimi-K2.6 l1_p80" transcript
 * (512 -> 508 along H with pad 2, dil 2, kH 5; 512 -> 496 along W with pad 4,
 * dil 3, kW 9).  Returns 0 when no output position exists (the numerator is
 * negative, i.e. the dilated filter is wider than the padded input). */
int oracle_output_dim(int in, int pad, int dil, int k, int stride)
{
    long long num = (long long)in + 2LL * pad - (long long)dil * (k - 1) - 1;
    if (in <= 0 || k <= 0 || stride <= 0 || dil <= 0 || pad < 0) return -1;
    if (num < 0) return 0;
    return (int)(num / stride + 1);
}

static int shape_ok(int N, int C, int H, int W, int K, int R, int S, int ph,
                    int pw, int sh, int sw, int dh, int dw, int *P, int *Q)
{
    if (N <= 0 || C <= 0 || K <= 0) return 0;
    *P = oracle_output_dim(H, ph, dh, R, sh);
    *Q = oracle_output_dim(W, pw, dw, S, sw);
    return *P > 0 && *Q > 0;
}

/* One int8 output accumulator, summed in int64 over (c, r, s). */
static int64_t acc_i8_point(const int8_t *x, const int8_t *w, int n, int k,
                            int p, int q, int C, int H, int W, int R, int S,
                            int ph, int pw, int sh, int sw, int dh, int dw)
{
    int64_t acc = 0;
    for (int c = 0; c < C; ++c)
        for (int r = 0; r < R; ++r) {
            int h = p * sh - ph + r * dh;
            if (h < 0 || h >= H) continue; /* zero padding */
            for (int s = 0; s < S; ++s) {
                int ww = q * sw - pw + s * dw;
                if (ww < 0 || ww >= W) continue; /* zero padding */
                int64_t xv = x[(((size_t)n * C + c) * H + h) * W + ww];
                int64_t wv = w[(((size_t)k * C + c) * R + r) * S + s];
                acc += xv * wv;
            }
        }
    return acc;
}

/* Direct int8 convolution: x is logical NCHW int8, w is logical KCRS int8,
 * acc is logical NKPQ int64.  Returns ORACLE_OK or ORACLE_ERR_SHAPE. */
int oracle_conv2d_i8_acc(const int8_t *x, const int8_t *w, int64_t *acc,
                         int N, int C, int H, int W, int K, int R, int S,
                         int ph, int pw, int sh, int sw, int dh, int dw,
                         int nthreads)
{
    int P, Q;
    if (!shape_ok(N, C, H, W, K, R, S, ph, pw, sh, sw, dh, dw, &P, &Q))
        return ORACLE_ERR_SHAPE;
    (void)nthreads;
#ifdef _OPENMP
#pragma omp parallel for collapse(2) schedule(dynamic) num_threads(nthreads > 0 ? nthreads : 1)
#endif
    for (int n = 0; n < N; ++n)
        for (int k = 0; k < K; ++k)
            for (int p = 0; p < P; ++p)
                for (int q = 0; q < Q; ++q)
                    acc[(((size_t)n * K + k) * P + p) * Q + q] = acc_i8_point(
                        x, w, n, k, p, q, C, H, W, R, S, ph, pw, sh, sw, dh, dw);
    return ORACLE_OK;
}

/* Selected int8 accumulators: for each i < npts, (n,k,p,q) = pts[4i..4i+3]. */
int oracle_conv2d_i8_points(const int8_t *x, const int8_t *w, const int32_t *pts,
                            int64_t npts, int64_t *acc, int N, int C, int H,
                            int W, int K, int R, int S, int ph, int pw, int sh,
                            int sw, int dh, int dw, int nthreads)
{
    int P, Q;
    if (!shape_ok(N, C, H, W, K, R, S, ph, pw, sh, sw, dh, dw, &P, &Q))
        return ORACLE_ERR_SHAPE;
    for (int64_t i = 0; i < npts; ++i) {
        const int32_t *t = pts + 4 * i;
        if (t[0] < 0 || t[0] >= N || t[1] < 0 || t[1] >= K || t[2] < 0 ||
            t[2] >= P || t[3] < 0 || t[3] >= Q)
            return ORACLE_ERR_SHAPE;
    }
    (void)nthreads;
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
#endif
    for (int64_t i = 0; i < npts; ++i) {
        const int32_t *t = pts + 4 * i;
        acc[i] = acc_i8_point(x, w, t[0], t[1], t[2], t[3], C, H, W, R, S, ph,
                              pw, sh, sw, dh, dw);
    }
    return ORACLE_OK;
}

/* The int8 epilogue (alpha-only scaling, then clamp to int8):
 *   f = (float)acc          one int32 -> fp32 conversion, round to nearest even
 *   g = f * alpha           one fp32 multiply (never a division, never an FMA)
 *   r = rint(g)             round half to even (the current mode, asserted)
 *   y = clamp(r, -128, 127)
 * The accumulator must fit in int32 (the hardware accumulator width named by
 * the CUTLASS configuration's int32_t accumulator). */
int oracle_epilogue_i8(const int64_t *acc, int8_t *y, int64_t count, float alpha)
{
    if (fegetround() != FE_TONEAREST) return ORACLE_ERR_ROUNDING;
    for (int64_t i = 0; i < count; ++i)
        if (acc[i] > INT32_MAX || acc[i] < INT32_MIN) return ORACLE_ERR_RANGE;
    for (int64_t i = 0; i < count; ++i) {
        volatile float f = (float)(int32_t)acc[i];
        volatile float g = f * alpha;
        float r = rintf(g);
        if (r > 127.0f) r = 127.0f;
        if (r < -128.0f) r = -128.0f;
        y[i] = (int8_t)r;
    }
    return ORACLE_OK;
}

/* Per-output-channel epilogue variant: a scale alpha[k] and a bias bias[k]
 * for each output channel k (bias may be NULL for none).  Source: the
 * "rowwise scaled" operators named in the review thread of torchao issue
 * 1406 (PR 1515, CUTLASS-based W4A8/W4A4 GEMM), read as a scale per GEMM
 * column, which is an output channel here, plus a bias per column:
 *   y[n][k][p][q] = clamp(rint(fl32(fl32(fl32(acc) * alpha[k]) + bias[k])), -128, 127)
 * (one fp32 multiply, then one fp32 add; no fused multiply-add).  acc is
 * logical NKPQ int64 with plane = P*Q. */
int oracle_epilogue_i8_per_channel(const int64_t *acc, int8_t *y, int N, int K, int64_t plane,
                                   const float *alpha, const float *bias)
{
    if (fegetround() != FE_TONEAREST) return ORACLE_ERR_ROUNDING;
    if (N <= 0 || K <= 0 || plane <= 0) return ORACLE_ERR_SHAPE;
    for (int64_t i = 0; i < (int64_t)N * K * plane; ++i)
        if (acc[i] > INT32_MAX || acc[i] < INT32_MIN) return ORACLE_ERR_RANGE;
    for (int n = 0; n < N; ++n)
        for (int k = 0; k < K; ++k)
            for (int64_t j = 0; j < plane; ++j) {
                const int64_t i = ((int64_t)n * K + k) * plane + j;
                volatile float f = (float)(int32_t)acc[i];
                volatile float g = f * alpha[k];
                volatile float h = g + (bias ? bias[k] : 0.0f);
                float r = rintf(h);
                if (r > 127.0f) r = 127.0f;
                if (r < -128.0f) r = -128.0f;
                y[i] = (int8_t)r;
            }
    return ORACLE_OK;
}

/* fp32 per-output-channel variant: y = alpha[k] * acc + bias[k] (bias may be
 * NULL), computed in double from the double accumulator, rounded once. */
void oracle_epilogue_f32_per_channel(const double *acc, float *y, int N, int K, int64_t plane,
                                     const float *alpha, const float *bias)
{
    for (int n = 0; n < N; ++n)
        for (int k = 0; k < K; ++k)
            for (int64_t j = 0; j < plane; ++j) {
                const int64_t i = ((int64_t)n * K + k) * plane + j;
                y[i] = (float)((double)alpha[k] * acc[i] + (bias ? (double)bias[k] : 0.0));
            }
}

/* One fp32 output, each product exact in double, summed in double. */
static double acc_f32_point(const float *x, const float *w, int n, int k, int p,
                            int q, int C, int H, int W, int R, int S, int ph,
                            int pw, int sh, int sw, int dh, int dw)
{
    double acc = 0.0;
    for (int c = 0; c < C; ++c)
        for (int r = 0; r < R; ++r) {
            int h = p * sh - ph + r * dh;
            if (h < 0 || h >= H) continue;
            for (int s = 0; s < S; ++s) {
                int ww = q * sw - pw + s * dw;
                if (ww < 0 || ww >= W) continue;
                double xv = x[(((size_t)n * C + c) * H + h) * W + ww];
                double wv = w[(((size_t)k * C + c) * R + r) * S + s];
                acc += xv * wv;
            }
        }
    return acc;
}

/* Direct fp32 convolution: x NCHW fp32, w KCRS fp32, acc NKPQ double. */
int oracle_conv2d_f32_acc(const float *x, const float *w, double *acc, int N,
                          int C, int H, int W, int K, int R, int S, int ph,
                          int pw, int sh, int sw, int dh, int dw, int nthreads)
{
    int P, Q;
    if (!shape_ok(N, C, H, W, K, R, S, ph, pw, sh, sw, dh, dw, &P, &Q))
        return ORACLE_ERR_SHAPE;
    (void)nthreads;
#ifdef _OPENMP
#pragma omp parallel for collapse(2) schedule(dynamic) num_threads(nthreads > 0 ? nthreads : 1)
#endif
    for (int n = 0; n < N; ++n)
        for (int k = 0; k < K; ++k)
            for (int p = 0; p < P; ++p)
                for (int q = 0; q < Q; ++q)
                    acc[(((size_t)n * K + k) * P + p) * Q + q] = acc_f32_point(
                        x, w, n, k, p, q, C, H, W, R, S, ph, pw, sh, sw, dh, dw);
    return ORACLE_OK;
}

int oracle_conv2d_f32_points(const float *x, const float *w, const int32_t *pts,
                             int64_t npts, double *acc, int N, int C, int H,
                             int W, int K, int R, int S, int ph, int pw, int sh,
                             int sw, int dh, int dw, int nthreads)
{
    int P, Q;
    if (!shape_ok(N, C, H, W, K, R, S, ph, pw, sh, sw, dh, dw, &P, &Q))
        return ORACLE_ERR_SHAPE;
    for (int64_t i = 0; i < npts; ++i) {
        const int32_t *t = pts + 4 * i;
        if (t[0] < 0 || t[0] >= N || t[1] < 0 || t[1] >= K || t[2] < 0 ||
            t[2] >= P || t[3] < 0 || t[3] >= Q)
            return ORACLE_ERR_SHAPE;
    }
    (void)nthreads;
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
#endif
    for (int64_t i = 0; i < npts; ++i) {
        const int32_t *t = pts + 4 * i;
        acc[i] = acc_f32_point(x, w, t[0], t[1], t[2], t[3], C, H, W, R, S, ph,
                               pw, sh, sw, dh, dw);
    }
    return ORACLE_OK;
}

/* fp32 epilogue: y = (float)(alpha * acc), one rounding from double. */
void oracle_epilogue_f32(const double *acc, float *y, int64_t count, float alpha)
{
    for (int64_t i = 0; i < count; ++i) y[i] = (float)((double)alpha * acc[i]);
}

/* ---- Interleaved layouts (reading of the CUTLASS template names) ----------
 * NCxHWx<32>: [N][C/32][H][W][32] -- 32 consecutive channels of one pixel are
 *             contiguous; then W, H, the channel group, the image.
 * CxRSKx<32>: [C/32][R][S][K][32] -- 32 consecutive input channels of one
 *             (r, s, k) are contiguous; then K, S, R, the channel group.
 * Both require the interleaved dimension to be a multiple of 32.
 */
int oracle_nchw_to_nc32hw32(const int8_t *src, int8_t *dst, int N, int C, int H, int W)
{
    if (N <= 0 || C <= 0 || H <= 0 || W <= 0 || C % 32) return ORACLE_ERR_SHAPE;
    for (int n = 0; n < N; ++n)
        for (int c = 0; c < C; ++c)
            for (int h = 0; h < H; ++h)
                for (int w = 0; w < W; ++w)
                    dst[((((size_t)n * (C / 32) + c / 32) * H + h) * W + w) * 32 + c % 32] =
                        src[(((size_t)n * C + c) * H + h) * W + w];
    return ORACLE_OK;
}

int oracle_nc32hw32_to_nchw(const int8_t *src, int8_t *dst, int N, int C, int H, int W)
{
    if (N <= 0 || C <= 0 || H <= 0 || W <= 0 || C % 32) return ORACLE_ERR_SHAPE;
    for (int n = 0; n < N; ++n)
        for (int c = 0; c < C; ++c)
            for (int h = 0; h < H; ++h)
                for (int w = 0; w < W; ++w)
                    dst[(((size_t)n * C + c) * H + h) * W + w] =
                        src[((((size_t)n * (C / 32) + c / 32) * H + h) * W + w) * 32 + c % 32];
    return ORACLE_OK;
}

int oracle_kcrs_to_c32rsk32(const int8_t *src, int8_t *dst, int K, int C, int R, int S)
{
    if (K <= 0 || C <= 0 || R <= 0 || S <= 0 || C % 32) return ORACLE_ERR_SHAPE;
    for (int k = 0; k < K; ++k)
        for (int c = 0; c < C; ++c)
            for (int r = 0; r < R; ++r)
                for (int s = 0; s < S; ++s)
                    dst[((((size_t)(c / 32) * R + r) * S + s) * K + k) * 32 + c % 32] =
                        src[(((size_t)k * C + c) * R + r) * S + s];
    return ORACLE_OK;
}

int oracle_c32rsk32_to_kcrs(const int8_t *src, int8_t *dst, int K, int C, int R, int S)
{
    if (K <= 0 || C <= 0 || R <= 0 || S <= 0 || C % 32) return ORACLE_ERR_SHAPE;
    for (int k = 0; k < K; ++k)
        for (int c = 0; c < C; ++c)
            for (int r = 0; r < R; ++r)
                for (int s = 0; s < S; ++s)
                    dst[(((size_t)k * C + c) * R + r) * S + s] =
                        src[((((size_t)(c / 32) * R + r) * S + s) * K + k) * 32 + c % 32];
    return ORACLE_OK;
}

/* Number of OpenMP threads a parallel region would use (1 without OpenMP). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
