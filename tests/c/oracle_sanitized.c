/* Every entry point of oracle/conv_oracle.c on small, ragged problems, for a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer: an access
 * outside a buffer, a signed overflow or a bad shift in the oracle ends the
 * program with a sanitizer report.  The buffers are allocated to their exact
 * sizes, so any overrun is caught.  Also checks that the point-wise entry
 * points agree with the full ones and that the layout maps round-trip.
 * Prints "all ok" on success. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_output_dim(int in, int pad, int dil, int k, int stride);
int oracle_conv2d_i8_acc(const int8_t *x, const int8_t *w, int64_t *acc, int N, int C, int H,
                         int W, int K, int R, int S, int ph, int pw, int sh, int sw, int dh,
                         int dw, int nthreads);
int oracle_conv2d_i8_points(const int8_t *x, const int8_t *w, const int32_t *pts, int64_t npts,
                            int64_t *acc, int N, int C, int H, int W, int K, int R, int S,
                            int ph, int pw, int sh, int sw, int dh, int dw, int nthreads);
int oracle_epilogue_i8(const int64_t *acc, int8_t *y, int64_t count, float alpha);
int oracle_epilogue_i8_per_channel(const int64_t *acc, int8_t *y, int N, int K, int64_t plane,
                                   const float *alpha, const float *bias);
void oracle_epilogue_f32_per_channel(const double *acc, float *y, int N, int K, int64_t plane,
                                     const float *alpha, const float *bias);
int oracle_conv2d_f32_acc(const float *x, const float *w, double *acc, int N, int C, int H,
                          int W, int K, int R, int S, int ph, int pw, int sh, int sw, int dh,
                          int dw, int nthreads);
int oracle_conv2d_f32_points(const float *x, const float *w, const int32_t *pts, int64_t npts,
                             double *acc, int N, int C, int H, int W, int K, int R, int S,
                             int ph, int pw, int sh, int sw, int dh, int dw, int nthreads);
void oracle_epilogue_f32(const double *acc, float *y, int64_t count, float alpha);
int oracle_nchw_to_nc32hw32(const int8_t *src, int8_t *dst, int N, int C, int H, int W);
int oracle_nc32hw32_to_nchw(const int8_t *src, int8_t *dst, int N, int C, int H, int W);
int oracle_kcrs_to_c32rsk32(const int8_t *src, int8_t *dst, int K, int C, int R, int S);
int oracle_c32rsk32_to_kcrs(const int8_t *src, int8_t *dst, int K, int C, int R, int S);

#define CHECK(cond, what)                                             \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "FAILED: %s (line %d)\n", what, __LINE__);      \
      return 1;                                                       \
    }                                                                 \
  } while (0)

static uint32_t lcg = 2026u;
static int rnd(int lo, int hi) {
  lcg = lcg * 1664525u + 1013904223u;
  return lo + (int)((lcg >> 8) % (uint32_t)(hi - lo + 1));
}

/* One problem through every int8 and fp32 entry point. */
static int one_problem(int N, int C, int H, int W, int K, int R, int S, int ph, int pw, int sh,
                       int sw, int dh, int dw, int threads) {
  const int P = oracle_output_dim(H, ph, dh, R, sh), Q = oracle_output_dim(W, pw, dw, S, sw);
  if (P <= 0 || Q <= 0) return 0;
  const size_t nx = (size_t)N * C * H * W, nw = (size_t)K * C * R * S, ny = (size_t)N * K * P * Q;
  int8_t *x = malloc(nx), *w = malloc(nw), *y = malloc(ny);
  int64_t *acc = malloc(ny * sizeof *acc), *pacc = malloc(ny * sizeof *pacc);
  float *xf = malloc(nx * sizeof *xf), *wf = malloc(nw * sizeof *wf), *yf = malloc(ny * sizeof *yf);
  double *accf = malloc(ny * sizeof *accf), *paccf = malloc(ny * sizeof *paccf);
  int32_t *pts = malloc(ny * 4 * sizeof *pts);
  float *al = malloc(K * sizeof *al), *bi = malloc(K * sizeof *bi);
  CHECK(x && w && y && acc && pacc && xf && wf && yf && accf && paccf && pts && al && bi, "malloc");
  for (size_t i = 0; i < nx; ++i) xf[i] = (float)(x[i] = (int8_t)rnd(-128, 127));
  for (size_t i = 0; i < nw; ++i) wf[i] = (float)(w[i] = (int8_t)rnd(-128, 127));
  for (int k = 0; k < K; ++k) {
    al[k] = 0.001f * (float)rnd(1, 50);
    bi[k] = 0.5f * (float)rnd(-4, 4);
  }
  CHECK(oracle_conv2d_i8_acc(x, w, acc, N, C, H, W, K, R, S, ph, pw, sh, sw, dh, dw, threads) == 0,
        "conv2d_i8_acc");
  size_t np = 0;
  for (int n = 0; n < N; ++n)
    for (int k = 0; k < K; ++k)
      for (int p = 0; p < P; ++p)
        for (int q = 0; q < Q; ++q) {
          pts[4 * np] = n, pts[4 * np + 1] = k, pts[4 * np + 2] = p, pts[4 * np + 3] = q;
          ++np;
        }
  CHECK(oracle_conv2d_i8_points(x, w, pts, (int64_t)np, pacc, N, C, H, W, K, R, S, ph, pw, sh, sw,
                                dh, dw, threads) == 0 &&
            memcmp(acc, pacc, ny * sizeof *acc) == 0,
        "conv2d_i8_points equals the full result");
  CHECK(oracle_epilogue_i8(acc, y, (int64_t)ny, 1.0f / 4096) == 0, "epilogue_i8");
  CHECK(oracle_epilogue_i8_per_channel(acc, y, N, K, (int64_t)P * Q, al, bi) == 0 &&
            oracle_epilogue_i8_per_channel(acc, y, N, K, (int64_t)P * Q, al, NULL) == 0,
        "epilogue_i8_per_channel");
  CHECK(oracle_conv2d_f32_acc(xf, wf, accf, N, C, H, W, K, R, S, ph, pw, sh, sw, dh, dw, threads) == 0,
        "conv2d_f32_acc");
  CHECK(oracle_conv2d_f32_points(xf, wf, pts, (int64_t)np, paccf, N, C, H, W, K, R, S, ph, pw, sh,
                                 sw, dh, dw, threads) == 0 &&
            memcmp(accf, paccf, ny * sizeof *accf) == 0,
        "conv2d_f32_points equals the full result");
  for (size_t i = 0; i < ny; ++i) CHECK(accf[i] == (double)acc[i], "fp32 path equals int8 path");
  oracle_epilogue_f32(accf, yf, (int64_t)ny, -2.5f);
  oracle_epilogue_f32_per_channel(accf, yf, N, K, (int64_t)P * Q, al, bi);
  oracle_epilogue_f32_per_channel(accf, yf, N, K, (int64_t)P * Q, al, NULL);
  /* a point outside the output is rejected, not read */
  int32_t bad[4] = {0, 0, P, 0};
  CHECK(oracle_conv2d_i8_points(x, w, bad, 1, pacc, N, C, H, W, K, R, S, ph, pw, sh, sw, dh, dw,
                                1) != 0,
        "out-of-range point rejected");
  free(x), free(w), free(y), free(acc), free(pacc), free(xf), free(wf), free(yf);
  free(accf), free(paccf), free(pts), free(al), free(bi);
  return 0;
}

static int layouts(int N, int C, int H, int W, int K, int R, int S) {
  const size_t nx = (size_t)N * C * H * W, nw = (size_t)K * C * R * S;
  int8_t *a = malloc(nx), *b = malloc(nx), *c = malloc(nx);
  int8_t *fa = malloc(nw), *fb = malloc(nw), *fc = malloc(nw);
  CHECK(a && b && c && fa && fb && fc, "malloc");
  for (size_t i = 0; i < nx; ++i) a[i] = (int8_t)rnd(-128, 127);
  for (size_t i = 0; i < nw; ++i) fa[i] = (int8_t)rnd(-128, 127);
  CHECK(oracle_nchw_to_nc32hw32(a, b, N, C, H, W) == 0 && oracle_nc32hw32_to_nchw(b, c, N, C, H, W) == 0 &&
            memcmp(a, c, nx) == 0,
        "activation layout round trip");
  CHECK(oracle_kcrs_to_c32rsk32(fa, fb, K, C, R, S) == 0 && oracle_c32rsk32_to_kcrs(fb, fc, K, C, R, S) == 0 &&
            memcmp(fa, fc, nw) == 0,
        "filter layout round trip");
  CHECK(oracle_nchw_to_nc32hw32(a, b, N, C + 1, H, W) != 0, "C % 32 != 0 rejected");
  free(a), free(b), free(c), free(fa), free(fb), free(fc);
  return 0;
}

int main(void) {
  /* hand-picked edge shapes: 1x1 outputs, padding wider than the filter
   * reach, strides and dilations, a filter as wide as the padded input */
  if (one_problem(1, 32, 1, 1, 32, 1, 1, 0, 0, 1, 1, 1, 1, 1)) return 1;
  if (one_problem(2, 32, 5, 7, 33, 3, 3, 1, 1, 1, 1, 1, 1, 2)) return 1;
  if (one_problem(1, 3, 9, 8, 5, 5, 9, 2, 4, 1, 1, 2, 3, 1)) return 1;
  if (one_problem(2, 4, 7, 6, 3, 3, 2, 3, 0, 3, 2, 1, 2, 4)) return 1;
  if (one_problem(1, 2, 4, 4, 2, 4, 6, 0, 1, 1, 1, 1, 1, 1)) return 1;
  /* seeded random small shapes */
  for (int t = 0; t < 60; ++t) {
    const int R = rnd(1, 5), S = rnd(1, 5);
    if (one_problem(rnd(1, 2), rnd(1, 40), rnd(1, 9), rnd(1, 9), rnd(1, 6), R, S, rnd(0, 3),
                    rnd(0, 3), rnd(1, 3), rnd(1, 3), rnd(1, 3), rnd(1, 3), rnd(1, 3)))
      return 1;
  }
  if (layouts(2, 64, 3, 5, 7, 3, 2) || layouts(1, 32, 1, 1, 1, 1, 1)) return 1;
  CHECK(oracle_output_dim(5, 0, 1, 7, 1) == 0 && oracle_output_dim(0, 0, 1, 1, 1) < 0,
        "output_dim edge cases");
  printf("all ok\n");
  return 0;
}
