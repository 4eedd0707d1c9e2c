/* The C ABI used from plain C (no Python, no C++): every entry point of
 * include/convfprop.h that needs no GPU, and -- with "run" -- one int8 and
 * one fp32 convolution through the HIP runtime's C API, checked against the
 * CPU oracle (oracle/conv_oracle.c, linked in by the test that builds this).
 * Prints one "ok ..." line per check and exits non-zero on the first
 * failure. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "convfprop.h"

int oracle_conv2d_i8_acc(const int8_t *x, const int8_t *w, int64_t *acc, int N, int C, int H,
                         int W, int K, int R, int S, int ph, int pw, int sh, int sw, int dh,
                         int dw, int nthreads);
int oracle_epilogue_i8(const int64_t *acc, int8_t *y, int64_t count, float alpha);
int oracle_conv2d_f32_acc(const float *x, const float *w, double *acc, int N, int C, int H, int W,
                          int K, int R, int S, int ph, int pw, int sh, int sw, int dh, int dw,
                          int nthreads);

#define CHECK(cond, what)                                  \
  do {                                                     \
    if (!(cond)) {                                         \
      fprintf(stderr, "FAILED: %s (line %d)\n", what, __LINE__); \
      return 1;                                            \
    }                                                      \
    printf("ok %s\n", what);                               \
  } while (0)

#define HIPCHECK(call)                                     \
  do {                                                     \
    hipError_t e_ = (call);                                \
    if (e_ != hipSuccess) {                                \
      fprintf(stderr, "FAILED: %s -> %d\n", #call, (int)e_); \
      return 1;                                            \
    }                                                      \
  } while (0)

static uint32_t lcg = 12345u;
static int8_t rnd_i8(int lo, int hi) {
  lcg = lcg * 1664525u + 1013904223u;
  return (int8_t)(lo + (int)((lcg >> 8) % (uint32_t)(hi - lo + 1)));
}

static int host_checks(void) {
  conv2d_fprop_desc_t d = NULL;
  CHECK(conv2d_fprop_desc_create(&d, 1, 32, 8, 8, 32, 3, 3, 1, 1, 1, 1, 1, 1, CONV_DTYPE_INT8,
                                 CONV_LAYOUT_NC32HW32_C32RSK32) == CONV_OK && d,
        "desc_create int8 3x3");
  int P = 0, Q = 0;
  CHECK(conv2d_fprop_desc_get_output_dims(d, &P, &Q) == CONV_OK && P == 8 && Q == 8,
        "get_output_dims");
  char buf[256];
  CHECK(conv2d_fprop_desc_get_config(d, buf, sizeof buf) == CONV_OK &&
            strncmp(buf, "config=", 7) == 0,
        "get_config");
  CHECK(conv2d_fprop_num_configs(CONV_DTYPE_INT8) > 0 && conv2d_fprop_num_configs(CONV_DTYPE_FP32) > 0,
        "num_configs");
  CHECK(conv2d_fprop_desc_set_config(d, conv2d_fprop_num_configs(CONV_DTYPE_INT8)) ==
            CONV_ERR_UNSUPPORTED,
        "set_config out of range");
  CHECK(conv2d_fprop_run(d, NULL, NULL, NULL, 1.0f, 0) == CONV_ERR_NULL, "run rejects null");
  CHECK(conv2d_fprop_desc_destroy(d) == CONV_OK && conv2d_fprop_desc_destroy(NULL) == CONV_OK,
        "desc_destroy");
  d = NULL;
  CHECK(conv2d_fprop_desc_create(&d, 1, 48, 8, 8, 32, 3, 3, 1, 1, 1, 1, 1, 1, CONV_DTYPE_INT8,
                                 CONV_LAYOUT_NC32HW32_C32RSK32) != CONV_OK && d == NULL,
        "C not a multiple of 32 rejected");
  CHECK(conv_status_string(CONV_ERR_MISALIGNED) != NULL && strlen(conv_status_string(CONV_OK)) > 0,
        "status strings");
  return 0;
}

static int run_int8(void) {
  const int N = 2, C = 64, H = 9, W = 11, K = 96, R = 3, S = 3;
  const float alpha = 1.0f / 1024;
  conv2d_fprop_desc_t d;
  CHECK(conv2d_fprop_desc_create(&d, N, C, H, W, K, R, S, 1, 1, 1, 1, 1, 1, CONV_DTYPE_INT8,
                                 CONV_LAYOUT_NC32HW32_C32RSK32) == CONV_OK,
        "desc_create int8 run shape");
  int P, Q;
  conv2d_fprop_desc_get_output_dims(d, &P, &Q);
  const size_t xn = (size_t)N * C * H * W, wn = (size_t)K * C * R * S, yn = (size_t)N * K * P * Q;
  int8_t *x = malloc(xn), *w = malloc(wn), *y = malloc(yn), *ref = malloc(yn);
  int64_t *acc = malloc(yn * sizeof(int64_t));
  for (size_t i = 0; i < xn; ++i) x[i] = rnd_i8(-128, 127);
  for (size_t i = 0; i < wn; ++i) w[i] = rnd_i8(-128, 127);
  void *dx, *dxi, *dw, *dwi, *dyi, *dy;
  HIPCHECK(hipMalloc(&dx, xn));
  HIPCHECK(hipMalloc(&dxi, xn));
  HIPCHECK(hipMalloc(&dw, wn));
  HIPCHECK(hipMalloc(&dwi, wn));
  HIPCHECK(hipMalloc(&dyi, yn));
  HIPCHECK(hipMalloc(&dy, yn));
  HIPCHECK(hipMemcpy(dx, x, xn, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(dw, w, wn, hipMemcpyHostToDevice));
  CHECK(conv_nchw_to_nc32hw32_i8(dx, dxi, N, C, H, W, 0) == CONV_OK, "activation transform");
  CHECK(conv_kcrs_to_c32rsk32_i8(dw, dwi, K, C, R, S, 0) == CONV_OK, "filter transform");
  CHECK(conv2d_fprop_run(d, dxi, dwi, dyi, alpha, 0) == CONV_OK, "run int8");
  CHECK(conv_nc32hw32_to_nchw_i8(dyi, dy, N, K, P, Q, 0) == CONV_OK, "output transform");
  HIPCHECK(hipMemcpy(y, dy, yn, hipMemcpyDeviceToHost));
  CHECK(oracle_conv2d_i8_acc(x, w, acc, N, C, H, W, K, R, S, 1, 1, 1, 1, 1, 1, 1) == 0 &&
            oracle_epilogue_i8(acc, ref, (int64_t)yn, alpha) == 0,
        "oracle int8");
  CHECK(memcmp(y, ref, yn) == 0, "int8 output equals the oracle, byte for byte");
  hipFree(dx); hipFree(dxi); hipFree(dw); hipFree(dwi); hipFree(dyi); hipFree(dy);
  free(x); free(w); free(y); free(ref); free(acc);
  conv2d_fprop_desc_destroy(d);
  return 0;
}

static int run_fp32(void) {
  const int N = 1, C = 5, H = 13, W = 10, K = 40, R = 5, S = 3;
  conv2d_fprop_desc_t d;
  CHECK(conv2d_fprop_desc_create(&d, N, C, H, W, K, R, S, 2, 1, 1, 2, 2, 1, CONV_DTYPE_FP32,
                                 CONV_LAYOUT_NCHW_KCRS) == CONV_OK,
        "desc_create fp32 (padding, stride, dilation)");
  int P, Q;
  conv2d_fprop_desc_get_output_dims(d, &P, &Q);
  const size_t xn = (size_t)N * C * H * W, wn = (size_t)K * C * R * S, yn = (size_t)N * K * P * Q;
  float *x = malloc(xn * 4), *w = malloc(wn * 4), *y = malloc(yn * 4);
  double *acc = malloc(yn * sizeof(double));
  /* integer-valued operands in {-1, 0, 1}: every sum is exact in fp32 */
  for (size_t i = 0; i < xn; ++i) x[i] = (float)(rnd_i8(-1, 1));
  for (size_t i = 0; i < wn; ++i) w[i] = (float)(rnd_i8(-1, 1));
  void *dx, *dw, *dy;
  HIPCHECK(hipMalloc(&dx, xn * 4));
  HIPCHECK(hipMalloc(&dw, wn * 4));
  HIPCHECK(hipMalloc(&dy, yn * 4));
  HIPCHECK(hipMemcpy(dx, x, xn * 4, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(dw, w, wn * 4, hipMemcpyHostToDevice));
  CHECK(conv2d_fprop_run(d, dx, dw, dy, 1.0f, 0) == CONV_OK, "run fp32");
  HIPCHECK(hipMemcpy(y, dy, yn * 4, hipMemcpyDeviceToHost));
  CHECK(oracle_conv2d_f32_acc(x, w, acc, N, C, H, W, K, R, S, 2, 1, 1, 2, 2, 1, 1) == 0,
        "oracle fp32");
  size_t bad = 0;
  for (size_t i = 0; i < yn; ++i) bad += y[i] != (float)acc[i];
  CHECK(bad == 0, "fp32 output equals the oracle exactly on integer-valued operands");
  hipFree(dx); hipFree(dw); hipFree(dy);
  free(x); free(w); free(y); free(acc);
  conv2d_fprop_desc_destroy(d);
  return 0;
}

int main(int argc, char **argv) {
  if (host_checks()) return 1;
  if (argc > 1 && strcmp(argv[1], "run") == 0) {
    if (run_int8() || run_fp32()) return 1;
  }
  printf("all ok\n");
  return 0;
}
