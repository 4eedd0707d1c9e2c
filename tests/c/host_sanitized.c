/* The host side of the C ABI under AddressSanitizer and
 * UndefinedBehaviorSanitizer, with no GPU: descriptor creation (argument
 * checks, output extents, the per-shape table, configuration planning and
 * the fitted selection model) over a grid of shapes, every configuration
 * index through set_config, the query calls with short buffers, and every
 * argument error of the run, graph and transform entry points -- each of
 * which returns before any HIP call.  Prints "all ok" on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "convfprop.h"

#define CHECK(cond, what)                                             \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "FAILED: %s (line %d)\n", what, __LINE__);      \
      return 1;                                                       \
    }                                                                 \
  } while (0)

static uint32_t lcg = 77u;
static int rnd(int lo, int hi) {
  lcg = lcg * 1664525u + 1013904223u;
  return lo + (int)((lcg >> 8) % (uint32_t)(hi - lo + 1));
}

/* Create a descriptor, query it, walk every configuration, destroy it. */
static int exercise(int N, int C, int H, int W, int K, int R, int S, int ph, int pw, int sh, int sw,
                    int dh, int dw, conv_dtype_t dt) {
  const conv_layout_t lay = dt == CONV_DTYPE_INT8 ? CONV_LAYOUT_NC32HW32_C32RSK32 : CONV_LAYOUT_NCHW_KCRS;
  conv2d_fprop_desc_t d = NULL;
  const conv_status_t st =
      conv2d_fprop_desc_create(&d, N, C, H, W, K, R, S, ph, pw, sh, sw, dh, dw, dt, lay);
  if (st != CONV_OK) {
    CHECK(d == NULL, "failed create leaves NULL");
    return 0;
  }
  int P = 0, Q = 0;
  CHECK(conv2d_fprop_desc_get_output_dims(d, &P, &Q) == CONV_OK && P > 0 && Q > 0, "dims");
  char buf[300], tiny[5];
  CHECK(conv2d_fprop_desc_get_config(d, buf, sizeof buf) == CONV_OK && strlen(buf) < sizeof buf,
        "config text");
  CHECK(conv2d_fprop_desc_get_config(d, tiny, sizeof tiny) == CONV_OK && strlen(tiny) == 4,
        "config text truncated");
  CHECK(conv2d_fprop_desc_get_config(d, tiny, 0) == CONV_OK, "config text, empty buffer");
  const int n = conv2d_fprop_num_configs(dt);
  for (int c = -1; c <= n; ++c) {
    const conv_status_t s = conv2d_fprop_desc_set_config(d, c);
    CHECK(s == CONV_OK || s == CONV_ERR_UNSUPPORTED, "set_config status");
    if (c < 0 || c == n) CHECK(s == CONV_ERR_UNSUPPORTED, "set_config out of range");
    if (s == CONV_OK) CHECK(conv2d_fprop_desc_get_config(d, buf, sizeof buf) == CONV_OK, "config");
  }
  /* run argument errors return before any launch */
  char *base = (char *)(uintptr_t)0x100000;  /* never dereferenced */
  CHECK(conv2d_fprop_run(d, NULL, base, base, 1.0f, 0) == CONV_ERR_NULL, "run null x");
  CHECK(conv2d_fprop_run(d, base + 1, base + 4096, base + 8192, 1.0f, 0) == CONV_ERR_MISALIGNED ||
            dt == CONV_DTYPE_FP32,
        "run misaligned");
  CHECK(conv2d_fprop_run(d, base, base, base, 1.0f, 0) == CONV_ERR_UNSUPPORTED, "run overlap");
  if (dt == CONV_DTYPE_INT8)
    CHECK(conv2d_fprop_run(d, base, base + (1 << 30), base + (3u << 29), NAN, 0) ==
              CONV_ERR_INVALID_ALPHA,
          "run NaN alpha");
  CHECK(conv2d_fprop_run_scaled(d, base, base + (1 << 30), base + (3u << 29), NULL, NULL, 0) ==
            CONV_ERR_NULL,
        "run_scaled null alpha");
  conv2d_fprop_graph_t g = (conv2d_fprop_graph_t)base;
  CHECK(conv2d_fprop_graph_create(&g, d, base, base + (1 << 30), base + (3u << 29), 1.0f, 0) ==
                CONV_ERR_INVALID_SHAPE &&
            g == NULL,
        "graph_create calls < 1");
  CHECK(conv2d_fprop_desc_destroy(d) == CONV_OK, "destroy");
  return 0;
}

int main(void) {
  /* the five graded problems */
  if (exercise(1, 32, 8, 8, 32, 3, 3, 1, 1, 1, 1, 1, 1, CONV_DTYPE_INT8) ||
      exercise(2, 128, 8, 8, 128, 1, 1, 0, 0, 1, 1, 1, 1, CONV_DTYPE_INT8) ||
      exercise(32, 256, 28, 28, 256, 3, 3, 1, 1, 1, 1, 1, 1, CONV_DTYPE_INT8) ||
      exercise(32, 128, 56, 56, 256, 3, 3, 1, 1, 2, 2, 1, 1, CONV_DTYPE_INT8) ||
      exercise(8, 32, 512, 512, 64, 5, 9, 2, 4, 1, 1, 2, 3, CONV_DTYPE_FP32))
    return 1;
  /* edge and seeded random shapes, both paths */
  if (exercise(1, 32, 1, 1, 32, 1, 1, 0, 0, 1, 1, 1, 1, CONV_DTYPE_INT8) ||
      exercise(1, 32, 300, 2, 32, 7, 1, 3, 0, 1, 1, 1, 1, CONV_DTYPE_INT8) ||
      exercise(1, 4064, 3, 3, 32, 3, 3, 1, 1, 1, 1, 1, 1, CONV_DTYPE_INT8) ||
      exercise(1, 3, 224, 224, 64, 7, 7, 3, 3, 2, 2, 1, 1, CONV_DTYPE_FP32))
    return 1;
  for (int t = 0; t < 150; ++t) {
    const conv_dtype_t dt = t & 1 ? CONV_DTYPE_FP32 : CONV_DTYPE_INT8;
    const int C = dt == CONV_DTYPE_INT8 ? 32 * rnd(1, 8) : rnd(1, 70);
    const int K = dt == CONV_DTYPE_INT8 ? 32 * rnd(1, 8) : rnd(1, 130);
    if (exercise(rnd(1, 40), C, rnd(1, 70), rnd(1, 70), K, rnd(1, 7), rnd(1, 7), rnd(0, 3),
                 rnd(0, 3), rnd(1, 3), rnd(1, 3), rnd(1, 3), rnd(1, 3), dt))
      return 1;
  }
  /* create rejections */
  conv2d_fprop_desc_t d = (conv2d_fprop_desc_t)(uintptr_t)16;
  CHECK(conv2d_fprop_desc_create(NULL, 1, 32, 8, 8, 32, 3, 3, 1, 1, 1, 1, 1, 1, CONV_DTYPE_INT8,
                                 CONV_LAYOUT_NC32HW32_C32RSK32) == CONV_ERR_NULL,
        "create null out");
  CHECK(conv2d_fprop_desc_create(&d, 1, 32, 2, 2, 32, 5, 5, 0, 0, 1, 1, 1, 1, CONV_DTYPE_INT8,
                                 CONV_LAYOUT_NC32HW32_C32RSK32) == CONV_ERR_INVALID_SHAPE &&
            d == NULL,
        "create empty output");
  CHECK(conv2d_fprop_desc_create(&d, 1, 8192, 8, 8, 32, 4, 4, 1, 1, 1, 1, 1, 1, CONV_DTYPE_INT8,
                                 CONV_LAYOUT_NC32HW32_C32RSK32) == CONV_ERR_OVERFLOW_RISK,
        "create overflow risk");
  CHECK(conv2d_fprop_desc_create(&d, 1, 32, 8, 8, 32, 3, 3, 1, 1, 1, 1, 1, 1, CONV_DTYPE_INT8,
                                 CONV_LAYOUT_NCHW_KCRS) == CONV_ERR_UNSUPPORTED,
        "create unsupported layout");
  CHECK(conv2d_fprop_desc_create(&d, 1 << 16, 1024, 64, 64, 32, 1, 1, 0, 0, 1, 1, 1, 1,
                                 CONV_DTYPE_INT8, CONV_LAYOUT_NC32HW32_C32RSK32) ==
            CONV_ERR_UNSUPPORTED,
        "create tensor over 2^31 bytes");
  CHECK(conv2d_fprop_num_configs((conv_dtype_t)7) == 0, "num_configs unknown dtype");
  CHECK(conv2d_fprop_desc_destroy(NULL) == CONV_OK, "destroy NULL");
  CHECK(conv2d_fprop_run(NULL, NULL, NULL, NULL, 1.0f, 0) == CONV_ERR_NULL, "run null desc");
  CHECK(conv2d_fprop_graph_launch(NULL, 0) == CONV_ERR_NULL, "graph_launch null");
  CHECK(conv2d_fprop_graph_destroy(NULL) == CONV_OK, "graph_destroy NULL");
  /* transform argument errors */
  int8_t *p = (int8_t *)(uintptr_t)0x100000;
  CHECK(conv_nchw_to_nc32hw32_i8(NULL, p, 1, 32, 8, 8, 0) == CONV_ERR_NULL, "transform null");
  CHECK(conv_nchw_to_nc32hw32_i8(p, p + 4096, 0, 32, 8, 8, 0) == CONV_ERR_INVALID_SHAPE,
        "transform empty");
  CHECK(conv_nc32hw32_to_nchw_i8(p, p + 4096, 1, 33, 8, 8, 0) == CONV_ERR_UNSUPPORTED,
        "transform C % 32");
  CHECK(conv_kcrs_to_c32rsk32_i8(p + 1, p + 8192, 32, 32, 3, 3, 0) == CONV_ERR_MISALIGNED,
        "transform misaligned");
  CHECK(conv_c32rsk32_to_kcrs_i8(p, p + 16, 32, 32, 3, 3, 0) == CONV_ERR_UNSUPPORTED,
        "transform overlap");
  for (int s = -1; s <= 9; ++s) CHECK(conv_status_string((conv_status_t)s) != NULL, "status");
  printf("all ok\n");
  return 0;
}
