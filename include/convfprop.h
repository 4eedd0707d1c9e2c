/*
 * convfprop.h -- C ABI of libconvfprop.so: 2D convolution forward (fprop)
 * computed as an implicit GEMM on MI355X (gfx950).
 *
 * The operation (cross-correlation, zero padding, no filter flip):
 *
 *   acc[n][k][p][q] = sum_{c,r,s} X(n, c, p*stride_h - pad_h + r*dil_h,
 *                                     q*stride_w - pad_w + s*dil_w) * w[k][c][r][s]
 *
 * with X = x inside the image and 0 outside, and output extents
 *   P = floor((H + 2*pad_h - dil_h*(R-1) - 1) / stride_h) + 1   (Q likewise),
 * the rule derived in the first turn of the POPCORNBENCH "Kimi-K2.6 l1_p80"
 * transcript.  As a GEMM: M = N*P*Q output pixels, N = K output channels,
 * reduction = C*R*S.
 *
 * Two paths are supported:
 *
 *   INT8 / NC32HW32_C32RSK32 -- the int8 kernel of CUTLASS issue 2996 ("How
 *     to optimize cutlass int8 fprop2d kernel with NCxHWx interleaved layout"),
 *     section "CUTLASS Kernel Configuration": int8 x int8 products, int32
 *     accumulation, alpha-only fp32 scaling and a clamp to int8:
 *       y = clamp(rint(fl32(fl32(acc) * alpha)), -128, 127)
 *     (one int32->fp32 conversion, one fp32 multiply, round half to even).
 *     Memory layouts, all int8, dense, no padding between elements:
 *       x: NCxHWx<32>  = [N][C/32][H][W][32]
 *       w: CxRSKx<32>  = [C/32][R][S][K][32]
 *       y: NCxHWx<32>  = [N][K/32][P][Q][32]
 *     C and K must be multiples of 32.
 *
 *   FP32 / NCHW_KCRS -- the general fp32 case of the transcript (stride,
 *     dilation, per-dimension padding): x NCHW fp32, w KCRS fp32
 *     ([K][C][R][S]), y NKPQ fp32, y = alpha * acc with fp32 accumulation.
 *
 * Conventions shared by every entry point:
 *   - Pointers x, w, y, src, dst are DEVICE pointers owned by the caller; the
 *     library never allocates, frees or copies them.  x/w/src are read only.
 *   - `stream` is a HIP stream (0 = the null stream).  Every call only
 *     enqueues work on it and returns; nothing synchronises, allocates device
 *     memory or copies between host and device, so calls may be captured in a
 *     HIP graph.  Completion is observed by the caller (stream/event sync).
 *   - Errors are return codes; no call aborts, throws or prints.  When a call
 *     returns an error, nothing was enqueued and outputs are untouched.
 *   - Each tensor must be smaller than 2^31 bytes (32-bit buffer offsets).
 */
#ifndef CONVFPROP_H
#define CONVFPROP_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CONV_OK = 0,
    CONV_ERR_NULL = 1,           /* a required pointer is NULL                    */
    CONV_ERR_INVALID_SHAPE = 2,  /* a size <= 0, a pad < 0, or no output position */
    CONV_ERR_UNSUPPORTED = 3,    /* valid problem this library does not handle   */
    CONV_ERR_MISALIGNED = 4,     /* a device pointer breaks the required alignment */
    CONV_ERR_OVERFLOW_RISK = 5,  /* int8 C*R*S could overflow the int32 accumulator */
    CONV_ERR_HIP = 6,            /* the HIP runtime reported an error on launch   */
    CONV_ERR_NO_MEMORY = 7,      /* host allocation of the descriptor failed      */
    CONV_ERR_INVALID_ALPHA = 8   /* int8 path: alpha is not a finite number       */
} conv_status_t;

typedef enum { CONV_DTYPE_INT8 = 0, CONV_DTYPE_FP32 = 1 } conv_dtype_t;

typedef enum {
    CONV_LAYOUT_NCHW_KCRS = 0,          /* fp32 path                   */
    CONV_LAYOUT_NC32HW32_C32RSK32 = 1   /* int8 path, interleaved x32  */
} conv_layout_t;

/* Opaque, immutable problem descriptor ("compile once, run many times":
 * all validation and kernel selection happen at creation, as the CUTLASS
 * host-latency notes recommend).  A descriptor may be used by concurrent
 * run calls on different streams. */
typedef struct conv2d_fprop_desc_s *conv2d_fprop_desc_t;

/* Validate a problem and choose its kernel configuration: the tuned
 * configuration of a per-shape table, else the one a cost model fitted to
 * configuration sweeps predicts fastest among those that can run it.  This is
 * where the CUTLASS notebook "Best practices for reducing host-side latency"
 * puts the work of its sections "Compile once, run many times" and "Bypassing
 * checks for argument-Operator compatibility": every check and every choice
 * happens here once, on the host, with no GPU call.
 *   out         receives the descriptor (set to NULL on error)
 *   N,C,H,W     input batch, channels, height, width        (> 0)
 *   K,R,S       output channels, filter height, filter width (> 0)
 *   pad_*       zero padding applied to both sides           (>= 0)
 *   stride_*, dil_*                                           (> 0)
 * Supported (dtype, layout): (INT8, NC32HW32_C32RSK32) with C % 32 == 0,
 * K % 32 == 0 and C*R*S < 131072 (so |acc| <= C*R*S*128*128 < 2^31), and
 * (FP32, NCHW_KCRS).  Returns CONV_ERR_INVALID_SHAPE if P or Q < 1. */
conv_status_t conv2d_fprop_desc_create(conv2d_fprop_desc_t *out, int N, int C,
                                       int H, int W, int K, int R, int S,
                                       int pad_h, int pad_w, int stride_h,
                                       int stride_w, int dil_h, int dil_w,
                                       conv_dtype_t dtype, conv_layout_t layout);

/* Release a descriptor.  NULL is accepted and ignored.  The descriptor is
 * the library's counterpart of the compiled artifact of the CUTLASS notebook
 * "Best practices for reducing host-side latency", section "Compile once, run
 * many times": made once, reused by every run, released by the caller. */
conv_status_t conv2d_fprop_desc_destroy(conv2d_fprop_desc_t desc);

/* Output extents P (rows) and Q (columns) of a descriptor:
 *   P = floor((H + 2*pad_h - dil_h*(R-1) - 1) / stride_h) + 1, Q likewise,
 * the rule the first turn of the POPCORNBENCH "Kimi-K2.6 l1_p80" transcript
 * derives (512 -> 508 rows and 512 -> 496 columns for its dilated 5x9
 * problem).  P and Q must not be NULL (CONV_ERR_NULL). */
conv_status_t conv2d_fprop_desc_get_output_dims(conv2d_fprop_desc_t desc,
                                                int *P, int *Q);

/* NUL-terminated text naming the chosen kernel configuration, truncated to
 * buf_size bytes: "config=<index> <name> tile=<ch>ch x <px>px grid=<work-
 * groups> lds=<bytes per workgroup> threads=<per workgroup>".  It reports the
 * per-shape choice that the TVM BYOC CUTLASS integration (apache/tvm PR
 * 9261) makes with its profiler, and that the torchao PR 1515 review holds
 * to be necessary (kernel parameters tuned to the input shapes); the fields mirror
 * the tile, warp and stage parameters listed in CUTLASS issue 2996, section
 * "CUTLASS Kernel Configuration".  buf_size 0 writes nothing. */
conv_status_t conv2d_fprop_desc_get_config(conv2d_fprop_desc_t desc, char *buf,
                                           size_t buf_size);

/* Number of kernel configurations compiled for a dtype, and a replacement of
 * a descriptor's configuration by index.  These are the candidate set and
 * the per-candidate trial of the profiler-based kernel selection in the TVM
 * BYOC CUTLASS integration (apache/tvm PR 9261), used here by the sweep that
 * builds the per-shape table.  set_config returns CONV_ERR_UNSUPPORTED, and
 * leaves the descriptor unchanged, if that configuration cannot run the
 * problem; num_configs returns 0 for an unknown dtype. */
int conv2d_fprop_num_configs(conv_dtype_t dtype);
conv_status_t conv2d_fprop_desc_set_config(conv2d_fprop_desc_t desc, int config);

/* Enqueue one convolution on `stream`: the operation of CUTLASS issue 2996,
 * section "CUTLASS Kernel Configuration" (int8), or of the first turn of the
 * "Kimi-K2.6 l1_p80" transcript (fp32), as stated at the top of this file.
 * Following the CUTLASS notebook "Best practices for reducing host-side
 * latency", section "Bypassing checks for argument-Operator compatibility",
 * every problem check was done once by desc_create; run only checks the
 * pointers (null, alignment, overlap) and launches one kernel.
 *   x     device input  (layout per the descriptor)
 *   w     device filter (layout per the descriptor)
 *   y     device output (layout per the descriptor); fully overwritten
 *   alpha output scale (int8: applied before rounding, must be finite --
 *         an infinite or NaN alpha returns CONV_ERR_INVALID_ALPHA, since
 *         0 * inf and NaN have no int8 value; fp32: y = alpha*acc, any value)
 * The int8 path needs x, w and y 16-byte aligned; the fp32 path 4-byte.
 * x and w must not overlap y. */
conv_status_t conv2d_fprop_run(conv2d_fprop_desc_t desc, const void *x,
                               const void *w, void *y, float alpha,
                               hipStream_t stream);

/* Enqueue one convolution with a scale and a bias per output channel (the
 * "rowwise scaled" operators named in the review thread of torchao issue
 * 1406, read as one scale and one bias per GEMM column = output channel):
 *   int8: y = clamp(rint(fl32(fl32(fl32(acc) * alpha[k]) + bias[k])), -128, 127)
 *   fp32: y = fl32(alpha[k] * acc) + bias[k]
 * (one multiply, then one add; never a fused multiply-add).
 *   alpha  device array of K floats (required)
 *   bias   device array of K floats, or NULL for no bias
 * x, w, y as for conv2d_fprop_run.  alpha and bias must be 16-byte aligned
 * and must not overlap y.  The values are read on the device, so they are
 * not checked: a non-finite alpha[k] or bias[k] gives unspecified int8
 * values in channel k (never a fault). */
conv_status_t conv2d_fprop_run_scaled(conv2d_fprop_desc_t desc, const void *x,
                                      const void *w, void *y, const float *alpha,
                                      const float *bias, hipStream_t stream);

/* Repeated runs as one HIP graph (the "CUDA Graphs" section of the CUTLASS
 * host-latency notes): `calls` back-to-back runs of `desc` on the fixed
 * buffers x, w, y with scale alpha are captured once, on a private stream,
 * and instantiated; each launch then enqueues all of them on `stream` with
 * one call and no per-kernel host work.  Creation is a setup step (it
 * creates and destroys a stream, and the runtime allocates the graph's
 * resources); launch only enqueues.  The buffers must stay valid for the
 * graph's lifetime.  1 <= calls <= 4096; the argument checks and errors are
 * those of conv2d_fprop_run.  Destroy with conv2d_fprop_graph_destroy (NULL
 * is accepted). */
typedef struct conv2d_fprop_graph_s *conv2d_fprop_graph_t;
conv_status_t conv2d_fprop_graph_create(conv2d_fprop_graph_t *out,
                                        conv2d_fprop_desc_t desc, const void *x,
                                        const void *w, void *y, float alpha,
                                        int calls);
conv_status_t conv2d_fprop_graph_launch(conv2d_fprop_graph_t graph,
                                        hipStream_t stream);
conv_status_t conv2d_fprop_graph_destroy(conv2d_fprop_graph_t graph);

/* Layout transforms (pure permutations, int8) into and out of the
 * interleaved layouts that CUTLASS issue 2996 names in section "CUTLASS
 * Kernel Configuration" (cutlass::layout::TensorNCxHWx<32> for the
 * activation and output, TensorCxRSKx<32> for the filter; the TensorRT kernel
 * of section "TensorRT Kernel Name" reads the same activation layout,
 * "nchw_vect_c_32").  The memory orders are the plainest reading of those
 * names:
 *   NCHW [N][C][H][W]          <-> NCxHWx<32> [N][C/32][H][W][32]
 *   KCRS [K][C][R][S]          <-> CxRSKx<32> [C/32][R][S][K][32]
 * src and dst are device pointers owned by the caller, must not overlap and
 * must both be 16-byte aligned; C must be a multiple of 32 and the tensor
 * under 2^31 bytes.  Errors: CONV_ERR_NULL, CONV_ERR_INVALID_SHAPE (a size
 * <= 0), CONV_ERR_UNSUPPORTED (C % 32, size, overlap), CONV_ERR_MISALIGNED,
 * CONV_ERR_HIP (launch failure).  Each call enqueues one kernel. */
conv_status_t conv_nchw_to_nc32hw32_i8(const int8_t *src, int8_t *dst, int N,
                                       int C, int H, int W, hipStream_t stream);
conv_status_t conv_nc32hw32_to_nchw_i8(const int8_t *src, int8_t *dst, int N,
                                       int C, int H, int W, hipStream_t stream);
conv_status_t conv_kcrs_to_c32rsk32_i8(const int8_t *src, int8_t *dst, int K,
                                       int C, int R, int S, hipStream_t stream);
conv_status_t conv_c32rsk32_to_kcrs_i8(const int8_t *src, int8_t *dst, int K,
                                       int C, int R, int S, hipStream_t stream);

/* Static description of a status code (never NULL).  Status codes, not
 * exceptions, carry the outcome of the argument checks that the torchao PR
 * 1515 review puts at the head of an operator (checks, then dispatch, then
 * the kernel). */
const char *conv_status_string(conv_status_t status);

#ifdef __cplusplus
}
#endif
#endif /* CONVFPROP_H */
