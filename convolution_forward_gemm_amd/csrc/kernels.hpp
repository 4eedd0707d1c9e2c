// kernels.hpp -- internal interface between the C ABI (api.hip) and the
// kernel translation units.  Not installed; callers use include/convfprop.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fastdiv.hpp"

namespace convfprop {

// Register-filter halo kernel: how many filter taps ahead of its use each
// wave loads a tap's filter fragments.  The prologue stages that many taps
// in LDS, once per workgroup, before the first MFMA; the kernel and the
// planner (which sizes that LDS) share this count.  Four measured best on
// the 3x3 workloads: a shorter prologue, and enough lead for the ring's loads
// (eight, six, four, three, two and one were tried).
__host__ __device__ constexpr int halo_filter_ahead(int rs) { return rs - 1 < 4 ? rs - 1 : 4; }

// Problem constants of the int8 kernel, precomputed on the host once per
// descriptor.  Byte counts are < 2^31 (checked at descriptor creation).
struct I8Params {
  int M;        // N*P*Q output pixels (GEMM M)
  int PQ, Q;    // output plane size and width
  int H, W, HW; // input height, width, plane size
  int CB;       // C/32 input channel blocks
  int K, KBLK;  // output channels and K/32
  int R, S, RS; // filter height, width, taps per channel block
  int ntaps;    // CB*R*S reduction steps of 32 channels
  int ph, pw, sh, sw, dh, dw;
  int k_tiles;  // workgroup tiles along K
  uint32_t x_bytes, w_bytes, y_bytes;
  float alpha;
  // Per-output-channel scale and bias (device arrays of K floats), or null:
  // then every channel uses alpha and no bias.
  const float *alpha_k, *bias_k;
  // Halo kernel only (see conv_i8_halo.hip): virtual rows per image, halo
  // columns, halo DMA blocks per half-plane, LDS bytes per stage and total.
  int N, HV, WV;
  int halo_dpp;      // 1 KiB LDS-DMA blocks per half-plane
  int halo_bytes;    // both half-planes
  int stage_bytes;   // filter taps + halo of one channel block
  int lds_bytes;     // dynamic LDS of one workgroup
  int pro_off;       // register-filter kernel: LDS offset of the prologue's filter taps
  int P;             // output rows per image
  // Division by the problem's extents in the halo kernels' prologues: by Q,
  // P*Q, HV, k_tiles, WV and the vertical stride (see fastdiv.hpp).
  FastDiv fd_q, fd_pq, fd_hv, fd_kt, fd_wv, fd_sh;
};

typedef hipError_t (*I8LaunchFn)(const int8_t *x, const int8_t *w, int8_t *y,
                                 const I8Params &p, int grid, hipStream_t s);

struct I8Config {
  const char *name;
  int bm;       // output channels per workgroup
  int bn;       // output pixels per workgroup
  int threads;
  int lds_bytes;
  int kt;        // taps per stage (kind 4: channel blocks; kind 5: reduction taps)
  int rs_outer;  // 1: needs (C/32) % kt == 0
  I8LaunchFn launch;
  // Halo kernels (kind 1, 2): compiled filter size, waves, stages, and the
  // most halo DMA blocks per wave per stage they can issue.
  int kind;      // 0: per-tap fragment ring, 1: LDS activation halo + LDS
                 // filter taps, 2: LDS activation halo + filter in registers,
                 // 3: one-pass kernel for small problems (whole reduction in LDS),
                 // 4: the same unrolled for one filter size and channel count
                 // (fr x fs taps over kt channel blocks), in registers,
                 // 5: the same for any problem of exactly kt reduction taps
  int fr, fs, nwaves, ns, hj;
  int pw;   // kind 2: halo row pitch in LDS (0: the halo width; > 0: fixed, dilation 1)
  int cps;  // kind 2: channel blocks per ring stage (C/32 must be a multiple)
  int al;   // kind 2: 1 = filter taps in the LDS ring too, 0 = in registers
  int swz;  // kind 2: swizzled halo rows (pitch pw, a power of two) for horizontal
            // stride swz (1 or 2); 0 = row-major halo
  int rg;   // kind 2 with swz: 1 = the halo comes through registers (coalesced
            // row-major loads, scattered LDS writes), not LDS-DMA
};

// Host-only tables (not const: a const namespace-scope object would also be
// emitted for the device and reference host launch functions).
extern I8Config kI8Configs[];
extern int kNumI8Configs;
extern I8Config kI8HaloConfigs[];
extern int kNumI8HaloConfigs;
extern I8Config kI8SmallConfigs[];
extern int kNumI8SmallConfigs;

// Problem constants of the fp32 kernel.
struct F32Params {
  int M, PQ, Q;
  int C, H, W, HW;
  int K, R, S;
  int ph, pw, sh, sw, dh, dw;
  int k_tiles;
  uint32_t x_bytes, w_bytes;
  float alpha;
  const float *alpha_k, *bias_k;  // per-output-channel scale and bias, or null
  int P;                          // output rows per image
  FastDiv fd_kt, fd_p;            // division by k_tiles and by P (row-halo kernel)
};

typedef hipError_t (*F32LaunchFn)(const float *x, const float *w, float *y,
                                  const F32Params &p, int grid, hipStream_t s);

struct F32Config {
  const char *name;
  int bm, bn, threads, lds_bytes;
  int max_rs;   // largest R*S it runs (double-buffered staging holds a chunk
                // in registers), 0 = any
  F32LaunchFn launch;
  int nk;       // > 0: runs only problems of exactly nk MFMA steps,
                // ceil(C*R*S / 2) (the unrolled tiny kernel)
  int kind;     // 0: staged weights / direct activations, 1: row halo in LDS
  int fr, fs, fdh, fdw, pitch;  // kind 1: compiled filter size, dilation, row pitch
  int dma16;    // kind 1: 16-byte row DMA (pw and W multiples of 4)
};

extern F32Config kF32Configs[];
extern int kNumF32Configs;
extern F32Config kF32HaloConfigs[];
extern int kNumF32HaloConfigs;

// Layout transforms (transforms.hip).
hipError_t launch_nchw_to_nc32(const int8_t *src, int8_t *dst, int N, int C,
                               int HW, hipStream_t s);
hipError_t launch_nc32_to_nchw(const int8_t *src, int8_t *dst, int N, int C,
                               int HW, hipStream_t s);
hipError_t launch_kcrs_to_c32rsk(const int8_t *src, int8_t *dst, int K, int C,
                                 int RS, hipStream_t s);
hipError_t launch_c32rsk_to_kcrs(const int8_t *src, int8_t *dst, int K, int C,
                                 int RS, hipStream_t s);

}  // namespace convfprop
