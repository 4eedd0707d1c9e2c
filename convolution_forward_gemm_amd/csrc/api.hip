// api.hip -- the C ABI of libconvfprop.so (declared in include/convfprop.h).
//
// Host-side structure follows two lessons of the CUTLASS notebook "Best
// practices for reducing host-side latency": validate and resolve the kernel
// once ("Compile once, run many times", "Bypassing checks"), so that the run
// call is a pointer check plus one kernel launch; and keep run free of
// allocation, synchronisation and host copies so it can be captured into a
// graph ("CUDA Graphs").  The operator shape (argument checks, then dispatch
// of run-time types to compiled instantiations, then the kernel) is the one
// the torchao PR 1515 review describes for CUTLASS-based operators.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <new>

#include "convfprop.h"
#include "kernels.hpp"

using namespace convfprop;

struct conv2d_fprop_desc_s {
  int N, C, H, W, K, R, S, ph, pw, sh, sw, dh, dw, P, Q;
  conv_dtype_t dtype;
  conv_layout_t layout;
  int config;
  int grid;
  int64_t x_bytes, w_bytes, y_bytes;
  I8Params i8;
  F32Params f32;
};

namespace {

constexpr int64_t kMaxTensorBytes = (int64_t(1) << 31) - 1;

// floor((in + 2*pad - dil*(k-1) - 1) / stride) + 1, or <= 0 if nothing fits.
int64_t out_extent(int64_t in, int64_t pad, int64_t dil, int64_t k, int64_t stride) {
  const int64_t num = in + 2 * pad - dil * (k - 1) - 1;
  if (num < 0) return 0;
  return num / stride + 1;
}

// The integer a C caller passed for an enum parameter.  C lets any int value
// through an enum type; in C++ reading an enum object whose value lies
// outside the enumerators' range is undefined, so the bits are copied out
// instead of loading the enum.
template <typename E>
int enum_bits(const E &e) {
  static_assert(sizeof(E) == sizeof(int), "C enums are int-sized");
  int v;
  memcpy(&v, &e, sizeof v);
  return v;
}

bool ranges_overlap(const void *a, int64_t an, const void *b, int64_t bn) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)bn && b0 < a0 + (uintptr_t)an;
}

// int8 configurations: the per-tap ring kernels, the halo kernels, then the
// one-pass kernels for small problems.
int num_i8_configs() { return kNumI8Configs + kNumI8HaloConfigs + kNumI8SmallConfigs; }

const I8Config *i8_config(int cfg) {
  if (cfg < 0) return nullptr;
  if (cfg < kNumI8Configs) return &kI8Configs[cfg];
  cfg -= kNumI8Configs;
  if (cfg < kNumI8HaloConfigs) return &kI8HaloConfigs[cfg];
  cfg -= kNumI8HaloConfigs;
  if (cfg < kNumI8SmallConfigs) return &kI8SmallConfigs[cfg];
  return nullptr;
}

// fp32 configurations: the staged-weight kernels (and tiny ones), then the
// row-halo kernels.
int num_f32_configs() { return kNumF32Configs + kNumF32HaloConfigs; }

const F32Config *f32_config(int cfg) {
  if (cfg < 0) return nullptr;
  if (cfg < kNumF32Configs) return &kF32Configs[cfg];
  cfg -= kNumF32Configs;
  if (cfg < kNumF32HaloConfigs) return &kF32HaloConfigs[cfg];
  return nullptr;
}

// Index of the configuration with this name, or -1.
int find_config(conv_dtype_t dtype, const char *name) {
  if (dtype == CONV_DTYPE_INT8) {
    for (int i = 0; i < num_i8_configs(); ++i)
      if (strcmp(i8_config(i)->name, name) == 0) return i;
  } else {
    for (int i = 0; i < num_f32_configs(); ++i)
      if (strcmp(f32_config(i)->name, name) == 0) return i;
  }
  return -1;
}

// Per-shape table: the configuration chosen for a problem by sweep, by
// name.  Other shapes are planned by the selection model below.
struct ShapeEntry {
  conv_dtype_t dtype;
  int N, C, H, W, K, R, S, ph, pw, sh, sw, dh, dw;
  const char *config;
};

const ShapeEntry kShapeTable[] = {
    // int8 3x3 N1 C32 8x8 K32 and 1x1 N2 C128 8x8 K128: launch-latency
    // bound, chosen by back-to-back time per call (graph replay); one wave
    // per 32x32 tile loads its whole reduction straight into registers in
    // one memory round trip, each MFMA waiting only for its own tap
    // (unrolled for the filter size and channel count)
    {CONV_DTYPE_INT8, 1, 32, 8, 8, 32, 3, 3, 1, 1, 1, 1, 1, 1,
     "i8_tiny_unrolled_r3s3_cb1_mfma32x32x32_frag1x1"},
    {CONV_DTYPE_INT8, 2, 128, 8, 8, 128, 1, 1, 0, 0, 1, 1, 1, 1,
     "i8_tiny_unrolled_r1s1_cb4_mfma32x32x32_frag1x1"},
    // int8 3x3 N32 C256 28x28 K256: activation halo in LDS, swizzled rows of
    // pitch 32 (bank-conflict-free fragment reads), filter fragments in
    // registers, 128 ch x 224 px tiles (224 workgroups), 8 waves of 32
    // channels with 4 + 3 pixel fragments per SIMD
    {CONV_DTYPE_INT8, 32, 256, 28, 28, 256, 3, 3, 1, 1, 1, 1, 1, 1,
     "i8_halo_regfilter_mfma32x32x32_wg4x2_frag1x4_r3s3_ring4_hj2_pitch32_cps1_pt7_swz"},
    // int8 3x3 stride-2 N32 C128 56x56 K256: the same kernel with a 64-pixel
    // halo row pitch (one row per DMA block) and a 3-stage ring, 256 ch x
    // 128 px tiles: all output channels in one workgroup, so each pixel
    // tile's halo is fetched once, not once per 128-channel half
    {CONV_DTYPE_INT8, 32, 128, 56, 56, 256, 3, 3, 1, 1, 2, 2, 1, 1,
     "i8_halo_regfilter_mfma32x32x32_wg4x2_frag2x2_r3s3_ring3_hj4_pitch64_cps1"},
    // fp32 5x9 dilated N8 C32 512x512 K64: one output row per workgroup, its
    // five input rows and the weights of a channel pair staged in LDS, every
    // tap's operand at an immediate offset; 8 waves of 64 ch x 64 px, one
    // weight buffer (72 KB: two workgroups per CU), rows by 16-byte LDS-DMA
    {CONV_DTYPE_FP32, 8, 32, 512, 512, 64, 5, 9, 2, 4, 1, 1, 2, 3,
     "f32_rowhalo_mfma32x32x2_8waves_frag2x2_r5s9_dil2x3_pitch520_wsingle_dma16"},
};

int lookup_shape(const conv2d_fprop_desc_s &d) {
  for (const ShapeEntry &e : kShapeTable)
    if (e.dtype == d.dtype && e.N == d.N && e.C == d.C && e.H == d.H && e.W == d.W &&
        e.K == d.K && e.R == d.R && e.S == d.S && e.ph == d.ph && e.pw == d.pw &&
        e.sh == d.sh && e.sw == d.sw && e.dh == d.dh && e.dw == d.dw)
      return find_config(d.dtype, e.config);
  return -1;
}

// Configuration-selection model for shapes without a table entry, fitted to
// shape-grid sweeps (fit_select.py): per configuration, its workgroups per
// CU and the coefficients k[0..6] of its predicted time
//   t_us = k0 + R * (k1 + k2 * W + k3 * L + k4 * C / 100 + k5 * Rf * Sf / 10)
//          + k6 * grid * W / 1000,
//   R = ceil(grid / (256 * occupancy)) (rounds of workgroups), W = bm * bn *
//   C * Rf * Sf / 1e6 (a tile's multiply-adds), L = C * Rf * Sf / 1e3.
struct SelectModel {
  conv_dtype_t dtype;
  const char *name;
  int occ;
  float k[7];
};
const SelectModel kSelectModel[] = {
#include "select_model.inc"
    {CONV_DTYPE_INT8, nullptr, 0, {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}},  // end of table
};

int f32_lds_bytes(const conv2d_fprop_desc_s &d, int cfg) {
  const F32Config &c = *f32_config(cfg);
  return c.kind == 1 ? c.lds_bytes : c.lds_bytes * d.R * d.S;
}


// Halo geometry of the LDS-halo kernel for this problem and tile width.
// Returns false if its LDS or per-wave load budget does not fit.
bool plan_halo(const conv2d_fprop_desc_s &d, const I8Config &c, int64_t M, I8Params &p) {
  if (d.R != c.fr || d.S != c.fs) return false;
  const int64_t HV = (int64_t)d.H + 2 * d.ph;
  const int64_t WV = (int64_t)(d.Q - 1) * d.sw + (int64_t)(d.S - 1) * d.dw + 1;
  const int64_t PQ = (int64_t)d.P * d.Q;
  // Virtual row of the first filter row of output pixel m.
  auto vrow = [&](int64_t m) { return (m / PQ) * HV + ((m % PQ) / d.Q) * d.sh; };
  int64_t rows = 0;
  for (int64_t m0 = 0; m0 < M; m0 += c.bn) {
    const int64_t m1 = (m0 + c.bn < M ? m0 + c.bn : M) - 1;
    const int64_t r = vrow(m1) - vrow(m0) + (int64_t)(d.R - 1) * d.dh + 1;
    if (r > rows) rows = r;
  }
  if (c.kind == 2 && c.swz) {
    // swizzled rows: a power-of-two pitch holding the row (its even and odd
    // columns in separate halves at stride 2); any dilation (each lane keeps
    // its per-tap offsets)
    if (d.sw != c.swz) return false;  // compiled for one horizontal stride
    const int64_t need = d.sw == 2 ? 2 * ((WV + 1) / 2) : WV;
    if (need > c.pw) return false;
  } else if (c.pw > 0 && (WV > c.pw || d.dh != 1 || d.dw != 1)) {
    return false;
  }
  const int64_t pitch = c.pw > 0 ? c.pw : WV;   // halo row pitch in LDS, pixels
  // 1 KiB blocks per half-plane: of the LDS layout, or (halo through
  // registers) of the row-major rows of WV pixels the loads bring
  const int64_t dpp = c.rg ? (rows * WV + 63) / 64 : (rows * pitch + 63) / 64;
  const int64_t hblk = 2 * dpp;
  if ((hblk + c.nwaves - 1) / c.nwaves > c.hj) return false;
  // registers: every row of the halo has its slots in half a ring slot
  if (c.rg && rows * pitch > (int64_t)c.hj * c.nwaves * 32) return false;
  // kind 1 (and kind 2 with al) stages the filter taps of a stage's channel
  // blocks in LDS too; kind 2 otherwise keeps them in registers
  const int64_t cps = c.kind == 2 && c.cps > 1 ? c.cps : 1;
  if ((d.C / 32) % cps != 0) return false;
  const int64_t filt =
      c.kind == 1 || (c.kind == 2 && c.al) ? (int64_t)d.R * d.S * (c.bm / 32) * 1024 * cps : 0;
  // a swizzled halo takes the space of every halo DMA slot of the
  // configuration (a compile-time stage size); others only what they use
  const int64_t halo_cap = c.kind == 2 && c.swz ? (int64_t)c.hj * c.nwaves * 1024 : hblk * 1024;
  const int64_t stage = filt + halo_cap * cps;
  int64_t lds = c.ns * stage + 1024;
  // kind 2: the prologue stages the filter of its first halo_filter_ahead
  // taps once in LDS, in the last ring slot (first written at the end of
  // stage 0) if it fits there
  const int64_t apro =
      c.kind == 2 && !c.al ? (int64_t)halo_filter_ahead(d.R * d.S) * (c.bm / 32) * 1024 : 0;
  int64_t pro_off = (c.ns - 1) * stage;
  // (a halo through registers writes the next slot during the first stage,
  // while slower waves may still copy the prologue filter out: its own space)
  if (apro > stage || c.rg) {
    pro_off = lds;
    lds += apro;
  }
  if (lds > 160 * 1024) return false;
  if ((int64_t)d.N * HV > 0x7fffffff) return false;
  p.HV = (int)HV;
  p.WV = (int)WV;
  p.halo_dpp = (int)dpp;
  p.halo_bytes = (int)halo_cap;
  p.stage_bytes = (int)stage;
  p.lds_bytes = (int)lds;
  p.pro_off = (int)pro_off;
  p.fd_hv = make_fastdiv((uint32_t)HV);
  p.fd_wv = make_fastdiv((uint32_t)WV);
  return true;
}

// Fill the launch parameters for configuration `cfg`; false if it cannot run.
bool plan(conv2d_fprop_desc_s &d, int cfg) {
  const int64_t M = (int64_t)d.N * d.P * d.Q;
  if (d.dtype == CONV_DTYPE_INT8) {
    const I8Config *cp = i8_config(cfg);
    if (!cp) return false;
    const I8Config &c = *cp;
    if (c.kind == 0 && c.rs_outer && (d.C / 32) % c.kt != 0) return false;
    const int64_t mt = (M + c.bn - 1) / c.bn, kt = (d.K + c.bm - 1) / c.bm;
    if (mt * kt > 0x7fffffff) return false;
    I8Params &p = d.i8;
    p.M = (int)M;
    p.PQ = d.P * d.Q;
    p.Q = d.Q;
    p.H = d.H;
    p.W = d.W;
    p.HW = d.H * d.W;
    p.CB = d.C / 32;
    p.K = d.K;
    p.KBLK = d.K / 32;
    p.R = d.R;
    p.S = d.S;
    p.RS = d.R * d.S;
    p.ntaps = p.CB * p.RS;
    p.ph = d.ph; p.pw = d.pw; p.sh = d.sh; p.sw = d.sw; p.dh = d.dh; p.dw = d.dw;
    p.k_tiles = (int)kt;
    p.P = d.P;
    p.fd_q = make_fastdiv((uint32_t)d.Q);
    p.fd_pq = make_fastdiv((uint32_t)(d.P * d.Q));
    p.fd_kt = make_fastdiv((uint32_t)kt);
    p.fd_sh = make_fastdiv((uint32_t)d.sh);
    p.fd_hv = p.fd_wv = make_fastdiv(1u);
    p.x_bytes = (uint32_t)d.x_bytes;
    p.w_bytes = (uint32_t)d.w_bytes;
    p.y_bytes = (uint32_t)d.y_bytes;
    p.alpha = 1.0f;
    p.N = d.N;
    p.HV = p.WV = p.halo_dpp = p.halo_bytes = p.stage_bytes = 0;
    p.lds_bytes = c.lds_bytes;
    if ((c.kind == 1 || c.kind == 2) && !plan_halo(d, c, M, p)) return false;
    if (c.kind == 4) {  // unrolled for one filter size and channel count; no LDS
      if (d.R != c.fr || d.S != c.fs || d.C / 32 != c.kt) return false;
      p.lds_bytes = 0;
    }
    if (c.kind == 5) {  // unrolled for exactly kt reduction taps; no LDS
      if (p.ntaps != c.kt) return false;
      p.lds_bytes = 0;
    }
    if (c.kind == 3) {  // the whole reduction in LDS: ntaps filter + pixel fragments
      // every fragment's DMA is in flight at once: at most 63 (vmcnt range)
      const int64_t loads = (int64_t)p.ntaps * (1 + c.bn / 32);
      if (loads > 63) return false;
      p.lds_bytes = (int)(loads * 1024);
    }
    d.grid = (int)(mt * kt);
  } else {
    const F32Config *cp = f32_config(cfg);
    if (!cp) return false;
    const F32Config &c = *cp;
    if (f32_lds_bytes(d, cfg) > 160 * 1024) return false;
    if (c.max_rs > 0 && d.R * d.S > c.max_rs) return false;
    if (c.nk > 0 && ((int64_t)d.C * d.R * d.S + 1) / 2 != c.nk) return false;
    int64_t mt = (M + c.bn - 1) / c.bn;
    const int64_t kt = (d.K + c.bm - 1) / c.bm;
    if (c.kind == 1) {
      // row halo: compiled filter size and dilation, a whole output row per
      // workgroup, the taps of a row within the compiled row pitch
      if (d.R != c.fr || d.S != c.fs || d.dh != c.fdh || d.dw != c.fdw) return false;
      if (d.Q > c.bn) return false;
      const int64_t wv = (int64_t)(d.Q - 1) * d.sw + (int64_t)(d.S - 1) * d.dw + 1;
      if (wv > c.pitch) return false;
      // 16-byte row DMA: whole 4-column quads in or out of the image, 16-byte
      // aligned rows
      if (c.dma16 && (d.pw % 4 != 0 || d.W % 4 != 0)) return false;
      mt = (int64_t)d.N * d.P;  // one output row per workgroup
    }
    if (mt * kt > 0x7fffffff) return false;
    F32Params &p = d.f32;
    p.M = (int)M;
    p.PQ = d.P * d.Q;
    p.Q = d.Q;
    p.C = d.C;
    p.H = d.H;
    p.W = d.W;
    p.HW = d.H * d.W;
    p.K = d.K;
    p.R = d.R;
    p.S = d.S;
    p.ph = d.ph; p.pw = d.pw; p.sh = d.sh; p.sw = d.sw; p.dh = d.dh; p.dw = d.dw;
    p.k_tiles = (int)kt;
    p.x_bytes = (uint32_t)d.x_bytes;
    p.w_bytes = (uint32_t)d.w_bytes;
    p.alpha = 1.0f;
    p.P = d.P;
    p.fd_kt = make_fastdiv((uint32_t)kt);
    p.fd_p = make_fastdiv((uint32_t)d.P);
    d.grid = (int)(mt * kt);
  }
  d.config = cfg;
  return true;
}

// Dynamic LDS bytes and threads of one workgroup of the planned launch.
int desc_lds_bytes(const conv2d_fprop_desc_s &d) {
  return d.dtype == CONV_DTYPE_INT8 ? d.i8.lds_bytes : f32_lds_bytes(d, d.config);
}
int desc_threads(const conv2d_fprop_desc_s &d) {
  return d.dtype == CONV_DTYPE_INT8 ? i8_config(d.config)->threads : f32_config(d.config)->threads;
}

const char *config_name(conv_dtype_t dtype, int cfg) {
  return dtype == CONV_DTYPE_INT8 ? i8_config(cfg)->name : f32_config(cfg)->name;
}

// Predicted microseconds of a planned descriptor under its configuration's
// model entry; negative if the configuration has none.
double select_time(const conv2d_fprop_desc_s &d) {
  const char *name = config_name(d.dtype, d.config);
  for (const SelectModel &m : kSelectModel) {
    if (!m.name || m.dtype != d.dtype || strcmp(m.name, name) != 0) continue;
    const int lds = desc_lds_bytes(d), threads = desc_threads(d);
    int occ = m.occ;
    if (lds > 0 && 163840 / lds < occ) occ = 163840 / lds;
    const int tlim = 2048 / threads > 1 ? 2048 / threads : 1;
    if (tlim < occ) occ = tlim;
    if (occ < 1) occ = 1;
    const int bm = d.dtype == CONV_DTYPE_INT8 ? i8_config(d.config)->bm : f32_config(d.config)->bm;
    const int bn = d.dtype == CONV_DTYPE_INT8 ? i8_config(d.config)->bn : f32_config(d.config)->bn;
    const double R = (double)((d.grid + 256 * occ - 1) / (256 * occ));
    const double crs = (double)d.C * d.R * d.S;
    const double W = (double)bm * bn * crs / 1e6, L = crs / 1e3;
    return m.k[0] +
           R * (m.k[1] + m.k[2] * W + m.k[3] * L + m.k[4] * d.C / 100.0 + m.k[5] * d.R * d.S / 10.0) +
           m.k[6] * d.grid * W / 1000.0;
  }
  return -1.0;
}

// The configuration with the least predicted time among those that plan for
// the problem (earlier configurations win ties); false if none has a model.
bool plan_by_model(conv2d_fprop_desc_s &d) {
  const int n = d.dtype == CONV_DTYPE_INT8 ? num_i8_configs() : num_f32_configs();
  int best = -1;
  double best_t = 0.0;
  for (int c = 0; c < n; ++c) {
    conv2d_fprop_desc_s trial = d;
    if (!plan(trial, c)) continue;
    const double t = select_time(trial);
    if (t < 0.0) continue;
    if (best < 0 || t < best_t) best = c, best_t = t;
  }
  return best >= 0 && plan(d, best);
}

}  // namespace

extern "C" {

const char *conv_status_string(conv_status_t status) {
  switch (enum_bits(status)) {
    case CONV_OK: return "CONV_OK: success";
    case CONV_ERR_NULL: return "CONV_ERR_NULL: a required pointer is NULL";
    case CONV_ERR_INVALID_SHAPE: return "CONV_ERR_INVALID_SHAPE: invalid sizes or empty output";
    case CONV_ERR_UNSUPPORTED: return "CONV_ERR_UNSUPPORTED: problem not supported by this library";
    case CONV_ERR_MISALIGNED: return "CONV_ERR_MISALIGNED: a pointer breaks the required alignment";
    case CONV_ERR_OVERFLOW_RISK: return "CONV_ERR_OVERFLOW_RISK: C*R*S could overflow the int32 accumulator";
    case CONV_ERR_HIP: return "CONV_ERR_HIP: the HIP runtime reported an error";
    case CONV_ERR_NO_MEMORY: return "CONV_ERR_NO_MEMORY: host allocation failed";
    case CONV_ERR_INVALID_ALPHA: return "CONV_ERR_INVALID_ALPHA: int8 alpha must be finite";
  }
  return "unknown conv_status_t";
}

conv_status_t conv2d_fprop_desc_create(conv2d_fprop_desc_t *out, int N, int C,
                                       int H, int W, int K, int R, int S,
                                       int pad_h, int pad_w, int stride_h,
                                       int stride_w, int dil_h, int dil_w,
                                       conv_dtype_t dtype, conv_layout_t layout) {
  if (!out) return CONV_ERR_NULL;
  *out = nullptr;
  if (N <= 0 || C <= 0 || H <= 0 || W <= 0 || K <= 0 || R <= 0 || S <= 0 ||
      pad_h < 0 || pad_w < 0 || stride_h <= 0 || stride_w <= 0 || dil_h <= 0 ||
      dil_w <= 0)
    return CONV_ERR_INVALID_SHAPE;
  const int64_t P = out_extent(H, pad_h, dil_h, R, stride_h);
  const int64_t Q = out_extent(W, pad_w, dil_w, S, stride_w);
  if (P < 1 || Q < 1) return CONV_ERR_INVALID_SHAPE;

  const int dt = enum_bits(dtype), lay = enum_bits(layout);
  int64_t esize;
  if (dt == CONV_DTYPE_INT8 && lay == CONV_LAYOUT_NC32HW32_C32RSK32) {
    if (C % 32 != 0 || K % 32 != 0) return CONV_ERR_UNSUPPORTED;
    // |acc| <= C*R*S * 128 * 128 must stay below 2^31.
    if ((int64_t)C * R * S >= 131072) return CONV_ERR_OVERFLOW_RISK;
    esize = 1;
  } else if (dt == CONV_DTYPE_FP32 && lay == CONV_LAYOUT_NCHW_KCRS) {
    esize = 4;
  } else {
    return CONV_ERR_UNSUPPORTED;
  }
  const int64_t xb = (int64_t)N * C * H * W * esize;
  const int64_t wb = (int64_t)K * C * R * S * esize;
  const int64_t yb = (int64_t)N * K * P * Q * esize;
  if (xb > kMaxTensorBytes || wb > kMaxTensorBytes || yb > kMaxTensorBytes)
    return CONV_ERR_UNSUPPORTED;

  conv2d_fprop_desc_s *d = new (std::nothrow) conv2d_fprop_desc_s();
  if (!d) return CONV_ERR_NO_MEMORY;
  d->N = N; d->C = C; d->H = H; d->W = W; d->K = K; d->R = R; d->S = S;
  d->ph = pad_h; d->pw = pad_w; d->sh = stride_h; d->sw = stride_w;
  d->dh = dil_h; d->dw = dil_w; d->P = (int)P; d->Q = (int)Q;
  d->dtype = dtype;
  d->layout = layout;
  d->x_bytes = xb;
  d->w_bytes = wb;
  d->y_bytes = yb;

  bool ok = false;
  const int cfg = lookup_shape(*d);
  if (cfg >= 0) ok = plan(*d, cfg);
  if (!ok) ok = plan_by_model(*d);
  if (!ok) {  // try every compiled configuration before giving up
    const int n = dtype == CONV_DTYPE_INT8 ? num_i8_configs() : num_f32_configs();
    for (int c = 0; c < n && !ok; ++c) ok = plan(*d, c);
  }
  if (!ok) {
    delete d;
    return CONV_ERR_UNSUPPORTED;
  }
  *out = d;
  return CONV_OK;
}

conv_status_t conv2d_fprop_desc_destroy(conv2d_fprop_desc_t desc) {
  delete desc;
  return CONV_OK;
}

conv_status_t conv2d_fprop_desc_get_output_dims(conv2d_fprop_desc_t d, int *P, int *Q) {
  if (!d || !P || !Q) return CONV_ERR_NULL;
  *P = d->P;
  *Q = d->Q;
  return CONV_OK;
}

conv_status_t conv2d_fprop_desc_get_config(conv2d_fprop_desc_t d, char *buf, size_t n) {
  if (!d || !buf) return CONV_ERR_NULL;
  if (n == 0) return CONV_OK;
  const bool i8 = d->dtype == CONV_DTYPE_INT8;
  const char *name = i8 ? i8_config(d->config)->name : f32_config(d->config)->name;
  const int bm = i8 ? i8_config(d->config)->bm : f32_config(d->config)->bm;
  const int bn = i8 ? i8_config(d->config)->bn : f32_config(d->config)->bn;
  snprintf(buf, n, "config=%d %s tile=%dch x %dpx grid=%d lds=%d threads=%d", d->config, name,
           bm, bn, d->grid, desc_lds_bytes(*d), desc_threads(*d));
  return CONV_OK;
}

int conv2d_fprop_num_configs(conv_dtype_t dtype) {
  const int dt = enum_bits(dtype);
  if (dt == CONV_DTYPE_INT8) return num_i8_configs();
  if (dt == CONV_DTYPE_FP32) return num_f32_configs();
  return 0;
}

conv_status_t conv2d_fprop_desc_set_config(conv2d_fprop_desc_t d, int config) {
  if (!d) return CONV_ERR_NULL;
  conv2d_fprop_desc_s trial = *d;
  if (!plan(trial, config)) return CONV_ERR_UNSUPPORTED;
  *d = trial;
  return CONV_OK;
}

static conv_status_t run_impl(conv2d_fprop_desc_t d, const void *x, const void *w, void *y,
                              float alpha, const float *alpha_k, const float *bias_k,
                              hipStream_t stream) {
  hipError_t e;
  if (d->dtype == CONV_DTYPE_INT8) {
    I8Params p = d->i8;
    p.alpha = alpha;
    p.alpha_k = alpha_k;
    p.bias_k = bias_k;
    e = i8_config(d->config)->launch((const int8_t *)x, (const int8_t *)w, (int8_t *)y, p,
                                     d->grid, stream);
  } else {
    F32Params p = d->f32;
    p.alpha = alpha;
    p.alpha_k = alpha_k;
    p.bias_k = bias_k;
    e = f32_config(d->config)->launch((const float *)x, (const float *)w, (float *)y, p,
                                      d->grid, stream);
  }
  return e == hipSuccess ? CONV_OK : CONV_ERR_HIP;
}

static conv_status_t check_run(conv2d_fprop_desc_t d, const void *x, const void *w,
                               const void *y) {
  if (!d || !x || !w || !y) return CONV_ERR_NULL;
  const uintptr_t align = d->dtype == CONV_DTYPE_INT8 ? 16 : 4;
  if (((uintptr_t)x | (uintptr_t)w | (uintptr_t)y) & (align - 1)) return CONV_ERR_MISALIGNED;
  if (ranges_overlap(x, d->x_bytes, y, d->y_bytes) ||
      ranges_overlap(w, d->w_bytes, y, d->y_bytes))
    return CONV_ERR_UNSUPPORTED;
  return CONV_OK;
}

conv_status_t conv2d_fprop_run(conv2d_fprop_desc_t d, const void *x, const void *w,
                               void *y, float alpha, hipStream_t stream) {
  const conv_status_t st = check_run(d, x, w, y);
  if (st != CONV_OK) return st;
  if (d->dtype == CONV_DTYPE_INT8 && !isfinite(alpha)) return CONV_ERR_INVALID_ALPHA;
  return run_impl(d, x, w, y, alpha, nullptr, nullptr, stream);
}

conv_status_t conv2d_fprop_run_scaled(conv2d_fprop_desc_t d, const void *x, const void *w,
                                      void *y, const float *alpha, const float *bias,
                                      hipStream_t stream) {
  const conv_status_t st = check_run(d, x, w, y);
  if (st != CONV_OK) return st;
  if (!alpha) return CONV_ERR_NULL;
  if (((uintptr_t)alpha | (uintptr_t)bias) & 15) return CONV_ERR_MISALIGNED;
  const int64_t kb = (int64_t)d->K * 4;
  if (ranges_overlap(alpha, kb, y, d->y_bytes) || (bias && ranges_overlap(bias, kb, y, d->y_bytes)))
    return CONV_ERR_UNSUPPORTED;
  return run_impl(d, x, w, y, 1.0f, alpha, bias, stream);
}

// ---- graph capture of repeated runs ----------------------------------------
struct conv2d_fprop_graph_s {
  hipGraphExec_t exec = nullptr;
};

conv_status_t conv2d_fprop_graph_create(conv2d_fprop_graph_t *out, conv2d_fprop_desc_t d,
                                        const void *x, const void *w, void *y, float alpha,
                                        int calls) {
  if (!out) return CONV_ERR_NULL;
  *out = nullptr;
  conv_status_t st = check_run(d, x, w, y);
  if (st != CONV_OK) return st;
  if (d->dtype == CONV_DTYPE_INT8 && !isfinite(alpha)) return CONV_ERR_INVALID_ALPHA;
  if (calls < 1 || calls > 4096) return CONV_ERR_INVALID_SHAPE;
  conv2d_fprop_graph_s *g = new (std::nothrow) conv2d_fprop_graph_s();
  if (!g) return CONV_ERR_NO_MEMORY;
  // capture on a private stream, so the caller's streams are untouched
  hipStream_t s = nullptr;
  hipGraph_t graph = nullptr;
  st = CONV_ERR_HIP;
  if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) == hipSuccess) {
    if (hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal) == hipSuccess) {
      conv_status_t rs = CONV_OK;
      for (int i = 0; i < calls && rs == CONV_OK; ++i)
        rs = run_impl(d, x, w, y, alpha, nullptr, nullptr, s);
      const hipError_t ec = hipStreamEndCapture(s, &graph);
      if (rs == CONV_OK && ec == hipSuccess &&
          hipGraphInstantiate(&g->exec, graph, nullptr, nullptr, 0) == hipSuccess)
        st = CONV_OK;
      if (graph) (void)hipGraphDestroy(graph);
    }
    (void)hipStreamDestroy(s);
  }
  if (st != CONV_OK) {
    delete g;
    return st;
  }
  *out = g;
  return CONV_OK;
}

conv_status_t conv2d_fprop_graph_launch(conv2d_fprop_graph_t g, hipStream_t stream) {
  if (!g) return CONV_ERR_NULL;
  return hipGraphLaunch(g->exec, stream) == hipSuccess ? CONV_OK : CONV_ERR_HIP;
}

conv_status_t conv2d_fprop_graph_destroy(conv2d_fprop_graph_t g) {
  if (!g) return CONV_OK;
  const hipError_t e = hipGraphExecDestroy(g->exec);
  delete g;
  return e == hipSuccess ? CONV_OK : CONV_ERR_HIP;
}

// ---- layout transforms ----------------------------------------------------
static conv_status_t check_transform(const int8_t *src, int8_t *dst, int a, int C, int b,
                                     int c) {
  if (!src || !dst) return CONV_ERR_NULL;
  if (a <= 0 || C <= 0 || b <= 0 || c <= 0) return CONV_ERR_INVALID_SHAPE;
  if (C % 32 != 0) return CONV_ERR_UNSUPPORTED;
  const int64_t bytes = (int64_t)a * C * b * c;
  if (bytes > kMaxTensorBytes) return CONV_ERR_UNSUPPORTED;
  if (((uintptr_t)src | (uintptr_t)dst) & 15) return CONV_ERR_MISALIGNED;
  if (ranges_overlap(src, bytes, dst, bytes)) return CONV_ERR_UNSUPPORTED;
  return CONV_OK;
}

conv_status_t conv_nchw_to_nc32hw32_i8(const int8_t *src, int8_t *dst, int N, int C,
                                       int H, int W, hipStream_t stream) {
  conv_status_t s = check_transform(src, dst, N, C, H, W);
  if (s != CONV_OK) return s;
  return launch_nchw_to_nc32(src, dst, N, C, H * W, stream) == hipSuccess ? CONV_OK
                                                                           : CONV_ERR_HIP;
}

conv_status_t conv_nc32hw32_to_nchw_i8(const int8_t *src, int8_t *dst, int N, int C,
                                       int H, int W, hipStream_t stream) {
  conv_status_t s = check_transform(src, dst, N, C, H, W);
  if (s != CONV_OK) return s;
  return launch_nc32_to_nchw(src, dst, N, C, H * W, stream) == hipSuccess ? CONV_OK
                                                                           : CONV_ERR_HIP;
}

conv_status_t conv_kcrs_to_c32rsk32_i8(const int8_t *src, int8_t *dst, int K, int C,
                                       int R, int S, hipStream_t stream) {
  conv_status_t s = check_transform(src, dst, K, C, R, S);
  if (s != CONV_OK) return s;
  return launch_kcrs_to_c32rsk(src, dst, K, C, R * S, stream) == hipSuccess ? CONV_OK
                                                                             : CONV_ERR_HIP;
}

conv_status_t conv_c32rsk32_to_kcrs_i8(const int8_t *src, int8_t *dst, int K, int C,
                                       int R, int S, hipStream_t stream) {
  conv_status_t s = check_transform(src, dst, K, C, R, S);
  if (s != CONV_OK) return s;
  return launch_c32rsk_to_kcrs(src, dst, K, C, R * S, stream) == hipSuccess ? CONV_OK
                                                                             : CONV_ERR_HIP;
}

}  // extern "C"
