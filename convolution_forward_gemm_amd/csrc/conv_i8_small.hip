// conv_i8_small.hip -- int8 implicit-GEMM conv fprop for problems too small
// to fill the GPU (latency bound: a few workgroups, a reduction of a few
// dozen 32-channel taps).
//
// The operation and the epilogue are those of CUTLASS issue 2996 ("How to
// optimize cutlass int8 fprop2d kernel with NCxHWx interleaved layout"),
// section "CUTLASS Kernel Configuration", as in conv_i8.hip.  For these
// shapes the time is launch, the memory round trips before the first MFMA,
// and instruction fetch of a cold kernel; the matrix work is a few hundred
// nanoseconds.  So:
//   - one wave per workgroup computes one 32-channel x (32*FP)-pixel tile,
//     needing no barrier;
//   - a rolled loop issues the LDS-DMA of every tap's filter and pixel
//     fragments at once (one memory round trip), and one vmcnt(0) waits for
//     all of them;
//   - a rolled loop then runs the taps (ds_read + MFMA);
//   - loops stay rolled so that the kernel's code is a few hundred bytes.
// Every fragment's DMA is in flight at once, so ntaps * (1 + FP) <= 63 (the
// vmcnt range); the reduction then needs at most 63 KiB of LDS.
#include "common.hpp"
#include "epilogue_i8.hpp"
#include "kernels.hpp"

namespace convfprop {

template <int FP, bool PC>
__global__ void __launch_bounds__(64)
conv_i8_small_kernel(const int8_t *__restrict__ x, const int8_t *__restrict__ w,
                     int8_t *__restrict__ y, I8Params p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int lane = threadIdx.x;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int ktile = blockIdx.x % p.KBLK;
  const int mtile = blockIdx.x / p.KBLK;
  const int m0 = mtile * 32 * FP;

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, p.x_bytes);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, p.w_bytes);

  // filter: this lane's output channel, its 16 input channels of a tap
  const uint32_t a_off = (uint32_t)((ktile * 32 + l32) * 32 + 16 * half);
  // pixels: origin of the filter window per fragment (or out of range)
  int h0[FP], w0[FP];
  uint32_t pbase[FP];
#pragma unroll
  for (int i = 0; i < FP; ++i) {
    const int m = m0 + 32 * i + l32;
    if (m < p.M) {
      const int n = m / p.PQ;
      const int pq = m - n * p.PQ;
      const int op = pq / p.Q;
      const int oq = pq - op * p.Q;
      h0[i] = op * p.sh - p.ph;
      w0[i] = oq * p.sw - p.pw;
      pbase[i] = (uint32_t)(n * p.CB * p.HW * 32 + 16 * half);
    } else {
      h0[i] = -(1 << 28);  // every tap out of range
      w0[i] = 0;
      pbase[i] = 0;
    }
  }

  // One pass over every tap: filter fragment to slot g of the filter area,
  // pixel fragments to slots g of the pixel area.  Taps in (cb, r, s) order.
  unsigned char *const fa = lds;
  unsigned char *const pa = lds + p.ntaps * 1024;
  const int KB32 = p.K * 32;
  int r = 0, s = 0, cb = 0;
#pragma nounroll
  for (int g = 0; g < p.ntaps; ++g) {
    lds_dma16(wr, fa + g * 1024, a_off, g * KB32);
#pragma unroll
    for (int i = 0; i < FP; ++i) {
      const int h = h0[i] + r * p.dh;
      const int ww = w0[i] + s * p.dw;
      const bool in = (unsigned)h < (unsigned)p.H && (unsigned)ww < (unsigned)p.W;
      const uint32_t off = in ? pbase[i] + (uint32_t)(((cb * p.H + h) * p.W + ww) * 32) : OOB_OFFSET;
      lds_dma16(xr, pa + (g * FP + i) * 1024, off, 0);
    }
    if (++s == p.S) {
      s = 0;
      if (++r == p.R) {
        r = 0;
        ++cb;
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) expcnt(0) lgkmcnt(0): all taps landed
  asm volatile("" ::: "memory");

  v16i acc[1][FP];
#pragma unroll
  for (int i = 0; i < FP; ++i) acc[0][i] = v16i{0};
#pragma nounroll
  for (int g = 0; g < p.ntaps; ++g) {
    const v4i a = *reinterpret_cast<const v4i *>(fa + g * 1024 + lane * 16);
#pragma unroll
    for (int i = 0; i < FP; ++i) {
      const v4i b = *reinterpret_cast<const v4i *>(pa + (g * FP + i) * 1024 + lane * 16);
      acc[0][i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[0][i], 0, 0, 0);
    }
  }

  store_i8_tile<PC, 1, FP>(acc, y, p, m0, ktile, lane);
}

template <int FP, bool PC>
static hipError_t launch_i8_small_pc(const int8_t *x, const int8_t *w, int8_t *y, const I8Params &p,
                                     int grid, hipStream_t s) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void *>(&conv_i8_small_kernel<FP, PC>),
      hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (attr != hipSuccess) return attr;
  return launch_kernel(&conv_i8_small_kernel<FP, PC>, dim3(grid), dim3(64), p.lds_bytes, s, x, w, y,
                     p);
}

template <int FP>
static hipError_t launch_i8_small(const int8_t *x, const int8_t *w, int8_t *y, const I8Params &p,
                                  int grid, hipStream_t s) {
  return p.alpha_k ? launch_i8_small_pc<FP, true>(x, w, y, p, grid, s)
                   : launch_i8_small_pc<FP, false>(x, w, y, p, grid, s);
}

// Fully unrolled one-pass variant for one filter size and channel count
// (R x S taps over CB channel blocks, fixed at compile time), one 32 x 32
// tile per wave.  Every tap's filter and pixel fragments are loaded straight
// into registers, in tap order; each MFMA then waits only for its own tap's
// two loads (the compiler's in-order vmcnt accounting), so the matrix work
// starts when the first tap lands rather than after the last, and no LDS
// round trip sits between the loads and the MFMAs.  Even and odd taps
// accumulate separately (two independent MFMA chains) and are summed at
// the end; integer sums, so the result is the same.
template <int R, int S, int CB, bool PC>
__global__ void __launch_bounds__(64)
conv_i8_tiny_kernel(const int8_t *__restrict__ x, const int8_t *__restrict__ w,
                    int8_t *__restrict__ y, I8Params p) {
  constexpr int NT = R * S * CB;
  const int lane = threadIdx.x;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int ktile = blockIdx.x % p.KBLK;
  const int mtile = blockIdx.x / p.KBLK;
  const int m0 = mtile * 32;

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, p.x_bytes);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, p.w_bytes);
  const uint32_t a_off = (uint32_t)((ktile * 32 + l32) * 32 + 16 * half);
  int h0 = -(1 << 28), w0 = 0;
  uint32_t pbase = 0;
  const int m = m0 + l32;
  if (m < p.M) {
    const int n = m / p.PQ;
    const int pq = m - n * p.PQ;
    const int op = pq / p.Q;
    const int oq = pq - op * p.Q;
    h0 = op * p.sh - p.ph;
    w0 = oq * p.sw - p.pw;
    pbase = (uint32_t)(n * CB * p.HW * 32 + 16 * half);
  }
  const int KB32 = p.K * 32;
  v4i a[NT], b[NT];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int g = (cb * R + r) * S + s;
        a[g] = load_b128_s(wr, a_off, g * KB32);
        const int h = h0 + r * p.dh;
        const int ww = w0 + s * p.dw;
        const bool in = (unsigned)h < (unsigned)p.H && (unsigned)ww < (unsigned)p.W;
        b[g] = load_b128(xr, in ? pbase + (uint32_t)(((cb * p.H + h) * p.W + ww) * 32) : OOB_OFFSET);
      }
  // every load goes out before the first MFMA (the scheduler would otherwise
  // trade registers for loads issued behind earlier waits: several memory
  // round trips instead of one)
  __builtin_amdgcn_sched_barrier(0);
  v16i acc[2] = {v16i{0}, v16i{0}};
#pragma unroll
  for (int g = 0; g < NT; ++g)
    acc[g & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[g], b[g], acc[g & 1], 0, 0, 0);
  v16i sum[1][1] = {{acc[0] + acc[1]}};
  store_i8_tile<PC, 1, 1>(sum, y, p, m0, ktile, lane);
}

template <int R, int S, int CB, bool PC>
static hipError_t launch_i8_tiny_pc(const int8_t *x, const int8_t *w, int8_t *y, const I8Params &p,
                                    int grid, hipStream_t s) {
  return launch_kernel(&conv_i8_tiny_kernel<R, S, CB, PC>, dim3(grid), dim3(64), 0, s, x, w, y, p);
}

template <int R, int S, int CB>
static hipError_t launch_i8_tiny(const int8_t *x, const int8_t *w, int8_t *y, const I8Params &p,
                                 int grid, hipStream_t s) {
  return p.alpha_k ? launch_i8_tiny_pc<R, S, CB, true>(x, w, y, p, grid, s)
                   : launch_i8_tiny_pc<R, S, CB, false>(x, w, y, p, grid, s);
}

// The same for any problem with exactly NT reduction taps (channel blocks x
// filter taps): the (cb, r, s) walk runs at run time, the load and MFMA
// sequence is unrolled for NT.
template <int NT, bool PC>
__global__ void __launch_bounds__(64)
conv_i8_tinyn_kernel(const int8_t *__restrict__ x, const int8_t *__restrict__ w,
                     int8_t *__restrict__ y, I8Params p) {
  const int lane = threadIdx.x;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int ktile = blockIdx.x % p.KBLK;
  const int mtile = blockIdx.x / p.KBLK;
  const int m0 = mtile * 32;

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, p.x_bytes);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, p.w_bytes);
  const uint32_t a_off = (uint32_t)((ktile * 32 + l32) * 32 + 16 * half);
  int h0 = -(1 << 28), w0 = 0;
  uint32_t pbase = 0;
  const int m = m0 + l32;
  if (m < p.M) {
    const int n = m / p.PQ;
    const int pq = m - n * p.PQ;
    const int op = pq / p.Q;
    const int oq = pq - op * p.Q;
    h0 = op * p.sh - p.ph;
    w0 = oq * p.sw - p.pw;
    pbase = (uint32_t)(n * p.CB * p.HW * 32 + 16 * half);
  }
  const int KB32 = p.K * 32;
  v4i a[NT], b[NT];
  int cb = 0, r = 0, s = 0;
#pragma unroll
  for (int g = 0; g < NT; ++g) {
    a[g] = load_b128_s(wr, a_off, g * KB32);
    const int h = h0 + r * p.dh;
    const int ww = w0 + s * p.dw;
    const bool in = (unsigned)h < (unsigned)p.H && (unsigned)ww < (unsigned)p.W;
    b[g] = load_b128(xr, in ? pbase + (uint32_t)(((cb * p.H + h) * p.W + ww) * 32) : OOB_OFFSET);
    if (++s == p.S) {
      s = 0;
      if (++r == p.R) {
        r = 0;
        ++cb;
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // every load before the first MFMA
  v16i acc[2] = {v16i{0}, v16i{0}};
#pragma unroll
  for (int g = 0; g < NT; ++g)
    acc[g & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[g], b[g], acc[g & 1], 0, 0, 0);
  v16i sum[1][1] = {{acc[0] + acc[1]}};
  store_i8_tile<PC, 1, 1>(sum, y, p, m0, ktile, lane);
}

template <int NT, bool PC>
static hipError_t launch_i8_tinyn_pc(const int8_t *x, const int8_t *w, int8_t *y, const I8Params &p,
                                     int grid, hipStream_t s) {
  return launch_kernel(&conv_i8_tinyn_kernel<NT, PC>, dim3(grid), dim3(64), 0, s, x, w, y, p);
}

template <int NT>
static hipError_t launch_i8_tinyn(const int8_t *x, const int8_t *w, int8_t *y, const I8Params &p,
                                  int grid, hipStream_t s) {
  return p.alpha_k ? launch_i8_tinyn_pc<NT, true>(x, w, y, p, grid, s)
                   : launch_i8_tinyn_pc<NT, false>(x, w, y, p, grid, s);
}

// kind 5: exactly kt reduction taps (C/32 * R * S)
#define I8_TINYN_CFG(NT)                                                            \
  I8Config {                                                                        \
    "i8_tiny_unrolled_taps" #NT "_mfma32x32x32_frag1x1", 32, 32, 64, 0, NT, 0,      \
        &launch_i8_tinyn<NT>, 5, 0, 0, 1, 1, 0, 0, 1                                \
  }

// kind 4: fr x fs filter and kt channel blocks exactly
#define I8_TINY_CFG(R, S, CB)                                                       \
  I8Config {                                                                        \
    "i8_tiny_unrolled_r" #R "s" #S "_cb" #CB "_mfma32x32x32_frag1x1", 32, 32, 64, 0, CB, 0, \
        &launch_i8_tiny<R, S, CB>, 4, R, S, 1, 1, 0, 0, 1                           \
  }

#define I8_SMALL_CFG(FP)                                                            \
  I8Config {                                                                        \
    "i8_small_onepass_mfma32x32x32_frag1x" #FP, 32, 32 * FP, 64, 0, 0, 0,           \
        &launch_i8_small<FP>, 3, 0, 0, 1, 1, 0, 0, 1                                \
  }

I8Config kI8SmallConfigs[] = {
    I8_SMALL_CFG(1),  // 32 ch x 32 px per wave
    I8_SMALL_CFG(2),  // 32 ch x 64 px per wave
    I8_TINY_CFG(3, 3, 1),  // 3x3 over 32 channels
    I8_TINY_CFG(1, 1, 4),  // 1x1 over 128 channels
    // any filter, exactly NT = C/32 * R * S reduction taps
    I8_TINYN_CFG(2), I8_TINYN_CFG(3), I8_TINYN_CFG(4), I8_TINYN_CFG(6), I8_TINYN_CFG(8),
    I8_TINYN_CFG(9), I8_TINYN_CFG(12), I8_TINYN_CFG(16), I8_TINYN_CFG(18), I8_TINYN_CFG(25),
    I8_TINYN_CFG(27), I8_TINYN_CFG(36),
};
int kNumI8SmallConfigs = sizeof(kI8SmallConfigs) / sizeof(kI8SmallConfigs[0]);

}  // namespace convfprop
