// conv_i8.hip -- int8 implicit-GEMM conv2d fprop for gfx950 (MI355X).
//
// What is computed (CUTLASS issue 2996, "How to optimize cutlass int8
// fprop2d kernel with NCxHWx interleaved layout", section "CUTLASS Kernel
// Configuration"): int8 x int8 products accumulated in int32 over the
// reduction C*R*S, then the alpha-only epilogue with a clamp to int8,
//   y = clamp(rint(fl32(fl32(acc) * alpha)), -128, 127),
// with x in NCxHWx<32> ([N][C/32][H][W][32]), w in CxRSKx<32>
// ([C/32][R][S][K][32]) and y in NCxHWx<32> ([N][K/32][P][Q][32]).
//
// How (MI355X design, not the page's Ampere one):
//   * The GEMM is computed transposed, D[k][m] = W[k][:] . X[:][m]: MFMA rows
//     are output channels and MFMA columns are output pixels.  With
//     v_mfma_i32_32x32x32_i8 each lane then ends up holding four consecutive
//     output channels of one pixel per accumulator quad, which packs into one
//     32-bit store of the NCxHWx<32> output with no shuffle.
//   * The reduction runs over "taps" t = (c/32, r, s): one 32-byte channel
//     vector each, which is exactly the K=32 of one MFMA.  In both
//     interleaved layouts the 32 bytes of a tap are contiguous, so every
//     operand fragment is a 16-byte load per lane (lane l: row/column l%32,
//     bytes 16*(l/32)..+16).  Both MFMA operands use that same K split, so
//     the dot product is the same whatever order the hardware pairs the
//     bytes in -- integer sums are exact.
//   * The activation iterator is implicit im2col: per lane, the pixel's
//     (n, h0 = p*sh - ph, w0 = q*sw - pw) is decoded once; per tap only a
//     wave-uniform offset is added and two unsigned compares decide padding.
//     Padded taps, pixels past M and channels past K load from an offset past
//     the end of the buffer, which the buffer unit returns as zeros.
//   * LDS holds each fragment in lane order (1 KiB per 32x32-byte block), so
//     both ds_write_b128 and ds_read_b128 touch 64 consecutive 16-byte slots:
//     no bank conflicts, no swizzle arithmetic.  Two stages of KT taps
//     alternate (global->VGPR prefetch of the next stage overlaps the MFMAs
//     of the current one; one barrier per stage).
//   * The epilogue converts, scales, rounds half-to-even and saturates in
//     registers, then writes four channels per 32-bit store.
#include "common.hpp"
#include "epilogue_i8.hpp"
#include "kernels.hpp"

namespace convfprop {

template <int WK, int WP, int FK, int FP, int KT, int NS>
struct I8Tile {
  static constexpr int NWAVES = WK * WP;
  static constexpr int THREADS = 64 * NWAVES;
  static constexpr int KB = WK * FK;  // 32-channel blocks per workgroup
  static constexpr int PB = WP * FP;  // 32-pixel blocks per workgroup
  static constexpr int BM = 32 * KB;  // output channels per workgroup
  static constexpr int BN = 32 * PB;  // output pixels per workgroup
  // Blocks of one stage are split over the waves (filter and pixel side).
  static_assert(KT % 2 == 0, "fragment double-buffering needs an even tap count per stage");
  static_assert(NS >= 3, "the ring needs a stage being read, one landed and one in flight");
  static_assert((KB * KT) % NWAVES == 0, "filter blocks must split over waves");
  static_assert((PB * KT) % NWAVES == 0, "pixel blocks must split over waves");
  static_assert(KB >= NWAVES ? KB % NWAVES == 0 : (NWAVES % KB == 0 && KT % (NWAVES / KB) == 0), "filter split");
  static_assert(PB >= NWAVES ? PB % NWAVES == 0 : (NWAVES % PB == 0 && KT % (NWAVES / PB) == 0), "pixel split");
  static constexpr int WLOADS = KB * KT / NWAVES;   // 1 KiB filter blocks per wave per stage
  static constexpr int XLOADS = PB * KT / NWAVES;   // 1 KiB pixel blocks per wave per stage
  static constexpr int NL = WLOADS + XLOADS;        // LDS-DMA instructions per wave per stage
  static_assert(NL * (NS - 2) < 64, "vmcnt counts at most 63 outstanding loads");
  static constexpr int NPX = PB >= NWAVES ? PB / NWAVES : 1;  // distinct pixels per lane
  static constexpr int NKC = KB >= NWAVES ? KB / NWAVES : 1;  // distinct channels per lane
  static constexpr int STAGE_BYTES = (KB + PB) * KT * 1024;
  static constexpr int LDS_BYTES = NS * STAGE_BYTES;
};

// Which (block, tap-in-stage) a wave's j-th load of a stage covers.
template <int NB, int NWAVES, int KT>
__device__ __forceinline__ void split_block(int wave, int j, int &blk_slot, int &blk, int &t) {
  if constexpr (NB >= NWAVES) {
    constexpr int per = NB / NWAVES;
    blk_slot = j % per;
    blk = wave + NWAVES * blk_slot;
    t = j / per;
  } else {
    constexpr int rep = NWAVES / NB;
    blk_slot = 0;
    blk = wave % NB;
    t = wave / NB + rep * j;
  }
}

// s_waitcnt with vmcnt(VM), lgkmcnt(0), expcnt untouched (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | ((VM >> 4) << 14));
}

// Workgroup barrier WITHOUT the release/acquire fence of __syncthreads():
// that fence would make the compiler drain every outstanding load (vmcnt(0))
// and so empty the LDS ring.  Visibility of LDS data is established by the
// explicit waits before it; the empty asm keeps the compiler from moving
// memory operations across.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Increments of the activation tap offset when the filter position moves
// by one tap: along S, at the end of a filter row, at the end of a channel
// block.  Offsets are bytes into NCxHWx<32> relative to the pixel's origin.
struct TapSteps {
  int S, R, dh, dw;
  int ds, dr, dcb;  // xoff increments: next s, row wrap, channel-block wrap
};

__device__ __forceinline__ TapSteps make_tap_steps(const I8Params &p) {
  TapSteps t;
  t.S = p.S;
  t.R = p.R;
  t.dh = p.dh;
  t.dw = p.dw;
  t.ds = 32 * p.dw;
  t.dr = 32 * (p.dh * p.W - p.S * p.dw);
  t.dcb = 32 * (p.HW - p.R * p.dh * p.W);
  return t;
}

// Wave-uniform position in the tap sequence t = (cb, r, s), s fastest (the
// tap order of CxRSKx<32>).  Stepping is branch-free: increments and selects.
struct TapWalker {
  int tap, s, r, rdh, sdw, xoff;  // xoff = 32*(cb*HW + r*dh*W + s*dw)
  __device__ __forceinline__ void reset() { tap = s = r = rdh = sdw = xoff = 0; }
  __device__ __forceinline__ void step(const TapSteps &k) {
    ++tap;
    ++s;
    sdw += k.dw;
    xoff += k.ds;
    const bool ws = s == k.S;
    s = ws ? 0 : s;
    sdw = ws ? 0 : sdw;
    r += ws ? 1 : 0;
    rdh += ws ? k.dh : 0;
    xoff += ws ? k.dr : 0;
    const bool wr = r == k.R;
    r = wr ? 0 : r;
    rdh = wr ? 0 : rdh;
    xoff += wr ? k.dcb : 0;
  }
};

// What a stage's loads need to know about one of its taps.
struct TapDesc {
  int live;  // tap < ntaps
  int rdh, sdw, xoff;
};

template <int KT>
__device__ __forceinline__ TapDesc pick_tap(const TapDesc (&td)[KT], int t) {
  TapDesc d = td[0];
#pragma unroll
  for (int i = 1; i < KT; ++i)
    if (t == i) d = td[i];  // folds away when t is a compile-time constant
  return d;
}

// RSO selects the reduction order.  false: taps t = (cb, r, s), s fastest,
// any shape (a wave-uniform walker tracks the tap).  true: (r, s) outer and
// the channel block inner, which needs C/32 % KT == 0: every stage then has a
// single filter position, so the padding mask is evaluated once per stage and
// the KT loads of a lane differ only in a wave-uniform offset.
template <int WK, int WP, int FK, int FP, int KT, int NS, bool RSO, bool PC>
__global__ void __launch_bounds__(64 * WK * WP)
conv_i8_kernel(const int8_t *__restrict__ x, const int8_t *__restrict__ w,
               int8_t *__restrict__ y, I8Params p) {
  using T = I8Tile<WK, WP, FK, FP, KT, NS>;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;   // which 16-byte half of a 32-byte tap vector
  const int l32 = lane & 31;

  // Logical tile (XCD-aware order: consecutive ids share pixel rows).
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int ktile = tile % p.k_tiles;
  const int mtile = tile / p.k_tiles;
  const int k0 = ktile * T::BM;
  const int m0 = mtile * T::BN;

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, p.x_bytes);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, p.w_bytes);

  // ---- per-lane pixel decode (implicit im2col, done once) ----------------
  int px_base[T::NPX], px_h0[T::NPX], px_w0[T::NPX];
#pragma unroll
  for (int i = 0; i < T::NPX; ++i) {
    int pb = (T::PB >= T::NWAVES) ? wave + T::NWAVES * i : wave % T::PB;
    int m = m0 + 32 * pb + l32;
    if (m < p.M) {
      int n = m / p.PQ;
      int pq = m - n * p.PQ;
      int op = pq / p.Q;
      int oq = pq - op * p.Q;
      int h0 = op * p.sh - p.ph;
      int w0 = oq * p.sw - p.pw;
      px_h0[i] = h0;
      px_w0[i] = w0;
      px_base[i] = ((n * p.CB * p.H + h0) * p.W + w0) * 32 + 16 * half;
    } else {
      px_h0[i] = -0x40000000;  // never inside the image: always masked
      px_w0[i] = -0x40000000;
      px_base[i] = 0;
    }
  }
  // ---- per-lane filter channel (fixed across taps) -----------------------
  // The lane's offset within a tap's K x 32 block; channels past K read zeros.
  uint32_t wv[T::NKC];
#pragma unroll
  for (int i = 0; i < T::NKC; ++i) {
    int kb = (T::KB >= T::NWAVES) ? wave + T::NWAVES * i : wave % T::KB;
    int k = k0 + 32 * kb + l32;
    wv[i] = k < p.K ? (uint32_t)(k * 32 + 16 * half) : OOB_OFFSET;
  }

  const int ntaps = p.ntaps;
  const int nstages = (ntaps + KT - 1) / KT;
  const int tap_stride_w = p.K * 32;  // bytes between consecutive taps of w
  const int HW32 = p.HW * 32;         // bytes between channel blocks of x

  // Global -> LDS loads (LDS-DMA) of one stage into ring slot stage % NS.
  // Each instruction moves one 1 KiB fragment block: lane l's 16 bytes land
  // at block + 16*l, which is the MFMA operand order.  The per-lane part of
  // the address is the voffset, a wave-uniform part may go in the soffset.
  // Padded taps, pixels past M and channels past K use OOB_OFFSET as voffset
  // and the buffer unit writes zeros.  The range check sees voffset only, so
  // every in-range access must have a non-negative voffset of its own.
  // soff is wave-uniform by construction (lds_dma16 states so to the
  // compiler, which then keeps it in an SGPR).
  auto dma = [&](__amdgpu_buffer_rsrc_t r, unsigned char *dst, uint32_t voff, int soff) {
    lds_dma16(r, dst, voff, soff);
  };

  // (cb, r, s) walker state for the generic order.
  const TapSteps steps = make_tap_steps(p);
  TapWalker walker;
  walker.reset();
  // (r, s)-outer state: the next stage's first channel block and position.
  int ld_cb0 = 0, ld_rs = 0, ld_s = 0, ld_rdh = 0, ld_sdw = 0, ld_xrs = 0;

  // Stages past the end are still issued, with every lane out of range: they
  // zero-fill the slot of an already consumed stage.  This keeps the loop body
  // free of branches (so the scheduler can interleave it) and the wait counts
  // exact.  An out-of-range voffset makes the whole access out of range, so
  // no address past a buffer is ever formed.
  auto load_next_stage = [&](int stage) {
    unsigned char *base = lds + (stage % NS) * T::STAGE_BYTES;
    unsigned char *xb = base + T::KB * KT * 1024;
    const bool live = stage < nstages;
    if constexpr (RSO) {
      uint32_t xv[T::NPX];  // this stage's padding decision per pixel
#pragma unroll
      for (int i = 0; i < T::NPX; ++i) {
        const int h = px_h0[i] + ld_rdh;
        const int ww = px_w0[i] + ld_sdw;
        // The filter-position part goes into voffset: the buffer range check
        // applies to voffset alone, and a padded pixel's origin (h0 or w0 < 0)
        // is a negative offset that only the in-image tap makes valid.
        xv[i] = (live && (unsigned)h < (unsigned)p.H && (unsigned)ww < (unsigned)p.W)
                    ? (uint32_t)(px_base[i] + ld_xrs)
                    : OOB_OFFSET;
      }
#pragma unroll
      for (int j = 0; j < T::XLOADS; ++j) {
        int slot, blk, t;
        split_block<T::PB, T::NWAVES, KT>(wave, j, slot, blk, t);
        dma(xr, xb + (t * T::PB + blk) * 1024, xv[slot], (ld_cb0 + t) * HW32);
      }
#pragma unroll
      for (int j = 0; j < T::WLOADS; ++j) {
        int slot, blk, t;
        split_block<T::KB, T::NWAVES, KT>(wave, j, slot, blk, t);
        dma(wr, base + (t * T::KB + blk) * 1024, live ? wv[slot] : OOB_OFFSET,
            live ? ((ld_cb0 + t) * p.RS + ld_rs) * tap_stride_w : 0);
      }
      // advance by KT channel blocks; at the end of the blocks, to the next
      // filter position (selects, not branches: the body stays one block)
      ld_cb0 += KT;
      const bool wrap_cb = ld_cb0 == p.CB;
      ld_cb0 = wrap_cb ? 0 : ld_cb0;
      ld_rs += wrap_cb ? 1 : 0;
      ld_s += wrap_cb ? 1 : 0;
      ld_sdw += wrap_cb ? p.dw : 0;
      ld_xrs += wrap_cb ? 32 * p.dw : 0;
      const bool wrap_s = ld_s == p.S;
      ld_s = wrap_s ? 0 : ld_s;
      ld_sdw = wrap_s ? 0 : ld_sdw;
      ld_rdh += wrap_s ? p.dh : 0;
      ld_xrs += wrap_s ? 32 * (p.dh * p.W - p.S * p.dw) : 0;
    } else {
      TapDesc td[KT];
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        td[t].live = walker.tap < ntaps;
        td[t].rdh = walker.rdh;
        td[t].sdw = walker.sdw;
        td[t].xoff = walker.xoff;
        walker.step(steps);
      }
#pragma unroll
      for (int j = 0; j < T::XLOADS; ++j) {
        int slot, blk, t;
        split_block<T::PB, T::NWAVES, KT>(wave, j, slot, blk, t);
        const TapDesc d = pick_tap<KT>(td, t);
        const int h = px_h0[slot] + d.rdh;
        const int ww = px_w0[slot] + d.sdw;
        const bool ok = d.live && (unsigned)h < (unsigned)p.H && (unsigned)ww < (unsigned)p.W;
        dma(xr, xb + (t * T::PB + blk) * 1024,
            ok ? (uint32_t)(px_base[slot] + d.xoff) : OOB_OFFSET, 0);
      }
#pragma unroll
      for (int j = 0; j < T::WLOADS; ++j) {
        int slot, blk, t;
        split_block<T::KB, T::NWAVES, KT>(wave, j, slot, blk, t);
        // Taps past the reduction read tap 0's filter: their activations
        // are zero, so the product is zero either way.
        const int tap = stage * KT + t;
        dma(wr, base + (t * T::KB + blk) * 1024, live ? wv[slot] : OOB_OFFSET,
            tap < ntaps ? tap * tap_stride_w : 0);
      }
    }
  };

  const int wk = wave % WK;  // this wave's channel sub-tile
  const int wp = wave / WK;  // this wave's pixel sub-tile

  // MFMA operand fragments, double-buffered across taps so the LDS reads of
  // tap t+1 are in flight while the MFMAs of tap t run.
  v4i af[2][FK], bf[2][FP];
  auto read_frags = [&](int stage, int t, v4i (&a)[FK], v4i (&b)[FP]) {
    const unsigned char *base = lds + (stage % NS) * T::STAGE_BYTES;
    const unsigned char *xb = base + T::KB * KT * 1024;
#pragma unroll
    for (int i = 0; i < FK; ++i)
      a[i] = *reinterpret_cast<const v4i *>(base + ((t * T::KB + wk * FK + i) * 64 + lane) * 16);
#pragma unroll
    for (int i = 0; i < FP; ++i)
      b[i] = *reinterpret_cast<const v4i *>(xb + ((t * T::PB + wp * FP + i) * 64 + lane) * 16);
  };

  v16i acc[FK][FP];
#pragma unroll
  for (int a = 0; a < FK; ++a)
#pragma unroll
    for (int b = 0; b < FP; ++b) acc[a][b] = v16i{0};

  // Ring schedule.  Barrier B_k (all waves) certifies that stage k has landed
  // and that every wave has finished reading stage k-2; after it, the slot of
  // stage k-2 is refilled with stage k-2+NS.  B_{s+1} sits just before the
  // last tap of stage s, so the first fragments of stage s+1 are read while
  // that tap's MFMAs run.
#pragma unroll
  for (int s0 = 0; s0 < NS - 1; ++s0) load_next_stage(s0);
  wait_vm_lgkm0<T::NL * (NS - 2)>();  // stage 0 landed
  ring_barrier();
  read_frags(0, 0, af[0], bf[0]);

  for (int st = 0; st < nstages; ++st) {
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      if (t + 1 < KT) {
        read_frags(st, t + 1, af[(t + 1) & 1], bf[(t + 1) & 1]);
      } else {
        // stage st+1 landed: all but the NS-3 newest stages are complete
        wait_vm_lgkm0<T::NL * (NS - 3)>();
        ring_barrier();
        load_next_stage(st + NS - 1);          // into the slot of stage st-1
        read_frags(st + 1, 0, af[0], bf[0]);  // KT is even: tap 0 -> buffer 0
      }
#pragma unroll
      for (int a = 0; a < FK; ++a)
#pragma unroll
        for (int b = 0; b < FP; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[t & 1][a], bf[t & 1][b],
                                                            acc[a][b], 0, 0, 0);
      // A wave issues in order and stalls on an MFMA while the matrix unit is
      // busy, so LDS reads or loads placed after a run of MFMAs would wait for
      // the whole run.  Ask the scheduler for MFMA, LDS read, load, MFMA, ...
      // so the memory instructions of the next tap go out under this tap's
      // matrix work.
#pragma unroll
      for (int i = 0; i < FK * FP; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // one global load (LDS-DMA)
      }
    }
  }
  wait_vm_lgkm0<0>();  // no LDS-DMA may outlive the workgroup

  store_i8_tile<PC, FK, FP>(acc, y, p, m0 + 32 * wp * FP, k0 / 32 + wk * FK, lane);
}

// ---------------------------------------------------------------------------
// Configuration table.  Each entry is one compiled tile shape.
// ---------------------------------------------------------------------------
template <int WK, int WP, int FK, int FP, int KT, int NS, bool RSO, bool PC>
static hipError_t launch_i8_pc(const int8_t *x, const int8_t *w, int8_t *y,
                               const I8Params &p, int grid, hipStream_t s) {
  using T = I8Tile<WK, WP, FK, FP, KT, NS>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void *>(&conv_i8_kernel<WK, WP, FK, FP, KT, NS, RSO, PC>),
      hipFuncAttributeMaxDynamicSharedMemorySize, T::LDS_BYTES);
  if (attr != hipSuccess) return attr;
  return launch_kernel(&conv_i8_kernel<WK, WP, FK, FP, KT, NS, RSO, PC>, dim3(grid),
                     dim3(T::THREADS), T::LDS_BYTES, s, x, w, y, p);
}

// Launch with the per-output-channel epilogue when the call carries one.
template <int WK, int WP, int FK, int FP, int KT, int NS, bool RSO>
static hipError_t launch_i8(const int8_t *x, const int8_t *w, int8_t *y,
                            const I8Params &p, int grid, hipStream_t s) {
  return p.alpha_k ? launch_i8_pc<WK, WP, FK, FP, KT, NS, RSO, true>(x, w, y, p, grid, s)
                   : launch_i8_pc<WK, WP, FK, FP, KT, NS, RSO, false>(x, w, y, p, grid, s);
}

#define I8_CFG(WK, WP, FK, FP, KT, NS, RSO)                                     \
  I8Config {                                                                    \
    "i8_mfma32x32x32_wg" #WK "x" #WP "_frag" #FK "x" #FP "_kt" #KT "_ring" #NS  \
    "_rsouter_" #RSO,                                                           \
        I8Tile<WK, WP, FK, FP, KT, NS>::BM, I8Tile<WK, WP, FK, FP, KT, NS>::BN,  \
        I8Tile<WK, WP, FK, FP, KT, NS>::THREADS,                                \
        I8Tile<WK, WP, FK, FP, KT, NS>::LDS_BYTES, KT, RSO,                     \
        &launch_i8<WK, WP, FK, FP, KT, NS, RSO>, 0, 0, 0, WK * WP, NS, 0        \
  }

I8Config kI8Configs[] = {
    // generic tap order (any C/32)
    I8_CFG(2, 2, 2, 2, 2, 4, false),  // 0: 128 ch x 128 px, 4 waves of 64x64
    I8_CFG(1, 4, 2, 1, 4, 4, false),  // 1: 64 ch x 128 px, 4 waves of 64x32
    I8_CFG(1, 2, 1, 1, 2, 4, false),  // 2: 32 ch x 64 px, 2 waves (tiny problems)
    I8_CFG(1, 1, 1, 1, 2, 4, false),  // 3: 32 ch x 32 px, 1 wave
    I8_CFG(2, 2, 4, 2, 2, 4, false),  // 4: 256 ch x 128 px, 4 waves of 128x64
    // (r, s)-outer order (C/32 divisible by the taps per stage)
    I8_CFG(2, 2, 4, 2, 2, 4, true),   // 5: 256 ch x 128 px, 96 KiB ring
    I8_CFG(2, 2, 4, 2, 2, 6, true),   // 6: 256 ch x 128 px, 144 KiB ring
    I8_CFG(2, 2, 4, 2, 4, 3, true),   // 7: 256 ch x 128 px, 4 taps per stage
    I8_CFG(1, 4, 4, 2, 2, 6, true),   // 8: 128 ch x 256 px, 4 waves of 128x64
    I8_CFG(2, 2, 2, 2, 2, 4, true),   // 9: 128 ch x 128 px, 64 KiB ring
    I8_CFG(2, 2, 2, 2, 4, 4, true),   // 10: 128 ch x 128 px, 4 taps per stage
    I8_CFG(2, 4, 2, 2, 2, 6, true),   // 11: 128 ch x 256 px, 8 waves of 64x64
    I8_CFG(4, 2, 2, 2, 2, 6, true),   // 12: 256 ch x 128 px, 8 waves of 64x64
    I8_CFG(2, 4, 2, 2, 4, 3, true),   // 13: 128 ch x 256 px, 8 waves, 4 taps per stage
    I8_CFG(1, 2, 1, 1, 2, 4, true),   // 14: 32 ch x 64 px, 2 waves
    // tiny problems: every stage of a 3x3 / C32 reduction issued up front,
    // so the operands arrive in one memory round trip
    I8_CFG(1, 1, 1, 1, 4, 4, false),  // 15: 9 taps in 3 stages
    I8_CFG(1, 2, 1, 1, 4, 4, false),  // 16: 32 ch x 64 px, 2 waves
    I8_CFG(1, 1, 1, 1, 6, 3, false),  // 17: 9 taps in 2 stages
    I8_CFG(1, 2, 1, 1, 6, 3, false),  // 18
    I8_CFG(2, 2, 1, 1, 4, 4, true),   // 19: 64 ch x 64 px, 4 waves
};
int kNumI8Configs = sizeof(kI8Configs) / sizeof(kI8Configs[0]);

}  // namespace convfprop
