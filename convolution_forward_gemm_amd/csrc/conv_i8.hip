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
#include "kernels.hpp"

namespace convfprop {

template <int WK, int WP, int FK, int FP, int KT>
struct I8Tile {
  static constexpr int NWAVES = WK * WP;
  static constexpr int THREADS = 64 * NWAVES;
  static constexpr int KB = WK * FK;  // 32-channel blocks per workgroup
  static constexpr int PB = WP * FP;  // 32-pixel blocks per workgroup
  static constexpr int BM = 32 * KB;  // output channels per workgroup
  static constexpr int BN = 32 * PB;  // output pixels per workgroup
  // Blocks of one stage handled per wave (filter and pixel side).
  static_assert((KB * KT) % NWAVES == 0, "filter blocks must split over waves");
  static_assert((PB * KT) % NWAVES == 0, "pixel blocks must split over waves");
  static_assert(KB >= NWAVES ? KB % NWAVES == 0 : (NWAVES % KB == 0 && KT % (NWAVES / KB) == 0), "filter split");
  static_assert(PB >= NWAVES ? PB % NWAVES == 0 : (NWAVES % PB == 0 && KT % (NWAVES / PB) == 0), "pixel split");
  static constexpr int WLOADS = KB * KT / NWAVES;
  static constexpr int XLOADS = PB * KT / NWAVES;
  static constexpr int NPX = PB >= NWAVES ? PB / NWAVES : 1;  // distinct pixels per lane
  static constexpr int NKC = KB >= NWAVES ? KB / NWAVES : 1;  // distinct channels per lane
  static constexpr int STAGE_BYTES = (KB + PB) * KT * 1024;
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
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

template <int WK, int WP, int FK, int FP, int KT>
__global__ void __launch_bounds__(64 * WK * WP)
conv_i8_kernel(const int8_t *__restrict__ x, const int8_t *__restrict__ w,
               int8_t *__restrict__ y, I8Params p) {
  using T = I8Tile<WK, WP, FK, FP, KT>;
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
  int wk_off[T::NKC];
  bool wk_ok[T::NKC];
#pragma unroll
  for (int i = 0; i < T::NKC; ++i) {
    int kb = (T::KB >= T::NWAVES) ? wave + T::NWAVES * i : wave % T::KB;
    int k = k0 + 32 * kb + l32;
    wk_ok[i] = k < p.K;
    wk_off[i] = k * 32 + 16 * half;
  }

  const int ntaps = p.ntaps;
  const int nstages = (ntaps + KT - 1) / KT;
  const int tap_stride_w = p.K * 32;  // bytes between consecutive taps of w

  v4i xbuf[T::XLOADS];
  v4i wbuf[T::WLOADS];

  // Tap t -> (cb, r, s) with s fastest, matching CxRSKx<32>'s tap order.
  auto issue_loads = [&](int stage) {
#pragma unroll
    for (int j = 0; j < T::XLOADS; ++j) {
      int slot, blk, t;
      split_block<T::PB, T::NWAVES, KT>(wave, j, slot, blk, t);
      int tap = stage * KT + t;
      uint32_t off = OOB_OFFSET;
      if (tap < ntaps) {
        int cb = tap / p.RS;
        int rs = tap - cb * p.RS;
        int r = rs / p.S;
        int s = rs - r * p.S;
        int h = px_h0[slot] + r * p.dh;
        int ww = px_w0[slot] + s * p.dw;
        if ((unsigned)h < (unsigned)p.H && (unsigned)ww < (unsigned)p.W)
          off = (uint32_t)(px_base[slot] + (cb * p.HW + r * p.dh * p.W + s * p.dw) * 32);
      }
      xbuf[j] = load_b128(xr, off);
    }
#pragma unroll
    for (int j = 0; j < T::WLOADS; ++j) {
      int slot, blk, t;
      split_block<T::KB, T::NWAVES, KT>(wave, j, slot, blk, t);
      int tap = stage * KT + t;
      uint32_t off = OOB_OFFSET;
      if (tap < ntaps && wk_ok[slot]) off = (uint32_t)(tap * tap_stride_w + wk_off[slot]);
      wbuf[j] = load_b128(wr, off);
    }
  };

  // LDS stage layout: [filter: t][kb][lane] then [pixels: t][pb][lane], 16 B each.
  auto store_stage = [&](int buf) {
    unsigned char *base = lds + buf * T::STAGE_BYTES;
#pragma unroll
    for (int j = 0; j < T::WLOADS; ++j) {
      int slot, blk, t;
      split_block<T::KB, T::NWAVES, KT>(wave, j, slot, blk, t);
      *reinterpret_cast<v4i *>(base + ((t * T::KB + blk) * 64 + lane) * 16) = wbuf[j];
    }
    unsigned char *xb = base + T::KB * KT * 1024;
#pragma unroll
    for (int j = 0; j < T::XLOADS; ++j) {
      int slot, blk, t;
      split_block<T::PB, T::NWAVES, KT>(wave, j, slot, blk, t);
      *reinterpret_cast<v4i *>(xb + ((t * T::PB + blk) * 64 + lane) * 16) = xbuf[j];
    }
  };

  const int wk = wave % WK;  // this wave's channel sub-tile
  const int wp = wave / WK;  // this wave's pixel sub-tile

  v16i acc[FK][FP];
#pragma unroll
  for (int a = 0; a < FK; ++a)
#pragma unroll
    for (int b = 0; b < FP; ++b) acc[a][b] = v16i{0};

  issue_loads(0);
  store_stage(0);
  __syncthreads();

  for (int st = 0; st < nstages; ++st) {
    const int cur = st & 1;
    const bool more = st + 1 < nstages;
    if (more) issue_loads(st + 1);

    const unsigned char *base = lds + cur * T::STAGE_BYTES;
    const unsigned char *xb = base + T::KB * KT * 1024;
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      v4i af[FK], bf[FP];
#pragma unroll
      for (int a = 0; a < FK; ++a)
        af[a] = *reinterpret_cast<const v4i *>(base + ((t * T::KB + wk * FK + a) * 64 + lane) * 16);
#pragma unroll
      for (int b = 0; b < FP; ++b)
        bf[b] = *reinterpret_cast<const v4i *>(xb + ((t * T::PB + wp * FP + b) * 64 + lane) * 16);
#pragma unroll
      for (int a = 0; a < FK; ++a)
#pragma unroll
        for (int b = 0; b < FP; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[a], bf[b], acc[a][b], 0, 0, 0);
    }
    if (more) store_stage(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: int32 -> fp32 -> *alpha -> rint -> clamp -> int8 --------
  // Accumulator layout of v_mfma_i32_32x32x32_i8: lane l, register i holds
  // D[row = 8*(i/4) + 4*(l/32) + i%4][col = l%32].  Rows are channels, so the
  // quad i = 4g..4g+3 is channels 8g + 4*(l/32) + 0..3 of pixel l%32.
  const float alpha = p.alpha;
#pragma unroll
  for (int b = 0; b < FP; ++b) {
    const int m = m0 + 32 * (wp * FP + b) + l32;
    if (m >= p.M) continue;
    const int n = m / p.PQ;
    const int pq = m - n * p.PQ;
#pragma unroll
    for (int a = 0; a < FK; ++a) {
      const int kb = k0 / 32 + wk * FK + a;
      if (kb >= p.KBLK) continue;
      int8_t *dst = y + ((size_t)(n * p.KBLK + kb) * p.PQ + pq) * 32 + 4 * half;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint32_t packed = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float f = (float)acc[a][b][4 * g + e];
          f = f * alpha;
          f = __builtin_rintf(f);
          f = __builtin_fminf(__builtin_fmaxf(f, -128.0f), 127.0f);
          packed |= ((uint32_t)(int)f & 0xffu) << (8 * e);
        }
        *reinterpret_cast<uint32_t *>(dst + 8 * g) = packed;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Configuration table.  Each entry is one compiled tile shape.
// ---------------------------------------------------------------------------
template <int WK, int WP, int FK, int FP, int KT>
static hipError_t launch_i8(const int8_t *x, const int8_t *w, int8_t *y,
                            const I8Params &p, int grid, hipStream_t s) {
  using T = I8Tile<WK, WP, FK, FP, KT>;
  hipLaunchKernelGGL((conv_i8_kernel<WK, WP, FK, FP, KT>), dim3(grid),
                     dim3(T::THREADS), T::LDS_BYTES, s, x, w, y, p);
  return hipGetLastError();
}

#define I8_CFG(WK, WP, FK, FP, KT)                                              \
  I8Config {                                                                    \
    "i8_mfma32x32x32_wg" #WK "x" #WP "_frag" #FK "x" #FP "_kt" #KT "_st2",     \
        I8Tile<WK, WP, FK, FP, KT>::BM, I8Tile<WK, WP, FK, FP, KT>::BN,         \
        I8Tile<WK, WP, FK, FP, KT>::THREADS, I8Tile<WK, WP, FK, FP, KT>::LDS_BYTES, \
        &launch_i8<WK, WP, FK, FP, KT>                                          \
  }

I8Config kI8Configs[] = {
    I8_CFG(2, 2, 2, 2, 2),  // 0: 128 ch x 128 px, 4 waves of 64x64
    I8_CFG(1, 4, 2, 1, 4),  // 1: 64 ch x 128 px, 4 waves of 64x32
    I8_CFG(1, 2, 1, 1, 2),  // 2: 32 ch x 64 px, 2 waves (tiny problems)
    I8_CFG(2, 2, 2, 4, 2),  // 3: 128 ch x 256 px, 4 waves of 64x128
    I8_CFG(2, 2, 4, 2, 2),  // 4: 256 ch x 128 px, 4 waves of 128x64
    I8_CFG(1, 1, 1, 1, 1),  // 5: 32 ch x 32 px, 1 wave
};
int kNumI8Configs = sizeof(kI8Configs) / sizeof(kI8Configs[0]);

}  // namespace convfprop
