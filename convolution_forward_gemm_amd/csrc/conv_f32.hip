// conv_f32.hip -- fp32 implicit-GEMM conv2d fprop for gfx950 (MI355X).
//
// What is computed: the general convolution of the POPCORNBENCH "Kimi-K2.6
// l1_p80" transcript (first turn: stride, per-dimension padding and dilation;
// NCHW input, [C_out][C_in][kH][kW] weights), y = alpha * acc in fp32.
//
// How:
//   * Transposed GEMM on fp32 MFMA (v_mfma_f32_32x32x2_f32): MFMA rows are
//     output channels, columns are output pixels, so each accumulator register
//     of a lane holds one channel of one pixel and 32 lanes store 32
//     consecutive pixels of one NCHW output row (128-byte runs).
//   * Reduction order (c, r, s) is regrouped as: for a chunk of CC input
//     channels, for each tap (r, s), for channel pairs -- the two K-slots of
//     one MFMA take channels c and c+1 of the same tap.  Per lane the tap
//     decides padding once (two unsigned compares against the pixel's
//     h0 = p*sh - ph, w0 = q*sw - pw); each channel pair then only adds the
//     plane size to the offset.  Masked lanes read past the buffer end and
//     get zeros.
//   * Weights of a channel chunk are staged once per workgroup into LDS,
//     transposed to [c][r][s][k] (row pitch BM+1) so that an MFMA operand is
//     32 consecutive floats (conflict-free ds_read_b32); the staging reads
//     each output channel's contiguous run of the chunk with whole waves.
//     With DB = 1 the staging is double-buffered: the next chunk's weights
//     are loaded into registers at the start of a chunk, written to the
//     other LDS buffer at its end, and one barrier per chunk separates the
//     two (CC*R*S <= 64*MAXJ).  The activation operand is read
//     straight from global memory (L1/L2 serve the R*S-fold reuse), with a
//     software pipeline of DEPTH taps in flight.
#include "common.hpp"
#include "kernels.hpp"

namespace convfprop {

template <int FK, int FP, int CC, int DEPTH, int NW = 4, int DB = 0>
struct F32Tile {
  static constexpr int NWAVES = NW;
  static constexpr int THREADS = 64 * NW;
  static constexpr int BM = 32 * FK;           // output channels per workgroup
  static constexpr int BN = 32 * FP * NWAVES;  // output pixels per workgroup
  static constexpr int PAIRS = CC / 2;         // MFMAs per tap per fragment
  static constexpr int LDP = BM + 1;           // LDS row pitch of the staged weights
  static constexpr int ROWS = THREADS / 64;    // output channels per staging pass
  static constexpr int KI = BM / ROWS;         // staging passes per 64-weight segment
  static constexpr int MAXJ = 4;               // DB: 64-weight segments held in registers
  static_assert(CC % 2 == 0, "channel chunk must hold whole pairs");
  static_assert(THREADS % 64 == 0 && BM % (THREADS / 64) == 0, "staging rows per pass");
};

// FULLC: C is a multiple of CC, so every chunk holds CC channels and the
// activation loads take the once-per-pixel mask (instantiated per launch).
template <int FK, int FP, int CC, int DEPTH, int NW, int DB, bool FULLC>
__global__ void __launch_bounds__(64 * NW)
conv_f32_kernel(const float *__restrict__ x, const float *__restrict__ w,
                float *__restrict__ y, F32Params p) {
  using T = F32Tile<FK, FP, CC, DEPTH, NW, DB>;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  float *wl = reinterpret_cast<float *>(lds_raw);  // [CC][R][S][LDP]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int ktile = tile % p.k_tiles;
  const int mtile = tile / p.k_tiles;
  const int k0 = ktile * T::BM;
  const int m0 = mtile * T::BN;

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, p.x_bytes);
  const int RS = p.R * p.S;

  // Per-lane pixel decode, once.
  int px_base[FP], px_h0[FP], px_w0[FP];
#pragma unroll
  for (int b = 0; b < FP; ++b) {
    int m = m0 + 32 * (wave * FP + b) + l32;
    if (m < p.M) {
      int n = m / p.PQ;
      int pq = m - n * p.PQ;
      int op = pq / p.Q;
      int oq = pq - op * p.Q;
      px_h0[b] = op * p.sh - p.ph;
      px_w0[b] = oq * p.sw - p.pw;
      px_base[b] = n * p.C * p.HW + px_h0[b] * p.W + px_w0[b];
    } else {
      px_h0[b] = -0x40000000;
      px_w0[b] = -0x40000000;
      px_base[b] = 0;
    }
  }

  v16f acc[FK][FP];
#pragma unroll
  for (int a = 0; a < FK; ++a)
#pragma unroll
    for (int b = 0; b < FP; ++b) acc[a][b] = v16f{0.0f};

  const int crs = CC * RS;  // weights of one output channel in a chunk
  const float alpha = p.alpha;

  // DB: the next chunk's weights, thread (jl, kr) holding W[k0 + kr + ki*ROWS]
  // [c0 ..)[j = ji*64 + jl] (the same element-to-thread map as the staging
  // loop below), and the LDS buffer the current chunk reads.
  float wnext[DB ? T::MAXJ : 1][DB ? T::KI : 1];
  auto wload = [&](int c0n) {
    const int jl = tid & 63;
    const int kr = tid >> 6;
#pragma unroll
    for (int ji = 0; ji < (DB ? T::MAXJ : 1); ++ji) {
      const int j = ji * 64 + jl;
      const int c = c0n + j / RS;
#pragma unroll
      for (int ki = 0; ki < (DB ? T::KI : 1); ++ki) {
        const int k = k0 + kr + ki * T::ROWS;
        wnext[ji][ki] = (j < crs && k < p.K && c < p.C) ? w[((size_t)k * p.C + c0n) * RS + j] : 0.0f;
      }
    }
  };
  // LDS row of weight j = cc*R*S + tap of a chunk: rows go tap-major
  // ([r][s][cc][k]), so the channel-pair stride of the MFMA operand reads is
  // a compile-time constant (immediate offsets) and one add per tap moves
  // them to the next tap
  auto wrow = [&](int j) { return (j % RS) * CC + j / RS; };
  auto wstore = [&](float *buf) {
    const int jl = tid & 63;
    const int kr = tid >> 6;
#pragma unroll
    for (int ji = 0; ji < (DB ? T::MAXJ : 1); ++ji) {
      const int j = ji * 64 + jl;
      if (j < crs) {
#pragma unroll
        for (int ki = 0; ki < (DB ? T::KI : 1); ++ki) buf[wrow(j) * T::LDP + kr + ki * T::ROWS] = wnext[ji][ki];
      }
    }
  };
  if constexpr (DB) {
    wload(0);
    wstore(wl);
    __syncthreads();
  }

  for (int c0 = 0, chunk = 0; c0 < p.C; c0 += CC, ++chunk) {
    float *wcur = wl + (DB ? (chunk & 1) * crs * T::LDP : 0);
    // ---- stage W[k0 .. k0+BM)[c0 .. c0+CC)[r][s] into LDS as [cc][r][s][k].
    // For one output channel the chunk's CC*R*S weights are contiguous in
    // global memory: a wave reads 64 consecutive of them (one row segment)
    // and writes them down an LDS column; the odd row pitch BM+1 keeps
    // those writes on 64 different banks.  No division per element.
    if constexpr (!DB) {
    __syncthreads();
      constexpr int ROWS = T::THREADS / 64;  // output channels per pass
      const int jl = tid & 63;
      const int kr = tid >> 6;
      for (int j0 = 0; j0 < crs; j0 += 64) {
        const int j = j0 + jl;
        const int c = c0 + j / RS;
        const int row = wrow(j);
#pragma unroll 4
        for (int kk = kr; kk < T::BM; kk += ROWS) {
          const int k = k0 + kk;
          float v = 0.0f;
          if (j < crs && k < p.K && c < p.C) v = w[((size_t)k * p.C + c0) * RS + j];
          if (j < crs) wl[row * T::LDP + kk] = v;
        }
      }
    __syncthreads();
    }

    // ---- taps of this chunk, software-pipelined DEPTH deep ---------------
    // For each tap a lane loads T::PAIRS values per pixel fragment: channel
    // c0 + 2*i + half for pair i.  The loader walks (r, s) incrementally.
    // The tap loop is branch-free: it runs a whole number of DEPTH-blocks,
    // and taps past R*S load zeros (and read the last tap's weights), so
    // they add nothing.
    uint32_t chan_off[T::PAIRS];
    bool chan_ok[T::PAIRS];
#pragma unroll
    for (int i = 0; i < T::PAIRS; ++i) {
      const int c = c0 + 2 * i + half;
      chan_ok[i] = c < p.C;
      chan_off[i] = (uint32_t)(c * p.HW);
    }
    uint32_t px_vo[FP];
#pragma unroll
    for (int b = 0; b < FP; ++b) px_vo[b] = (uint32_t)(px_base[b] + half * p.HW) * 4u;
    float ring[DEPTH][T::PAIRS][FP];
    int ld_r = 0, ld_s = 0, ld_tap = 0;
    // With every channel of the chunk present (FULL) a lane masks its pixel
    // once per tap and the channel pair's plane offset rides in the
    // wave-uniform soffset; otherwise each (pixel, pair) is masked.
    auto load_next = [&](float (&dst)[T::PAIRS][FP], auto full_c) {
      constexpr bool FULL = decltype(full_c)::value;
      const bool live = ld_tap < RS;
      const int rdh = ld_r * p.dh, sdw = ld_s * p.dw;
#pragma unroll
      for (int b = 0; b < FP; ++b) {
        const int h = px_h0[b] + rdh;
        const int ww = px_w0[b] + sdw;
        // bitwise, not short-circuit, so that no branch is formed
        const bool ok = live & ((unsigned)h < (unsigned)p.H) & ((unsigned)ww < (unsigned)p.W);
        if constexpr (FULL) {
          // byte offset: the pixel's own part (channel c0 + half folded in)
          // plus the tap's wave-uniform part; uint32 wrap-around is exact
          const uint32_t vo = ok ? px_vo[b] + (uint32_t)(rdh * p.W + sdw) * 4u : OOB_OFFSET;
#pragma unroll
          for (int i = 0; i < T::PAIRS; ++i)
            dst[i][b] = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(xr, vo, (c0 + 2 * i) * p.HW * 4, 0));
        } else {
          const uint32_t base = (uint32_t)(px_base[b] + rdh * p.W + sdw);
#pragma unroll
          for (int i = 0; i < T::PAIRS; ++i)
            dst[i][b] = load_f32(xr, (ok & chan_ok[i]) ? (base + chan_off[i]) * 4u : OOB_OFFSET);
        }
      }
      ++ld_tap;
      if (++ld_s == p.S) {
        ld_s = 0;
        ++ld_r;
      }
    };

    const bool has_next = c0 + CC < p.C;
    auto taps = [&](auto full_c) {
#pragma unroll
    for (int d = 0; d < DEPTH - 1; ++d) load_next(ring[d], full_c);
    // DB: the next chunk's weights go out behind the first activation taps,
    // a whole chunk ahead of their use
    if (DB && has_next) wload(c0 + CC);

    const int rs_blocks = (RS + DEPTH - 1) / DEPTH;
    for (int blk = 0; blk < rs_blocks; ++blk) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        const int tt = blk * DEPTH + d;
        // prefetch DEPTH-1 taps ahead into the slot freed last step; the
        // scheduling barrier keeps the loads at the head of the tap (the
        // scheduler would otherwise sink them next to their use)
        load_next(ring[(d + DEPTH - 1) % DEPTH], full_c);
        __builtin_amdgcn_sched_barrier(0);
        const int ttw = tt < RS ? tt : RS - 1;
#pragma unroll
        for (int i = 0; i < T::PAIRS; ++i) {
          float af[FK];
#pragma unroll
          for (int a = 0; a < FK; ++a)
            af[a] = wcur[(ttw * CC + 2 * i + half) * T::LDP + 32 * a + l32];
#pragma unroll
          for (int a = 0; a < FK; ++a)
#pragma unroll
            for (int b = 0; b < FP; ++b)
              acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[a], ring[d][i][b],
                                                               acc[a][b], 0, 0, 0);
        }
      }
    }
    };
    // one variant per kernel: two copies of the tap loop in one kernel
    // would raise its register use past the occupancy the tiles assume
    taps(std::integral_constant<bool, FULLC>{});
    if constexpr (DB) {
      // the other buffer was last read in the previous chunk, before the
      // barrier that ended it
      if (has_next) wstore(wl + ((chunk + 1) & 1) * crs * T::LDP);
      __syncthreads();
    }
  }

  // ---- epilogue: y[n][k][p][q] = alpha * acc (+ per channel: alpha[k] * acc
  // + bias[k], one multiply then one add) --------------------------------------
  // Accumulator layout of v_mfma_f32_32x32x2_f32: lane l, register i holds
  // D[row = 8*(i/4) + 4*(l/32) + i%4][col = l%32]; rows are channels.
  const float *alpha_k = p.alpha_k, *bias_k = p.bias_k;
#pragma unroll
  for (int b = 0; b < FP; ++b) {
    const int m = m0 + 32 * (wave * FP + b) + l32;
    if (m >= p.M) continue;
    const int n = m / p.PQ;
    const int pq = m - n * p.PQ;
#pragma unroll
    for (int a = 0; a < FK; ++a)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int k = k0 + 32 * a + 8 * (i / 4) + 4 * half + (i % 4);
        if (k < p.K) {
          float v = (alpha_k ? alpha_k[k] : alpha) * acc[a][b][i];
          if (bias_k) v = v + bias_k[k];
          y[((size_t)n * p.K + k) * p.PQ + pq] = v;
        }
      }
  }
}

template <int FK, int FP, int CC, int DEPTH, int NW, int DB>
static hipError_t launch_f32(const float *x, const float *w, float *y,
                             const F32Params &p, int grid, hipStream_t s) {
  using T = F32Tile<FK, FP, CC, DEPTH, NW, DB>;
  const int lds = CC * p.R * p.S * T::LDP * 4 * (DB ? 2 : 1);
  static const hipError_t attr_full = hipFuncSetAttribute(
      reinterpret_cast<const void *>(&conv_f32_kernel<FK, FP, CC, DEPTH, NW, DB, true>),
      hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  static const hipError_t attr_part = hipFuncSetAttribute(
      reinterpret_cast<const void *>(&conv_f32_kernel<FK, FP, CC, DEPTH, NW, DB, false>),
      hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (attr_full != hipSuccess) return attr_full;
  if (attr_part != hipSuccess) return attr_part;
  if (p.C % CC == 0)
    return launch_kernel(&conv_f32_kernel<FK, FP, CC, DEPTH, NW, DB, true>, dim3(grid),
                         dim3(T::THREADS), lds, s, x, w, y, p);
  return launch_kernel(&conv_f32_kernel<FK, FP, CC, DEPTH, NW, DB, false>, dim3(grid),
                       dim3(T::THREADS), lds, s, x, w, y, p);
}

#define F32_CFG_W(FK, FP, CC, DEPTH, NW, DB, NAME)                                   \
  F32Config {                                                                        \
    NAME, F32Tile<FK, FP, CC, DEPTH, NW, DB>::BM, F32Tile<FK, FP, CC, DEPTH, NW, DB>::BN, \
        64 * NW, CC * 4 * F32Tile<FK, FP, CC, DEPTH, NW, DB>::LDP * (DB ? 2 : 1),      \
        DB ? 64 * F32Tile<FK, FP, CC, DEPTH, NW, DB>::MAXJ / CC : 0,                  \
        &launch_f32<FK, FP, CC, DEPTH, NW, DB>                                         \
  }
// Tiny problems (a reduction of at most a few dozen MFMA steps, e.g. the
// first layer of a network on 3 input channels): one wave per 32-channel x
// 32-pixel tile loads every step's filter and pixel values straight into
// registers -- all before the first MFMA -- and runs the NK MFMAs with two
// accumulator chains.  Reduction index j = 2*step + (lane / 32) walks
// (c, r, s) in KCRS order; each lane advances its own (c, r, s) by two per
// step.  Indices past C*R*S, channels past K, pixels past M and padding read
// zeros.  fp32 sums in a different order than the staged kernel: the result
// obeys the same tolerance.
template <int NK>
__global__ void __launch_bounds__(64)
conv_f32_tiny_kernel(const float *__restrict__ x, const float *__restrict__ w,
                     float *__restrict__ y, F32Params p) {
  const int lane = threadIdx.x;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int ktile = blockIdx.x % p.k_tiles;
  const int mtile = blockIdx.x / p.k_tiles;
  const int k0 = ktile * 32, m0 = mtile * 32;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, p.x_bytes);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, p.w_bytes);
  const int RS = p.R * p.S, CRS = p.C * RS;

  int h0 = -0x40000000, w0 = -0x40000000, xbase = 0;
  const int m = m0 + l32;
  if (m < p.M) {
    const int n = m / p.PQ;
    const int pq = m - n * p.PQ;
    const int op = pq / p.Q;
    const int oq = pq - op * p.Q;
    h0 = op * p.sh - p.ph;
    w0 = oq * p.sw - p.pw;
    xbase = n * p.C * p.HW;
  }
  const int k = k0 + l32;
  const bool kok = k < p.K;
  const uint32_t wrow = (uint32_t)(k * CRS);
  // this lane's reduction index j = half at step 0
  int c = 0, r = 0, s = 0;
  auto adv = [&]() {
    if (++s == p.S) {
      s = 0;
      if (++r == p.R) {
        r = 0;
        ++c;
      }
    }
  };
  if (half) adv();
  float a[NK], b[NK];
#pragma unroll
  for (int g = 0; g < NK; ++g) {
    const int j = 2 * g + half;
    const bool jok = j < CRS;
    a[g] = load_f32(wr, (kok & jok) ? (wrow + j) * 4u : OOB_OFFSET);
    const int h = h0 + r * p.dh, ww = w0 + s * p.dw;
    const bool ok = jok & ((unsigned)h < (unsigned)p.H) & ((unsigned)ww < (unsigned)p.W);
    b[g] = load_f32(xr, ok ? (uint32_t)(xbase + c * p.HW + h * p.W + ww) * 4u : OOB_OFFSET);
    adv();
    adv();
  }
  __builtin_amdgcn_sched_barrier(0);  // every load before the first MFMA
  v16f acc[2] = {v16f{0.0f}, v16f{0.0f}};
#pragma unroll
  for (int g = 0; g < NK; ++g)
    acc[g & 1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[g], b[g], acc[g & 1], 0, 0, 0);
  // epilogue as in conv_f32_kernel: register i holds channel
  // 8*(i/4) + 4*half + i%4 of pixel l32
  if (m < p.M) {
    const int n = m / p.PQ;
    const int pq = m - n * p.PQ;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kk = k0 + 8 * (i / 4) + 4 * half + (i % 4);
      if (kk < p.K) {
        const float sum = acc[0][i] + acc[1][i];
        float v = (p.alpha_k ? p.alpha_k[kk] : p.alpha) * sum;
        if (p.bias_k) v = v + p.bias_k[kk];
        y[((size_t)n * p.K + kk) * p.PQ + pq] = v;
      }
    }
  }
}

template <int NK>
static hipError_t launch_f32_tiny(const float *x, const float *w, float *y, const F32Params &p,
                                  int grid, hipStream_t s) {
  return launch_kernel(&conv_f32_tiny_kernel<NK>, dim3(grid), dim3(64), 0, s, x, w, y, p);
}

#define F32_TINY_CFG(NK) \
  F32Config { "f32_tiny_unrolled_steps" #NK "_mfma32x32x2_frag1x1", 32, 32, 64, 0, 0, &launch_f32_tiny<NK>, NK }

#define F32_CFG(FK, FP, CC, DEPTH) \
  F32_CFG_W(FK, FP, CC, DEPTH, 4, 0, "f32_mfma32x32x2_frag" #FK "x" #FP "_cc" #CC "_depth" #DEPTH)
#define F32_CFG16(FK, FP, CC, DEPTH) \
  F32_CFG_W(FK, FP, CC, DEPTH, 16, 0, \
            "f32_mfma32x32x2_16waves_frag" #FK "x" #FP "_cc" #CC "_depth" #DEPTH)
#define F32_CFG8(FK, FP, CC, DEPTH) \
  F32_CFG_W(FK, FP, CC, DEPTH, 8, 0, \
            "f32_mfma32x32x2_8waves_frag" #FK "x" #FP "_cc" #CC "_depth" #DEPTH)
#define F32_CFG16_DB(FK, FP, CC, DEPTH) \
  F32_CFG_W(FK, FP, CC, DEPTH, 16, 1, \
            "f32_mfma32x32x2_16waves_frag" #FK "x" #FP "_cc" #CC "_depth" #DEPTH "_dbuf")

// lds_bytes here is per filter tap (times R*S at launch).
F32Config kF32Configs[] = {
    F32_CFG(2, 2, 4, 3),  // 0: 64 ch x 256 px
    F32_CFG(1, 2, 4, 3),  // 1: 32 ch x 256 px
    F32_CFG(2, 1, 8, 3),  // 2: 64 ch x 128 px, 8-channel chunks
    F32_CFG(2, 2, 4, 5),  // 3: 64 ch x 256 px, deeper activation prefetch
    F32_CFG(2, 2, 4, 2),  // 4: 64 ch x 256 px, shallower prefetch
    F32_CFG8(2, 2, 4, 3),  // 5: 64 ch x 512 px, 8 waves: half the weight staging per pixel
    F32_CFG8(2, 2, 2, 3),  // 6: the same with 2-channel chunks
    F32_CFG16(2, 2, 4, 3), // 7: 64 ch x 1024 px, 16 waves
    F32_CFG8(2, 2, 4, 5),  // 8: 8 waves, deeper activation prefetch
    F32_CFG8(2, 2, 8, 3),  // 9: 8 waves, 8-channel chunks
    // 10: config 7 with double-buffered weight staging.  Its two weight
    // buffers (94 KB at 5x9) leave room for one workgroup per CU, which with
    // 16 waves keeps four per SIMD; an 8-wave workgroup with two buffers
    // drops to two waves per SIMD and runs 7% slower than config 5.
    F32_CFG16_DB(2, 2, 4, 3),
    // tiny problems, exactly NK = ceil(C*R*S / 2) MFMA steps (on 3 input
    // channels: 1x1, 3x3, 5x5, 5x9, 7x7)
    F32_TINY_CFG(2), F32_TINY_CFG(14), F32_TINY_CFG(38), F32_TINY_CFG(68), F32_TINY_CFG(74),
};
int kNumF32Configs = sizeof(kF32Configs) / sizeof(kF32Configs[0]);

}  // namespace convfprop
