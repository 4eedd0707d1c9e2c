// conv_f32_halo.hip -- fp32 implicit-GEMM conv2d fprop for gfx950 with the
// activation rows of an output row staged in LDS (filter size and dilation
// fixed at compile time).
//
// What is computed is the general fp32 convolution of the POPCORNBENCH
// "Kimi-K2.6 l1_p80" transcript (first turn: stride, per-dimension padding
// and dilation; NCHW input, [C_out][C_in][kH][kW] weights), y = alpha * acc.
// This kernel serves the transcript's own shape family: a 5x9 filter with
// dilation (2, 3), every output row of which reads exactly R input rows.
//
// How:
//   * One workgroup computes one output row (n, p) for BM output channels:
//     NW waves, each FK x FP fragments of v_mfma_f32_32x32x2_f32 (rows =
//     output channels, columns = 32 consecutive output pixels; the MFMA's
//     two K slots take input channels c and c+1 of one tap).
//   * Per input-channel pair the workgroup stages, in LDS:
//       - the R input rows the output row reads, p*sh - ph + r*DH, one
//         PITCH-float row each, as [channel of the pair][r][column], column
//         j holding input column j - pw (zeros outside the image), brought in
//         by LDS-DMA: 16 bytes per lane (whole 4-column quads, when pw and W
//         are multiples of 4; 2% faster on the 512 x 512 problem than 4
//         bytes per lane) or 4 bytes per lane, out-of-image lanes reading
//         zeros through an out-of-range offset;
//       - the pair's weights transposed to [channel of the pair][tap][k],
//         loaded into registers a pair ahead (eight threads per output
//         channel, each element at a constant offset from the thread's
//         base) and written to LDS.
//     The tap (r, s) operand of pixel q is then at r*PITCH + q*sw + s*DW:
//     the lane's pixel is its address register, the tap an immediate offset.
//     The loop body is one LDS read per MFMA, no address arithmetic; the
//     reads of tap t+1 are scheduled ahead of tap t's MFMAs.
//   * Two row stages: the next pair's rows go out (LDS-DMA) and its weights
//     are loaded into registers at the start of a pair; both land behind the
//     pair's R*S*FK*FP MFMAs per wave.  With one weight buffer (WDB = 0) the
//     weights are written between two barriers at the pair's end, with two
//     (WDB = 1) after one.
//   * Bank-conflict-free reads: a plane (one channel) of rows or of weights
//     is a multiple of 64 floats plus 32, so the two lane halves (channels c
//     and c+1) read disjoint banks; weight tap rows are BM + 8 floats, so the
//     transposing writes of a wave (8 channels x 8 taps) hit 64 banks.
//   * Registers: 114-126 VGPRs, four waves per SIMD: two workgroups per CU
//     (with one weight buffer), each hiding the other's staging and
//     barriers.
#include "common.hpp"
#include "kernels.hpp"

namespace convfprop {

template <int FK, int FP, int NW, int R, int S, int DH, int DW, int PITCH, int WDB, int D16 = 0>
struct F32HaloTile {
  static constexpr int THREADS = 64 * NW;
  static constexpr int BM = 32 * FK;       // output channels per workgroup
  static constexpr int BN = 32 * FP * NW;  // output pixels of the row covered
  static constexpr int RS = R * S;
  static constexpr int ROWF = R * PITCH;                      // floats of one plane's rows
  // D16: rows come in by 16-byte LDS-DMA (256 floats per instruction; the
  // problem keeps pw and W multiples of 4), else by 4-byte LDS-DMA
  static constexpr int DBLK = D16 ? 256 : 64;                 // floats per DMA instruction
  static constexpr int BPP = (ROWF + DBLK - 1) / DBLK;        // DMA blocks per plane
  static constexpr int PLANE = BPP * DBLK + 32;               // >= BPP*DBLK, = 32 (mod 64)
  static constexpr int ACT = 2 * PLANE;                       // floats: the pair's rows
  // weights of a pair as [ci][t][kk]: tap rows of KP = BM + 1 floats (= 1 mod
  // 64 for BM = 64: the transposing writes of consecutive taps land on
  // consecutive banks) in channel planes of CIS floats (= 32 mod 64: the two
  // lane halves of an operand read hit disjoint banks)
  // Eight threads per output channel stage its 2*RS weights; tap rows of
  // BM + 8 floats put a wave's writes (eight channels, each thread's taps
  // 8 apart) on 64 distinct banks.
  static constexpr int KP = BM + 8;
  static constexpr int CIS = (RS * KP + 31) / 64 * 64 + 32 >= RS * KP ? (RS * KP + 31) / 64 * 64 + 32
                                                                     : (RS * KP + 31) / 64 * 64 + 96;
  static constexpr int WT = 2 * CIS;                          // floats: the pair's weights
  // rows are double-buffered; the weights too with WDB = 1, else one buffer
  // rewritten between two barriers per pair (less LDS: two workgroups per CU)
  static constexpr int WOFF = 2 * ACT;                        // first weight buffer
  static constexpr int LDS_BYTES = (2 * ACT + (WDB ? 2 : 1) * WT) * 4;
  static constexpr int DMA_BLOCKS = 2 * BPP;                  // per pair
  static constexpr int DJ = (DMA_BLOCKS + NW - 1) / NW;       // DMAs per wave per pair
  static constexpr int WELEM = BM * 2 * RS;                   // weights per pair
  static constexpr int WJ = (2 * RS + 7) / 8;                 // weights per thread
  static_assert(THREADS == 8 * BM, "eight threads per output channel");
  static_assert(PLANE >= BPP * DBLK && PLANE % 64 == 32, "plane pitch");
  static_assert(!D16 || PITCH % 4 == 0, "16-byte DMA blocks hold whole rows' quads");
  static_assert(CIS % 64 == 32 && CIS >= RS * KP, "weight channel plane pitch");
  static_assert(LDS_BYTES <= 160 * 1024, "two stages must fit in LDS");
  static_assert(DJ < 64, "vmcnt range");
};

template <int FK, int FP, int NW, int R, int S, int DH, int DW, int PITCH, int WDB, int D16>
__global__ void __launch_bounds__(64 * NW)
conv_f32_halo_kernel(const float *__restrict__ x, const float *__restrict__ w,
                     float *__restrict__ y, F32Params p) {
  using T = F32HaloTile<FK, FP, NW, R, S, DH, DW, PITCH, WDB, D16>;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  float *lds = reinterpret_cast<float *>(lds_raw);  // [2][ACT rows] [1 or 2][WT weights]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;

  // workgroup -> (k tile, image, output row); neighbouring rows share an XCD
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int row = fast_div(tile, p.fd_kt);  // n * P + p
  const int ktile = tile - row * p.k_tiles;
  const int k0 = ktile * T::BM;
  const int n = fast_div(row, p.fd_p);
  const int op = row - n * p.P;

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, p.x_bytes);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, p.w_bytes);
  const int HW = p.HW;
  const int NPAIR = (p.C + 1) >> 1;

  // ---- activation DMA sources: lane l of block g = plane * BPP + b loads
  // float f = 64 b + l of the plane, row f / PITCH, column f % PITCH; the
  // pair's first channel plane offset rides in the wave-uniform soffset ----
  uint32_t a_off[T::DJ];
  int a_dst[T::DJ];  // float offset in a stage, or -1 for none
#pragma unroll
  for (int j = 0; j < T::DJ; ++j) {
    const int g = j * NW + wave;
    uint32_t off = OOB_OFFSET;
    int dst = -1;
    if (g < T::DMA_BLOCKS) {
      const int pl = g >= T::BPP;
      const int b = g - pl * T::BPP;
      const int f = b * T::DBLK + lane * (D16 ? 4 : 1);
      const int r = f / PITCH;
      const int col = f - r * PITCH;
      const int h = op * p.sh - p.ph + r * DH;
      const int iw = col - p.pw;
      if (r < R && (unsigned)h < (unsigned)p.H && (unsigned)iw < (unsigned)p.W)
        off = (uint32_t)((((n * p.C + pl) * p.H + h) * p.W + iw) * 4);
      dst = pl * T::PLANE + b * T::DBLK;
    }
    a_off[j] = off;
    a_dst[j] = dst;
  }
  // channels past C (odd C, last pair) load zeros
  auto issue_act = [&](int pair, float *stage) __attribute__((always_inline)) {
    const int c0 = 2 * pair;
#pragma unroll
    for (int j = 0; j < T::DJ; ++j) {
      if (a_dst[j] < 0) continue;  // wave-uniform
      const bool ok = c0 + (a_dst[j] >= T::PLANE) < p.C;
      if constexpr (D16)
        lds_dma16(xr, reinterpret_cast<unsigned char *>(stage + a_dst[j]), ok ? a_off[j] : OOB_OFFSET,
                  c0 * HW * 4);
      else
        lds_dma4(xr, stage + a_dst[j], ok ? a_off[j] : OOB_OFFSET, c0 * HW * 4);
    }
  };

  // ---- weights of a pair: element e = kk * 2*RS + ci * RS + t of the
  // pair's contiguous run per output channel, into LDS [ci][t][kk] --------
  // Thread tid stages output channel k0 + tid/8, elements part + 8j
  // (part = tid % 8) of the pair's contiguous 2*RS-float run: one base
  // offset per thread, the pair in the wave-uniform soffset, the element a
  // constant.  (Spreading consecutive threads over consecutive elements
  // instead needs a division per element and ~20 more VGPRs, which kept the
  // kernel at three waves per SIMD: one workgroup per CU, 7% slower.)
  float wreg[T::WJ];
  const int w_kk = tid >> 3, w_part = tid & 7;
  const uint32_t w_base =
      k0 + w_kk < p.K ? (uint32_t)(((k0 + w_kk) * p.C * T::RS + w_part) * 4) : OOB_OFFSET;
  auto load_w = [&](int pair) __attribute__((always_inline)) {
    const int soff = __builtin_amdgcn_readfirstlane(2 * pair * T::RS * 4);
#pragma unroll
    for (int j = 0; j < T::WJ; ++j)
      wreg[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(wr, w_base + 32 * j, soff, 0));
  };
  // into [ci][t][kk]; a second channel past C (odd C, last pair) is zero
  auto store_w = [&](float *wt, int pair) __attribute__((always_inline)) {
    const bool c1 = 2 * pair + 1 < p.C;
    float *wb = wt + w_part * T::KP + w_kk;
#pragma unroll
    for (int j = 0; j < T::WJ; ++j) {
      const int lo = 8 * j;  // this element is tap lo + part of the run
      if (lo + 7 < T::RS) {
        wb[lo * T::KP] = wreg[j];
      } else if (lo >= T::RS) {
        if (w_part + lo < 2 * T::RS) wb[T::CIS + (lo - T::RS) * T::KP] = c1 ? wreg[j] : 0.0f;
      } else if (w_part + lo < T::RS) {
        wb[lo * T::KP] = wreg[j];
      } else {
        wb[T::CIS + (lo - T::RS) * T::KP] = c1 ? wreg[j] : 0.0f;
      }
    }
  };

  // ---- per-lane operand offsets (floats from a stage's base) ------------
  // A (weights): output channel k0 + 32a + l32, pair channel `half`, from a
  // weight buffer's base; B (rows): plane `half`, column q * sw (the tap adds
  // r*PITCH + s*DW), from a row buffer's base
  int b_base[FP];
#pragma unroll
  for (int b = 0; b < FP; ++b) b_base[b] = half * T::PLANE + (32 * (wave * FP + b) + l32) * p.sw;
  const int a_base = half * T::CIS + l32;

  v16f acc[FK][FP];
#pragma unroll
  for (int a = 0; a < FK; ++a)
#pragma unroll
    for (int b = 0; b < FP; ++b) acc[a][b] = v16f{0.0f};

  // prologue: pair 0 into row buffer 0 and weight buffer 0
  issue_act(0, lds);
  load_w(0);
  store_w(lds + T::WOFF, 0);
  __builtin_amdgcn_s_waitcnt(0);  // the LDS-DMAs of pair 0 (and every other count) done
  __syncthreads();

  for (int pair = 0; pair < NPAIR; ++pair) {
    float *cur = lds + (pair & 1) * T::ACT;
    float *nxt = lds + ((pair + 1) & 1) * T::ACT;
    float *wcur = lds + T::WOFF + (WDB ? (pair & 1) * T::WT : 0);
    float *wnxt = lds + T::WOFF + (WDB ? ((pair + 1) & 1) * T::WT : 0);
    const bool more = pair + 1 < NPAIR;
    // the other row buffer (and weight buffer) was last read in the previous
    // pair, before the barrier that ended it
    if (more) {
      issue_act(pair + 1, nxt);
      load_w(pair + 1);
    }
    float af[2][FK], bf[2][FP];
    auto read_ops = [&](int t, float (&av)[FK], float (&bv)[FP]) __attribute__((always_inline)) {
      const int r = t / S, s = t - (t / S) * S;
#pragma unroll
      for (int a = 0; a < FK; ++a) av[a] = wcur[a_base + t * T::KP + 32 * a];
#pragma unroll
      for (int b = 0; b < FP; ++b) bv[b] = cur[b_base[b] + r * PITCH + s * DW];
    };
    read_ops(0, af[0], bf[0]);
#pragma unroll
    for (int t = 0; t < T::RS; ++t) {
      if (t + 1 < T::RS) read_ops(t + 1, af[(t + 1) & 1], bf[(t + 1) & 1]);
#pragma unroll
      for (int a = 0; a < FK; ++a)
#pragma unroll
        for (int b = 0; b < FP; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[t & 1][a], bf[t & 1][b], acc[a][b], 0, 0,
                                                           0);
      // the next tap's LDS reads go out ahead of this tap's MFMAs, so their
      // latency hides behind them
      if (t + 1 < T::RS) __builtin_amdgcn_sched_group_barrier(0x100, FK + FP, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, FK * FP, 0);
    }
    if constexpr (WDB) {
      if (more) store_w(wnxt, pair + 1);
    } else {
      __syncthreads();  // every wave is done with this pair's weights
      if (more) store_w(wnxt, pair + 1);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's DMAs of the next pair have landed
    __syncthreads();
  }

  // ---- epilogue: y[n][k][p][q] = alpha * acc (per channel: alpha[k] * acc
  // + bias[k], one multiply then one add); lane l, register i of a fragment
  // holds channel 8*(i/4) + 4*(l/32) + i%4 of pixel l%32 --------------------
  const float alpha = p.alpha;
  const float *alpha_k = p.alpha_k, *bias_k = p.bias_k;
  float *yrow = y + ((size_t)n * p.K) * p.PQ + (size_t)op * p.Q;
#pragma unroll
  for (int b = 0; b < FP; ++b) {
    const int q = 32 * (wave * FP + b) + l32;
    if (q >= p.Q) continue;
#pragma unroll
    for (int a = 0; a < FK; ++a)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int k = k0 + 32 * a + 8 * (i / 4) + 4 * half + (i % 4);
        if (k < p.K) {
          float v = (alpha_k ? alpha_k[k] : alpha) * acc[a][b][i];
          if (bias_k) v = v + bias_k[k];
          yrow[(size_t)k * p.PQ + q] = v;
        }
      }
  }
}

template <int FK, int FP, int NW, int R, int S, int DH, int DW, int PITCH, int WDB, int D16>
static hipError_t launch_f32_halo(const float *x, const float *w, float *y, const F32Params &p,
                                  int grid, hipStream_t s) {
  using T = F32HaloTile<FK, FP, NW, R, S, DH, DW, PITCH, WDB, D16>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void *>(&conv_f32_halo_kernel<FK, FP, NW, R, S, DH, DW, PITCH, WDB, D16>),
      hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (attr != hipSuccess) return attr;
  return launch_kernel(&conv_f32_halo_kernel<FK, FP, NW, R, S, DH, DW, PITCH, WDB, D16>, dim3(grid),
                       dim3(T::THREADS), T::LDS_BYTES, s, x, w, y, p);
}

#define F32_HALO_CFG(FK, FP, NW, R, S, DH, DW, PITCH, WDB, D16, SUFFIX)                      \
  F32Config {                                                                            \
    "f32_rowhalo_mfma32x32x2_" #NW "waves_frag" #FK "x" #FP "_r" #R "s" #S "_dil" #DH "x" #DW \
    "_pitch" #PITCH SUFFIX,                                                              \
        F32HaloTile<FK, FP, NW, R, S, DH, DW, PITCH, WDB, D16>::BM,                        \
        F32HaloTile<FK, FP, NW, R, S, DH, DW, PITCH, WDB, D16>::BN, 64 * NW,               \
        F32HaloTile<FK, FP, NW, R, S, DH, DW, PITCH, WDB, D16>::LDS_BYTES, 0,              \
        &launch_f32_halo<FK, FP, NW, R, S, DH, DW, PITCH, WDB, D16>, 0, 1, R, S, DH, DW,   \
        PITCH, D16                                                                       \
  }

F32Config kF32HaloConfigs[] = {
    // the transcript's 5x9 filter with dilation (2, 3): rows of up to 520
    // columns (a 512-wide output row's taps span 496 + 24 columns); one
    // weight buffer (72 KB, two workgroups per CU), rows by 16-byte LDS-DMA
    // where the padding and width keep 4-column quads whole (the faster),
    // else by 4-byte LDS-DMA
    F32_HALO_CFG(2, 2, 8, 5, 9, 2, 3, 520, 0, 1, "_wsingle_dma16"),
    F32_HALO_CFG(2, 2, 8, 5, 9, 2, 3, 520, 0, 0, "_wsingle"),
    F32_HALO_CFG(2, 2, 8, 5, 9, 2, 3, 520, 1, 0, ""),   // two weight buffers, 98 KB
};
int kNumF32HaloConfigs = sizeof(kF32HaloConfigs) / sizeof(kF32HaloConfigs[0]);

}  // namespace convfprop
