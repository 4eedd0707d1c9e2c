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
//     transposed to [c][r][s][k] so that an MFMA operand is 32 consecutive
//     floats (conflict-free ds_read_b32).  The activation operand is read
//     straight from global memory (L1/L2 serve the R*S-fold reuse), with a
//     software pipeline of DEPTH taps in flight.
#include "common.hpp"
#include "kernels.hpp"

namespace convfprop {

template <int FK, int FP, int CC, int DEPTH>
struct F32Tile {
  static constexpr int NWAVES = 4;
  static constexpr int THREADS = 256;
  static constexpr int BM = 32 * FK;           // output channels per workgroup
  static constexpr int BN = 32 * FP * NWAVES;  // output pixels per workgroup
  static constexpr int PAIRS = CC / 2;         // MFMAs per tap per fragment
  static_assert(CC % 2 == 0, "channel chunk must hold whole pairs");
};

template <int FK, int FP, int CC, int DEPTH>
__global__ void __launch_bounds__(256)
conv_f32_kernel(const float *__restrict__ x, const float *__restrict__ w,
                float *__restrict__ y, F32Params p) {
  using T = F32Tile<FK, FP, CC, DEPTH>;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  float *wl = reinterpret_cast<float *>(lds_raw);  // [CC][R][S][BM]

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

  const int chunk_elems = CC * RS * T::BM;
  const float alpha = p.alpha;

  for (int c0 = 0; c0 < p.C; c0 += CC) {
    // ---- stage W[k0 .. k0+BM)[c0 .. c0+CC)[r][s] into LDS as [cc][r][s][k].
    __syncthreads();
    for (int e = tid; e < chunk_elems; e += T::THREADS) {
      int kk = e % T::BM;
      int rest = e / T::BM;  // = cc*RS + rs
      int cc = rest / RS;
      int rs = rest - cc * RS;
      int k = k0 + kk, c = c0 + cc;
      float v = 0.0f;
      if (k < p.K && c < p.C) v = w[((size_t)k * p.C + c) * RS + rs];
      wl[e] = v;
    }
    __syncthreads();

    // ---- taps of this chunk, software-pipelined DEPTH deep ---------------
    // Tap index tt = r*S + s.  For each tap, a lane loads T::PAIRS values per
    // pixel fragment: channel c0 + 2*i + half for pair i.
    float ring[DEPTH][T::PAIRS][FP];
    auto load_tap = [&](int tt, float (&dst)[T::PAIRS][FP]) {
      int r = tt / p.S;
      int s = tt - r * p.S;
#pragma unroll
      for (int b = 0; b < FP; ++b) {
        int h = px_h0[b] + r * p.dh;
        int ww = px_w0[b] + s * p.dw;
        bool ok = (unsigned)h < (unsigned)p.H && (unsigned)ww < (unsigned)p.W;
        int base = px_base[b] + r * p.dh * p.W + s * p.dw;
#pragma unroll
        for (int i = 0; i < T::PAIRS; ++i) {
          int c = c0 + 2 * i + half;
          uint32_t off = (ok && c < p.C) ? (uint32_t)(base + c * p.HW) * 4u : OOB_OFFSET;
          dst[i][b] = load_f32(xr, off);
        }
      }
    };

#pragma unroll
    for (int d = 0; d < DEPTH - 1; ++d)
      if (d < RS) load_tap(d, ring[d]);

    for (int tt0 = 0; tt0 < RS; tt0 += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        const int tt = tt0 + d;
        if (tt >= RS) break;
        // prefetch tap tt + DEPTH - 1 into the slot freed last step
        const int pf = tt + DEPTH - 1;
        if (pf < RS) load_tap(pf, ring[(d + DEPTH - 1) % DEPTH]);
#pragma unroll
        for (int i = 0; i < T::PAIRS; ++i) {
          float af[FK];
#pragma unroll
          for (int a = 0; a < FK; ++a)
            af[a] = wl[((2 * i + half) * RS + tt) * T::BM + 32 * a + l32];
#pragma unroll
          for (int a = 0; a < FK; ++a)
#pragma unroll
            for (int b = 0; b < FP; ++b)
              acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[a], ring[d][i][b],
                                                               acc[a][b], 0, 0, 0);
        }
      }
    }
  }

  // ---- epilogue: y[n][k][p][q] = alpha * acc ------------------------------
  // Accumulator layout of v_mfma_f32_32x32x2_f32: lane l, register i holds
  // D[row = 8*(i/4) + 4*(l/32) + i%4][col = l%32]; rows are channels.
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
        if (k < p.K) y[((size_t)n * p.K + k) * p.PQ + pq] = alpha * acc[a][b][i];
      }
  }
}

template <int FK, int FP, int CC, int DEPTH>
static hipError_t launch_f32(const float *x, const float *w, float *y,
                             const F32Params &p, int grid, hipStream_t s) {
  using T = F32Tile<FK, FP, CC, DEPTH>;
  const int lds = CC * p.R * p.S * T::BM * 4;
  hipLaunchKernelGGL((conv_f32_kernel<FK, FP, CC, DEPTH>), dim3(grid),
                     dim3(T::THREADS), lds, s, x, w, y, p);
  return hipGetLastError();
}

#define F32_CFG(FK, FP, CC, DEPTH)                                             \
  F32Config {                                                                  \
    "f32_mfma32x32x2_frag" #FK "x" #FP "_cc" #CC "_depth" #DEPTH,             \
        F32Tile<FK, FP, CC, DEPTH>::BM, F32Tile<FK, FP, CC, DEPTH>::BN, 256,   \
        CC * 4 * F32Tile<FK, FP, CC, DEPTH>::BM, 0, &launch_f32<FK, FP, CC, DEPTH> \
  }

// lds_bytes here is per filter tap (times R*S at launch).
F32Config kF32Configs[] = {
    F32_CFG(2, 2, 4, 3),  // 0: 64 ch x 256 px
    F32_CFG(1, 2, 4, 3),  // 1: 32 ch x 256 px
    F32_CFG(2, 1, 8, 3),  // 2: 64 ch x 128 px, 8-channel chunks
};
int kNumF32Configs = sizeof(kF32Configs) / sizeof(kF32Configs[0]);

}  // namespace convfprop
