// transforms.hip -- int8 layout permutations between the logical layouts and
// the interleaved ones the int8 kernel consumes (CUTLASS issue 2996, section
// "CUTLASS Kernel Configuration": TensorNCxHWx<32> activations/outputs and
// TensorCxRSKx<32> filters).  Memory orders:
//   NCHW       [N][C][H][W]        <->  NCxHWx<32>  [N][C/32][H][W][32]
//   KCRS       [K][C][R][S]        <->  CxRSKx<32>  [C/32][R][S][K][32]
// These are HBM-bound copies: every byte is read once and written once.  The
// activation transforms are a 32 x HW byte transpose per (n, c/32), staged
// through an LDS tile so that both sides move whole 16-byte vectors: rows of
// HW bytes on the NCHW side, 32-byte channel vectors on the interleaved side.
#include "common.hpp"
#include "kernels.hpp"

namespace convfprop {

constexpr int TP = 256;        // pixels per workgroup tile (one per thread)
constexpr int TPITCH = TP + 16;  // LDS row pitch: rows stay 16-byte aligned

// 32 bytes of an LDS channel column (channels 0..31 of pixel j) packed into
// two 16-byte vectors, channel c at byte c.
__device__ __forceinline__ void gather_column(const int8_t (*tile)[TPITCH], int j, v4i &lo,
                                              v4i &hi) {
  uint32_t d[8];
#pragma unroll
  for (int q = 0; q < 8; ++q)
    d[q] = (uint32_t)(uint8_t)tile[4 * q][j] | (uint32_t)(uint8_t)tile[4 * q + 1][j] << 8 |
           (uint32_t)(uint8_t)tile[4 * q + 2][j] << 16 | (uint32_t)(uint8_t)tile[4 * q + 3][j] << 24;
  lo = v4i{(int)d[0], (int)d[1], (int)d[2], (int)d[3]};
  hi = v4i{(int)d[4], (int)d[5], (int)d[6], (int)d[7]};
}

// grid: ceil(HW/TP) * N*C/32 workgroups (tile index fastest); block 256.
// Read: each thread one 32-byte run of one channel row (two 16-byte loads
// when the row is 16-byte aligned and the run is whole).  Write: each thread
// one pixel's 32-channel vector (two 16-byte stores, consecutive threads
// consecutive pixels).
__global__ void __launch_bounds__(256)
nchw_to_nc32_kernel(const int8_t *__restrict__ src, int8_t *__restrict__ dst,
                    int C, int HW) {
  __shared__ __attribute__((aligned(16))) int8_t tile[32][TPITCH];
  const int t = threadIdx.x;
  const int hw_tiles = (HW + TP - 1) / TP;
  const int ncb = blockIdx.x / hw_tiles;  // n*CB + cb
  const int hw0 = (blockIdx.x - ncb * hw_tiles) * TP;
  const int CB = C / 32;
  const int n = ncb / CB, cb = ncb - n * CB;
  {
    const int ci = t >> 3, j0 = (t & 7) * 32;
    const int8_t *row = src + ((size_t)(n * C + cb * 32 + ci)) * HW + hw0 + j0;
    if ((HW & 15) == 0 && hw0 + j0 + 32 <= HW) {
      const v4i *r16 = reinterpret_cast<const v4i *>(row);
      *reinterpret_cast<v4i *>(&tile[ci][j0]) = r16[0];
      *reinterpret_cast<v4i *>(&tile[ci][j0 + 16]) = r16[1];
    } else {
#pragma unroll
      for (int e = 0; e < 32; ++e) tile[ci][j0 + e] = (hw0 + j0 + e < HW) ? row[e] : 0;
    }
  }
  __syncthreads();
  if (hw0 + t < HW) {
    v4i lo, hi;
    gather_column(tile, t, lo, hi);
    v4i *out = reinterpret_cast<v4i *>(dst + ((size_t)ncb * HW + hw0 + t) * 32);
    out[0] = lo;
    out[1] = hi;
  }
}

// The inverse permutation: each thread loads one pixel's 32-channel vector
// (two 16-byte loads) and writes it down an LDS column; then each thread
// stores a 32-byte run of one channel row (two 16-byte stores when aligned
// and whole).
__global__ void __launch_bounds__(256)
nc32_to_nchw_kernel(const int8_t *__restrict__ src, int8_t *__restrict__ dst,
                    int C, int HW) {
  __shared__ __attribute__((aligned(16))) int8_t tile[32][TPITCH];
  const int t = threadIdx.x;
  const int hw_tiles = (HW + TP - 1) / TP;
  const int ncb = blockIdx.x / hw_tiles;  // n*CB + cb
  const int hw0 = (blockIdx.x - ncb * hw_tiles) * TP;
  const int CB = C / 32;
  const int n = ncb / CB, cb = ncb - n * CB;
  if (hw0 + t < HW) {
    const v4i *in = reinterpret_cast<const v4i *>(src + ((size_t)ncb * HW + hw0 + t) * 32);
    const v4i lo = in[0], hi = in[1];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        tile[4 * q + e][t] = (int8_t)((uint32_t)lo[q] >> (8 * e));
        tile[16 + 4 * q + e][t] = (int8_t)((uint32_t)hi[q] >> (8 * e));
      }
  }
  __syncthreads();
  {
    const int ci = t >> 3, j0 = (t & 7) * 32;
    int8_t *row = dst + ((size_t)(n * C + cb * 32 + ci)) * HW + hw0 + j0;
    if ((HW & 15) == 0 && hw0 + j0 + 32 <= HW) {
      v4i *r16 = reinterpret_cast<v4i *>(row);
      r16[0] = *reinterpret_cast<const v4i *>(&tile[ci][j0]);
      r16[1] = *reinterpret_cast<const v4i *>(&tile[ci][j0 + 16]);
    } else {
#pragma unroll
      for (int e = 0; e < 32; ++e)
        if (hw0 + j0 + e < HW) row[e] = tile[ci][j0 + e];
    }
  }
}

// One thread per 4 output bytes (4 consecutive input channels of one k, tap).
__global__ void __launch_bounds__(256)
kcrs_to_c32rsk_kernel(const int8_t *__restrict__ src, int8_t *__restrict__ dst,
                      int K, int C, int RS, int total4) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= total4) return;
  const int o = i * 4;                 // byte offset in dst
  const int ci = o & 31;
  const int rest = o >> 5;             // (cb*RS + rs)*K + k
  const int k = rest % K;
  const int cbrs = rest / K;
  const int rs = cbrs % RS;
  const int cb = cbrs / RS;
  const int c = cb * 32 + ci;
  uint32_t v = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    v |= (uint32_t)(uint8_t)src[((size_t)k * C + c + e) * RS + rs] << (8 * e);
  *reinterpret_cast<uint32_t *>(dst + o) = v;
}

// One thread per output byte of KCRS.
__global__ void __launch_bounds__(256)
c32rsk_to_kcrs_kernel(const int8_t *__restrict__ src, int8_t *__restrict__ dst,
                      int K, int C, int RS, int total) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int rs = i % RS;
  const int kc = i / RS;
  const int c = kc % C;
  const int k = kc / C;
  dst[i] = src[(((size_t)(c >> 5) * RS + rs) * K + k) * 32 + (c & 31)];
}

hipError_t launch_nchw_to_nc32(const int8_t *src, int8_t *dst, int N, int C,
                               int HW, hipStream_t s) {
  dim3 grid(((HW + TP - 1) / TP) * N * (C / 32));
  return launch_kernel(&nchw_to_nc32_kernel, grid, dim3(256), 0, s, src, dst, C, HW);
}

hipError_t launch_nc32_to_nchw(const int8_t *src, int8_t *dst, int N, int C,
                               int HW, hipStream_t s) {
  dim3 grid(((HW + TP - 1) / TP) * N * (C / 32));
  return launch_kernel(&nc32_to_nchw_kernel, grid, dim3(256), 0, s, src, dst, C, HW);
}

hipError_t launch_kcrs_to_c32rsk(const int8_t *src, int8_t *dst, int K, int C,
                                 int RS, hipStream_t s) {
  const int total4 = K * C * RS / 4;
  return launch_kernel(&kcrs_to_c32rsk_kernel, dim3((total4 + 255) / 256), dim3(256),
                     0, s, src, dst, K, C, RS, total4);
}

hipError_t launch_c32rsk_to_kcrs(const int8_t *src, int8_t *dst, int K, int C,
                                 int RS, hipStream_t s) {
  const int total = K * C * RS;
  return launch_kernel(&c32rsk_to_kcrs_kernel, dim3((total + 255) / 256), dim3(256),
                     0, s, src, dst, K, C, RS, total);
}

}  // namespace convfprop
