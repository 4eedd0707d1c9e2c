// transforms.hip -- int8 layout permutations between the logical layouts and
// the interleaved ones the int8 kernel consumes (CUTLASS issue 2996, section
// "CUTLASS Kernel Configuration": TensorNCxHWx<32> activations/outputs and
// TensorCxRSKx<32> filters).  Memory orders:
//   NCHW       [N][C][H][W]        <->  NCxHWx<32>  [N][C/32][H][W][32]
//   KCRS       [K][C][R][S]        <->  CxRSKx<32>  [C/32][R][S][K][32]
// These are HBM-bound copies: every byte is read once and written once.  The
// activation transform is a 32 x HW transpose per (n, c/32), staged through
// an LDS tile so that both the reads (rows of HW bytes) and the writes
// (32-byte channel vectors) stay coalesced.
#include "common.hpp"
#include "kernels.hpp"

namespace convfprop {

constexpr int TP = 64;  // pixels per workgroup tile

// grid: ceil(HW/TP) * N*C/32 workgroups (tile index fastest); block 256.
__global__ void __launch_bounds__(256)
nchw_to_nc32_kernel(const int8_t *__restrict__ src, int8_t *__restrict__ dst,
                    int C, int HW) {
  __shared__ int8_t tile[32][TP + 8];
  const int t = threadIdx.x;
  const int hw_tiles = (HW + TP - 1) / TP;
  const int ncb = blockIdx.x / hw_tiles;  // n*CB + cb
  const int hw0 = (blockIdx.x - ncb * hw_tiles) * TP;
  const int CB = C / 32;
  const int n = ncb / CB, cb = ncb - n * CB;
  {
    const int ci = t >> 3, j8 = (t & 7) * 8;
    const int8_t *row = src + ((size_t)(n * C + cb * 32 + ci)) * HW + hw0 + j8;
    if ((HW & 7) == 0 && hw0 + j8 + 8 <= HW) {
      uint64_t v = *reinterpret_cast<const uint64_t *>(row);
#pragma unroll
      for (int e = 0; e < 8; ++e) tile[ci][j8 + e] = (int8_t)(v >> (8 * e));
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) tile[ci][j8 + e] = (hw0 + j8 + e < HW) ? row[e] : 0;
    }
  }
  __syncthreads();
  {
    const int j = t >> 2, cg = (t & 3) * 8;
    if (hw0 + j < HW) {
      uint64_t v = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) v |= (uint64_t)(uint8_t)tile[cg + e][j] << (8 * e);
      *reinterpret_cast<uint64_t *>(dst + ((size_t)ncb * HW + hw0 + j) * 32 + cg) = v;
    }
  }
}

__global__ void __launch_bounds__(256)
nc32_to_nchw_kernel(const int8_t *__restrict__ src, int8_t *__restrict__ dst,
                    int C, int HW) {
  __shared__ int8_t tile[32][TP + 8];
  const int t = threadIdx.x;
  const int hw_tiles = (HW + TP - 1) / TP;
  const int ncb = blockIdx.x / hw_tiles;  // n*CB + cb
  const int hw0 = (blockIdx.x - ncb * hw_tiles) * TP;
  const int CB = C / 32;
  const int n = ncb / CB, cb = ncb - n * CB;
  {
    const int j = t >> 2, cg = (t & 3) * 8;
    if (hw0 + j < HW) {
      uint64_t v = *reinterpret_cast<const uint64_t *>(src + ((size_t)ncb * HW + hw0 + j) * 32 + cg);
#pragma unroll
      for (int e = 0; e < 8; ++e) tile[cg + e][j] = (int8_t)(v >> (8 * e));
    }
  }
  __syncthreads();
  {
    const int ci = t >> 3, j8 = (t & 7) * 8;
    int8_t *row = dst + ((size_t)(n * C + cb * 32 + ci)) * HW + hw0 + j8;
    if ((HW & 7) == 0 && hw0 + j8 + 8 <= HW) {
      uint64_t v = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) v |= (uint64_t)(uint8_t)tile[ci][j8 + e] << (8 * e);
      *reinterpret_cast<uint64_t *>(row) = v;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (hw0 + j8 + e < HW) row[e] = tile[ci][j8 + e];
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
  hipLaunchKernelGGL(nchw_to_nc32_kernel, grid, dim3(256), 0, s, src, dst, C, HW);
  return hipGetLastError();
}

hipError_t launch_nc32_to_nchw(const int8_t *src, int8_t *dst, int N, int C,
                               int HW, hipStream_t s) {
  dim3 grid(((HW + TP - 1) / TP) * N * (C / 32));
  hipLaunchKernelGGL(nc32_to_nchw_kernel, grid, dim3(256), 0, s, src, dst, C, HW);
  return hipGetLastError();
}

hipError_t launch_kcrs_to_c32rsk(const int8_t *src, int8_t *dst, int K, int C,
                                 int RS, hipStream_t s) {
  const int total4 = K * C * RS / 4;
  hipLaunchKernelGGL(kcrs_to_c32rsk_kernel, dim3((total4 + 255) / 256), dim3(256),
                     0, s, src, dst, K, C, RS, total4);
  return hipGetLastError();
}

hipError_t launch_c32rsk_to_kcrs(const int8_t *src, int8_t *dst, int K, int C,
                                 int RS, hipStream_t s) {
  const int total = K * C * RS;
  hipLaunchKernelGGL(c32rsk_to_kcrs_kernel, dim3((total + 255) / 256), dim3(256),
                     0, s, src, dst, K, C, RS, total);
  return hipGetLastError();
}

}  // namespace convfprop
