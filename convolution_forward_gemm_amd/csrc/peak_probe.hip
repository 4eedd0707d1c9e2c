// peak_probe.hip -- measured throughput ceilings of one MI355X (gfx950),
// for the roofline of the conv kernels: int8 / fp32 MFMA rate, LDS read
// bandwidth, L2 -> CU load bandwidth (to VGPRs and LDS-DMA), HBM copy rate.
// Every kernel touches only its own buffers, at in-bounds offsets.
// Build: hipcc --offload-arch=gfx950 -O3 peak_probe.hip -o peak_probe
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdio.h>

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
#define LDS __attribute__((address_space(3)))

#define CHECK(x)                                                          \
  do {                                                                    \
    hipError_t e_ = (x);                                                  \
    if (e_ != hipSuccess) {                                               \
      printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 1;                                                           \
    }                                                                     \
  } while (0)

// Four independent accumulator chains per wave keep the matrix unit busy.
__global__ void __launch_bounds__(256) mfma_i8(v16i *out, int iters) {
  int t = threadIdx.x;
  v4i a = {t, 1, 2, 3}, b = {4, 5, 6, t};
  v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c3, 0, 0, 0);
  }
  out[blockIdx.x * 256 + t] = c0 + c1 + c2 + c3;
}

// Eight chains, operands rotating through registers as in the conv kernels'
// inner loop (one wave per SIMD when launched with one workgroup per CU).
__global__ void __launch_bounds__(256) mfma_i8_8chain(v16i *out, int iters) {
  int t = threadIdx.x;
  v4i a0 = {t, 1, 2, 3}, a1 = {t, 7, 2, 3}, b0 = {4, 5, 6, t}, b1 = {4, 9, 6, t};
  v4i b2 = {1, 5, 6, t}, b3 = {4, 5, 3, t};
  v16i c[8] = {};
  for (int i = 0; i < iters; ++i) {
    c[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, b0, c[0], 0, 0, 0);
    c[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, b0, c[1], 0, 0, 0);
    c[2] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, b1, c[2], 0, 0, 0);
    c[3] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, b1, c[3], 0, 0, 0);
    c[4] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, b2, c[4], 0, 0, 0);
    c[5] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, b2, c[5], 0, 0, 0);
    c[6] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, b3, c[6], 0, 0, 0);
    c[7] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, b3, c[7], 0, 0, 0);
  }
  v16i s = {};
  for (int k = 0; k < 8; ++k) s += c[k];
  out[blockIdx.x * 256 + t] = s;
}

// Eight chains whose operands are uniform random int8 (read from a buffer)
// and change from one MFMA to the next, as real data does.  The matrix
// unit's rate depends on the operand bits: the constant, mostly-zero
// operands above run faster than data like the conv workloads'.
__global__ void __launch_bounds__(256) mfma_i8_rand(const v4i *__restrict__ src, v16i *out, int iters) {
  int t = threadIdx.x;
  v4i a[4], b[4];
  for (int k = 0; k < 4; ++k) {
    a[k] = src[(k * 256 + t) & 2047];
    b[k] = src[((k + 4) * 256 + t) & 2047];
  }
  v16i c[8] = {};
  for (int i = 0; i < iters; i += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        c[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[(j + u) & 3], b[((j >> 1) + u) & 3], c[j], 0, 0, 0);
  }
  v16i s = {};
  for (int k = 0; k < 8; ++k) s += c[k];
  out[blockIdx.x * 256 + t] = s;
}

// The same random operands on the 16 x 16 x 64 int8 MFMA (half the work
// per instruction, twice the instructions for the same operations).
__global__ void __launch_bounds__(256) mfma_i8_rand16(const v4i *__restrict__ src, v16i *out, int iters) {
  int t = threadIdx.x;
  v4i a[4], b[4];
  for (int k = 0; k < 4; ++k) {
    a[k] = src[(k * 256 + t) & 2047];
    b[k] = src[((k + 4) * 256 + t) & 2047];
  }
  v4i c[16] = {};
  for (int i = 0; i < iters; i += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        c[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[(j + u) & 3], b[((j >> 2) + u) & 3], c[j], 0, 0, 0);
  }
  v4i s = {};
  for (int k = 0; k < 16; ++k) s += c[k];
  out[blockIdx.x * 256 + t] = v16i{s[0], s[1], s[2], s[3]};
}

// The same with K independent v_add_u32 issued by the wave after every
// MFMA: how much vector ALU work one wave can hide behind its own MFMAs.
template <int K>
__global__ void __launch_bounds__(256) mfma_i8_valu(v16i *out, int *out2, int iters) {
  int t = threadIdx.x;
  v4i a0 = {t, 1, 2, 3}, a1 = {t, 7, 2, 3}, b0 = {4, 5, 6, t}, b1 = {4, 9, 6, t};
  v16i c[8] = {};
  int x[8];
  for (int k = 0; k < 8; ++k) x[k] = t * (k + 1);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      c[m] = __builtin_amdgcn_mfma_i32_32x32x32_i8((m & 1) ? a1 : a0, (m & 2) ? b1 : b0, c[m], 0, 0, 0);
#pragma unroll
      for (int k = 0; k < K; ++k) asm volatile("v_add_u32 %0, %0, %1" : "+v"(x[k % 8]) : "v"(t));
    }
  }
  v16i s = {};
  for (int k = 0; k < 8; ++k) s += c[k];
  out[blockIdx.x * 256 + t] = s;
  int xs = 0;
  for (int k = 0; k < 8; ++k) xs += x[k];
  out2[blockIdx.x * 256 + t] = xs;
}

// (A __global__ function's host-side address is a launch handle, not a
// callable stub: each instantiation is launched by name.)
template <int K>
static int run_valu(int ncu, int iters, void *out, void *out2, hipEvent_t e0, hipEvent_t e1) {
  CHECK(hipEventRecord(e0));
  hipLaunchKernelGGL(mfma_i8_valu<K>, dim3(ncu), dim3(256), 0, 0, (v16i *)out, (int *)out2, iters);
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  float ms;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  printf("int8 MFMA, 1 wave/SIMD, %d v_add per MFMA : %8.1f TOPS\n", K,
         2.0 * 32 * 32 * 32 * 8 * (double)iters * ncu * 4 / ms / 1e9);
  return 0;
}

__global__ void __launch_bounds__(256) mfma_f32(v16f *out, int iters) {
  float a = threadIdx.x, b = 1.0f;
  v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c3, 0, 0, 0);
  }
  out[blockIdx.x * 256 + threadIdx.x] = c0 + c1 + c2 + c3;
}

// fp32 MFMA with normally distributed operands that change from one MFMA to
// the next (the fp32 workload's data), eight accumulator chains.
__global__ void __launch_bounds__(256) mfma_f32_rand(const float *__restrict__ src, v16f *out, int iters) {
  const int t = threadIdx.x;
  float a[4], b[4];
  for (int k = 0; k < 4; ++k) {
    a[k] = src[(k * 256 + t) & 4095];
    b[k] = src[((k + 4) * 256 + t) & 4095];
  }
  v16f c[8] = {};
  for (int i = 0; i < iters; i += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        c[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[(j + u) & 3], b[((j >> 1) + u) & 3], c[j], 0, 0, 0);
  }
  v16f s = {};
  for (int k = 0; k < 8; ++k) s += c[k];
  out[blockIdx.x * 256 + t] = s;
}

// ds_read_b128 with lane-contiguous addresses (the conv kernels' pattern).
__global__ void __launch_bounds__(256) lds_read(v4i *out, int iters) {
  __shared__ v4i buf[4096];  // 64 KiB
  for (int i = threadIdx.x; i < 4096; i += 256) buf[i] = v4i{i, i, i, i};
  __syncthreads();
  v4i acc = {};
  int base = (threadIdx.x >> 6) * 1024 + (threadIdx.x & 63);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= buf[(base + j * 64 + i * 8) & 4095];
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc;
}

// 1 KiB per wave per load from an L2-resident window, into VGPRs.
__global__ void __launch_bounds__(256) l2_to_vgpr(const char *src, int win, int iters, v4i *out) {
  __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)src, (short)0, win, 0x00020000);
  int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  unsigned off = ((blockIdx.x * 4 + wave) * 8192u + lane * 16u) % (unsigned)win;
  v4i acc = {};
  for (int i = 0; i < iters; ++i) {
    v4i v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, (off + j * 1024u) % (unsigned)win, 0, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= v[j];
    off = (off + 8192u) % (unsigned)win;
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc;
}

// The same loads straight into LDS (buffer_load ... lds), 3 stages in flight.
__global__ void __launch_bounds__(256) l2_to_lds(const char *src, int win, int iters, v4i *out) {
  __shared__ v4i ring[4][8][64];
  __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)src, (short)0, win, 0x00020000);
  int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  unsigned off = ((blockIdx.x * 4 + wave) * 8192u + lane * 16u) % (unsigned)win;
  v4i acc = {};
  for (int i = 0; i < iters; ++i) {
    int st = i & 3;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS void *)&ring[st][wave * 2 + j][0], 16,
                                               (off + j * 1024u) % (unsigned)win, 0, 0, 0);
    off = (off + 8192u) % (unsigned)win;
    __builtin_amdgcn_s_waitcnt((6 & 15) | (7 << 4) | (15 << 8));  // vmcnt(6)
    acc ^= ring[(i + 1) & 3][wave * 2][lane];
  }
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  out[blockIdx.x * 256 + threadIdx.x] = acc;
}

// Launch floor: a kernel that does nothing, and one that copies 2 KiB from
// HBM-resident memory (a tiny kernel's minimum: launch + one round trip).
__global__ void empty_kernel() {}
__global__ void tiny_copy(const v4i *__restrict__ in, v4i *__restrict__ out) {
  out[threadIdx.x] = in[threadIdx.x];
}

__global__ void copy_kernel(const v4i *__restrict__ in, v4i *__restrict__ out, size_t n) {
  size_t i = blockIdx.x * (size_t)256 + threadIdx.x;
  size_t stride = (size_t)gridDim.x * 256;
  for (; i < n; i += stride) out[i] = in[i];
}

// HBM streaming with enough bytes in flight: every thread issues U 16-byte
// loads (coalesced across the grid: element i + u * stride) before its U
// stores, non-temporal so the 256 MB Infinity Cache is not what is measured
// (n is a multiple of U * stride).
template <int U>
__global__ void __launch_bounds__(256) copy_unrolled(const v4i *__restrict__ in,
                                                     v4i *__restrict__ out, size_t n) {
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = blockIdx.x * (size_t)256 + threadIdx.x; i < n; i += U * stride) {
    v4i v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(in + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_nontemporal_store(v[u], out + i + u * stride);
  }
}
template <int U>
__global__ void __launch_bounds__(256) read_unrolled(const v4i *__restrict__ in, v4i *__restrict__ out,
                                                     size_t n) {
  const size_t stride = (size_t)gridDim.x * 256;
  v4i acc = v4i{0, 0, 0, 0};
  for (size_t i = blockIdx.x * (size_t)256 + threadIdx.x; i < n; i += U * stride) {
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= __builtin_nontemporal_load(in + i + u * stride);
  }
  if (acc[0] == 0x7fffffff && acc[1] == 0x13579) out[0] = acc;  // keeps the loads; never true here
}

int main() {
  setvbuf(stdout, nullptr, _IOLBF, 0);  // each line reaches a redirected log at once
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  const int ncu = prop.multiProcessorCount;
  const double clk = prop.clockRate * 1e3;  // Hz
  printf("device %s, %d CUs, max clock %.0f MHz\n", prop.gcnArchName, ncu, clk / 1e6);
  void *out;
  CHECK(hipMalloc(&out, (size_t)ncu * 8 * 256 * 64 * 4));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  float ms;
  const int grid = ncu * 2, iters = 20000;

  hipLaunchKernelGGL(mfma_i8, dim3(grid), dim3(256), 0, 0, (v16i *)out, 100);
  CHECK(hipDeviceSynchronize());
  CHECK(hipEventRecord(e0));
  hipLaunchKernelGGL(mfma_i8, dim3(grid), dim3(256), 0, 0, (v16i *)out, iters);
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  printf("int8 MFMA v_mfma_i32_32x32x32_i8 : %8.1f TOPS\n",
         2.0 * 32 * 32 * 32 * 4 * (double)iters * grid * 4 / ms / 1e9);

  // one wave per SIMD (one workgroup of 4 waves per CU)
  for (int chains : {4, 8}) {
    CHECK(hipEventRecord(e0));
    if (chains == 4)
      hipLaunchKernelGGL(mfma_i8, dim3(ncu), dim3(256), 0, 0, (v16i *)out, iters);
    else
      hipLaunchKernelGGL(mfma_i8_8chain, dim3(ncu), dim3(256), 0, 0, (v16i *)out, iters / 2);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    printf("int8 MFMA, 1 wave/SIMD, %d chains : %8.1f TOPS\n", chains,
           2.0 * 32 * 32 * 32 * 4 * (double)iters * ncu * 4 / ms / 1e9);
  }

  // uniform random operands, on every CU and on 196 (the c3 grid)
  {
    v4i *rnd;
    CHECK(hipMalloc(&rnd, 2048 * sizeof(v4i)));
    static int host[2048 * 4];
    unsigned st = 12345u;
    for (int i = 0; i < 2048 * 4; ++i) {
      st = st * 1664525u + 1013904223u;
      host[i] = (int)st;
    }
    CHECK(hipMemcpy(rnd, host, sizeof(host), hipMemcpyHostToDevice));
    const int rit = iters / 2;  // a multiple of 4
    for (int g : {ncu, ncu < 196 ? ncu : 196}) {
      hipLaunchKernelGGL(mfma_i8_rand, dim3(g), dim3(256), 0, 0, (const v4i *)rnd, (v16i *)out, 100);
      CHECK(hipDeviceSynchronize());
      CHECK(hipEventRecord(e0));
      for (int r = 0; r < 4; ++r)
        hipLaunchKernelGGL(mfma_i8_rand, dim3(g), dim3(256), 0, 0, (const v4i *)rnd, (v16i *)out, rit);
      CHECK(hipEventRecord(e1));
      CHECK(hipEventSynchronize(e1));
      CHECK(hipEventElapsedTime(&ms, e0, e1));
      const double tops = 4 * 2.0 * 32 * 32 * 32 * 8 * (double)rit * g * 4 / ms / 1e9;
      printf("int8 MFMA, random operands, %3d CUs : %8.1f TOPS (%.1f per-CU rate x %d CUs)\n", g, tops,
             tops / g * ncu, ncu);
      CHECK(hipEventRecord(e0));
      for (int r = 0; r < 4; ++r)
        hipLaunchKernelGGL(mfma_i8_rand16, dim3(g), dim3(256), 0, 0, (const v4i *)rnd, (v16i *)out, rit);
      CHECK(hipEventRecord(e1));
      CHECK(hipEventSynchronize(e1));
      CHECK(hipEventElapsedTime(&ms, e0, e1));
      printf("int8 MFMA 16x16x64, random operands, %3d CUs : %8.1f TOPS\n", g,
             4 * 2.0 * 16 * 16 * 64 * 16 * (double)rit * g * 4 / ms / 1e9);
    }
    CHECK(hipFree(rnd));
  }

  // vector ALU work hidden behind one wave's own MFMAs
  {
    void *out2;
    CHECK(hipMalloc(&out2, (size_t)ncu * 256 * 4));
    if (run_valu<0>(ncu, iters / 8, out, out2, e0, e1) || run_valu<2>(ncu, iters / 8, out, out2, e0, e1) ||
        run_valu<4>(ncu, iters / 8, out, out2, e0, e1) || run_valu<8>(ncu, iters / 8, out, out2, e0, e1))
      return 1;
    CHECK(hipFree(out2));
  }

  CHECK(hipEventRecord(e0));
  hipLaunchKernelGGL(mfma_f32, dim3(grid), dim3(256), 0, 0, (v16f *)out, iters / 4);
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  printf("fp32 MFMA v_mfma_f32_32x32x2_f32 : %8.1f TFLOPS\n",
         2.0 * 32 * 32 * 2 * 4 * (double)(iters / 4) * grid * 4 / ms / 1e9);

  {
    // normally distributed fp32 operands (Box-Muller on a fixed LCG stream)
    float *rf;
    CHECK(hipMalloc(&rf, 4096 * sizeof(float)));
    static float host[4096];
    unsigned st = 777u;
    for (int i = 0; i < 4096; i += 2) {
      st = st * 1664525u + 1013904223u;
      const double u1 = ((st >> 8) + 1.0) / 16777217.0;
      st = st * 1664525u + 1013904223u;
      const double u2 = (st >> 8) / 16777216.0;
      const double r = sqrt(-2.0 * log(u1));
      host[i] = (float)(r * cos(6.283185307179586 * u2));
      host[i + 1] = (float)(r * sin(6.283185307179586 * u2));
    }
    CHECK(hipMemcpy(rf, host, sizeof(host), hipMemcpyHostToDevice));
    const int fit = iters / 4;  // a multiple of 4
    hipLaunchKernelGGL(mfma_f32_rand, dim3(ncu), dim3(256), 0, 0, (const float *)rf, (v16f *)out, 100);
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0));
    for (int r = 0; r < 4; ++r)
      hipLaunchKernelGGL(mfma_f32_rand, dim3(ncu), dim3(256), 0, 0, (const float *)rf, (v16f *)out, fit);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    printf("fp32 MFMA, N(0,1) operands, %3d CUs : %8.1f TFLOPS\n", ncu,
           4 * 2.0 * 32 * 32 * 2 * 8 * (double)fit * ncu * 4 / ms / 1e9);
    CHECK(hipFree(rf));
  }

  for (int wgs = 1; wgs <= 2; ++wgs) {
    const int g = ncu * wgs;
    hipLaunchKernelGGL(lds_read, dim3(g), dim3(256), 0, 0, (v4i *)out, 100);
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL(lds_read, dim3(g), dim3(256), 0, 0, (v4i *)out, iters);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    const double bytes = 16.0 * 8 * (double)iters * g * 256;
    printf("LDS ds_read_b128, %d WG/CU          : %8.1f B/clk/CU\n", wgs, bytes / (ms * 1e-3) / ncu / clk);
  }

  const int win = 2 << 20;  // L2-resident window
  char *src;
  CHECK(hipMalloc(&src, win));
  CHECK(hipMemset(src, 3, win));
  for (int wgs = 1; wgs <= 2; ++wgs) {
    const int g = ncu * wgs, it = 4000;
    hipLaunchKernelGGL(l2_to_vgpr, dim3(g), dim3(256), 0, 0, src, win, 10, (v4i *)out);
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL(l2_to_vgpr, dim3(g), dim3(256), 0, 0, src, win, it, (v4i *)out);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    double bytes = (double)g * 4 * it * 8192;
    printf("L2 -> VGPR loads, %d WG/CU         : %8.1f B/clk/CU\n", wgs, bytes / (ms * 1e-3) / ncu / clk);
    hipLaunchKernelGGL(l2_to_lds, dim3(g), dim3(256), 0, 0, src, win, 10, (v4i *)out);
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL(l2_to_lds, dim3(g), dim3(256), 0, 0, src, win, it, (v4i *)out);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    bytes = (double)g * 4 * it * 2048;
    printf("L2 -> LDS (LDS-DMA), %d WG/CU      : %8.1f B/clk/CU\n", wgs, bytes / (ms * 1e-3) / ncu / clk);
  }

  const size_t n = (size_t)1 << 26;  // 1 GiB of 16-byte elements
  void *a, *b;
  CHECK(hipMalloc(&a, n * 16));
  CHECK(hipMalloc(&b, n * 16));
  CHECK(hipMemset(a, 1, n * 16));
  hipLaunchKernelGGL(copy_kernel, dim3(ncu * 16), dim3(256), 0, 0, (const v4i *)a, (v4i *)b, n);
  CHECK(hipDeviceSynchronize());
  CHECK(hipEventRecord(e0));
  for (int r = 0; r < 5; ++r)
    hipLaunchKernelGGL(copy_kernel, dim3(ncu * 16), dim3(256), 0, 0, (const v4i *)a, (v4i *)b, n);
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  printf("HBM copy 1 GiB (read + write)      : %8.1f GB/s  (one 16-byte load in flight per thread)\n",
         5 * 2.0 * n * 16 / ms / 1e6);
  {  // 8 loads in flight per thread, non-temporal; grid: 8 workgroups per CU
    const int g = ncu * 8;
    const size_t per = (size_t)g * 256 * 8;  // elements per pass of the grid
    const size_t nn = n / per * per;
    hipLaunchKernelGGL(copy_unrolled<8>, dim3(g), dim3(256), 0, 0, (const v4i *)a, (v4i *)b, nn);
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0));
    for (int r = 0; r < 5; ++r)
      hipLaunchKernelGGL(copy_unrolled<8>, dim3(g), dim3(256), 0, 0, (const v4i *)a, (v4i *)b, nn);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    printf("HBM copy 1 GiB, 8 loads in flight   : %8.1f GB/s (read + write)\n", 5 * 2.0 * nn * 16 / ms / 1e6);
    hipLaunchKernelGGL(read_unrolled<8>, dim3(g), dim3(256), 0, 0, (const v4i *)a, (v4i *)b, nn);
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0));
    for (int r = 0; r < 5; ++r)
      hipLaunchKernelGGL(read_unrolled<8>, dim3(g), dim3(256), 0, 0, (const v4i *)a, (v4i *)b, nn);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    printf("HBM read 1 GiB, 8 loads in flight   : %8.1f GB/s\n", 5 * 1.0 * nn * 16 / ms / 1e6);
  }

  // back-to-back launches on one stream, device time per launch
  for (int kind = 0; kind < 2; ++kind) {
    const int calls = 2000;
    for (int i = 0; i < 50; ++i) {
      if (kind == 0) hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, 0);
      else hipLaunchKernelGGL(tiny_copy, dim3(1), dim3(128), 0, 0, (const v4i *)a, (v4i *)b);
    }
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0));
    for (int i = 0; i < calls; ++i) {
      if (kind == 0) hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, 0);
      else hipLaunchKernelGGL(tiny_copy, dim3(1), dim3(128), 0, 0, (const v4i *)a, (v4i *)b);
    }
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    printf("%s, back-to-back       : %8.3f us per launch\n",
           kind == 0 ? "empty kernel       " : "2 KiB copy kernel  ", ms * 1e3 / calls);
  }
  return 0;
}
