// common.hpp -- device helpers shared by the gfx950 kernels of libconvfprop.
//
// Buffer resources: every global operand is read through a raw buffer
// descriptor (base, num_records = size in bytes).  An offset at or beyond
// num_records makes the load return zero, which is how the implicit-GEMM
// iterators express zero padding, ragged tiles and reduction tails without a
// branch: a masked lane simply asks for offset OOB_OFFSET.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <type_traits>

namespace convfprop {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Offset used by masked lanes: above every valid tensor size (< 2^31 bytes).
constexpr uint32_t OOB_OFFSET = 0x80000000u;

// Word 3 of a gfx9 buffer descriptor: 32-bit data format, raw (unswizzled)
// addressing.  With stride 0 the range check is offset < num_records.
constexpr int BUFFER_FLAGS = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base,
                                                            uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                           (int)bytes, BUFFER_FLAGS);
}

__device__ __forceinline__ v4i load_b128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// 16-byte load with a wave-uniform soffset added to the per-lane offset.
__device__ __forceinline__ v4i load_b128_s(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, __builtin_amdgcn_readfirstlane(soff), 0);
}

__device__ __forceinline__ float load_f32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// One LDS-DMA load: 64 lanes x 16 bytes from the buffer into LDS at dst +
// 16*lane (dst wave-uniform).  The per-lane offset is voff, a wave-uniform
// offset soff is added to it; an out-of-range voff writes zeros.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, unsigned char *dst,
                                          uint32_t voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 16,
                                           voff, __builtin_amdgcn_readfirstlane(soff), 0, 0);
}

// The same with 4 bytes per lane: 64 consecutive floats at dst.
__device__ __forceinline__ void lds_dma4(__amdgpu_buffer_rsrc_t r, float *dst, uint32_t voff,
                                         int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 4,
                                           voff, __builtin_amdgcn_readfirstlane(soff), 0, 0);
}

// Launch-grid remap that keeps neighbouring logical tiles on one XCD.
// Workgroups are dispatched round-robin over the 8 XCDs (wg b -> XCD b % 8),
// each with its own L2.  XCD x runs wgs x, x+8, x+16, ...; this bijection
// hands XCD x a contiguous range of logical tile ids, so tiles that share
// operand rows (adjacent ids) also share an L2.
__device__ __forceinline__ int xcd_remap(int b, int total) {
  constexpr int NXCD = 8;
  int q = total / NXCD, r = total % NXCD;
  int x = b % NXCD, i = b / NXCD;
  return x * q + (x < r ? x : r) + i;
}

// Host side: launch one kernel and return the status of that launch alone.
// hipLaunchKernel reports the launch's own outcome; reading hipGetLastError()
// after a launch would instead return (and clear) an error that an earlier,
// unrelated HIP call of the caller left pending, and misreport a launch that
// was in fact enqueued.  The arguments are converted to the kernel's
// parameter types and passed by address, as the launch API expects.
template <typename... KArgs, typename... Args>
inline hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds,
                                hipStream_t stream, Args &&...args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  std::tuple<std::remove_cv_t<std::remove_reference_t<KArgs>>...> values(
      std::forward<Args>(args)...);
  return std::apply(
      [&](auto &...v) {
        void *argv[] = {static_cast<void *>(&v)...};
        return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, argv, lds,
                               stream);
      },
      values);
}

}  // namespace convfprop
