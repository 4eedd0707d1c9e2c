// fastdiv.hpp -- division by a run-time constant as a multiply-high and a
// shift (Granlund and Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994, the round-up method).
//
// A kernel's prologue divides pixel and row indices by problem extents (Q,
// P*Q, the virtual image height, the number of channel tiles).  A general
// 32-bit division by a value held in a register compiles to ~15-20
// instructions; the descriptor computes the magic number once on the host,
// and the kernel pays two.
//
// For a divisor d >= 1 that is not a power of two, with l = ceil(log2 d) and
// m = ceil(2^(31+l) / d) (< 2^32 because d > 2^(l-1)):
//   m*d - 2^(31+l) < d <= 2^l,
// so floor(m * x / 2^(31+l)) = floor(x / d) for every 0 <= x < 2^31, i.e.
//   x / d = mulhi32(x, m) >> (l - 1).
// A power of two d = 2^l is a plain shift (stored as magic 0).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convfprop {

struct FastDiv {
  uint32_t magic;  // 0: d is a power of two
  int shift;
};

// Host side: the magic number of divisor d (1 <= d < 2^31).
inline FastDiv make_fastdiv(uint32_t d) {
  int l = 0;
  while ((1u << l) < d) ++l;  // l = ceil(log2 d)
  if ((1u << l) == d) return FastDiv{0u, l};
  const uint64_t m = ((uint64_t(1) << (31 + l)) + d - 1) / d;
  return FastDiv{(uint32_t)m, l - 1};
}

// x / d for 0 <= x < 2^31.
__host__ __device__ inline int fast_div(int x, FastDiv f) {
  const uint32_t u = (uint32_t)x;
#ifdef __HIP_DEVICE_COMPILE__
  const uint32_t hi = __umulhi(u, f.magic);
#else
  const uint32_t hi = (uint32_t)(((uint64_t)u * f.magic) >> 32);
#endif
  return (int)((f.magic ? hi : u) >> f.shift);
}

}  // namespace convfprop
