// epilogue_i8.hpp -- the fused int8 epilogue shared by the int8 kernels.
//
// CUTLASS issue 2996 ("How to optimize cutlass int8 fprop2d kernel with
// NCxHWx interleaved layout"), section "CUTLASS Kernel Configuration": the
// int32 accumulator is scaled by an fp32 alpha only and clamped to int8
// (LinearCombinationClamp, OnlyAlphaScaling).  Order, one rounding per step:
//   f = fl32(acc)  (round to nearest even)
//   g = f * alpha  (one fp32 multiply; the build forbids FMA contraction)
//   r = rint(g)    (round half to even)
//   y = clamp(r, -128, 127)
// The caller guarantees a finite alpha (the C ABI rejects others).
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace convfprop {

// The epilogue of one accumulator as fp32 bits whose low byte is the int8
// result.  Clamping before rounding gives the same value as clamping after
// it (the bounds are integers and rint is monotone), and adding 1.5 * 2^23
// to a value in [-128, 127] rounds it to an integer, ties to even, exactly as
// rint does (the sum's unit in the last place is 1), leaving that integer in
// two's complement in the low mantissa bits.  Bit-identical to
// clamp(rint(fl32(fl32(acc) * alpha))) for every finite alpha.
__device__ __forceinline__ uint32_t i8_epilogue_bits(int acc, float alpha) {
  const float f = (float)acc;
  const float g = f * alpha;
  const float c = __builtin_amdgcn_fmed3f(g, -128.0f, 127.0f);
  return __builtin_bit_cast(uint32_t, c + 12582912.0f);
}

// Low bytes of four words, packed little-endian (v_perm_b32 byte selects).
__device__ __forceinline__ uint32_t pack_low_bytes(uint32_t b0, uint32_t b1, uint32_t b2,
                                                   uint32_t b3) {
  const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// Stores an FK x FP grid of 32x32 MFMA accumulator tiles (rows = output
// channels, columns = output pixels) into y in NCxHWx<32> over K.
// Accumulator layout of v_mfma_i32_32x32x32_i8: lane l, register i holds
// D[row = 8*(i/4) + 4*(l/32) + i%4][col = l%32], so the quad i = 4g..4g+3
// packs into the dword at byte 8g + 4*(l/32) of pixel l%32's 32 channels.
// Lanes l and l+32 together hold a pixel's 32 bytes; two lane-half swaps
// (v_permlane32_swap) give lane l bytes 0..15 and lane l+32 bytes 16..31,
// so each tile leaves in one 16-byte store per lane: 32 consecutive pixels,
// 1 KiB contiguous when they share an image.
//   m_base: first pixel of fragment column 0; kb_base: first 32-channel
//   block of fragment row 0.  Pixels past M and blocks past K/32 are skipped.
// One 32x32 accumulator tile (rows = output channels of 32-channel block
// kb, columns = output pixels m_col .. m_col+31) into y in NCxHWx<32> over K.
__device__ __forceinline__ void store_i8_frag(const v16i &v, int8_t *__restrict__ y,
                                              const I8Params &p, int m_col, int kb, int lane) {
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const float alpha = p.alpha;
  const int m = m_col + l32;
  uint32_t d[4];
#pragma unroll
  for (int g = 0; g < 4; ++g)
    d[g] = pack_low_bytes(i8_epilogue_bits(v[4 * g + 0], alpha), i8_epilogue_bits(v[4 * g + 1], alpha),
                          i8_epilogue_bits(v[4 * g + 2], alpha), i8_epilogue_bits(v[4 * g + 3], alpha));
  // (upper half of d0) <-> (lower half of d2), likewise d1 / d3; every lane
  // takes part, before any per-lane predicate
  const auto s02 = __builtin_amdgcn_permlane32_swap(d[0], d[2], false, false);
  const auto s13 = __builtin_amdgcn_permlane32_swap(d[1], d[3], false, false);
  if (kb < p.KBLK && m < p.M) {
    const int n = m / p.PQ;
    const int pq = m - n * p.PQ;
    int8_t *dst = y + ((size_t)(n * p.KBLK + kb) * p.PQ + pq) * 32 + 16 * half;
    *reinterpret_cast<v4i *>(dst) = v4i{(int)s02[0], (int)s02[1], (int)s13[0], (int)s13[1]};
  }
}

// An FK x FP grid of tiles: fragment (a, b) covers channel block kb_base + a
// and pixels m_base + 32*b ...
template <int FK, int FP>
__device__ __forceinline__ void store_i8_tile(const v16i (&acc)[FK][FP], int8_t *__restrict__ y,
                                              const I8Params &p, int m_base, int kb_base,
                                              int lane) {
#pragma unroll
  for (int b = 0; b < FP; ++b)
#pragma unroll
    for (int a = 0; a < FK; ++a) store_i8_frag(acc[a][b], y, p, m_base + 32 * b, kb_base + a, lane);
}

}  // namespace convfprop
