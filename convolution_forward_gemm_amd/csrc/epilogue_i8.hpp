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
//
// Per-output-channel variant (the "rowwise scaled" operators named in the
// review thread of torchao issue 1406): a scale alpha[k] and a bias bias[k]
// for output channel k, applied as
//   y = clamp(rint(fl32(fl32(fl32(acc) * alpha[k]) + bias[k])), -128, 127)
// (one fp32 multiply, then one fp32 add).  The kernels take it as a
// compile-time flag PC, so the scalar path carries none of its code.
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

// The per-output-channel variant: one multiply, then one add, then as above.
__device__ __forceinline__ uint32_t i8_epilogue_bits(int acc, float alpha, float bias) {
  const float f = (float)acc;
  const float g = f * alpha;
  const float h = g + bias;
  const float c = __builtin_amdgcn_fmed3f(h, -128.0f, 127.0f);
  return __builtin_bit_cast(uint32_t, c + 12582912.0f);
}

// Low bytes of four words, packed little-endian (v_perm_b32 byte selects).
__device__ __forceinline__ uint32_t pack_low_bytes(uint32_t b0, uint32_t b1, uint32_t b2,
                                                   uint32_t b3) {
  const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// Byte offset in y (NCxHWx<32> over K) of output pixel m's first 32-channel
// block, plus this lane half's 16 bytes; OOB_OFFSET for pixels past M, so
// that their stores are dropped.  Adding kb * PQ * 32 moves to block kb.
__device__ __forceinline__ uint32_t i8_pixel_yoff(const I8Params &p, int m, int half) {
  if (m >= p.M) return OOB_OFFSET;
  const int n = fast_div(m, p.fd_pq);
  const int pq = m - n * p.PQ;
  return (uint32_t)((n * p.KBLK * p.PQ + pq) * 32 + 16 * half);
}

// Cache policy of the y stores: sc0 | sc1 (system scope) writes them
// through the XCD's L2 while the workgroup still computes.  With the default
// write-back policy the whole output sits dirty in the L2s when the last
// workgroup ends, and the kernel's end-of-grid release writes it back
// (6.4 MB on the 3x3 N32 C256 H28 workload) before the kernel counts as
// done: 15.3 -> 14.7 us there, 11.1 -> 10.4 us on the stride-2 C128 H56 one.
constexpr int kYStorePolicy = 1 | 16;

// One 32x32 accumulator tile (rows = output channels of 32-channel block
// kb, columns = 32 output pixels) into y in NCxHWx<32> over K.
// Accumulator layout of v_mfma_i32_32x32x32_i8: lane l, register i holds
// D[row = 8*(i/4) + 4*(l/32) + i%4][col = l%32], so the quad i = 4g..4g+3
// packs into the dword at byte 8g + 4*(l/32) of pixel l%32's 32 channels.
// Lanes l and l+32 together hold a pixel's 32 bytes; two lane-half swaps
// (v_permlane32_swap) give lane l bytes 0..15 and lane l+32 bytes 16..31,
// so the tile leaves in one 16-byte store per lane: 32 consecutive pixels,
// 1 KiB contiguous when they share an image.  yoff is i8_pixel_yoff() of
// the lane's pixel; the store goes through a buffer descriptor over y, so
// pixels past M and blocks past K/32 (offset OOB_OFFSET) are dropped
// without a branch.
template <bool PC>
__device__ __forceinline__ void store_i8_frag(const v16i &v, __amdgpu_buffer_rsrc_t yr,
                                              uint32_t yoff, int kb, const I8Params &p) {
  uint32_t d[4];
  if constexpr (PC) {
    // register 4g + j of this lane holds output channel kb*32 + 8g + 4*half + j
    const int K4 = p.KBLK * 32 * 4;  // bytes of a per-channel array; blocks past it read 0
    const __amdgpu_buffer_rsrc_t ar = make_rsrc(p.alpha_k, K4);
    const __amdgpu_buffer_rsrc_t br = make_rsrc(p.bias_k, p.bias_k ? K4 : 0);
    const uint32_t base = (uint32_t)((kb * 32 + 4 * (__lane_id() >> 5)) * 4);
    v4f al[4], bi[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      al[g] = __builtin_bit_cast(v4f, load_b128(ar, base + 32 * g));
      bi[g] = __builtin_bit_cast(v4f, load_b128(br, base + 32 * g));
    }
#pragma unroll
    for (int g = 0; g < 4; ++g)
      d[g] = pack_low_bytes(i8_epilogue_bits(v[4 * g + 0], al[g][0], bi[g][0]),
                            i8_epilogue_bits(v[4 * g + 1], al[g][1], bi[g][1]),
                            i8_epilogue_bits(v[4 * g + 2], al[g][2], bi[g][2]),
                            i8_epilogue_bits(v[4 * g + 3], al[g][3], bi[g][3]));
  } else {
    const float alpha = p.alpha;
#pragma unroll
    for (int g = 0; g < 4; ++g)
      d[g] = pack_low_bytes(i8_epilogue_bits(v[4 * g + 0], alpha), i8_epilogue_bits(v[4 * g + 1], alpha),
                            i8_epilogue_bits(v[4 * g + 2], alpha), i8_epilogue_bits(v[4 * g + 3], alpha));
  }
  // (upper half of d0) <-> (lower half of d2), likewise d1 / d3
  const auto s02 = __builtin_amdgcn_permlane32_swap(d[0], d[2], false, false);
  const auto s13 = __builtin_amdgcn_permlane32_swap(d[1], d[3], false, false);
  const uint32_t off = kb < p.KBLK && yoff != OOB_OFFSET ? yoff + (uint32_t)(kb * p.PQ * 32) : OOB_OFFSET;
  __builtin_amdgcn_raw_buffer_store_b128(v4i{(int)s02[0], (int)s02[1], (int)s13[0], (int)s13[1]},
                                         yr, off, 0, kYStorePolicy);
}

// An FK x FP grid of tiles: fragment (a, b) covers channel block kb_base + a
// and pixels m_base + 32*b ...
template <bool PC, int FK, int FP>
__device__ __forceinline__ void store_i8_tile(const v16i (&acc)[FK][FP], int8_t *__restrict__ y,
                                              const I8Params &p, int m_base, int kb_base,
                                              int lane) {
  const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, p.y_bytes);
#pragma unroll
  for (int b = 0; b < FP; ++b) {
    const uint32_t yoff = i8_pixel_yoff(p, m_base + 32 * b + (lane & 31), lane >> 5);
#pragma unroll
    for (int a = 0; a < FK; ++a) store_i8_frag<PC>(acc[a][b], yr, yoff, kb_base + a, p);
  }
}

}  // namespace convfprop
