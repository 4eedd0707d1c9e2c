// halo_swizzle.hpp -- bank-conflict-free placement of the LDS activation halo.
//
// The halo kernels (conv_i8_halo.hip) stage, per 32-channel block, every input
// row and column that a tile's output pixels read (the implicit-GEMM
// activation tile of CUTLASS issue 2996, section "CUTLASS Kernel
// Configuration", fetched once per channel block instead of once per filter
// tap).  Each halo slot is 16 bytes (one half of a pixel's 32-channel
// vector).  A pixel fragment read is 32 lanes reading the slots of 32
// consecutive output pixels at one filter tap.
//
// LDS serves a 16-byte-per-lane read in groups of lanes; two lanes of a group
// that hit the same bank (slot index mod 16 for 64 four-byte banks, mod 8 for
// 32) are serialised.  In a plain row-major halo the lanes of a fragment are
// contiguous only until the fragment wraps to the next output row: the wrap
// skips the halo's padding columns (and, for a stride-2 problem, every lane
// is two slots from the next).  The layout here keeps every fragment
// contiguous modulo 16 for every tap:
//
//  - columns: with a horizontal stride of 2 the even columns of a row come
//    first, then the odd ones (each in its half of the row), so the lanes of
//    a fragment step by one slot;
//  - rows: row v (absolute virtual row) is rotated within its pitch by
//      rot(v) = (Q * (n * P + (v - n * HV) / sh)) mod 16,   n = v / HV,
//    which advances by Q (mod 16) per output row, exactly what the output
//    pixels' linear index advances by.  Then the slot of output pixel i at
//    tap (r, s) is congruent to i + const(r, s) modulo 16: any 16 (or 8)
//    consecutive lanes hit 16 (or 8) different banks, across row wraps and
//    image boundaries alike.
//
// The pitch is a power of two >= 16 (32 or 64 slots), so the rotation is a
// bijection of each row's slots and the congruence survives the wrap-around.
// Host and device share these functions: the planner sizes the halo with
// them and a CPU test checks bijectivity and conflict-freedom.
#pragma once

#include <hip/hip_runtime.h>

namespace convfprop {

// Rotation (0..15 slots) of absolute virtual row v.  HV: virtual rows per
// image (H + 2*pad_h), P, Q: output extents, sh: vertical stride.
__host__ __device__ inline int halo_rot(int v, int HV, int P, int Q, int sh) {
  const int n = v / HV;
  return (Q * (n * P + (v - n * HV) / sh)) & 15;
}

// Position of halo column c within a row before rotation: with a horizontal
// stride of 2, even columns take the first half of the pitch, odd ones the
// second.
__host__ __device__ inline int halo_split(int c, int sw, int pitch) {
  return sw == 2 ? (c & 1) * (pitch >> 1) + (c >> 1) : c;
}

// Inverse of halo_split; -1 for a position that holds no column of the row
// (width WV).
__host__ __device__ inline int halo_unsplit(int cs, int sw, int pitch, int WV) {
  int c;
  if (sw == 2) {
    const int h = pitch >> 1;
    c = cs < h ? 2 * cs : 2 * (cs - h) + 1;
  } else {
    c = cs;
  }
  return c < WV ? c : -1;
}

// Slot (within one half-plane) of halo row vrel (relative to the tile's first
// row v_lo) and column c.
__host__ __device__ inline int halo_slot(int vrel, int c, int v_lo, int HV, int P, int Q, int sh,
                                         int sw, int pitch) {
  const int rot = halo_rot(v_lo + vrel, HV, P, Q, sh);
  return vrel * pitch + ((halo_split(c, sw, pitch) + rot) & (pitch - 1));
}

// The same slot from the reading side, without a division by HV: output
// pixel m (row index m / Q = n * P + op, column oq) at filter row r reads
// virtual row n * HV + op * sh + r * dh, which lies in image n (the rows a
// valid output pixel reads never pass its image's last virtual row), so its
// rotation is Q * (n * P + op + floor(r * dh / sh)) mod 16 =
// (m - oq + Q * floor(r * dh / sh)) mod 16.  vrel is that row relative to
// v_lo, c the column oq * sw + s * dw, rdh_sh = floor(r * dh / sh).
__host__ __device__ inline int halo_slot_of_pixel(int vrel, int c, int m, int oq, int Q,
                                                  int rdh_sh, int sw, int pitch) {
  const int rot = (m - oq + Q * rdh_sh) & 15;
  return vrel * pitch + ((halo_split(c, sw, pitch) + rot) & (pitch - 1));
}

// The column held at position j (0 <= j < pitch) of a row rotated by rot, or
// -1: the inverse of the rotation and the column split, for a caller that has
// the row's rotation already.
__host__ __device__ inline int halo_column_at(int j, int rot, int sw, int pitch, int WV) {
  return halo_unsplit((j - rot) & (pitch - 1), sw, pitch, WV);
}

// Inverse: the column stored in slot `slot` of a half-plane, or -1 if the slot
// holds none; *vrel receives its row.
__host__ __device__ inline int halo_slot_column(int slot, int v_lo, int HV, int P, int Q, int sh,
                                                int sw, int pitch, int WV, int *vrel) {
  const int row = slot / pitch;
  const int j = slot - row * pitch;
  *vrel = row;
  return halo_column_at(j, halo_rot(v_lo + row, HV, P, Q, sh), sw, pitch, WV);
}

}  // namespace convfprop
