// CPU check of the swizzled halo layout (csrc/halo_swizzle.hpp, the same
// header the gfx950 kernel includes).  For a problem and a tile width:
//  - bijection: within each halo row, every column gets its own slot of the
//    row, and halo_slot_column inverts halo_slot;
//  - conflict freedom: for every tile, every 32-pixel fragment and every
//    filter tap, the slots that the fragment's lanes read are distinct
//    modulo 16 within each aligned group of 16 lanes and modulo 8 within each
//    aligned group of 8 (LDS banks for 16-byte reads, for either bank count);
//  - the plain row-major layout of the same halo is reported for contrast.
// Usage: halo_swizzle_check N H W R S ph pw sh sw dh dw bn pitch
// Prints "ok <fragments> <conflicting groups of the plain layout>" or FAIL.
#include <stdio.h>
#include <stdlib.h>

#include <set>
#include <vector>

#include "halo_swizzle.hpp"

using namespace convfprop;

static int out_dim(int in, int pad, int dil, int k, int stride) {
  return (in + 2 * pad - dil * (k - 1) - 1) / stride + 1;
}

// true if the slots of the lanes in `lanes` are distinct modulo `mod`
static bool distinct(const std::vector<int> &slots, int lo, int n, int mod) {
  std::set<int> seen;
  for (int i = lo; i < lo + n && i < (int)slots.size(); ++i) {
    if (slots[i] < 0) continue;  // lane past the output
    if (!seen.insert(slots[i] % mod).second) return false;
  }
  return true;
}

int main(int argc, char **argv) {
  if (argc != 14) {
    fprintf(stderr, "usage: N H W R S ph pw sh sw dh dw bn pitch\n");
    return 2;
  }
  int a[13];
  for (int i = 0; i < 13; ++i) a[i] = atoi(argv[i + 1]);
  const int N = a[0], H = a[1], W = a[2], R = a[3], S = a[4], ph = a[5], pw = a[6], sh = a[7],
            sw = a[8], dh = a[9], dw = a[10], bn = a[11], pitch = a[12];
  const int P = out_dim(H, ph, dh, R, sh), Q = out_dim(W, pw, dw, S, sw);
  const int HV = H + 2 * ph, WV = (Q - 1) * sw + (S - 1) * dw + 1;
  const long M = (long)N * P * Q;
  if ((sw == 2 ? 2 * ((WV + 1) / 2) : WV) > pitch) {
    printf("FAIL row of %d columns does not fit pitch %d\n", WV, pitch);
    return 1;
  }
  long frags = 0, plain_conflicts = 0;
  for (long m0 = 0; m0 < M; m0 += bn) {
    const int n_first = (int)(m0 / (P * Q));
    const int p_first = (int)((m0 % (P * Q)) / Q);
    const int v_lo = n_first * HV + p_first * sh;
    const long m1 = (m0 + bn < M ? m0 + bn : M) - 1;
    const int v_hi = (int)(m1 / (P * Q)) * HV + (int)((m1 % (P * Q)) / Q) * sh + (R - 1) * dh;
    const int rows = v_hi - v_lo + 1;
    // bijection of every row
    for (int vr = 0; vr < rows; ++vr) {
      std::set<int> used;
      for (int c = 0; c < WV; ++c) {
        const int slot = halo_slot(vr, c, v_lo, HV, P, Q, sh, sw, pitch);
        if (slot < vr * pitch || slot >= (vr + 1) * pitch || !used.insert(slot).second) {
          printf("FAIL slot %d of row %d column %d\n", slot, vr, c);
          return 1;
        }
        int back_row = -1;
        const int back = halo_slot_column(slot, v_lo, HV, P, Q, sh, sw, pitch, WV, &back_row);
        if (back != c || back_row != vr) {
          printf("FAIL inverse of slot %d: row %d column %d, expected %d %d\n", slot, back_row,
                 back, vr, c);
          return 1;
        }
      }
      for (int j = 0; j < pitch; ++j) {  // slots holding no column decode to -1
        int rr;
        const int c = halo_slot_column(vr * pitch + j, v_lo, HV, P, Q, sh, sw, pitch, WV, &rr);
        if (c >= 0 && halo_slot(vr, c, v_lo, HV, P, Q, sh, sw, pitch) != vr * pitch + j) {
          printf("FAIL slot %d decodes to column %d of another slot\n", vr * pitch + j, c);
          return 1;
        }
      }
    }
    // conflicts of every fragment at every tap
    for (long f0 = m0; f0 <= m1; f0 += 32) {
      for (int r = 0; r < R; ++r)
        for (int s = 0; s < S; ++s) {
          std::vector<int> swz(32, -1), plain(32, -1);
          for (int l = 0; l < 32; ++l) {
            const long m = f0 + l;
            if (m > m1) break;
            const int n = (int)(m / (P * Q)), pq = (int)(m % (P * Q));
            const int op = pq / Q, oq = pq % Q;
            const int vr = n * HV + op * sh + r * dh - v_lo;
            const int c = oq * sw + s * dw;
            swz[l] = halo_slot(vr, c, v_lo, HV, P, Q, sh, sw, pitch);
            // the reading side's division-free form must give the same slot
            if (halo_slot_of_pixel(vr, c, (int)m, oq, Q, r * dh / sh, sw, pitch) != swz[l]) {
              printf("FAIL pixel %ld tap (%d,%d): reader slot differs\n", m, r, s);
              return 1;
            }
            plain[l] = vr * pitch + c;
          }
          for (int g = 0; g < 32; g += 16)
            if (!distinct(swz, g, 16, 16)) {
              printf("FAIL fragment at pixel %ld tap (%d,%d): lanes %d..%d share a bank\n", f0, r,
                     s, g, g + 15);
              return 1;
            }
          for (int g = 0; g < 32; g += 8)
            if (!distinct(swz, g, 8, 8)) {
              printf("FAIL fragment at pixel %ld tap (%d,%d): lanes %d..%d share a bank (8)\n", f0,
                     r, s, g, g + 7);
              return 1;
            }
          for (int g = 0; g < 32; g += 16) plain_conflicts += !distinct(plain, g, 16, 16);
          ++frags;
        }
    }
  }
  printf("ok %ld %ld\n", frags, plain_conflicts);
  return 0;
}
