// conv_i8_halo.hip -- int8 implicit-GEMM conv2d fprop for gfx950 with an
// LDS-resident activation halo (filter size fixed at compile time).
//
// What is computed is the same as conv_i8.hip (CUTLASS issue 2996, "How to
// optimize cutlass int8 fprop2d kernel with NCxHWx interleaved layout",
// section "CUTLASS Kernel Configuration"): int8 products, int32 sums over
// C*R*S, the alpha / rint / saturate epilogue, NCxHWx<32> / CxRSKx<32>.
//
// How it differs from the per-tap ring of conv_i8.hip: a stage is one
// 32-channel block.  It holds the R*S filter taps of the workgroup's output
// channels and, once, the input halo those channels' output pixels read:
// every input row and column any of the R*S taps touches.  All R*S taps then
// read their pixel fragments from that one halo with per-lane LDS addresses,
// instead of each tap bringing its own copy from L2.  For a 3x3 filter this
// cuts the bytes a workgroup pulls from L2 per tap by about half and the
// activation load instructions several-fold; the L2 -> CU path, not the
// matrix unit, is what bounds the per-tap design.  (The filter-size
// specialisation mirrors the "t1r3s3" in the TensorRT kernel name quoted in
// the same issue, section "TensorRT Kernel Name".)
//
// Halo geometry.  Rows are "virtual": image n owns rows n*HV .. n*HV+HV-1
// with HV = H + 2*pad_h, the first and last pad_h of them being zero
// padding.  Output pixel (n, p, q) with filter tap (r, s) reads virtual row
// n*HV + p*sh + r*dh and column q*sw + s*dw (column c is input column
// c - pad_w).  A workgroup's pixels, even across an image boundary, thus read
// one contiguous range of virtual rows starting at V_lo (its first pixel's
// row); the rows and columns outside the image are loaded as zeros.  The
// halo is stored as two half-planes, bytes 0..15 and 16..31 of each 32-channel
// vector, each [row][col][16 B]: a fragment read is 32 consecutive 16-byte
// slots per half-wave, conflict-free.
#include <type_traits>

#include "common.hpp"
#include "epilogue_i8.hpp"
#include "halo_swizzle.hpp"
#include "kernels.hpp"


namespace convfprop {

template <int WK, int WP, int FK, int FP, int R, int S, int NS, int HJ>
struct HaloTile {
  static constexpr int NWAVES = WK * WP;
  static constexpr int THREADS = 64 * NWAVES;
  static constexpr int KB = WK * FK;
  static constexpr int PB = WP * FP;
  static constexpr int BM = 32 * KB;
  static constexpr int BN = 32 * PB;
  static constexpr int RS = R * S;
  static constexpr int FBLK = RS * KB;                          // filter blocks per stage
  static constexpr int FJ = (FBLK + NWAVES - 1) / NWAVES;       // filter DMAs per wave
  static constexpr int NL = FJ + HJ;                            // DMAs per wave per stage
  static constexpr int FILT_BYTES = FBLK * 1024;
  static_assert(NS >= 3, "the ring needs a stage being read, one landed and one in flight");
  static_assert(NL * (NS - 2) < 64, "vmcnt counts at most 63 outstanding loads");
};

// s_waitcnt vmcnt(VM) lgkmcnt(0) (gfx9 encoding), and a barrier without the
// fence of __syncthreads (which would drain every LDS-DMA in flight).
template <int VM>
__device__ __forceinline__ void halo_wait() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | ((VM >> 4) << 14));
}
__device__ __forceinline__ void halo_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int WK, int WP, int FK, int FP, int R, int S, int NS, int HJ, bool PC>
__global__ void __launch_bounds__(64 * WK * WP)
conv_i8_halo_kernel(const int8_t *__restrict__ x, const int8_t *__restrict__ w,
                    int8_t *__restrict__ y, I8Params p) {
  using T = HaloTile<WK, WP, FK, FP, R, S, NS, HJ>;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

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
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, p.w_bytes);

  const int HV = p.HV, WV = p.WV;
  const int plane = p.halo_dpp * 1024;  // bytes per half-plane
  const int hblk = 2 * p.halo_dpp;      // halo DMA blocks per stage
  unsigned char *dummy = lds + NS * p.stage_bytes;  // 1 KiB sink for padding DMAs

  // First virtual row of the workgroup's halo (wave-uniform).
  const int n_first = m0 / p.PQ;
  const int p_first = (m0 - n_first * p.PQ) / p.Q;
  const int v_lo = n_first * HV + p_first * p.sh;

  // ---- per-lane halo DMA sources (channel block 0), fixed for all stages --
  uint32_t hv_off[HJ];
  int hv_dst[HJ];  // LDS offset within the halo, or -1 for the sink
#pragma unroll
  for (int j = 0; j < HJ; ++j) {
    const int g = j * T::NWAVES + wave;  // this wave's j-th halo block
    uint32_t off = OOB_OFFSET;
    int dst = -1;
    if (g < hblk) {
      const int hp = g >= p.halo_dpp;               // half-plane
      const int slot = (g - hp * p.halo_dpp) * 64 + lane;
      const int row = slot / WV;
      const int col = slot - row * WV;
      const int v = v_lo + row;
      const int n = v / HV;
      const int ih = v - n * HV - p.ph;
      const int iw = col - p.pw;
      if (n < p.N && (unsigned)ih < (unsigned)p.H && (unsigned)iw < (unsigned)p.W)
        off = (uint32_t)(((n * p.CB * p.H + ih) * p.W + iw) * 32 + hp * 16);
      dst = hp * plane + (g - hp * p.halo_dpp) * 1024;
    }
    hv_off[j] = off;
    hv_dst[j] = dst;
  }

  // ---- per-lane filter DMA sources: block g = (tap, kb) ------------------
  uint32_t fv_off[T::FJ];
#pragma unroll
  for (int j = 0; j < T::FJ; ++j) {
    const int g = j * T::NWAVES + wave;
    const int kb = g % T::KB;
    const int k = k0 + 32 * kb + l32;
    fv_off[j] = (g < T::FBLK && k < p.K) ? (uint32_t)(k * 32 + 16 * half) : OOB_OFFSET;
  }

  // ---- per-lane pixel fragment addresses inside the halo -----------------
  const int wk = wave % WK;
  const int wp = wave / WK;
  int b_addr[FP];
#pragma unroll
  for (int i = 0; i < FP; ++i) {
    const int m = m0 + 32 * (wp * FP + i) + l32;
    int a = 0;  // pixels past M read any valid slot; their columns are not stored
    if (m < p.M) {
      const int n = m / p.PQ;
      const int pq = m - n * p.PQ;
      const int op = pq / p.Q;
      const int oq = pq - op * p.Q;
      a = ((n * HV + op * p.sh - v_lo) * WV + oq * p.sw) * 16;
    }
    b_addr[i] = T::FILT_BYTES + half * plane + a;
  }
  // LDS offset of tap t = (r, s) relative to the pixel's tap (0, 0).
  int tap_off[T::RS];
#pragma unroll
  for (int t = 0; t < T::RS; ++t) tap_off[t] = ((t / S) * p.dh * WV + (t % S) * p.dw) * 16;

  const int CB = p.CB;
  const int HW32 = p.HW * 32;
  const int KB32 = p.K * 32;

  // Issue the DMAs of channel block `st` into ring slot st % NS.  Blocks
  // past the reduction are issued with every lane out of range (they zero a
  // consumed slot) so that every wave always has exactly NL loads per stage.
  auto issue_stage = [&](int st) {
    unsigned char *base = lds + (st % NS) * p.stage_bytes;
    const bool live = st < CB;
#pragma unroll
    for (int j = 0; j < HJ; ++j) {
      unsigned char *dst = hv_dst[j] >= 0 ? base + T::FILT_BYTES + hv_dst[j] : dummy;
      lds_dma16(xr, dst, live ? hv_off[j] : OOB_OFFSET, live ? st * HW32 : 0);
    }
#pragma unroll
    for (int j = 0; j < T::FJ; ++j) {
      const int g = j * T::NWAVES + wave;
      const int tap = g / T::KB;
      const int kb = g - tap * T::KB;
      unsigned char *dst = g < T::FBLK ? base + (tap * T::KB + kb) * 1024 : dummy;
      lds_dma16(wr, dst, live ? fv_off[j] : OOB_OFFSET,
                live && g < T::FBLK ? (st * T::RS + tap) * KB32 : 0);
    }
  };

  v4i af[2][FK], bf[2][FP];
  auto read_frags = [&](int st, int t, v4i (&a)[FK], v4i (&b)[FP]) {
    const unsigned char *base = lds + (st % NS) * p.stage_bytes;
#pragma unroll
    for (int i = 0; i < FK; ++i)
      a[i] = *reinterpret_cast<const v4i *>(base + ((t * T::KB + wk * FK + i) * 64 + lane) * 16);
#pragma unroll
    for (int i = 0; i < FP; ++i)
      b[i] = *reinterpret_cast<const v4i *>(base + b_addr[i] + tap_off[t]);
  };

  v16i acc[FK][FP];
#pragma unroll
  for (int a = 0; a < FK; ++a)
#pragma unroll
    for (int b = 0; b < FP; ++b) acc[a][b] = v16i{0};

  // Ring schedule as in conv_i8.hip: barrier B_k certifies stage k landed and
  // stage k-2 fully read; B_{st+1} sits before the last tap of stage st.
#pragma unroll
  for (int s0 = 0; s0 < NS - 1; ++s0) issue_stage(s0);
  halo_wait<T::NL * (NS - 2)>();
  halo_barrier();
  read_frags(0, 0, af[0], bf[0]);

  // One stage; PAR is the fragment buffer of its tap 0 (R*S may be odd).
  auto stage = [&](auto par_c, int st) {
    constexpr int PAR = decltype(par_c)::value;
#pragma unroll
    for (int t = 0; t < T::RS; ++t) {
      const int cur = (t + PAR) & 1;
      const int nxt = (t + 1 + PAR) & 1;
      if (t + 1 < T::RS) {
        read_frags(st, t + 1, af[nxt], bf[nxt]);
      } else {
        halo_wait<T::NL * (NS - 3)>();
        halo_barrier();
        issue_stage(st + NS - 1);
        read_frags(st + 1, 0, af[nxt], bf[nxt]);
      }
#pragma unroll
      for (int a = 0; a < FK; ++a)
#pragma unroll
        for (int b = 0; b < FP; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[cur][a], bf[cur][b], acc[a][b], 0, 0, 0);
#pragma unroll
      for (int i = 0; i < FK * FP; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // one LDS-DMA load
      }
    }
  };
  using Par0 = std::integral_constant<int, 0>;
  using Par1 = std::integral_constant<int, 1>;
  if constexpr (T::RS % 2 == 0) {
    for (int st = 0; st < CB; ++st) stage(Par0{}, st);
  } else {
    for (int st = 0; st < CB; st += 2) {
      stage(Par0{}, st);
      if (st + 1 < CB) stage(Par1{}, st + 1);
    }
  }
  halo_wait<0>();  // no LDS-DMA may outlive the workgroup

  store_i8_tile<PC, FK, FP>(acc, y, p, m0 + 32 * wp * FP, k0 / 32 + wk * FK, lane);
}

// ---------------------------------------------------------------------------
// Variant with the filter operand in registers.  Each wave loads its own
// MFMA filter fragments straight from global memory (16 bytes per lane, the
// MFMA operand order of CxRSKx<32>), AHEAD taps ahead (halo_filter_ahead),
// into a ring of RS register slots; LDS holds only the activation halo.  This halves the LDS
// bytes read per MFMA -- with 64-wide fragments LDS reads, not the matrix
// unit, bound the all-LDS variant -- and shrinks a stage to the halo alone.
//
// Wait accounting: the halo LDS-DMAs and the filter loads share vmcnt, which
// retires in issue order, so a wait for a halo batch may only count loads
// that are certain to issue after that batch and before the wait.  The
// compiler may move a filter load later (into the block that uses it) but
// not earlier, so each count below is a lower bound under any such move:
//   prologue (stage 0's halo batch and the filter of taps 0..AHEAD-1, both
//   by LDS-DMA; no register loads):
//                             0                -> both have landed.  Stages
//                             1..NS-2 are issued only after this wait, so at
//                             kernel start stage 0 does not share the memory
//                             system with the later stages' halos.
//   end of stage st (before issuing stage st+NS-1; stage st+1 must have
//   landed):                  (NS-3)*HJ*CPS + TPS*FK
// The second counts the later halo batches plus the stage's own TPS*FK
// filter loads (TPS = R*S*CPS taps per stage), which precede the wait in one
// straight-line block: the stage loop has no conditional stage (an odd last
// stage runs after it).
//
// PW > 0 fixes the halo's row pitch in LDS at PW pixels (>= the halo width)
// and the dilation at 1, so every tap's offset inside the halo is a
// compile-time constant: the LDS reads take it as an immediate and the
// inner loop needs no address arithmetic.  PW = 0 keeps the pitch at the
// halo width and any dilation.
//
// AL = 1 moves the filter operand into the ring too: each stage also holds
// the filter of its TPS taps for the workgroup's KB channel blocks (block
// t*KB + kb, 1 KiB, MFMA operand order), brought in by LDS-DMA once per
// workgroup, and the waves read both operands from LDS one tap ahead.  The
// waves that share output channels then no longer each pull the same
// filter bytes from L2 (WP copies per workgroup), at the cost of LDS reads.
// With no register loads, every vmcnt event is an LDS-DMA.  The NB DMAs of
// stage st+NS-1 go out one per tap during stage st (its ring slot held
// stage st-1, which the barrier at the end of stage st-1 released), so the
// wait at the end of stage st counts NS-2 whole batches.
//
// SW = 1 or 2 lays the halo out swizzled (halo_swizzle.hpp) for problems of
// that horizontal stride; the layout's arithmetic is then straight-line code.
template <int WK, int WP, int FK, int FP, int R, int S, int NS, int HJ, int PW = 0,
          int CPS = 1, int AL = 0, int SW = 0, int PT = 0, int RG = 0>
struct HaloAdTile {
  static constexpr int NWAVES = WK * WP;
  static constexpr int THREADS = 64 * NWAVES;
  static constexpr int KB = WK * FK;
  static constexpr int PB = WP * FP;
  // Pixel fragments in the tile.  PT < WP*FP leaves the last wave column
  // FPL < FP fragments: with WK = 4, WP = 2, FP = 4, PT = 7 the two waves of
  // a SIMD (waves w and w+4) own 4 + 3 fragments of the same 32 channels,
  // 7 blocks per SIMD for a 128 x 224 tile.
  static constexpr int PTILE = PT ? PT : PB;
  static constexpr int FPL = PTILE - FP * (WP - 1);
  static_assert(FPL >= 1 && FPL <= FP, "only the last wave column may be short");
  static_assert(PTILE == PB || CPS == 1, "a short wave column needs one channel block per stage");
  static constexpr int BM = 32 * KB;
  static constexpr int BN = 32 * PTILE;
  static constexpr int RS = R * S;
  static constexpr int AHEAD = halo_filter_ahead(RS);
  static constexpr int TPS = RS * CPS;  // taps per stage
  static constexpr int WAIT0 = 0;
  // The prologue brings the filter of taps 0..AHEAD-1 into LDS once per
  // workgroup (AHEAD*KB blocks of 1 KiB, AJ per wave) instead of once per
  // wave: the waves that share output channels would otherwise each load it.
  static constexpr int APRO_BLK = AHEAD * KB;
  static constexpr int APRO_BYTES = APRO_BLK * 1024;
  static constexpr int AJ = AL ? 0 : (APRO_BLK + NWAVES - 1) / NWAVES;
  // AL = 1: filter blocks per stage and filter DMAs per wave per stage
  static constexpr int FBLK = TPS * KB;
  static constexpr int FJ = AL ? (FBLK + NWAVES - 1) / NWAVES : 0;
  // AL = 1: DMAs per wave per stage; they go out one per tap through the
  // stage NS-1 ahead (its slot was freed by the previous stage barrier)
  static constexpr int NB = HJ * CPS + FJ;
  static constexpr int WAITL = AL ? (NS - 2) * NB : (NS - 3) * HJ * CPS + TPS * FK;
  static_assert(NS >= 3 || (AL && NS == 2) || (RG && NS == 2),
                "the ring needs a stage being read, one landed and one in flight (a two-slot "
                "ring, filter in LDS only, issues a whole stage at the start of the one before; "
                "with the halo through registers, the registers hold the one in flight)");
  static_assert(!RG || (SW && !AL && CPS == 1), "register-staged halo: swizzled, filter in registers");
  static_assert(WAIT0 < 64 && WAITL < 64, "vmcnt counts at most 63 outstanding loads");
  static_assert(SW >= 0 && SW <= 2, "swizzled halo for horizontal stride 1 or 2");
  static_assert(!SW || (PW >= 16 && (PW & (PW - 1)) == 0),
                "the swizzled halo rotates rows within a power-of-two pitch");
  // Swizzled halo: every stage takes the ring slot space of the most halo
  // DMA blocks the configuration issues (HB per channel block), so a slot's
  // base is a compile-time constant and folds, with the lane's tap offset
  // register, into the LDS read's immediate offset.
  static constexpr int HB = HJ * NWAVES * 1024;
  static constexpr int SB = CPS * HB + (AL ? FBLK * 1024 : 0);
  static constexpr int UNROLL = (TPS % 2) ? (NS % 2 ? 2 * NS : NS) : NS;  // lcm(NS, parity)
  static_assert(!SW || (NS - 1) * SB < 2 * 65536, "slot bases past 128 KiB");
};

template <int WK, int WP, int FK, int FP, int R, int S, int NS, int HJ, int PW, int CPS, int AL,
          int SW, int PT, int RG, bool PC>
__global__ void __launch_bounds__(64 * WK * WP)
conv_i8_halo_ad_kernel(const int8_t *__restrict__ x, const int8_t *__restrict__ w,
                       int8_t *__restrict__ y, I8Params p) {
  using T = HaloAdTile<WK, WP, FK, FP, R, S, NS, HJ, PW, CPS, AL, SW, PT, RG>;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int mtile = fast_div(tile, p.fd_kt);
  const int ktile = tile - mtile * p.k_tiles;
  const int k0 = ktile * T::BM;
  const int m0 = mtile * T::BN;

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, p.x_bytes);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, p.w_bytes);

  const int HV = p.HV, WV = p.WV;
  const int WVL = PW > 0 ? PW : WV;  // halo row pitch in LDS, pixels
  // half-plane offset in a ring slot (RG: half of the slot; p.halo_dpp then
  // counts the row-major blocks the registers bring per half-plane)
  const int plane = RG ? T::SB / 2 : p.halo_dpp * 1024;
  const int hblk = 2 * p.halo_dpp;
  unsigned char *dummy = lds + NS * p.stage_bytes;

  const int n_first = fast_div(m0, p.fd_pq);
  const int p_first = fast_div(m0 - n_first * p.PQ, p.fd_q);
  const int v_lo = n_first * HV + p_first * p.sh;

  // ---- per-lane halo DMA sources (channel block 0) ------------------------
  // Lane l of halo block g writes slot 64*g' + l of its half-plane; it loads
  // the halo column that the layout puts in that slot.
  uint32_t hv_off[HJ];
  int hv_dst[HJ];
#pragma unroll
  for (int j = 0; j < HJ; ++j) {
    const int g = j * T::NWAVES + wave;
    uint32_t off = OOB_OFFSET;
    int dst = -1;
    if constexpr (RG) {
      // register-staged halo: lane l of block g loads element
      // q = 64 (g - hp*dpp) + l of its half-plane in row-major order (rows
      // of WV columns: consecutive lanes, consecutive pixels) and later
      // writes it to that element's swizzled slot; lanes past the slot's
      // capacity write nothing
      if (g < hblk) {
        const int hp = g >= p.halo_dpp;
        // (consecutive lanes take consecutive pixels: coalesced loads; at
        // stride 2 an even and an odd column share an LDS bank, so the writes
        // conflict two ways.  Giving each 16 lanes columns of one parity
        // instead makes the writes conflict-free but the loads strided, and
        // the kernel slower.)
        const int q = (g - hp * p.halo_dpp) * 64 + lane;
        const int row = fast_div(q, p.fd_wv);
        const int col = q - row * WV;
        if (row * PW < T::SB / 32) {
          const int v = v_lo + row;
          const int n = fast_div(v, p.fd_hv);
          const int ih = v - n * HV - p.ph;
          const int iw = col - p.pw;
          if (n < p.N && (unsigned)ih < (unsigned)p.H && (unsigned)iw < (unsigned)p.W)
            off = (uint32_t)(((n * p.CB * p.H + ih) * p.W + iw) * 32 + hp * 16);
          const int rot = (p.Q * (n * p.P + fast_div(v - n * HV, p.fd_sh))) & 15;
          dst = hp * plane + 16 * (row * PW + ((halo_split(col, SW, PW) + rot) & (PW - 1)));
        }
      }
      hv_off[j] = off;
      hv_dst[j] = dst;
      continue;
    }
    if constexpr (PW == 64) {
      // A block of 64 slots is one whole row: its image, bounds, base offset
      // and rotation are the same for the whole wave (scalar work); a lane
      // adds only its column.  (At pitch 32 a block holds two rows, and the
      // per-lane form below times the same.)
      if (g < hblk) {
        const int hp = g >= p.halo_dpp;
        const int gb = g - hp * p.halo_dpp;
        const int v = v_lo + gb;
        const int n = fast_div(v, p.fd_hv);
        const int ih = v - n * HV - p.ph;
        const bool row_ok = n < p.N && (unsigned)ih < (unsigned)p.H;
        // + 32 * column gives the offset of input column (column - pad_w)
        const uint32_t rbase = ((uint32_t)((n * p.CB * p.H + ih) * p.W) - (uint32_t)p.pw) * 32u + hp * 16;
        const int rot = SW ? (p.Q * (n * p.P + fast_div(v - n * HV, p.fd_sh))) & 15 : 0;
        const int col = SW ? halo_column_at(lane, rot, SW, PW, WV) : (lane < WV ? lane : -1);
        if (col >= 0 && row_ok && (unsigned)(col - p.pw) < (unsigned)p.W) off = rbase + (uint32_t)col * 32u;
        dst = hp * plane + gb * 1024;
      }
      hv_off[j] = off;
      hv_dst[j] = dst;
      continue;
    }
    if (g < hblk) {
      const int hp = g >= p.halo_dpp;
      const int slot = (g - hp * p.halo_dpp) * 64 + lane;
      int row, col;
      if constexpr (SW) {
        row = slot / PW;
      } else {
        row = PW > 0 ? slot / PW : fast_div(slot, p.fd_wv);
        col = slot - row * WVL;
        if (col >= WV) col = -1;
      }
      const int v = v_lo + row;
      const int n = fast_div(v, p.fd_hv);
      if constexpr (SW) {  // the row's rotation (halo_rot), then the inverse swizzle
        const int rot = (p.Q * (n * p.P + fast_div(v - n * HV, p.fd_sh))) & 15;
        col = halo_column_at(slot & (PW - 1), rot, SW, PW, WV);
      }
      const int ih = v - n * HV - p.ph;
      const int iw = col - p.pw;
      if (col >= 0 && n < p.N && (unsigned)ih < (unsigned)p.H && (unsigned)iw < (unsigned)p.W)
        off = (uint32_t)(((n * p.CB * p.H + ih) * p.W + iw) * 32 + hp * 16);
      dst = hp * plane + (g - hp * p.halo_dpp) * 1024;
    }
    hv_off[j] = off;
    hv_dst[j] = dst;
  }

  const int wk = wave % WK;
  const int wp = wave / WK;

  // Per-lane operand and output offsets: declared here, worked out once
  // stage 0's DMAs are out (below), so that the DMAs wait only for their own
  // source offsets.
  uint32_t a_off[FK];        // filter fragments (channels past K read zeros)
  int b_addr_c[CPS][FP];     // pixel fragments in the halo, per channel block of a stage
  int tap_off[T::RS];
  uint32_t y_off[FP];        // output offsets of the wave's pixel fragments
  const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, p.y_bytes);
  // Swizzled halo: a tap's slot is no fixed distance from the pixel's, so
  // each lane keeps the LDS offset of every (fragment, tap) it reads.
  int b_tap[SW ? FP : 1][SW ? T::RS : 1];  // filled after the first DMAs are out (below)
  // LDS offset of fragment i at tap t of the stage (t < TPS) from the slot base
  auto b_off = [&](int i, int t) __attribute__((always_inline)) -> int  {
    if constexpr (SW)
      return b_tap[i][t % T::RS] + (t / T::RS) * p.halo_bytes;
    else
      return b_addr_c[t / T::RS][i] + tap_off[t % T::RS];
  };

  const int CB = p.CB;
  const int ntaps = CB * T::RS;
  const int HW32 = p.HW * 32;
  const int KB32 = p.K * 32;

  const int NST = CB / CPS;  // stages (the plan keeps CB a multiple of CPS)

  // AL = 1: the stage's filter follows its CPS halos; this wave's filter
  // DMA j carries block g = j*NWAVES + wave = t*KB + kb of the stage.
  const int filt_off = SW ? CPS * T::HB : CPS * p.halo_bytes;
  uint32_t fv_off[T::FJ > 0 ? T::FJ : 1];
#pragma unroll
  for (int j = 0; j < T::FJ; ++j) {
    const int g = j * T::NWAVES + wave;
    const int k = k0 + 32 * (g % T::KB) + l32;
    fv_off[j] = g < T::FBLK && k < p.K ? (uint32_t)(k * 32 + 16 * half) : OOB_OFFSET;
  }

  auto issue_stage = [&](int st) __attribute__((always_inline)) {
    unsigned char *base = lds + (st % NS) * p.stage_bytes;
    const bool live = st < NST;
#pragma unroll
    for (int c = 0; c < CPS; ++c)
#pragma unroll
      for (int j = 0; j < HJ; ++j) {
        unsigned char *dst = hv_dst[j] >= 0 ? base + c * p.halo_bytes + hv_dst[j] : dummy;
        lds_dma16(xr, dst, live ? hv_off[j] : OOB_OFFSET, live ? (st * CPS + c) * HW32 : 0);
      }
#pragma unroll
    for (int j = 0; j < T::FJ; ++j) {
      const int g = j * T::NWAVES + wave;
      const int t = g / T::KB;
      const bool ok = g < T::FBLK;
      lds_dma16(wr, ok ? base + filt_off + g * 1024 : dummy, live ? fv_off[j] : OOB_OFFSET,
                live && ok ? (st * T::TPS + t) * KB32 : 0);
    }
  };

  // RG = 1: stage st's halo into registers (coalesced 16-byte loads), and
  // from registers into ring slot K (scattered 16-byte LDS writes)
  v4i hreg[RG ? HJ : 1];
  auto load_halo = [&](int st) __attribute__((always_inline)) {
    const bool live = st < NST;
#pragma unroll
    for (int j = 0; j < HJ; ++j) hreg[j] = load_b128_s(xr, live ? hv_off[j] : OOB_OFFSET, live ? st * HW32 : 0);
  };
  auto write_halo = [&](int K) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < HJ; ++j)
      if (hv_dst[j] >= 0) *reinterpret_cast<v4i *>(lds + K * T::SB + hv_dst[j]) = hreg[j];
  };

  // AL = 1: the d-th of the NB DMAs of stage st (halo blocks, then filter)
  auto issue_dma = [&](int st, int d) __attribute__((always_inline)) {
    unsigned char *base = lds + (st % NS) * p.stage_bytes;
    const bool live = st < NST;
    if (d < HJ * CPS) {
      const int c = d / HJ, j = d % HJ;
      unsigned char *dst = hv_dst[j] >= 0 ? base + c * p.halo_bytes + hv_dst[j] : dummy;
      lds_dma16(xr, dst, live ? hv_off[j] : OOB_OFFSET, live ? (st * CPS + c) * HW32 : 0);
    } else {
      const int j = d - HJ * CPS;
      const int g = j * T::NWAVES + wave;
      const int t = g / T::KB;
      const bool ok = g < T::FBLK;
      lds_dma16(wr, ok ? base + filt_off + g * 1024 : dummy, live ? fv_off[j] : OOB_OFFSET,
                live && ok ? (st * T::TPS + t) * KB32 : 0);
    }
  };

  // Filter fragments of global tap g = cb*RS + t into a register slot; taps
  // past the end (prefetched, never used) re-read the last one.
  v4i aring[T::RS][FK];
  auto load_a = [&](int g, v4i (&dst)[FK]) __attribute__((always_inline)) {
    const int soff = (g < ntaps ? g : ntaps - 1) * KB32;
#pragma unroll
    for (int i = 0; i < FK; ++i) dst[i] = load_b128_s(wr, a_off[i], soff);
  };

  // Reads of stage st, held in ring slot K = st % NS.  slot_c is
  // Slot<K> when K is known at compile time (the swizzled kernels' unrolled
  // ring), else Slot<-1>.  With a compile-time K the slot base is an
  // immediate: below 64 KiB it goes straight into the read's offset field;
  // above, the lane's offset register carries 64 KiB (b_tap_hi) and the
  // immediate the rest.
  int b_tap_hi[SW ? FP : 1][SW ? T::RS : 1];
  auto slot_base = [&](auto slot_c, int st) __attribute__((always_inline)) -> const unsigned char *  {
    constexpr int K = decltype(slot_c)::value;
    if constexpr (SW && K >= 0)
      return lds + K * T::SB;
    else
      return lds + (st % NS) * p.stage_bytes;
  };
  v4i af[2][FK];
  auto read_a = [&](auto slot_c, int st, int t, v4i (&a)[FK]) __attribute__((always_inline)) {  // AL = 1; t: tap within the stage
    const unsigned char *base = slot_base(slot_c, st) + filt_off;
#pragma unroll
    for (int i = 0; i < FK; ++i)
      a[i] = *reinterpret_cast<const v4i *>(base + ((t * T::KB + wk * FK + i) * 64 + lane) * 16);
  };

  // b: the wave's pixel fragments (FP, or FPL in a short wave column)
  auto read_b = [&](auto slot_c, int st, int t, auto &b) __attribute__((always_inline)) {  // t: tap within the stage
    constexpr int K = decltype(slot_c)::value;
    constexpr int NF = std::extent_v<std::remove_reference_t<decltype(b)>>;
    if constexpr (SW && K >= 0 && K * T::SB >= 65536) {
      const unsigned char *base = lds + K * T::SB - 65536;
#pragma unroll
      for (int i = 0; i < NF; ++i)
        b[i] = *reinterpret_cast<const v4i *>(base + b_tap_hi[i][t % T::RS] + (t / T::RS) * T::HB);
    } else if constexpr (SW && K >= 0) {
      const unsigned char *base = lds + K * T::SB;
#pragma unroll
      for (int i = 0; i < NF; ++i)
        b[i] = *reinterpret_cast<const v4i *>(base + b_tap[i][t % T::RS] + (t / T::RS) * T::HB);
    } else {
      const unsigned char *base = slot_base(slot_c, st);
#pragma unroll
      for (int i = 0; i < NF; ++i) b[i] = *reinterpret_cast<const v4i *>(base + b_off(i, t));
    }
  };
  using RtSlot = std::integral_constant<int, -1>;

  // Prologue: stage 0's halo and the filter of taps 0..AHEAD-1 (block
  // g = tap*KB + kb at pro_off + g KiB, the MFMA operand order), then the
  // other stages once those have landed.  pro_off is a ring slot that is
  // first written at the end of stage 0, or space of its own (always with
  // the halo through registers, which writes the next slot during stage 0).
  if constexpr (RG)
    load_halo(0);
  else
    issue_stage(0);
  unsigned char *apro = lds + p.pro_off;
#pragma unroll
  for (int j = 0; j < T::AJ; ++j) {  // AL = 0 only (AJ = 0 otherwise)
    const int g = j * T::NWAVES + wave;
    const int tap = g / T::KB;
    const int kb = g - tap * T::KB;
    const int k = k0 + 32 * kb + l32;
    const bool ok = g < T::APRO_BLK;
    lds_dma16(wr, ok ? apro + g * 1024 : dummy,
              ok && k < p.K ? (uint32_t)(k * 32 + 16 * half) : OOB_OFFSET, ok ? tap * KB32 : 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  // ---- per-lane filter fragment offsets --------------------------------
#pragma unroll
  for (int i = 0; i < FK; ++i) {
    const int k = k0 + 32 * (wk * FK + i) + l32;
    a_off[i] = k < p.K ? (uint32_t)(k * 32 + 16 * half) : OOB_OFFSET;
  }
  // ---- per-lane pixel fragment addresses inside the halo -----------------
  if constexpr (!SW) {
#pragma unroll
    for (int i = 0; i < FP; ++i) {
      const int m = m0 + 32 * (wp * FP + i) + l32;
      int a = 0;
      if (m < p.M) {
        const int n = fast_div(m, p.fd_pq);
        const int pq = m - n * p.PQ;
        const int op = fast_div(pq, p.fd_q);
        const int oq = pq - op * p.Q;
        a = ((n * HV + op * p.sh - v_lo) * WVL + oq * p.sw) * 16;
      }
      // the halo of the stage's c-th channel block sits c * halo_bytes further
#pragma unroll
      for (int c = 0; c < CPS; ++c) b_addr_c[c][i] = half * plane + a + c * p.halo_bytes;
    }
#pragma unroll
    for (int t = 0; t < T::RS; ++t)
      tap_off[t] = PW > 0 ? ((t / S) * PW + (t % S)) * 16 : ((t / S) * p.dh * WV + (t % S) * p.dw) * 16;
  }
  // output offsets (decoded here, off the epilogue's critical path)
#pragma unroll
  for (int i = 0; i < FP; ++i) y_off[i] = i8_pixel_yoff(p, m0 + 32 * (wp * FP + i) + l32, half);
  // Swizzled halo: the lanes' tap offsets are worked out while stage 0's
  // DMAs are in flight, off the path to their issue.
  if constexpr (SW) {
    int rdh_sh[R];  // floor(r * dh / sh), wave-uniform
#pragma unroll
    for (int r = 0; r < R; ++r) rdh_sh[r] = fast_div(r * p.dh, p.fd_sh);
#pragma unroll
    for (int i = 0; i < FP; ++i) {
      int m = m0 + 32 * (wp * FP + i) + l32;
      if (m >= p.M) m = m0;  // pixels past M read the tile's first pixel; never stored
      const int n = fast_div(m, p.fd_pq);
      const int pq = m - n * p.PQ;
      const int op = fast_div(pq, p.fd_q);
      const int oq = pq - op * p.Q;
      const int vrel = n * HV + op * p.sh - v_lo;
      if constexpr (SW == 1) {
        // halo_slot_of_pixel at stride 1, term by term: row r's base (a
        // multiple of 16 * PW, so the in-row part ORs in), the row's rotation
        // from the lane's output-row start, then two operations per tap
        const int rbase = half * plane + 16 * PW * vrel;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int rot = (m - oq + p.Q * rdh_sh[r]) & 15;
          const int w16 = (oq + rot) << 4;
          const int base = rbase + 16 * PW * r * p.dh;
#pragma unroll
          for (int s = 0; s < S; ++s)
            b_tap[i][r * S + s] = ((w16 + 16 * s * p.dw) & (16 * (PW - 1))) | base;
        }
      } else {
#pragma unroll
        for (int t = 0; t < T::RS; ++t)
          b_tap[i][t] = half * plane + 16 * halo_slot_of_pixel(vrel + (t / S) * p.dh,
                                                               oq * SW + (t % S) * p.dw, m, oq,
                                                               p.Q, rdh_sh[t / S], SW, PW);
      }
    }
  }
  if constexpr (SW && (NS - 1) * T::SB >= 65536) {  // some slot base needs it
#pragma unroll
    for (int i = 0; i < FP; ++i)
#pragma unroll
      for (int t = 0; t < T::RS; ++t) {
        b_tap_hi[i][t] = b_tap[i][t] + 65536;
        asm volatile("" : "+v"(b_tap_hi[i][t]));  // keep it a register of its own
      }
  }
  __builtin_amdgcn_sched_barrier(0);
  halo_wait<T::WAIT0>();
  if constexpr (RG) {
    write_halo(0);
    halo_wait<63>();  // the LDS writes
  }
  halo_barrier();
  if constexpr (RG) {
    load_halo(1);
  } else {
#pragma unroll
    for (int s0 = 1; s0 < NS - 1; ++s0) issue_stage(s0);
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (AL) {
    read_a(std::integral_constant<int, 0>{}, 0, 0, af[0]);
  } else {
#pragma unroll
    for (int g = 0; g < T::AHEAD; ++g)
#pragma unroll
      for (int i = 0; i < FK; ++i)
        aring[g][i] = *reinterpret_cast<const v4i *>(apro + ((g * T::KB + wk * FK + i) * 64 + lane) * 16);
  }

  // The main loop and the epilogue, for a wave of NF pixel fragments (FP, or
  // FPL in the last wave column of a short tile; both run the same stages,
  // waits and barriers).
  auto body = [&](auto nf_c) __attribute__((always_inline)) {
  constexpr int NF = decltype(nf_c)::value;
  v16i acc[FK][NF];
  v4i bf[2][NF];
  read_b(std::integral_constant<int, 0>{}, 0, 0, bf[0]);

  // One ring stage; PAR is the fragment buffer of its tap 0 (the stage's
  // taps may be odd), slot_c its ring slot (see read_b).
  auto stage = [&](auto par_c, auto slot_c, int st) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par_c)::value;
    constexpr int KS = decltype(slot_c)::value;
    using NextSlot = std::integral_constant<int, KS < 0 ? -1 : (KS + 1) % NS>;
#pragma unroll
    for (int t = 0; t < T::TPS; ++t) {
      const int cur = (t + PAR) & 1;
      const int nxt = (t + 1 + PAR) & 1;
      if constexpr (!AL) load_a(st * T::TPS + t + T::AHEAD, aring[(t + T::AHEAD) % T::RS]);
      if constexpr (RG) {
        // one register block of stage st+1 per tap into its slot (two slots:
        // it held stage st-1, released by that stage's barrier), then its
        // register reloaded with stage st+2's block; the compiler waits for
        // each load (issued a stage earlier) before its write
        constexpr int NEXT = KS >= 0 ? (KS + 1) % NS : -1;
        static_assert(NS == 2, "register-staged halo: a two-slot ring");
        if (t < HJ) {
          const int j = t;
          if (hv_dst[j] >= 0)
            *reinterpret_cast<v4i *>(lds + (NEXT >= 0 ? NEXT : (st + 1) % NS) * T::SB + hv_dst[j]) = hreg[j];
          const bool live = st + 2 < NST;
          hreg[j] = load_b128_s(xr, live ? hv_off[j] : OOB_OFFSET, live ? (st + 2) * HW32 : 0);
        }
      }
      if constexpr (AL) {
        if constexpr (NS == 2) {
          // two slots: the next stage's slot was freed by the barrier that
          // ended the previous stage; all its DMAs go out now and have the
          // whole stage to land
          if (t == 0) {
#pragma unroll
            for (int d = 0; d < T::NB; ++d) issue_dma(st + 1, d);
          }
        } else if (t + 1 < T::TPS) {
          // this tap's share of stage st+NS-1's DMAs (the rest at the last tap)
          if (t < T::NB) issue_dma(st + NS - 1, t);
        } else {
#pragma unroll
          for (int d = T::TPS - 1; d < T::NB; ++d) issue_dma(st + NS - 1, d);
        }
      }
      if (t + 1 < T::TPS) {
        if constexpr (AL) read_a(slot_c, st, t + 1, af[nxt]);
        read_b(slot_c, st, t + 1, bf[nxt]);
      } else {
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (RG) {
          static_assert(!RG || HJ <= T::TPS, "one register block per tap");
          halo_wait<63>();  // this stage's LDS writes (and reads) complete
          halo_barrier();
        } else {
          halo_wait<T::WAITL>();
          halo_barrier();
          if constexpr (!AL) issue_stage(st + NS - 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (AL) read_a(NextSlot{}, st + 1, 0, af[nxt]);
        read_b(NextSlot{}, st + 1, 0, bf[nxt]);
      }
      // Pixel-fragment-major order: fragment b of this tap is done after its
      // FK MFMAs, and the next tap's fragment b is read into its registers
      // right then, a whole tap ahead of its first use.
#pragma unroll
      for (int b = 0; b < NF; ++b)
#pragma unroll
        for (int a = 0; a < FK; ++a)
          acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(AL ? af[cur][a] : aring[t % T::RS][a],
                                                            bf[cur][b], acc[a][b], 0, 0, 0);
#pragma unroll
      for (int b = 0; b < NF; ++b) {
        __builtin_amdgcn_sched_group_barrier(0x008, FK, 0);  // fragment b's MFMAs
        if constexpr (AL) {
          // this tap's reads for the next: FP pixel and FK filter fragments
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          if (b < FK) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        } else {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
          if (b < FK) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one filter load
        }
      }
    }
  };
  using Par0 = std::integral_constant<int, 0>;
  using Par1 = std::integral_constant<int, 1>;
  // With one channel block per stage the last stage runs apart (below); the
  // ring loop runs the others.
  const int NRING = CPS == 1 ? NST - 1 : NST;
#pragma unroll
  for (int a = 0; a < FK; ++a)
#pragma unroll
    for (int b = 0; b < NF; ++b) acc[a][b] = v16i{0};
  if constexpr (SW) {
    // Unrolled over UNROLL = lcm(NS, tap parity) stages, so that every
    // stage's ring slot and parity are compile-time constants; the remainder
    // runs the same bodies behind a run-time guard.
    int st = 0;
    for (; st + T::UNROLL <= NRING; st += T::UNROLL) {
      [&]<int... Ks>(std::integer_sequence<int, Ks...>) {
        (stage(std::integral_constant<int, (T::TPS % 2) ? Ks % 2 : 0>{},
               std::integral_constant<int, Ks % NS>{}, st + Ks),
         ...);
      }(std::make_integer_sequence<int, T::UNROLL>{});
    }
    [&]<int... Ks>(std::integer_sequence<int, Ks...>) {
      ((st + Ks < NRING ? stage(std::integral_constant<int, (T::TPS % 2) ? Ks % 2 : 0>{},
                                std::integral_constant<int, Ks % NS>{}, st + Ks)
                        : void()),
       ...);
    }(std::make_integer_sequence<int, T::UNROLL - 1>{});
  } else if constexpr (T::TPS % 2 == 0) {
    for (int st = 0; st < NRING; ++st) stage(Par0{}, RtSlot{}, st);
  } else {
    int st = 0;
    for (; st + 1 < NRING; st += 2) {
      stage(Par0{}, RtSlot{}, st);
      stage(Par1{}, RtSlot{}, st + 1);
    }
    if (st < NRING) stage(Par0{}, RtSlot{}, st);
  }
  const int m_wave = m0 + 32 * wp * FP;
  const int kb_wave = k0 / 32 + wk * FK;
  if constexpr (CPS == 1) {
    // Last stage, pixel-fragment by pixel-fragment: once fragment b has all
    // its taps, its epilogue (vector ALU work and the store) overlaps the
    // MFMAs of fragment b+1.  The stage's halo landed at the previous
    // stage's wait; the ring holds the filter of its taps 0..AHEAD-1 and the
    // others are loaded here.
    const int st = NST - 1;
    if constexpr (!AL) {
#pragma unroll
      for (int g = T::AHEAD; g < T::RS; ++g) load_a(st * T::TPS + g, aring[g % T::RS]);
    }
    const unsigned char *base = lds + (st % NS) * p.stage_bytes;
#pragma unroll
    for (int b = 0; b < NF; ++b) {
      v4i bb[2], aa[2][FK];
      bb[0] = *reinterpret_cast<const v4i *>(base + b_off(b, 0));
      if constexpr (AL) read_a(RtSlot{}, st, 0, aa[0]);
#pragma unroll
      for (int t = 0; t < T::RS; ++t) {
        if (t + 1 < T::RS) {
          bb[(t + 1) & 1] = *reinterpret_cast<const v4i *>(base + b_off(b, t + 1));
          if constexpr (AL) read_a(RtSlot{}, st, t + 1, aa[(t + 1) & 1]);
        }
#pragma unroll
        for (int a = 0; a < FK; ++a)
          acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(AL ? aa[t & 1][a] : aring[t][a], bb[t & 1],
                                                            acc[a][b], 0, 0, 0);
      }
#pragma unroll
      for (int a = 0; a < FK; ++a) store_i8_frag<PC>(acc[a][b], yr, y_off[b], kb_wave + a, p);
    }
    halo_wait<0>();  // no LDS-DMA (of the ring's idle stages) may outlive the workgroup
  } else {
    halo_wait<0>();
    store_i8_tile<PC, FK, NF>(acc, y, p, m_wave, kb_wave, lane);
  }
  };  // body
  if constexpr (T::FPL == FP)
    body(std::integral_constant<int, FP>{});
  else if (wp == WP - 1)
    body(std::integral_constant<int, T::FPL>{});
  else
    body(std::integral_constant<int, FP>{});
}

template <int WK, int WP, int FK, int FP, int R, int S, int NS, int HJ, int PW, int CPS, int AL,
          int SW, int PT, int RG, bool PC>
static hipError_t launch_i8_halo_ad_pc(const int8_t *x, const int8_t *w, int8_t *y,
                                       const I8Params &p, int grid, hipStream_t s) {
  using T = HaloAdTile<WK, WP, FK, FP, R, S, NS, HJ, PW, CPS, AL, SW, PT, RG>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void *>(
          &conv_i8_halo_ad_kernel<WK, WP, FK, FP, R, S, NS, HJ, PW, CPS, AL, SW, PT, RG, PC>),
      hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (attr != hipSuccess) return attr;
  return launch_kernel(
      &conv_i8_halo_ad_kernel<WK, WP, FK, FP, R, S, NS, HJ, PW, CPS, AL, SW, PT, RG, PC>, dim3(grid),
      dim3(T::THREADS), p.lds_bytes, s, x, w, y, p);
}

template <int WK, int WP, int FK, int FP, int R, int S, int NS, int HJ, int PW, int CPS, int AL,
          int SW, int PT, int RG>
static hipError_t launch_i8_halo_ad(const int8_t *x, const int8_t *w, int8_t *y,
                                    const I8Params &p, int grid, hipStream_t s) {
  return p.alpha_k ? launch_i8_halo_ad_pc<WK, WP, FK, FP, R, S, NS, HJ, PW, CPS, AL, SW, PT, RG, true>(
                         x, w, y, p, grid, s)
                   : launch_i8_halo_ad_pc<WK, WP, FK, FP, R, S, NS, HJ, PW, CPS, AL, SW, PT, RG, false>(
                         x, w, y, p, grid, s);
}

template <int WK, int WP, int FK, int FP, int R, int S, int NS, int HJ, bool PC>
static hipError_t launch_i8_halo_pc(const int8_t *x, const int8_t *w, int8_t *y,
                                    const I8Params &p, int grid, hipStream_t s) {
  using T = HaloTile<WK, WP, FK, FP, R, S, NS, HJ>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void *>(&conv_i8_halo_kernel<WK, WP, FK, FP, R, S, NS, HJ, PC>),
      hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (attr != hipSuccess) return attr;
  return launch_kernel(&conv_i8_halo_kernel<WK, WP, FK, FP, R, S, NS, HJ, PC>, dim3(grid),
                     dim3(T::THREADS), p.lds_bytes, s, x, w, y, p);
}

template <int WK, int WP, int FK, int FP, int R, int S, int NS, int HJ>
static hipError_t launch_i8_halo(const int8_t *x, const int8_t *w, int8_t *y,
                                 const I8Params &p, int grid, hipStream_t s) {
  return p.alpha_k ? launch_i8_halo_pc<WK, WP, FK, FP, R, S, NS, HJ, true>(x, w, y, p, grid, s)
                   : launch_i8_halo_pc<WK, WP, FK, FP, R, S, NS, HJ, false>(x, w, y, p, grid, s);
}

#define I8_HALO_CFG(WK, WP, FK, FP, R, S, NS, HJ)                                     \
  I8Config {                                                                          \
    "i8_halo_mfma32x32x32_wg" #WK "x" #WP "_frag" #FK "x" #FP "_r" #R "s" #S "_ring" #NS, \
        HaloTile<WK, WP, FK, FP, R, S, NS, HJ>::BM, HaloTile<WK, WP, FK, FP, R, S, NS, HJ>::BN, \
        HaloTile<WK, WP, FK, FP, R, S, NS, HJ>::THREADS, 0, R * S, 0,                  \
        &launch_i8_halo<WK, WP, FK, FP, R, S, NS, HJ>, 1, R, S, WK * WP, NS, HJ        \
  }

#define I8_HALO_AD_CFG_X(KINDNAME, WK, WP, FK, FP, R, S, NS, HJ, PW, CPS, AL, SW, PT, RG, SUFFIX) \
  I8Config {                                                                          \
    "i8_halo_" KINDNAME "_mfma32x32x32_wg" #WK "x" #WP "_frag" #FK "x" #FP "_r" #R "s" #S \
    "_ring" #NS "_hj" #HJ "_pitch" #PW "_cps" #CPS SUFFIX,                              \
        HaloAdTile<WK, WP, FK, FP, R, S, NS, HJ, PW, CPS, AL, SW, PT, RG>::BM,              \
        HaloAdTile<WK, WP, FK, FP, R, S, NS, HJ, PW, CPS, AL, SW, PT, RG>::BN,              \
        HaloAdTile<WK, WP, FK, FP, R, S, NS, HJ, PW, CPS, AL, SW, PT, RG>::THREADS, 0, R * S, 0, \
        &launch_i8_halo_ad<WK, WP, FK, FP, R, S, NS, HJ, PW, CPS, AL, SW, PT, RG>, 2, R, S, \
        WK * WP, NS, HJ, PW, CPS, AL, SW, RG                                              \
  }
#define I8_HALO_AD_CFG(WK, WP, FK, FP, R, S, NS, HJ, PW, CPS) \
  I8_HALO_AD_CFG_X("regfilter", WK, WP, FK, FP, R, S, NS, HJ, PW, CPS, 0, 0, 0, 0, "")
#define I8_HALO_LF_CFG(WK, WP, FK, FP, R, S, NS, HJ, PW, CPS) \
  I8_HALO_AD_CFG_X("ldsfilter", WK, WP, FK, FP, R, S, NS, HJ, PW, CPS, 1, 0, 0, 0, "")
// swizzled (bank-conflict-free) halo: PW is the power-of-two row pitch
#define I8_HALO_AD_SWZ_CFG(WK, WP, FK, FP, R, S, NS, HJ, PW, CPS, SW) \
  I8_HALO_AD_CFG_X("regfilter", WK, WP, FK, FP, R, S, NS, HJ, PW, CPS, 0, SW, 0, 0, "_swz")
// tiles of PT pixel fragments (the last wave column short)
#define I8_HALO_AD_PT_CFG(WK, WP, FK, FP, R, S, NS, HJ, PW, SW, PT, SUFFIX) \
  I8_HALO_AD_CFG_X("regfilter", WK, WP, FK, FP, R, S, NS, HJ, PW, 1, 0, SW, PT, 0, "_pt" #PT SUFFIX)
// swizzled halo through registers (stride-2 problems: the DMA form would
// read every other pixel)
#define I8_HALO_AD_RG_CFG(WK, WP, FK, FP, R, S, NS, HJ, PW, PT, SUFFIX) \
  I8_HALO_AD_CFG_X("regfilter", WK, WP, FK, FP, R, S, NS, HJ, PW, 1, 0, 2, PT, 1, "_swz_rg" SUFFIX)

I8Config kI8HaloConfigs[] = {
    I8_HALO_CFG(2, 4, 2, 2, 3, 3, 3, 4),  // 128 ch x 256 px, 8 waves of 64x64
    I8_HALO_CFG(1, 4, 4, 2, 3, 3, 3, 6),  // 128 ch x 256 px, 4 waves of 128x64
    I8_HALO_CFG(2, 2, 2, 2, 3, 3, 3, 6),  // 128 ch x 128 px, 4 waves of 64x64
    I8_HALO_CFG(1, 4, 2, 2, 3, 3, 3, 6),  // 64 ch x 256 px, 4 waves of 64x64
    // filter fragments in registers, LDS holds the halo only
    I8_HALO_AD_CFG(2, 2, 2, 4, 3, 3, 4, 8, 0, 1),  // 128 ch x 256 px, 4 waves of 64x128
    I8_HALO_AD_CFG(2, 4, 2, 2, 3, 3, 4, 4, 0, 1),  // 128 ch x 256 px, 8 waves of 64x64
    I8_HALO_AD_CFG(2, 2, 2, 4, 3, 3, 3, 16, 0, 1), // 128 ch x 256 px, 4 waves, large halos
    I8_HALO_AD_CFG(2, 2, 2, 2, 3, 3, 4, 8, 0, 1),  // 128 ch x 128 px, 4 waves of 64x64
    I8_HALO_AD_CFG(2, 4, 2, 2, 3, 3, 3, 8, 0, 1),  // 128 ch x 256 px, 8 waves, large halos
    // halo DMA slots sized to the halo (few idle slots), deeper rings
    I8_HALO_AD_CFG(2, 4, 2, 2, 3, 3, 4, 2, 0, 1),
    I8_HALO_AD_CFG(2, 4, 2, 2, 3, 3, 6, 2, 0, 1),
    I8_HALO_AD_CFG(2, 2, 2, 4, 3, 3, 4, 4, 0, 1),
    I8_HALO_AD_CFG(2, 2, 2, 4, 3, 3, 6, 4, 0, 1),
    I8_HALO_AD_CFG(2, 4, 2, 2, 3, 3, 3, 6, 0, 1),
    I8_HALO_AD_CFG(2, 2, 2, 4, 3, 3, 3, 11, 0, 1),
    // fixed LDS row pitch, dilation 1: immediate tap offsets
    I8_HALO_AD_CFG(2, 4, 2, 2, 3, 3, 4, 2, 32, 1),
    I8_HALO_AD_CFG(2, 2, 2, 4, 3, 3, 4, 4, 32, 1),
    I8_HALO_AD_CFG(2, 4, 2, 2, 3, 3, 3, 6, 64, 1),
    I8_HALO_AD_CFG(2, 2, 2, 4, 3, 3, 3, 12, 64, 1),
    // pitch = Q + 16 for Q = 28: a fragment that wraps to the next output
    // row skips a multiple of 256 bytes and keeps its LDS banks
    I8_HALO_AD_CFG(2, 4, 2, 2, 3, 3, 4, 3, 44, 1),
    I8_HALO_AD_CFG(2, 2, 2, 4, 3, 3, 4, 5, 44, 1),
    // two channel blocks per stage: half the ring waits and barriers
    I8_HALO_AD_CFG(2, 4, 2, 2, 3, 3, 3, 2, 32, 2),
    I8_HALO_AD_CFG(2, 4, 2, 2, 3, 3, 4, 2, 32, 2),
    I8_HALO_AD_CFG(2, 2, 2, 4, 3, 3, 3, 4, 32, 2),
    // filter in the LDS ring as well, fetched once per workgroup
    I8_HALO_LF_CFG(2, 4, 2, 2, 3, 3, 3, 2, 32, 1),   // 8 waves of 64x64
    I8_HALO_LF_CFG(2, 2, 2, 4, 3, 3, 3, 4, 32, 1),   // 4 waves of 64x128
    // small tiles for problems that give too few large ones (64 x 64,
    // 64 x 128, 128 x 64: four waves of one or two 32 x 32 fragments)
    I8_HALO_AD_CFG(2, 2, 1, 1, 3, 3, 4, 2, 32, 1),
    I8_HALO_AD_CFG(2, 2, 1, 2, 3, 3, 4, 2, 32, 1),
    I8_HALO_AD_CFG(2, 2, 2, 1, 3, 3, 4, 2, 32, 1),
    I8_HALO_AD_CFG(2, 2, 1, 1, 3, 3, 3, 4, 64, 1),
    I8_HALO_AD_CFG(2, 2, 1, 2, 3, 3, 3, 6, 64, 1),
    // the same with room for stride-2 halos (rows twice as far apart)
    I8_HALO_AD_CFG(2, 2, 1, 1, 3, 3, 3, 6, 64, 1),
    I8_HALO_AD_CFG(2, 2, 1, 2, 3, 3, 3, 9, 64, 1),
    // swizzled halo rows (bank-conflict-free fragment reads at any tap, row
    // wrap, image boundary; stride-2 columns split by parity)
    I8_HALO_AD_SWZ_CFG(2, 4, 2, 2, 3, 3, 4, 2, 32, 1, 1),   // 3x3 stride 1, like config 35
    I8_HALO_AD_SWZ_CFG(2, 4, 2, 2, 3, 3, 3, 6, 64, 1, 2),   // 3x3 stride 2, like config 37
    // stride 2 with the filter in a two-slot ring (fetched once per
    // workgroup; 2 x (42 KiB halo + 36 KiB filter) at pitch 57)
    I8_HALO_LF_CFG(2, 4, 2, 2, 3, 3, 2, 6, 57, 1),
    // 128 ch x 224 px: eight waves of 32 channels, 4 + 3 pixel fragments per
    // SIMD (7 blocks where 128 x 256 tiles give 8; 224 workgroups for the
    // 25088-pixel problems), each wave pulling one filter fragment per tap
    I8_HALO_AD_PT_CFG(4, 2, 1, 4, 3, 3, 4, 2, 32, 1, 7, "_swz"),
    I8_HALO_AD_PT_CFG(4, 2, 1, 4, 3, 3, 4, 2, 32, 0, 7, ""),
    I8_HALO_AD_PT_CFG(4, 2, 1, 4, 3, 3, 3, 6, 64, 0, 7, ""),
    // stride 2 with the swizzled halo through registers: two LDS slots, the
    // registers holding the stage in flight
    I8_HALO_AD_RG_CFG(2, 4, 2, 2, 3, 3, 2, 6, 64, 0, ""),
    // 256 ch x 128 px: every output channel of a K = 256 problem in one
    // workgroup, so each pixel tile's halo is fetched once, not once per
    // channel half (the same 64 x 64 waves and workgroup count)
    I8_HALO_AD_CFG(4, 2, 2, 2, 3, 3, 3, 4, 64, 1),
};
int kNumI8HaloConfigs = sizeof(kI8HaloConfigs) / sizeof(kI8HaloConfigs[0]);

}  // namespace convfprop
