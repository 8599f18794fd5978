// tile_gemm.hpp — the bf16 MFMA tile main loops shared by every GEMM-shaped kernel of the library.
//
// C[M x N] (fp32, in registers) = A[M x K] . B[N x K]^T, with both operands row-major and K
// contiguous ("TN").  One workgroup computes a TM x TN tile with WM x WN wavefronts; every
// wavefront owns a 128 x (16*NSUB) sub-tile made of 8 x NSUB accumulators of the gfx950
// instruction v_mfma_f32_16x16x32_bf16 (4 fp32 per lane each).  That instruction rather than
// the 32x32x16 one: it moves less accumulator data per flop, and under the chip's power limit the
// same MFMA stream on random data runs at a clock about 12% higher.
//
// Invariance contract.  For one output element the sequence of floating-point operations is
//   acc = C0;  for each 32-wide k slice in ascending order: acc = mfma(A[i, k32], B[j, k32], acc)
// whatever the main loop, its K step or stage count, the tile configuration, the element's
// position inside the tile, or M and N.  Padding past K is exact zeros.
//
// Data path.  Global -> LDS by direct loads (buffer_load_dwordx4 ... lds, 16 bytes per lane,
// out-of-range rows read as zero) into LDS slots with XOR-swizzled 16-byte chunks -> VGPR
// fragments (ds_read_b128) -> MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmh {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int MFMA_MN = 16;            // rows and columns of one MFMA output block
constexpr int MFMA_K = 32;             // k extent of one MFMA
constexpr int MSUB = 8;                // MFMA blocks per wavefront along M
constexpr int WAVE_M = MFMA_MN * MSUB; // rows of A per wavefront (128)
constexpr float LOG2E = 1.4426950408889634f;

// Offsets at or beyond this value are outside every buffer descriptor we build (all ranges are
// below 2^31 bytes), so the hardware returns zeros for them.
constexpr uint32_t OOB_OFFSET = 0x80000000u;

// Accumulator layout of one 16 x 16 output block: lane l holds column l % 16, and its register i
// holds row 4 * (l / 16) + i.
__device__ __forceinline__ int acc_row(int i, int lane) { return 4 * (lane >> 4) + i; }
__device__ __forceinline__ int acc_col(int lane) { return lane & 15; }

// Operand layout: lane l supplies row (A) or column (B) l % 16 of the block and the eight
// consecutive k values starting at 8 * (l / 16) of the 32-wide slice: one 16-byte chunk.
__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Workgroup tile order.  Consecutive workgroup ids are dealt round-robin to the 8 XCDs; xcd_range
// gives each XCD one contiguous range of logical tiles, and inside a range tiles go in groups of
// GROUP_M m-tiles by all n-tiles (group_coords), so the workgroups running together on one XCD
// share both their A rows and their B rows in that XCD's L2.
__device__ __forceinline__ void xcd_range(int xcd, int ntiles, int& start, int& count) {
  const int q = ntiles >> 3, rem = ntiles & 7;
  start = xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q;
  count = q + (xcd < rem ? 1 : 0);
}

template <int GROUP_M>
__device__ __forceinline__ void group_coords(int L, int n_mt, int n_nt, int& mt, int& nt) {
  const int per_group = GROUP_M * n_nt;
  const int g = L / per_group;
  const int first_m = g * GROUP_M;
  const int gm = min(GROUP_M, n_mt - first_m);
  const int in = L - g * per_group;
  mt = first_m + in % gm;
  nt = in / gm;
}

// Workgroup id -> (m tile, n tile) for a grid of one workgroup per tile.
template <int GROUP_M>
__device__ __forceinline__ void tile_coords(int bid, int nblk, int n_mt, int n_nt, int& mt, int& nt) {
  int start, count;
  xcd_range(bid & 7, nblk, start, count);
  group_coords<GROUP_M>(start + (bid >> 3), n_mt, n_nt, mt, nt);
}

// Dynamic tile queue of a persistent grid over one or two problems (problem 0's tiles are handed
// out before problem 1's).  Each XCD owns a contiguous share of each problem (xcd_range) and a
// counter ctr[x] in device memory, zeroed before the launch; counter value i on XCD x is the i-th
// tile of x's list "problem-0 share, then problem-1 share".  A workgroup on XCD x claims from
// ctr[x] and, once x's list is used up, from the other XCDs' counters.  Tiles are numbered
// 0 .. n0-1 for problem 0 and n0 .. n0+n1-1 for problem 1; -1 means no tile is left.  The queue
// decides only which workgroup computes a tile.  Only one thread per workgroup calls it.
struct TileQueue {
  int* ctr;
  int n0, n1;

  __device__ __forceinline__ int decode(int x, int i) const {
    int s0, c0, s1, c1;
    xcd_range(x, n0, s0, c0);
    if (i < c0) return s0 + i;
    xcd_range(x, n1, s1, c1);
    i -= c0;
    return i < c1 ? n0 + s1 + i : -1;
  }
  // raw claim on the own XCD's list (its result may be read much later)
  __device__ __forceinline__ int claim(int x) const { return atomicAdd(&ctr[x], 1); }
  // the tile of a raw claim, stealing from the other XCDs when the own list is used up
  __device__ __forceinline__ int resolve(int x, int raw) const {
    int t = decode(x, raw);
    for (int k = 1; t < 0 && k < 8; ++k) {
      const int y = (x + k) & 7;
      t = decode(y, atomicAdd(&ctr[y], 1));
    }
    return t;
  }
};

// Code placement of the ping-pong K loop.  The loop runs fastest when its first instruction sits
// 4 bytes past a 32-byte boundary (instruction fetch; at T=8192 the spread between placements
// measured 1.5%).  Every kernel that contains the loop starts with LOOP_PAD[id] no-ops, executed
// once per workgroup; the build measures where each loop landed in a first compile and sets the
// counts (LMH_LOOP_PADS), so the placement holds whatever code precedes the loop.  Kernel ids:
// 0-3 forward persistent (2 * temperature + sum_p2), 4-7 backward dz (2 * temperature +
// entropy gradient), 8 gradient GEMM, 9-12 forward K-split (2 * temperature + sum_p2).
#ifndef LMH_LOOP_PADS
#define LMH_LOOP_PADS 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0
#endif
constexpr int LOOP_PAD[13] = {LMH_LOOP_PADS};

template <int ID>
__device__ __forceinline__ void loop_placement_pad() {
  constexpr int n = LOOP_PAD[ID];
  if constexpr (n > 0) asm volatile(".rept %0\n\ts_nop 0\n\t.endr" ::"n"(n));
}

// Main loop selectors (see the two loops below).
constexpr int LOOP_SPREAD = 1;
constexpr int LOOP_PINGPONG = 2;

// Tile geometry and LDS staging.  A stage holds BK k-values of the tile's A rows then its B rows,
// BK*2 bytes per row in 16-byte chunks; logical chunk c of row r is stored at c ^ swz(r).
template <int WM_, int WN_, int NSUB_, int NS_, int BK_ = 64>
struct PipeCfg {
  static constexpr int WM = WM_, WN = WN_, NSUB = NSUB_, NS = NS_, BK = BK_;
  static constexpr int NWAVES = WM * WN;
  static constexpr int NTHREADS = 64 * NWAVES;
  static constexpr int TM = WAVE_M * WM;
  static constexpr int WAVE_N = MFMA_MN * NSUB;
  static constexpr int TN = WAVE_N * WN;
  static constexpr int ROW = BK * 2;               // bytes per staged row
  static constexpr int CPR = BK / 8;               // 16-byte chunks per row
  static constexpr int RPI = 1024 / ROW;           // rows per DMA instruction
  static constexpr int KSUB = BK / MFMA_K;         // MFMA k-slices per step
  static constexpr int A_IPW = TM / RPI / NWAVES;  // DMA instructions per wavefront per step
  static constexpr int B_IPW = TN / RPI / NWAVES;
  static constexpr int STAGE_BYTES = (TM + TN) * ROW;
  static constexpr int LDS_BYTES = NS * STAGE_BYTES;
  static_assert(BK == 32 || BK == 64 || BK == 128, "BK");
  static_assert(TM % (RPI * NWAVES) == 0 && TN % (RPI * NWAVES) == 0 && B_IPW >= 1, "DMA split");
  static_assert(NS >= 2 && (NS - 1) * (A_IPW + B_IPW) <= 63, "vmcnt range");
  // Conflict-free ds_read_b128 of 16 consecutive rows at one logical chunk: BK = 128 rows are
  // 256 B (one 256-byte bank line each), BK = 64 rows 128 B (two per line), BK = 32 rows 64 B
  // (four per line).
  __device__ static __forceinline__ int swz(int r) {
    return BK == 128 ? r & 15 : BK == 64 ? (r >> 1) & 7 : (r >> 2) & 3;
  }
  // byte offset inside a row of lane `lane`'s fragment chunk for k-slice s (fsw = swz(lane % 16))
  __device__ static __forceinline__ int koff(int s, int lane, int fsw) { return ((4 * s + (lane >> 4)) ^ fsw) << 4; }
};

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Buffer descriptor in SGPRs: base, 16-bit stride 0, num_records = bytes, gfx9 data format.
__device__ __forceinline__ u32x4 make_desc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  u32x4 d;
  d[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
  d[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
  d[2] = __builtin_amdgcn_readfirstlane(bytes);
  d[3] = 0x00020000u;
  return d;
}

// 16 bytes per lane from buffer offset `voff` into LDS at lds_base + 16 * lane.
//
// The loads are issued from inline assembly.  The compiler therefore neither counts them nor
// waits for them; the loops wait with explicit vmcnt values (loads return in order), and the
// compiler's own waits for other loads stay correct (extra outstanding loads only make a vmcnt
// wait stricter).  M0 (the LDS destination base) is written inside the same asm block.
__device__ __forceinline__ void dma16(u32x4 desc, uint32_t voff, uint32_t lds_base) {
  lds_base = __builtin_amdgcn_readfirstlane(lds_base);  // wavefront-uniform by construction
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(desc), "s"(lds_base)
      : "memory");
}

// ds_read_b64_tr_b16 at LDS byte address `addr` (8-byte aligned).  In each group of 16 lanes,
// lane i receives element i % 4 of the 8 bytes addressed by lane 4 e + i / 4 of its group as its
// element e: if those four lanes address four consecutive 4-element pieces of one row of a 2-byte
// matrix, and the group's lanes 4 e + q take row e, lane i gets column i of the 4 x 16 block.
__device__ __forceinline__ s16x4 ds_read_tr16(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(uintptr_t)addr);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Per-lane DMA geometry of a ring-staged tile: instruction d of a step moves RPI rows; the lane
// loads row (its block's first row + lane / CPR) and stores chunk lane % CPR, which holds logical
// chunk (lane % CPR) ^ swz(row).
template <class Cfg>
struct RingDma {
  static constexpr int NDMA = Cfg::A_IPW + Cfg::B_IPW;
  u32x4 da, db;
  uint32_t lds0;
  uint32_t off[NDMA];
  int lc[NDMA];
  int K, nk;

  __device__ __forceinline__ RingDma(const __bf16* A, int64_t lda, int rowsA, const __bf16* B, int64_t ldb, int rowsB,
                                     int K_, char* lds, int wave, int lane) {
    da = make_desc(A, (uint32_t)((int64_t)rowsA * lda * 2));
    db = make_desc(B, (uint32_t)((int64_t)rowsB * ldb * 2));
    lds0 = lds_addr(lds);
    K = K_;
    nk = (K + Cfg::BK - 1) / Cfg::BK;
    const int dl_row = lane / Cfg::CPR;
    const int dl_pc = lane % Cfg::CPR;
#pragma unroll
    for (int d = 0; d < NDMA; ++d) {
      const bool is_a = d < Cfg::A_IPW;
      const int i = is_a ? d : d - Cfg::A_IPW;
      const int r = (wave * (is_a ? Cfg::A_IPW : Cfg::B_IPW) + i) * Cfg::RPI + dl_row;
      lc[d] = dl_pc ^ Cfg::swz(r);
      off[d] = (uint32_t)(r * (is_a ? lda : ldb) * 2 + lc[d] * 16);
    }
  }
  // load instruction d of step kt into stage kt % NS; steps past the end and chunks past K read zeros
  __device__ __forceinline__ void dma(int d, int kt, int wave) const {
    const bool is_a = d < Cfg::A_IPW;
    const int i = is_a ? d : d - Cfg::A_IPW;
    const bool ok = kt < nk && kt * Cfg::BK + lc[d] * 8 < K;
    const uint32_t voff = ok ? off[d] + (uint32_t)kt * Cfg::ROW : OOB_OFFSET;
    const uint32_t dst = lds0 + (kt % Cfg::NS) * Cfg::STAGE_BYTES +
                         (is_a ? (wave * Cfg::A_IPW + i) * 1024 : Cfg::TM * Cfg::ROW + (wave * Cfg::B_IPW + i) * 1024);
    dma16(is_a ? da : db, voff, dst);
  }
  __device__ __forceinline__ void step(int kt, int wave) const {
#pragma unroll
    for (int d = 0; d < NDMA; ++d) dma(d, kt, wave);
  }
};

template <class Cfg>
__device__ __forceinline__ void load_frags(const char* base, int a_frow, int b_frow, int koff, bf16x8 (&af)[MSUB],
                                           bf16x8 (&bfr)[Cfg::NSUB]) {
#pragma unroll
  for (int m = 0; m < MSUB; ++m)
    af[m] = *reinterpret_cast<const bf16x8*>(base + a_frow + m * MFMA_MN * Cfg::ROW + koff);
#pragma unroll
  for (int n = 0; n < Cfg::NSUB; ++n)
    bfr[n] = *reinterpret_cast<const bf16x8*>(base + b_frow + n * MFMA_MN * Cfg::ROW + koff);
}

template <class Cfg>
__device__ __forceinline__ void mfma_block(const bf16x8 (&af)[MSUB], const bf16x8 (&bfr)[Cfg::NSUB],
                                           f32x4 (&acc)[MSUB][Cfg::NSUB]) {
#pragma unroll
  for (int m = 0; m < MSUB; ++m)
#pragma unroll
    for (int n = 0; n < Cfg::NSUB; ++n) acc[m][n] = mfma(af[m], bfr[n], acc[m][n]);
}

// =============================================================================================
// LOOP_SPREAD: a ring of NS stages with the loads of each step spread between its MFMAs.
// =============================================================================================
//
// Issuing a step's global -> LDS loads in one burst right after the barrier stalls every
// wavefront at the texture unit (a 1 KiB load instruction takes the unit many cycles) while the
// matrix pipe idles.  Here the step's NDMA load instructions are interleaved with its NMF MFMAs,
// one after every NMF/NDMA MFMAs, so address processing overlaps matrix work.  The stage being
// filled is (kt + NS - 1) % NS, retired by the barrier at the top of step kt; the data of step
// kt + 1 has NS - 2 further steps of slack, so NS >= 3.  Used for the HBM-bound small-T tiles,
// where deep prefetch of the weight stream matters most.

template <class Cfg>
__device__ __forceinline__ void tile_mainloop_spread(const __bf16* __restrict__ A, int64_t lda, int rowsA,
                                                     const __bf16* __restrict__ B, int64_t ldb, int rowsB, int K,
                                                     char* __restrict__ lds, f32x4 (&acc)[MSUB][Cfg::NSUB]) {
  constexpr int ROW = Cfg::ROW;
  constexpr int KSUB = Cfg::KSUB;
  constexpr int NS = Cfg::NS;
  constexpr int NDMA = RingDma<Cfg>::NDMA;
  constexpr int NMF = KSUB * MSUB * Cfg::NSUB;
  static_assert(NS >= 3, "the spread main loop needs at least three stages");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % Cfg::WM;
  const int wn = wave / Cfg::WM;
  const RingDma<Cfg> ring(A, lda, rowsA, B, ldb, rowsB, K, lds, wave, lane);

  const int fr = lane & 15;
  const int fsw = Cfg::swz(fr);
  const int a_frow = (wm * WAVE_M + fr) * ROW;
  const int b_frow = Cfg::TM * ROW + (wn * Cfg::WAVE_N + fr) * ROW;
  int koff[KSUB];
#pragma unroll
  for (int s = 0; s < KSUB; ++s) koff[s] = Cfg::koff(s, lane, fsw);

#pragma unroll
  for (int p = 0; p < NS - 1; ++p) ring.step(p, wave);

  for (int kt = 0; kt < ring.nk; ++kt) {
    wait_vmcnt<(NS - 2) * NDMA>();   // this thread's loads of step kt have landed
    __syncthreads();                 // ... everyone's; and stage (kt - 1) % NS is free again
    const char* base = lds + (kt % NS) * Cfg::STAGE_BYTES;
    const int kn = kt + NS - 1;      // the step refilled during this one
#pragma unroll
    for (int s = 0; s < KSUB; ++s) {
      bf16x8 af[MSUB], bfr[Cfg::NSUB];
      load_frags<Cfg>(base, a_frow, b_frow, koff[s], af, bfr);
#pragma unroll
      for (int m = 0; m < MSUB; ++m)
#pragma unroll
        for (int n = 0; n < Cfg::NSUB; ++n) {
          acc[m][n] = mfma(af[m], bfr[n], acc[m][n]);
          const int q = (s * MSUB + m) * Cfg::NSUB + n;   // MFMA index inside the step
#pragma unroll
          for (int d = 0; d < NDMA; ++d)
            if (d * NMF / NDMA == q) ring.dma(d, kn, wave);
        }
    }
  }
  wait_vmcnt<0>();   // trailing out-of-range loads still write LDS
  __syncthreads();
}

// =============================================================================================
// LOOP_PINGPONG: two groups of four wavefronts alternating between loads and MFMAs.
// =============================================================================================
//
// Eight wavefronts, two per SIMD (wavefronts w and w+4 share SIMD w % 4).  Group 0 = wavefronts
// 0-3, group 1 = 4-7; each has one wavefront per SIMD.  Every wavefront runs the same sequence
// "memory phase: issue global -> LDS loads, read the fragments of K step k from LDS | barrier |
// compute phase: the MFMAs of step k | barrier", but group 1 starts one barrier later, so in every
// phase one group issues MFMAs back to back from registers while the other works the memory
// system: each SIMD's matrix pipe is fed by one wavefront per phase without waiting on LDS.
// (Hardware barriers count arrivals, so the groups may sit at different barrier instructions as
// long as every wavefront executes the same number of them.)
//
// LDS: three A slots and two B slots of one K = 64 step each (256 rows x 128 B = 32 KB per slot,
// 160 KB in all).  The loads of a step are split between the groups so that neither memory phase
// carries a whole step: group 1 loads the A rows of step k+2 into A slot (k+2) % 3 during its
// memory phase of step k, and group 0 loads the B rows of step k+1 into B slot (k+1) % 2 during
// its memory phase of step k.  In phase terms (group 0 in even phases, group 1 one phase behind):
//   A slot (k+2) % 3 was last read in phases 2k-2 and 2k-1, and is needed again in phase 2k+4;
//   B slot (k+1) % 2 was last read in phases 2k-2 and 2k-1, and is needed again in phase 2k+2.
// Group 1 waits for its A loads of step k+1 at the end of its memory phase of step k (phase 2k+1);
// group 0 waits for its B loads of step k+1 at the end of its compute phase of step k (phase 2k+1).
// Every barrier is preceded by the wait for the wavefront's own LDS reads, so a slot is never
// overwritten while a read of it is in flight.  Loads of steps past the end are not issued, so
// when run() returns no load is in flight and a persistent caller may start() its next tile at
// once: those first loads then travel while the caller reduces the finished tile's accumulators.

// REMAT: start() derives the lane's load positions afresh from an opaque thread index, so a caller
// that runs several tiles with a register-heavy epilogue between them does not keep values derived
// from them (loop-invariant to the compiler) live across that epilogue.
template <class Cfg, bool REMAT = false>
struct PingPong {
  static_assert(Cfg::NWAVES == 8 && Cfg::WM == 2 && Cfg::BK == 64 && Cfg::TM == 256 && Cfg::TN == 256,
                "ping-pong loop: 8 wavefronts, 256 x 256 tile, K = 64 steps");
  static constexpr int ROW = Cfg::ROW;          // 128 bytes
  static constexpr int SLOT = 256 * ROW;        // 32 KB: one operand of one step
  static constexpr int B_BASE = 3 * SLOT;       // A slots 0..2, then B slots 0..1
  static constexpr int LDS_BYTES = 5 * SLOT;    // 160 KB
  static constexpr int DPW = 8;                 // DMA instructions per wavefront per step (8 rows each)
  static constexpr int KSUB = Cfg::KSUB;

  char* lds;
  int lane, group, wm, wn;
  bool loads_a;                                 // group 1 loads A, group 0 loads B
  uint32_t lds0;
  int blk0, lc_even, lc_odd;
  // per tile
  u32x4 desc;
  uint32_t row_off, blk_stride;
  int K, nk;

  __device__ __forceinline__ PingPong(char* lds_) : lds(lds_) { init_lane(threadIdx.x); }

  __device__ __forceinline__ void init_lane(int tid) {
    lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    group = wave >> 2;
    wm = wave % Cfg::WM;
    wn = wave / Cfg::WM;
    loads_a = group == 1;
    lds0 = lds_addr(lds);
    // wavefront wave % 4 of a group loads rows [64 (wave % 4), + 64) of its operand
    blk0 = (wave & 3) * DPW;                    // even, so block i has the parity of i
    const int dl_row = lane >> 3;
    const int dl_pc = lane & 7;
    lc_even = dl_pc ^ (dl_row >> 1);            // swz(row) = (row >> 1) & 7 for row = 8 blk + dl_row
    lc_odd = dl_pc ^ (4 + (dl_row >> 1));
  }

  // this group's operand of step kt into its slot; nothing is issued for kt >= nk
  __device__ __forceinline__ void dma_step(int kt) const {
    if (kt >= nk) return;
    const int k0 = kt * Cfg::BK;
    const bool ok_even = k0 + lc_even * 8 < K;
    const bool ok_odd = k0 + lc_odd * 8 < K;
    const uint32_t ve = row_off + lc_even * 16 + (uint32_t)kt * ROW;
    const uint32_t vo = row_off + lc_odd * 16 + (uint32_t)kt * ROW;
    const uint32_t sbase = lds0 + (loads_a ? (kt % 3) * SLOT : B_BASE + (kt & 1) * SLOT) + blk0 * 1024;
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      const bool ok = (i & 1) ? ok_odd : ok_even;
      const uint32_t voff = ((i & 1) ? vo : ve) + (uint32_t)i * blk_stride;
      dma16(desc, ok ? voff : OOB_OFFSET, sbase + i * 1024);
    }
  }

  // Set up a tile and issue its first loads (A of steps 0 and 1, B of step 0).  Requires every
  // slot to be free: before the first tile, or after run() of the previous tile.
  __device__ __forceinline__ void start(const __bf16* __restrict__ A, int64_t lda, int rowsA,
                                        const __bf16* __restrict__ B, int64_t ldb, int rowsB, int K_) {
    if constexpr (REMAT) {
      int tid = threadIdx.x;
      asm volatile("" : "+v"(tid));
      init_lane(tid);
    }
    desc = loads_a ? make_desc(A, (uint32_t)((int64_t)rowsA * lda * 2))
                   : make_desc(B, (uint32_t)((int64_t)rowsB * ldb * 2));
    const int64_t ld = loads_a ? lda : ldb;
    row_off = (uint32_t)((blk0 * 8 + (lane >> 3)) * ld * 2);
    // The first steps' load offsets do not depend on the tile (the tile is in the descriptor);
    // hiding row_off from the optimizer keeps it from hoisting them out of a persistent caller's
    // tile loop, where they would stay live (and spill) across the K loop.
    asm volatile("" : "+v"(row_off));
    blk_stride = (uint32_t)(8 * ld * 2);
    K = K_;
    nk = (K + Cfg::BK - 1) / Cfg::BK;
    dma_step(0);
    if (loads_a) dma_step(1);
  }

  // The K loop of the tile set up by start().  On return every wavefront has passed the same
  // number of barriers, every LDS read has completed and no load is in flight: all slots are free.
  __device__ __forceinline__ void run(f32x4 (&acc)[MSUB][Cfg::NSUB]) const {
    const int fr = lane & 15;
    const int fsw = Cfg::swz(fr);
    const int a_frow = (wm * WAVE_M + fr) * ROW;
    const int b_frow = (wn * Cfg::WAVE_N + fr) * ROW;
    bf16x8 fa[KSUB][MSUB], fb[KSUB][Cfg::NSUB];

    // step 0 published (group 1 may leave A of step 1 in flight)
    if (loads_a && nk > 1)
      wait_vmcnt<DPW>();
    else
      wait_vmcnt<0>();
    __syncthreads();
    if (group == 1) __syncthreads();  // group 1 runs one phase behind

    for (int kt = 0; kt < nk; ++kt) {
      // memory phase
      dma_step(loads_a ? kt + 2 : kt + 1);
      const char* abase = lds + (kt % 3) * SLOT;
      const char* bbase = lds + B_BASE + (kt & 1) * SLOT;
#pragma unroll
      for (int s = 0; s < KSUB; ++s) {
        const int ko = Cfg::koff(s, lane, fsw);
#pragma unroll
        for (int m = 0; m < MSUB; ++m)
          fa[s][m] = *reinterpret_cast<const bf16x8*>(abase + a_frow + m * MFMA_MN * ROW + ko);
#pragma unroll
        for (int n = 0; n < Cfg::NSUB; ++n)
          fb[s][n] = *reinterpret_cast<const bf16x8*>(bbase + b_frow + n * MFMA_MN * ROW + ko);
      }
      if (loads_a) {                    // group 1's A of step kt+1 has landed
        if (kt + 2 < nk)
          wait_vmcnt<DPW>();
        else
          wait_vmcnt<0>();
      }
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      // compute phase
#pragma unroll
      for (int s = 0; s < KSUB; ++s) mfma_block<Cfg>(fa[s], fb[s], acc);
      __builtin_amdgcn_sched_barrier(0);
      if (!loads_a) wait_vmcnt<0>();    // group 0's B of step kt+1 has landed
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    }
    if (group == 0) __syncthreads();    // same barrier count for both groups
  }
};

// One tile: start + run.
template <class Cfg>
__device__ __forceinline__ void tile_mainloop_pingpong(const __bf16* __restrict__ A, int64_t lda, int rowsA,
                                                       const __bf16* __restrict__ B, int64_t ldb, int rowsB,
                                                       int K, char* __restrict__ lds,
                                                       f32x4 (&acc)[MSUB][Cfg::NSUB]) {
  PingPong<Cfg> pp(lds);
  pp.start(A, lda, rowsA, B, ldb, rowsB, K);
  pp.run(acc);
}

}  // namespace lmh
