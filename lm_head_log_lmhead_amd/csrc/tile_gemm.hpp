// tile_gemm.hpp — the bf16 MFMA tile main loop shared by every GEMM-shaped kernel of the library.
//
// C[M x N] (fp32, in registers) = A[M x K] . B[N x K]^T, with both operands row-major and K
// contiguous ("TN").  One workgroup computes a TM x TN tile with WM x WN wavefronts; every
// wavefront owns a 128 x (32*NSUB) sub-tile made of 4 x NSUB accumulators of the gfx950
// instruction v_mfma_f32_32x32x16_bf16 (16 fp32 per lane each).
//
// Invariance contract.  For one output element the sequence of floating-point operations is
//   acc = C0;  for each 16-wide k slice in ascending order: acc = mfma(A[i, k16], B[j, k16], acc)
// whatever the main loop, its K step or stage count, the tile configuration, the element's
// position inside the tile, or M and N.  Padding past K is exact zeros.
//
// Data path.  Global -> LDS by direct loads (buffer_load_dwordx4 ... lds, 16 bytes per lane,
// out-of-range rows read as zero) into a ring of stages with XOR-swizzled 16-byte chunks ->
// VGPR fragments (ds_read_b128) -> MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmh {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int MSUB = 4;           // 32-row MFMA sub-tiles per wavefront along M (128 rows)
constexpr int WAVE_M = 32 * MSUB; // rows of A per wavefront
constexpr float LOG2E = 1.4426950408889634f;

// Offsets at or beyond this value are outside every buffer descriptor we build (all ranges are
// below 2^31 bytes), so the hardware returns zeros for them.
constexpr uint32_t OOB_OFFSET = 0x80000000u;

// Row (M index inside the wavefront sub-tile) held by accumulator register r of lane `lane` in
// a 32x32 MFMA output block; the column (N index) is lane & 31.
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Workgroup id -> (m tile, n tile).  Consecutive workgroup ids are dealt round-robin to the 8
// XCDs; the remap gives each XCD one contiguous range of logical tiles, and inside a range tiles
// go in groups of GROUP_M m-tiles by all n-tiles, so the workgroups running together on one XCD
// share both their A rows and their B rows in that XCD's L2.
template <int GROUP_M>
__device__ __forceinline__ void tile_coords(int bid, int nblk, int n_mt, int n_nt, int& mt, int& nt) {
  const int xcd = bid & 7;
  const int q = nblk >> 3, rem = nblk & 7;
  const int start = xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q;
  const int L = start + (bid >> 3);
  const int per_group = GROUP_M * n_nt;
  const int g = L / per_group;
  const int first_m = g * GROUP_M;
  const int gm = min(GROUP_M, n_mt - first_m);
  const int in = L - g * per_group;
  mt = first_m + in % gm;
  nt = in / gm;
}


// =============================================================================================
// Main loop v2: a ring of NS LDS stages of BK K-elements filled by direct global -> LDS loads.
// =============================================================================================
//
// Each stage holds the tile's A rows then B rows, BK*2 bytes per row in 16-byte chunks; logical
// chunk c of row r is stored at c ^ swz2(r).  Loads go straight from global memory to LDS
// (buffer_load_dwordx4 ... lds): one instruction moves 64 lanes x 16 bytes into one contiguous KiB
// of LDS, the lane -> (row, chunk) assignment applying the swizzle.  Stages are filled NS-1 steps
// ahead, so global latency hides behind NS-1 steps of MFMA work; one barrier per step both
// publishes the stage and retires the stage it overwrites.  With BK = 64 every row contributes a
// whole 128-byte line per step, so no line is fetched twice into L1.
//
// The loads are issued from inline assembly.  The compiler therefore neither counts them nor
// waits for them; the loop waits with explicit vmcnt values (loads return in order), and the
// compiler's own waits for other loads stay correct (extra outstanding loads only make a vmcnt
// wait stricter).  M0 (the LDS destination base) is written inside the same asm block.

template <int WM_, int WN_, int NSUB_, int NS_, int BK_ = 64>
struct PipeCfg {
  static constexpr int WM = WM_, WN = WN_, NSUB = NSUB_, NS = NS_, BK = BK_;
  static constexpr int NWAVES = WM * WN;
  static constexpr int NTHREADS = 64 * NWAVES;
  static constexpr int TM = WAVE_M * WM;
  static constexpr int WAVE_N = 32 * NSUB;
  static constexpr int TN = WAVE_N * WN;
  static constexpr int ROW = BK * 2;               // bytes per staged row
  static constexpr int CPR = BK / 8;               // 16-byte chunks per row
  static constexpr int RPI = 1024 / ROW;           // rows per DMA instruction
  static constexpr int KSUB = BK / 16;             // MFMA k-substeps per step
  static constexpr int A_IPW = TM / RPI / NWAVES;  // DMA instructions per wavefront per step
  static constexpr int B_IPW = TN / RPI / NWAVES;
  static constexpr int STAGE_BYTES = (TM + TN) * ROW;
  static constexpr int LDS_BYTES = NS * STAGE_BYTES;
  static constexpr int VMCNT_AHEAD = (NS - 2) * (A_IPW + B_IPW);  // loads allowed in flight
  static_assert(BK == 32 || BK == 64, "BK");
  static_assert(TM % (RPI * NWAVES) == 0 && TN % (RPI * NWAVES) == 0 && B_IPW >= 1, "DMA split");
  static_assert(NS >= 2 && (NS - 1) * (A_IPW + B_IPW) <= 63, "vmcnt range");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  // stored chunk of logical chunk c in row r is c ^ swz(r): conflict-free ds_read_b128 of 32 rows
  __device__ static __forceinline__ int swz(int r) { return BK == 64 ? (r >> 1) & 7 : (r >> 2) & 3; }
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
__device__ __forceinline__ void dma16(u32x4 desc, uint32_t voff, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(desc), "s"(lds_base)
      : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <class Cfg>
__device__ __forceinline__ void tile_mainloop2(const __bf16* __restrict__ A, int64_t lda, int rowsA,
                                               const __bf16* __restrict__ B, int64_t ldb, int rowsB, int K,
                                               char* __restrict__ lds, f32x16 (&acc)[MSUB][Cfg::NSUB]) {
  constexpr int ROW = Cfg::ROW;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % Cfg::WM;
  const int wn = wave / Cfg::WM;

  const u32x4 da = make_desc(A, (uint32_t)((int64_t)rowsA * lda * 2));
  const u32x4 db = make_desc(B, (uint32_t)((int64_t)rowsB * ldb * 2));
  const uint32_t lds0 = lds_addr(lds);

  // DMA lane assignment: lane -> (row lane / CPR of the instruction's RPI rows, stored chunk
  // lane % CPR), which holds logical chunk (lane % CPR) ^ swz(row).
  const int dl_row = lane / Cfg::CPR;
  const int dl_pc = lane % Cfg::CPR;
  uint32_t a_off[Cfg::A_IPW], b_off[Cfg::B_IPW];
  int a_lc[Cfg::A_IPW], b_lc[Cfg::B_IPW];
#pragma unroll
  for (int i = 0; i < Cfg::A_IPW; ++i) {
    const int r = (wave * Cfg::A_IPW + i) * Cfg::RPI + dl_row;
    a_lc[i] = dl_pc ^ Cfg::swz(r);
    a_off[i] = (uint32_t)(r * lda * 2 + a_lc[i] * 16);
  }
#pragma unroll
  for (int i = 0; i < Cfg::B_IPW; ++i) {
    const int r = (wave * Cfg::B_IPW + i) * Cfg::RPI + dl_row;
    b_lc[i] = dl_pc ^ Cfg::swz(r);
    b_off[i] = (uint32_t)(r * ldb * 2 + b_lc[i] * 16);
  }

  const int nk = (K + Cfg::BK - 1) / Cfg::BK;
  auto issue = [&](int kt) {
    const int st = kt % Cfg::NS;
    const bool kt_in = kt < nk;
    const int k0 = kt * Cfg::BK;
    const uint32_t kb = (uint32_t)kt * ROW;
    const uint32_t sbase = lds0 + st * Cfg::STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < Cfg::A_IPW; ++i)
      dma16(da, (kt_in && k0 + a_lc[i] * 8 < K) ? a_off[i] + kb : OOB_OFFSET, sbase + (wave * Cfg::A_IPW + i) * 1024);
#pragma unroll
    for (int i = 0; i < Cfg::B_IPW; ++i)
      dma16(db, (kt_in && k0 + b_lc[i] * 8 < K) ? b_off[i] + kb : OOB_OFFSET,
            sbase + Cfg::TM * ROW + (wave * Cfg::B_IPW + i) * 1024);
  };

  // Fragment reads: lane reads row (lane & 31) of a 32-row sub-tile, logical chunk 2s + lane/32;
  // sub-tile bases are multiples of 32 rows, so the swizzle of the row is swz(lane & 31).
  const int fr = lane & 31;
  const int fsw = Cfg::swz(fr);
  const int a_frow = (wm * WAVE_M + fr) * ROW;
  const int b_frow = Cfg::TM * ROW + (wn * Cfg::WAVE_N + fr) * ROW;
  int koff[Cfg::KSUB];
#pragma unroll
  for (int s = 0; s < Cfg::KSUB; ++s) koff[s] = (((2 * s) | (lane >> 5)) ^ fsw) << 4;

#pragma unroll
  for (int p = 0; p < Cfg::NS - 1; ++p) issue(p);

  for (int kt = 0; kt < nk; ++kt) {
    wait_vmcnt<Cfg::VMCNT_AHEAD>();   // this thread's loads of step kt have landed
    __syncthreads();                  // ... everyone's; and step kt-1's stage is free again
    issue(kt + Cfg::NS - 1);
    const char* base = lds + (kt % Cfg::NS) * Cfg::STAGE_BYTES;
#pragma unroll
    for (int s = 0; s < Cfg::KSUB; ++s) {
      bf16x8 af[MSUB], bfr[Cfg::NSUB];
#pragma unroll
      for (int m = 0; m < MSUB; ++m)
        af[m] = *reinterpret_cast<const bf16x8*>(base + a_frow + m * 32 * ROW + koff[s]);
#pragma unroll
      for (int n = 0; n < Cfg::NSUB; ++n)
        bfr[n] = *reinterpret_cast<const bf16x8*>(base + b_frow + n * 32 * ROW + koff[s]);
#pragma unroll
      for (int m = 0; m < MSUB; ++m)
#pragma unroll
        for (int n = 0; n < Cfg::NSUB; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[m], bfr[n], acc[m][n], 0, 0, 0);
    }
  }
  wait_vmcnt<0>();   // the trailing (out-of-range) loads still write LDS: drain them
  __syncthreads();
}

// =============================================================================================
// Main loop v3: the v2 ring with software-pipelined fragments.
// =============================================================================================
//
// The fragments are double buffered in registers: the ds_reads of k-substep s+1 are in flight
// while the MFMAs of substep s run, and the step's barrier sits between the last ds_read of the
// step and its last MFMAs, so the matrix pipe keeps working across the barrier and the first
// fragments of the next step load under those MFMAs.  Stage kt is refilled with step kt+NS right
// after that barrier (every read of stage kt has been issued by then), so NS = 2 stages of K = 64
// already give each load one step of slack.  Used with one or two wavefronts per SIMD.
//
// Per accumulator the MFMA sequence is unchanged (k ascending), so results are bit-identical to
// the other main loops.

template <class Cfg>
__device__ __forceinline__ void load_frags(const char* base, int a_frow, int b_frow, int koff, bf16x8 (&af)[MSUB],
                                           bf16x8 (&bfr)[Cfg::NSUB]) {
#pragma unroll
  for (int m = 0; m < MSUB; ++m) af[m] = *reinterpret_cast<const bf16x8*>(base + a_frow + m * 32 * Cfg::ROW + koff);
#pragma unroll
  for (int n = 0; n < Cfg::NSUB; ++n)
    bfr[n] = *reinterpret_cast<const bf16x8*>(base + b_frow + n * 32 * Cfg::ROW + koff);
}

template <class Cfg>
__device__ __forceinline__ void mfma_block(const bf16x8 (&af)[MSUB], const bf16x8 (&bfr)[Cfg::NSUB],
                                           f32x16 (&acc)[MSUB][Cfg::NSUB]) {
#pragma unroll
  for (int m = 0; m < MSUB; ++m)
#pragma unroll
    for (int n = 0; n < Cfg::NSUB; ++n)
      acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[m], bfr[n], acc[m][n], 0, 0, 0);
}

template <class Cfg>
__device__ __forceinline__ void tile_mainloop3(const __bf16* __restrict__ A, int64_t lda, int rowsA,
                                               const __bf16* __restrict__ B, int64_t ldb, int rowsB, int K,
                                               char* __restrict__ lds, f32x16 (&acc)[MSUB][Cfg::NSUB]) {
  constexpr int ROW = Cfg::ROW;
  constexpr int KSUB = Cfg::KSUB;
  constexpr int NS = Cfg::NS;
  constexpr int IPW = Cfg::A_IPW + Cfg::B_IPW;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % Cfg::WM;
  const int wn = wave / Cfg::WM;

  const u32x4 da = make_desc(A, (uint32_t)((int64_t)rowsA * lda * 2));
  const u32x4 db = make_desc(B, (uint32_t)((int64_t)rowsB * ldb * 2));
  const uint32_t lds0 = lds_addr(lds);

  const int dl_row = lane / Cfg::CPR;
  const int dl_pc = lane % Cfg::CPR;
  uint32_t a_off[Cfg::A_IPW], b_off[Cfg::B_IPW];
  int a_lc[Cfg::A_IPW], b_lc[Cfg::B_IPW];
#pragma unroll
  for (int i = 0; i < Cfg::A_IPW; ++i) {
    const int r = (wave * Cfg::A_IPW + i) * Cfg::RPI + dl_row;
    a_lc[i] = dl_pc ^ Cfg::swz(r);
    a_off[i] = (uint32_t)(r * lda * 2 + a_lc[i] * 16);
  }
#pragma unroll
  for (int i = 0; i < Cfg::B_IPW; ++i) {
    const int r = (wave * Cfg::B_IPW + i) * Cfg::RPI + dl_row;
    b_lc[i] = dl_pc ^ Cfg::swz(r);
    b_off[i] = (uint32_t)(r * ldb * 2 + b_lc[i] * 16);
  }
  const int nk = (K + Cfg::BK - 1) / Cfg::BK;
  auto issue = [&](int kt) {  // step kt -> stage kt % NS; steps past the end read zeros
    const bool kt_in = kt < nk;
    const int k0 = kt * Cfg::BK;
    const uint32_t kb = (uint32_t)kt * ROW;
    const uint32_t sbase = lds0 + (kt % NS) * Cfg::STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < Cfg::A_IPW; ++i)
      dma16(da, (kt_in && k0 + a_lc[i] * 8 < K) ? a_off[i] + kb : OOB_OFFSET, sbase + (wave * Cfg::A_IPW + i) * 1024);
#pragma unroll
    for (int i = 0; i < Cfg::B_IPW; ++i)
      dma16(db, (kt_in && k0 + b_lc[i] * 8 < K) ? b_off[i] + kb : OOB_OFFSET,
            sbase + Cfg::TM * ROW + (wave * Cfg::B_IPW + i) * 1024);
  };

  const int fr = lane & 31;
  const int fsw = Cfg::swz(fr);
  const int a_frow = (wm * WAVE_M + fr) * ROW;
  const int b_frow = Cfg::TM * ROW + (wn * Cfg::WAVE_N + fr) * ROW;
  int koff[KSUB];
#pragma unroll
  for (int s = 0; s < KSUB; ++s) koff[s] = (((2 * s) | (lane >> 5)) ^ fsw) << 4;

  // prologue: steps 0..NS-1 in flight, wait for step 0
#pragma unroll
  for (int p = 0; p < NS; ++p) issue(p);
  wait_vmcnt<(NS - 1) * IPW>();
  __syncthreads();
  bf16x8 fa[2][MSUB], fb[2][Cfg::NSUB];
  load_frags<Cfg>(lds, a_frow, b_frow, koff[0], fa[0], fb[0]);

  for (int kt = 0; kt < nk; ++kt) {
    const char* base = lds + (kt % NS) * Cfg::STAGE_BYTES;
    const char* nbase = lds + ((kt + 1) % NS) * Cfg::STAGE_BYTES;
#pragma unroll
    for (int s = 0; s < KSUB - 1; ++s) {
      load_frags<Cfg>(base, a_frow, b_frow, koff[s + 1], fa[(s + 1) & 1], fb[(s + 1) & 1]);
      mfma_block<Cfg>(fa[s & 1], fb[s & 1], acc);
    }
    // Every read of stage kt has been issued (the barrier waits for them): publish step kt+1
    // (its loads were issued NS-1 steps ago) and refill stage kt with step kt+NS.
    wait_vmcnt<(NS - 2) * IPW>();
    __syncthreads();
    issue(kt + NS);
    if (kt + 1 < nk) load_frags<Cfg>(nbase, a_frow, b_frow, koff[0], fa[0], fb[0]);
    mfma_block<Cfg>(fa[(KSUB - 1) & 1], fb[(KSUB - 1) & 1], acc);
  }
  wait_vmcnt<0>();   // trailing out-of-range loads still write LDS
  __syncthreads();
}

// =============================================================================================
// Main loop v4: the v2 ring with the DMA of each step spread between that step's MFMAs.
// =============================================================================================
//
// Issuing a step's global -> LDS loads in one burst right after the barrier stalls every
// wavefront at the texture unit (a 1 KiB load instruction takes the unit many cycles) while the
// matrix pipe idles.  Here the step's NDMA load instructions are interleaved with its NMF MFMAs,
// one after every NMF/NDMA MFMAs, so address processing overlaps matrix work.  The stage being
// filled is (kt + NS - 1) % NS, retired by the barrier at the top of step kt; the data of step
// kt + 1 has NS - 2 further steps of slack, so NS >= 3.

template <class Cfg>
__device__ __forceinline__ void tile_mainloop4(const __bf16* __restrict__ A, int64_t lda, int rowsA,
                                               const __bf16* __restrict__ B, int64_t ldb, int rowsB, int K,
                                               char* __restrict__ lds, f32x16 (&acc)[MSUB][Cfg::NSUB]) {
  constexpr int ROW = Cfg::ROW;
  constexpr int KSUB = Cfg::KSUB;
  constexpr int NS = Cfg::NS;
  constexpr int NDMA = Cfg::A_IPW + Cfg::B_IPW;
  constexpr int NMF = KSUB * MSUB * Cfg::NSUB;
  static_assert(NS >= 3, "v4 main loop needs at least three stages");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % Cfg::WM;
  const int wn = wave / Cfg::WM;

  const u32x4 da = make_desc(A, (uint32_t)((int64_t)rowsA * lda * 2));
  const u32x4 db = make_desc(B, (uint32_t)((int64_t)rowsB * ldb * 2));
  const uint32_t lds0 = lds_addr(lds);

  const int dl_row = lane / Cfg::CPR;
  const int dl_pc = lane % Cfg::CPR;
  uint32_t d_off[NDMA];
  int d_lc[NDMA];
#pragma unroll
  for (int d = 0; d < NDMA; ++d) {
    const bool is_a = d < Cfg::A_IPW;
    const int i = is_a ? d : d - Cfg::A_IPW;
    const int r = (wave * (is_a ? Cfg::A_IPW : Cfg::B_IPW) + i) * Cfg::RPI + dl_row;
    d_lc[d] = dl_pc ^ Cfg::swz(r);
    d_off[d] = (uint32_t)(r * (is_a ? lda : ldb) * 2 + d_lc[d] * 16);
  }
  const int nk = (K + Cfg::BK - 1) / Cfg::BK;
  // load instruction d of step kt (stage kt % NS)
  auto dma = [&](int d, int kt) {
    const bool is_a = d < Cfg::A_IPW;
    const int i = is_a ? d : d - Cfg::A_IPW;
    const bool ok = kt < nk && kt * Cfg::BK + d_lc[d] * 8 < K;
    const uint32_t voff = ok ? d_off[d] + (uint32_t)kt * ROW : OOB_OFFSET;
    const uint32_t dst = lds0 + (kt % NS) * Cfg::STAGE_BYTES +
                         (is_a ? (wave * Cfg::A_IPW + i) * 1024 : Cfg::TM * ROW + (wave * Cfg::B_IPW + i) * 1024);
    dma16(is_a ? da : db, voff, dst);
  };

  const int fr = lane & 31;
  const int fsw = Cfg::swz(fr);
  const int a_frow = (wm * WAVE_M + fr) * ROW;
  const int b_frow = Cfg::TM * ROW + (wn * Cfg::WAVE_N + fr) * ROW;
  int koff[KSUB];
#pragma unroll
  for (int s = 0; s < KSUB; ++s) koff[s] = (((2 * s) | (lane >> 5)) ^ fsw) << 4;

#pragma unroll
  for (int p = 0; p < NS - 1; ++p)
#pragma unroll
    for (int d = 0; d < NDMA; ++d) dma(d, p);

  for (int kt = 0; kt < nk; ++kt) {
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
          acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[m], bfr[n], acc[m][n], 0, 0, 0);
          const int q = (s * MSUB + m) * Cfg::NSUB + n;   // MFMA index inside the step
#pragma unroll
          for (int d = 0; d < NDMA; ++d)
            if (d * NMF / NDMA == q) dma(d, kn);
        }
    }
  }
  wait_vmcnt<0>();   // trailing out-of-range loads still write LDS
  __syncthreads();
}

// =============================================================================================
// Main loop v5: two groups of four wavefronts in ping-pong.
// =============================================================================================
//
// Eight wavefronts, two per SIMD (wavefronts w and w+4 share SIMD w % 4).  Group 0 = wavefronts
// 0-3, group 1 = 4-7; each has one wavefront per SIMD.  Every wavefront runs the same sequence
// "load the fragments of step k from LDS | barrier | 32 MFMAs of step k | barrier", but group 1
// starts one barrier later, so in every phase one group issues MFMAs back to back from registers
// while the other reads LDS: each SIMD's matrix pipe is fed by one wavefront per phase without
// waiting on LDS.  (Hardware barriers count arrivals, so the groups may sit at different barrier
// instructions as long as every wavefront executes the same number of them.)
//
//   phase 2k:    group 0 issues the global -> LDS loads of step k+1 into stage (k+1) % 2 (last read
//                in phases 2k-2 and 2k-1) and reads the fragments of step k; group 1 computes k-1
//   phase 2k+1:  group 0 computes step k, then waits for its loads of step k+1;
//                group 1 reads the fragments of step k
//
// Per accumulator the MFMA sequence is unchanged (k ascending), so results are bit-identical to the
// other main loops.

template <class Cfg>
__device__ __forceinline__ void tile_mainloop5(const __bf16* __restrict__ A, int64_t lda, int rowsA,
                                               const __bf16* __restrict__ B, int64_t ldb, int rowsB, int K,
                                               char* __restrict__ lds, f32x16 (&acc)[MSUB][Cfg::NSUB]) {
  static_assert(Cfg::NWAVES == 8 && Cfg::WM == 2 && Cfg::NS == 2 && Cfg::BK == 64, "v5: 8 wavefronts, 2 x K64");
  constexpr int ROW = Cfg::ROW;                   // 128 bytes
  constexpr int NBLK = (Cfg::TM + Cfg::TN) / 8;   // 8-row DMA blocks per stage
  constexpr int DPW = NBLK / 4;                   // DMA instructions per group-0 wavefront per step
  static_assert(Cfg::TM / 8 == 2 * DPW && Cfg::TN / 8 == 2 * DPW && DPW <= 31, "v5 DMA split");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;
  const int gw = wave & 3;
  const int wm = wave % Cfg::WM;
  const int wn = wave / Cfg::WM;

  // ---- global -> LDS (group 0): wavefronts 0,1 load the A rows, 2,3 the B rows
  const bool dma_a = gw < 2;
  const u32x4 desc = dma_a ? make_desc(A, (uint32_t)((int64_t)rowsA * lda * 2))
                           : make_desc(B, (uint32_t)((int64_t)rowsB * ldb * 2));
  const int64_t ld = dma_a ? lda : ldb;
  const int blk0 = (gw & 1) * DPW;                // first 8-row block (even: block parity = i parity)
  const uint32_t lds0 = lds_addr(lds);
  const uint32_t part = dma_a ? 0u : (uint32_t)(Cfg::TM * ROW);
  const int dl_row = lane >> 3;
  const int dl_pc = lane & 7;
  // the stored chunk of row r is c ^ ((r >> 1) & 7), r = 8 * (blk0 + i) + dl_row
  const int lc_even = dl_pc ^ (dl_row >> 1);
  const int lc_odd = dl_pc ^ (4 + (dl_row >> 1));
  const uint32_t row_off = (uint32_t)((blk0 * 8 + dl_row) * ld * 2);
  const uint32_t blk_stride = (uint32_t)(8 * ld * 2);
  const int nk = (K + Cfg::BK - 1) / Cfg::BK;
  auto dma_step = [&](int kt) {
    const bool kt_in = kt < nk;
    const int k0 = kt * Cfg::BK;
    const bool ok_even = kt_in && k0 + lc_even * 8 < K;
    const bool ok_odd = kt_in && k0 + lc_odd * 8 < K;
    const uint32_t ve = row_off + lc_even * 16 + (uint32_t)kt * ROW;
    const uint32_t vo = row_off + lc_odd * 16 + (uint32_t)kt * ROW;
    const uint32_t sbase = lds0 + (kt & 1) * Cfg::STAGE_BYTES + part + blk0 * 1024;
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      const bool ok = (i & 1) ? ok_odd : ok_even;
      const uint32_t voff = ((i & 1) ? vo : ve) + (uint32_t)i * blk_stride;
      dma16(desc, ok ? voff : OOB_OFFSET, sbase + i * 1024);
    }
  };

  // ---- the fragments of one whole step
  const int fr = lane & 31;
  const int fsw = (fr >> 1) & 7;
  const int a_frow = (wm * WAVE_M + fr) * ROW;
  const int b_frow = Cfg::TM * ROW + (wn * Cfg::WAVE_N + fr) * ROW;
  const int kx = lane >> 5;
  bf16x8 fa[4][MSUB], fb[4][Cfg::NSUB];

  if (group == 0) {
    dma_step(0);
    wait_vmcnt<0>();
  }
  __syncthreads();                 // step 0 published
  if (group == 1) __syncthreads(); // group 1 runs one phase behind

  for (int kt = 0; kt < nk; ++kt) {
    // memory phase
    if (group == 0) dma_step(kt + 1);
    const char* base = lds + (kt & 1) * Cfg::STAGE_BYTES;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int ko = (((2 * s) | kx) ^ fsw) << 4;
#pragma unroll
      for (int m = 0; m < MSUB; ++m) fa[s][m] = *reinterpret_cast<const bf16x8*>(base + a_frow + m * 32 * ROW + ko);
#pragma unroll
      for (int n = 0; n < Cfg::NSUB; ++n)
        fb[s][n] = *reinterpret_cast<const bf16x8*>(base + b_frow + n * 32 * ROW + ko);
    }
    // keep the phases apart: the scheduler must not move MFMAs (not memory operations) across
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    // compute phase
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int m = 0; m < MSUB; ++m)
#pragma unroll
        for (int n = 0; n < Cfg::NSUB; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s][m], fb[s][n], acc[m][n], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (group == 0) wait_vmcnt<0>();  // this wavefront's loads of step kt+1 have landed
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  }
  if (group == 0) __syncthreads(); // same barrier count for both groups
  wait_vmcnt<0>();                 // trailing out-of-range loads still write LDS
  __syncthreads();
}

// =============================================================================================
// Main loop v6: ping-pong on a ring of NS stages of K = 32, loads shared by both groups.
// =============================================================================================
//
// As v5, two groups of four wavefronts alternate between a memory phase and a compute phase, with
// group 1 one phase behind.  Here a step is K = 32 (16 MFMAs per wavefront) and every wavefront
// issues its own share of the global -> LDS loads of step k+2 in its memory phase of step k, so the
// texture unit gets one quarter of a step's bytes per phase instead of a whole step at once.
//
//   iteration k, memory phase:  loads of step k+2 into stage (k+2) % NS (last read two steps ago);
//                               fragments of step k from stage k % NS;
//                               group 1 then waits for its loads of step k+1
//   iteration k, compute phase: 16 MFMAs of step k; group 0 then waits for its loads of step k+1
//
// Each group's loads of step k+1 have landed before the barrier that precedes group 0's memory
// phase of step k+1 (group 0 waits at the end of its compute phase, group 1 at the end of its memory
// phase, one phase later in time), giving each load three to four phases of slack.

template <class Cfg>
__device__ __forceinline__ void tile_mainloop6(const __bf16* __restrict__ A, int64_t lda, int rowsA,
                                               const __bf16* __restrict__ B, int64_t ldb, int rowsB, int K,
                                               char* __restrict__ lds, f32x16 (&acc)[MSUB][Cfg::NSUB]) {
  static_assert(Cfg::NWAVES == 8 && Cfg::NS >= 3 && Cfg::BK == 32, "v6: 8 wavefronts, K32 ring");
  constexpr int ROW = Cfg::ROW;
  constexpr int NS = Cfg::NS;
  constexpr int NDMA = Cfg::A_IPW + Cfg::B_IPW;   // load instructions per wavefront per step
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;
  const int wm = wave % Cfg::WM;
  const int wn = wave / Cfg::WM;

  const u32x4 da = make_desc(A, (uint32_t)((int64_t)rowsA * lda * 2));
  const u32x4 db = make_desc(B, (uint32_t)((int64_t)rowsB * ldb * 2));
  const uint32_t lds0 = lds_addr(lds);
  const int dl_row = lane / Cfg::CPR;
  const int dl_pc = lane % Cfg::CPR;
  uint32_t d_off[NDMA];
  int d_lc[NDMA];
#pragma unroll
  for (int d = 0; d < NDMA; ++d) {
    const bool is_a = d < Cfg::A_IPW;
    const int i = is_a ? d : d - Cfg::A_IPW;
    const int r = (wave * (is_a ? Cfg::A_IPW : Cfg::B_IPW) + i) * Cfg::RPI + dl_row;
    d_lc[d] = dl_pc ^ Cfg::swz(r);
    d_off[d] = (uint32_t)(r * (is_a ? lda : ldb) * 2 + d_lc[d] * 16);
  }
  const int nk = (K + Cfg::BK - 1) / Cfg::BK;
  auto dma_step = [&](int kt) {
    const uint32_t sbase = lds0 + (kt % NS) * Cfg::STAGE_BYTES;
#pragma unroll
    for (int d = 0; d < NDMA; ++d) {
      const bool is_a = d < Cfg::A_IPW;
      const int i = is_a ? d : d - Cfg::A_IPW;
      const bool ok = kt < nk && kt * Cfg::BK + d_lc[d] * 8 < K;
      const uint32_t dst = sbase + (is_a ? (wave * Cfg::A_IPW + i) * 1024 : Cfg::TM * ROW + (wave * Cfg::B_IPW + i) * 1024);
      dma16(is_a ? da : db, ok ? d_off[d] + (uint32_t)kt * ROW : OOB_OFFSET, dst);
    }
  };

  const int fr = lane & 31;
  const int fsw = Cfg::swz(fr);
  const int a_frow = (wm * WAVE_M + fr) * ROW;
  const int b_frow = Cfg::TM * ROW + (wn * Cfg::WAVE_N + fr) * ROW;
  const int kx = lane >> 5;
  bf16x8 fa[2][MSUB], fb[2][Cfg::NSUB];

  dma_step(0);
  dma_step(1);
  wait_vmcnt<NDMA>();              // this wavefront's loads of step 0
  __syncthreads();                 // step 0 published
  if (group == 1) __syncthreads(); // group 1 runs one phase behind

  for (int kt = 0; kt < nk; ++kt) {
    // memory phase
    dma_step(kt + 2);
    const char* base = lds + (kt % NS) * Cfg::STAGE_BYTES;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int ko = (((2 * s) | kx) ^ fsw) << 4;
#pragma unroll
      for (int m = 0; m < MSUB; ++m) fa[s][m] = *reinterpret_cast<const bf16x8*>(base + a_frow + m * 32 * ROW + ko);
#pragma unroll
      for (int n = 0; n < Cfg::NSUB; ++n)
        fb[s][n] = *reinterpret_cast<const bf16x8*>(base + b_frow + n * 32 * ROW + ko);
    }
    if (group == 1) wait_vmcnt<NDMA>();   // group 1's loads of step kt+1 have landed
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    // compute phase
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int m = 0; m < MSUB; ++m)
#pragma unroll
        for (int n = 0; n < Cfg::NSUB; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s][m], fb[s][n], acc[m][n], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (group == 0) wait_vmcnt<NDMA>();   // group 0's loads of step kt+1 have landed
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  }
  if (group == 0) __syncthreads(); // same barrier count for both groups
  wait_vmcnt<0>();                 // trailing out-of-range loads still write LDS
  __syncthreads();
}

// =============================================================================================
// Main loop v7: ping-pong on K = 64 steps with separate A and B rings (3 + 2 slots of 32 KB).
// =============================================================================================
//
// As v5 (one K = 64 step per phase, full-step fragments in registers), but the global -> LDS loads
// of a step are split between the groups so that neither group's memory phase carries a whole
// step: group 1 loads the A rows (256 x 128 B) of step k+2 into A slot (k+2) % 3 during its memory
// phase of step k, and group 0 loads the B rows of step k+1 into B slot (k+1) % 2 during its memory
// phase of step k.  In phase terms (group 0 in even phases, group 1 one phase behind):
//   A slot (k+2) % 3 was last read in phases 2k-2 and 2k-1, and is needed again in phase 2k+4;
//   B slot (k+1) % 2 was last read in phases 2k-2 and 2k-1, and is needed again in phase 2k+2.
// Group 1 waits for its A loads of step k+1 at the end of its memory phase of step k (phase 2k+1);
// group 0 waits for its B loads of step k+1 at the end of its compute phase of step k (phase 2k+1).

template <class Cfg>
__device__ __forceinline__ void tile_mainloop7(const __bf16* __restrict__ A, int64_t lda, int rowsA,
                                               const __bf16* __restrict__ B, int64_t ldb, int rowsB, int K,
                                               char* __restrict__ lds, f32x16 (&acc)[MSUB][Cfg::NSUB]) {
  static_assert(Cfg::NWAVES == 8 && Cfg::WM == 2 && Cfg::BK == 64 && Cfg::TM == 256 && Cfg::TN == 256,
                "v7: 8 wavefronts, 256 x 256, K64");
  constexpr int ROW = Cfg::ROW;                 // 128 bytes
  constexpr int SLOT = 256 * ROW;               // 32 KB: one operand of one step
  constexpr int B_BASE = 3 * SLOT;              // A slots 0..2, then B slots 0..1
  constexpr int DPW = 8;                        // DMA instructions per wavefront per step (8 rows each)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;
  const int gw = wave & 3;
  const int wm = wave % Cfg::WM;
  const int wn = wave / Cfg::WM;

  // group 1 loads A, group 0 loads B; wavefront gw of a group loads rows [64 gw, 64 gw + 64)
  const bool loads_a = group == 1;
  const u32x4 desc = loads_a ? make_desc(A, (uint32_t)((int64_t)rowsA * lda * 2))
                             : make_desc(B, (uint32_t)((int64_t)rowsB * ldb * 2));
  const int64_t ld = loads_a ? lda : ldb;
  const uint32_t lds0 = lds_addr(lds);
  const int dl_row = lane >> 3;
  const int dl_pc = lane & 7;
  const int blk0 = gw * DPW;                    // even
  const int lc_even = dl_pc ^ (dl_row >> 1);
  const int lc_odd = dl_pc ^ (4 + (dl_row >> 1));
  const uint32_t row_off = (uint32_t)((blk0 * 8 + dl_row) * ld * 2);
  const uint32_t blk_stride = (uint32_t)(8 * ld * 2);
  const int nk = (K + Cfg::BK - 1) / Cfg::BK;
  auto dma_step = [&](int kt) {   // this group's operand of step kt into its slot
    const bool kt_in = kt < nk;
    const int k0 = kt * Cfg::BK;
    const bool ok_even = kt_in && k0 + lc_even * 8 < K;
    const bool ok_odd = kt_in && k0 + lc_odd * 8 < K;
    const uint32_t ve = row_off + lc_even * 16 + (uint32_t)kt * ROW;
    const uint32_t vo = row_off + lc_odd * 16 + (uint32_t)kt * ROW;
    const uint32_t sbase = lds0 + (loads_a ? (kt % 3) * SLOT : B_BASE + (kt & 1) * SLOT) + blk0 * 1024;
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      const bool ok = (i & 1) ? ok_odd : ok_even;
      const uint32_t voff = ((i & 1) ? vo : ve) + (uint32_t)i * blk_stride;
      dma16(desc, ok ? voff : OOB_OFFSET, sbase + i * 1024);
    }
  };

  const int fr = lane & 31;
  const int fsw = (fr >> 1) & 7;
  const int a_frow = (wm * WAVE_M + fr) * ROW;
  const int b_frow = (wn * Cfg::WAVE_N + fr) * ROW;
  const int kx = lane >> 5;
  bf16x8 fa[4][MSUB], fb[4][Cfg::NSUB];

  // prologue: A of steps 0 and 1 (group 1), B of step 0 (group 0); step 0 published
  dma_step(0);
  if (loads_a) {
    dma_step(1);
    wait_vmcnt<DPW>();
  } else {
    wait_vmcnt<0>();
  }
  __syncthreads();
  if (group == 1) __syncthreads();  // group 1 runs one phase behind

  for (int kt = 0; kt < nk; ++kt) {
    // memory phase
    dma_step(loads_a ? kt + 2 : kt + 1);
    const char* abase = lds + (kt % 3) * SLOT;
    const char* bbase = lds + B_BASE + (kt & 1) * SLOT;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int ko = (((2 * s) | kx) ^ fsw) << 4;
#pragma unroll
      for (int m = 0; m < MSUB; ++m) fa[s][m] = *reinterpret_cast<const bf16x8*>(abase + a_frow + m * 32 * ROW + ko);
#pragma unroll
      for (int n = 0; n < Cfg::NSUB; ++n)
        fb[s][n] = *reinterpret_cast<const bf16x8*>(bbase + b_frow + n * 32 * ROW + ko);
    }
    if (loads_a) wait_vmcnt<DPW>();   // group 1's A of step kt+1 has landed
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    // compute phase
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int m = 0; m < MSUB; ++m)
#pragma unroll
        for (int n = 0; n < Cfg::NSUB; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s][m], fb[s][n], acc[m][n], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (!loads_a) wait_vmcnt<0>();    // group 0's B of step kt+1 has landed
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  }
  if (group == 0) __syncthreads();    // same barrier count for both groups
  wait_vmcnt<0>();                    // trailing out-of-range loads still write LDS
  __syncthreads();
}

}  // namespace lmh
