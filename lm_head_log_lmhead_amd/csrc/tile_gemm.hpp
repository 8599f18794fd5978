// tile_gemm.hpp — the bf16 MFMA tile main loop shared by every GEMM-shaped kernel of the library.
//
// C[M x N] (fp32, in registers) = A[M x K] . B[N x K]^T, with both operands row-major and K
// contiguous ("TN").  One workgroup computes a TM x TN tile with WM x WN wavefronts; every
// wavefront owns a 128 x (32*NSUB) sub-tile made of 4 x NSUB accumulators of the gfx950
// instruction v_mfma_f32_32x32x16_bf16 (16 fp32 per lane each).
//
// Invariance contract.  For one output element the sequence of floating-point operations is
//   acc = C0;  for k-step ks = 0, 1, ...: for substep s = 0..3: acc = mfma(A[i, k16], B[j, k16], acc)
// with k-steps of 64 in ascending order.  It does not depend on the tile configuration, on the
// element's position inside the tile, or on M and N.  Padding past K is exact zeros.
//
// Data path.  Global -> VGPR (buffer loads, 16 bytes per lane, out-of-range rows read as zero)
// -> LDS (double buffered, XOR-swizzled 16-byte chunks to spread the fragment reads over the
// banks) -> VGPR fragments (ds_read_b128) -> MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmh {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int BK = 64;            // K elements per main-loop step (one 128-byte row segment)
constexpr int MSUB = 4;           // 32-row MFMA sub-tiles per wavefront along M (128 rows)
constexpr int WAVE_M = 32 * MSUB; // rows of A per wavefront
constexpr float LOG2E = 1.4426950408889634f;

// Offsets at or beyond this value are outside every buffer resource we build, so the hardware
// returns zeros for them.
constexpr uint32_t OOB_OFFSET = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // Raw buffer (stride 0); 0x00020000 is the gfx9 data-format word for untyped 32-bit access.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Physical 16-byte chunk of logical chunk c in LDS row r (8 chunks per 128-byte row) is
// c ^ swz(r).  LMH_LDS_SWIZZLE selects the row hash (a build-time tuning knob; every choice gives
// the same results, only the LDS bank pattern changes).
#ifndef LMH_LDS_SWIZZLE
#define LMH_LDS_SWIZZLE 1
#endif
__device__ __forceinline__ int swz(int r) {
#if LMH_LDS_SWIZZLE == 0
  return r & 7;
#else
  return (r >> 1) & 7;
#endif
}

template <int WM_, int WN_, int NSUB_>
struct TileCfg {
  static constexpr int WM = WM_, WN = WN_, NSUB = NSUB_;
  static constexpr int NWAVES = WM * WN;
  static constexpr int NTHREADS = 64 * NWAVES;
  static constexpr int TM = WAVE_M * WM;          // rows of A per workgroup
  static constexpr int WAVE_N = 32 * NSUB;        // rows of B per wavefront
  static constexpr int TN = WAVE_N * WN;          // rows of B per workgroup
  static constexpr int A_LOADS = TM * 8 / NTHREADS;  // 16-byte chunks per thread per k-step
  static constexpr int B_LOADS = TN * 8 / NTHREADS;
  static constexpr int STAGE_BYTES = (TM + TN) * BK * 2;
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
  static_assert(TM * 8 % NTHREADS == 0 && TN * 8 % NTHREADS == 0 && B_LOADS >= 1, "tile load split");
};

// Runs the whole K loop for one workgroup tile, continuing the accumulation chains already in
// `acc` (callers start them at zero, or at a previous partial result to extend a chain).  A points at the tile's first row, with `rowsA`
// valid rows (rows beyond read as zero) and a row pitch of `lda` elements; same for B.  `K` is the
// contraction length; chunks at k >= K read as zero (an 8-element chunk that straddles K is read
// as stored, so callers keep the elements past K inside such a chunk at zero).
template <class Cfg>
__device__ __forceinline__ void tile_mainloop(const __bf16* __restrict__ A, int64_t lda, int rowsA,
                                              const __bf16* __restrict__ B, int64_t ldb, int rowsB, int K,
                                              char* __restrict__ lds, f32x16 (&acc)[MSUB][Cfg::NSUB]) {
  constexpr int NT = Cfg::NTHREADS;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % Cfg::WM;
  const int wn = wave / Cfg::WM;

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (uint32_t)((int64_t)rowsA * lda * 2));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(B, (uint32_t)((int64_t)rowsB * ldb * 2));

  // Global -> LDS assignment: chunk q = tid + i*NT -> row q/8, logical chunk q%8 (= tid%8).
  const int lc = tid & 7;
  const int lrow0 = tid >> 3;
  constexpr int ROWS_PER_PASS = NT / 8;

  uint32_t a_goff[Cfg::A_LOADS], b_goff[Cfg::B_LOADS];
  int a_loff[Cfg::A_LOADS], b_loff[Cfg::B_LOADS];
#pragma unroll
  for (int i = 0; i < Cfg::A_LOADS; ++i) {
    const int r = lrow0 + i * ROWS_PER_PASS;
    a_goff[i] = (uint32_t)(r * lda * 2 + lc * 16);
    a_loff[i] = r * 128 + ((lc ^ swz(r)) << 4);
  }
#pragma unroll
  for (int i = 0; i < Cfg::B_LOADS; ++i) {
    const int r = lrow0 + i * ROWS_PER_PASS;
    b_goff[i] = (uint32_t)(r * ldb * 2 + lc * 16);
    b_loff[i] = Cfg::TM * 128 + r * 128 + ((lc ^ swz(r)) << 4);
  }

  // Fragment read offsets (bytes inside a stage) for this lane.
  const int fr = lane & 31;           // row inside a 32-row sub-tile
  const int fh = lane >> 5;           // which 8-element half of the 16-wide k slice
  const int fsw = swz(fr);            // sub-tile bases are multiples of 32 rows: same swizzle
  const int a_frow = (wm * WAVE_M + fr) * 128;
  const int b_frow = Cfg::TM * 128 + (wn * Cfg::WAVE_N + fr) * 128;
  int koff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) koff[s] = (((2 * s) | fh) ^ fsw) << 4;

  const int nk = (K + BK - 1) / BK;
  u32x4 ra_reg[Cfg::A_LOADS], rb_reg[Cfg::B_LOADS];

  auto gload = [&](int kt) {
    const uint32_t kb = (uint32_t)kt * (BK * 2);
    const bool kin = kt * BK + lc * 8 < K;
#pragma unroll
    for (int i = 0; i < Cfg::A_LOADS; ++i) ra_reg[i] = buffer_load16(ra, kin ? a_goff[i] + kb : OOB_OFFSET);
#pragma unroll
    for (int i = 0; i < Cfg::B_LOADS; ++i) rb_reg[i] = buffer_load16(rb, kin ? b_goff[i] + kb : OOB_OFFSET);
  };
  auto lstore = [&](int stage) {
    char* base = lds + stage * Cfg::STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < Cfg::A_LOADS; ++i) *reinterpret_cast<u32x4*>(base + a_loff[i]) = ra_reg[i];
#pragma unroll
    for (int i = 0; i < Cfg::B_LOADS; ++i) *reinterpret_cast<u32x4*>(base + b_loff[i]) = rb_reg[i];
  };

  if (nk > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int stage = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const char* base = lds + stage * Cfg::STAGE_BYTES;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 af[MSUB], bfr[Cfg::NSUB];
#pragma unroll
      for (int m = 0; m < MSUB; ++m)
        af[m] = *reinterpret_cast<const bf16x8*>(base + a_frow + m * 32 * 128 + koff[s]);
#pragma unroll
      for (int n = 0; n < Cfg::NSUB; ++n)
        bfr[n] = *reinterpret_cast<const bf16x8*>(base + b_frow + n * 32 * 128 + koff[s]);
#pragma unroll
      for (int m = 0; m < MSUB; ++m)
#pragma unroll
        for (int n = 0; n < Cfg::NSUB; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[m], bfr[n], acc[m][n], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(stage ^ 1);
    __syncthreads();
  }
}

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
// Main loop v2: a ring of NS LDS stages of BK = 32 filled by direct global -> LDS loads.
// =============================================================================================
//
// Each stage holds the tile's A rows then B rows, 64 bytes (32 bf16) per row, four 16-byte
// chunks per row with chunk c of row r stored at c ^ ((r >> 2) & 3).  Loads go straight from
// global memory to LDS (buffer_load_dwordx4 ... lds): one instruction moves 64 lanes x 16 bytes
// into one contiguous KiB of LDS (16 rows), the lane -> (row, chunk) assignment applying the
// swizzle.  Stages are filled NS-1 steps ahead, so global latency hides behind NS-1 steps of
// MFMA work; one barrier per step both publishes the stage and retires the stage it overwrites.
//
// The loads are issued from inline assembly.  The compiler therefore neither counts them nor
// waits for them; the loop waits with explicit vmcnt values (loads return in order), and the
// compiler's own waits for other loads stay correct (extra outstanding loads only make a vmcnt
// wait stricter).  M0 (the LDS destination base) is written inside the same asm block.

constexpr int BK2 = 32;          // K elements per step
constexpr int ROW2 = BK2 * 2;    // bytes per staged row

template <int WM_, int WN_, int NSUB_, int NS_>
struct PipeCfg {
  static constexpr int WM = WM_, WN = WN_, NSUB = NSUB_, NS = NS_;
  static constexpr int NWAVES = WM * WN;
  static constexpr int NTHREADS = 64 * NWAVES;
  static constexpr int TM = WAVE_M * WM;
  static constexpr int WAVE_N = 32 * NSUB;
  static constexpr int TN = WAVE_N * WN;
  static constexpr int A_IPW = TM / 16 / NWAVES;   // DMA instructions per wavefront per step
  static constexpr int B_IPW = TN / 16 / NWAVES;
  static constexpr int STAGE_BYTES = (TM + TN) * ROW2;
  static constexpr int LDS_BYTES = NS * STAGE_BYTES;
  static constexpr int VMCNT_AHEAD = (NS - 2) * (A_IPW + B_IPW);  // loads allowed in flight
  static_assert(TM % (16 * NWAVES) == 0 && TN % (16 * NWAVES) == 0 && B_IPW >= 1, "DMA split");
  static_assert(NS >= 2 && VMCNT_AHEAD <= 63, "vmcnt range");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
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
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % Cfg::WM;
  const int wn = wave / Cfg::WM;

  const u32x4 da = make_desc(A, (uint32_t)((int64_t)rowsA * lda * 2));
  const u32x4 db = make_desc(B, (uint32_t)((int64_t)rowsB * ldb * 2));
  const uint32_t lds0 = lds_addr(lds);

  // DMA lane assignment: lane -> (row lane/4 of the instruction's 16 rows, stored chunk lane%4),
  // which holds logical chunk (lane%4) ^ ((row >> 2) & 3) = (lane%4) ^ (lane/16).
  const int dl_row = lane >> 2;
  const int dl_chunk = (lane & 3) ^ (lane >> 4);
  uint32_t a_off[Cfg::A_IPW], b_off[Cfg::B_IPW];
#pragma unroll
  for (int i = 0; i < Cfg::A_IPW; ++i)
    a_off[i] = (uint32_t)(((wave * Cfg::A_IPW + i) * 16 + dl_row) * lda * 2 + dl_chunk * 16);
#pragma unroll
  for (int i = 0; i < Cfg::B_IPW; ++i)
    b_off[i] = (uint32_t)(((wave * Cfg::B_IPW + i) * 16 + dl_row) * ldb * 2 + dl_chunk * 16);

  const int nk = (K + BK2 - 1) / BK2;
  auto issue = [&](int kt) {
    const int st = kt % Cfg::NS;
    const bool kin = kt < nk && kt * BK2 + dl_chunk * 8 < K;
    const uint32_t kb = (uint32_t)kt * ROW2;
    const uint32_t sbase = lds0 + st * Cfg::STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < Cfg::A_IPW; ++i)
      dma16(da, kin ? a_off[i] + kb : OOB_OFFSET, sbase + (wave * Cfg::A_IPW + i) * 1024);
#pragma unroll
    for (int i = 0; i < Cfg::B_IPW; ++i)
      dma16(db, kin ? b_off[i] + kb : OOB_OFFSET, sbase + Cfg::TM * ROW2 + (wave * Cfg::B_IPW + i) * 1024);
  };

  // Fragment reads: lane reads row (lane & 31) of a 32-row sub-tile, logical chunk 2s + lane/32.
  const int fr = lane & 31;
  const int fsw = (lane >> 2) & 3;   // (row >> 2) & 3 for rows at multiples of 16 plus fr
  const int a_frow = (wm * WAVE_M + fr) * ROW2;
  const int b_frow = Cfg::TM * ROW2 + (wn * Cfg::WAVE_N + fr) * ROW2;
  int koff[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) koff[s] = (((2 * s) | (lane >> 5)) ^ fsw) << 4;

#pragma unroll
  for (int p = 0; p < Cfg::NS - 1; ++p) issue(p);

  for (int kt = 0; kt < nk; ++kt) {
    wait_vmcnt<Cfg::VMCNT_AHEAD>();   // this thread's loads of step kt have landed
    __syncthreads();                  // ... everyone's; and step kt-1's stage is free again
    issue(kt + Cfg::NS - 1);
    const char* base = lds + (kt % Cfg::NS) * Cfg::STAGE_BYTES;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 af[MSUB], bfr[Cfg::NSUB];
#pragma unroll
      for (int m = 0; m < MSUB; ++m)
        af[m] = *reinterpret_cast<const bf16x8*>(base + a_frow + m * 32 * ROW2 + koff[s]);
#pragma unroll
      for (int n = 0; n < Cfg::NSUB; ++n)
        bfr[n] = *reinterpret_cast<const bf16x8*>(base + b_frow + n * 32 * ROW2 + koff[s]);
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

}  // namespace lmh
