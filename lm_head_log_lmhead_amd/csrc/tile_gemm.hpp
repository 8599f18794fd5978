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

// Physical 16-byte chunk of logical chunk c in LDS row r (8 chunks per 128-byte row).
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

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

}  // namespace lmh
