// bwd.hip — backward kernels of the fused LM-head log-prob.
//
// The backward of sum_t g_t * logprob_t recomputes the logits instead of keeping them (SkyRL PR
// #1765 "[megatron] Triton backend for fused LM-head log-prob", design commit: per-chunk logits
// are recomputed in backward) and uses dz_tj = g_t * ([j == y_t] - p_tj) with p = exp(z - lse);
// a label outside the call's weight rows contributes no label term, so dz = -g * p there (same
// PR, precision-policy commit; streaming-backward commit: exp of the log-softmax, negated, times
// the upstream gradient, plus the upstream gradient at the label).  The rows are the vocabulary
// ids [vocab_start, vocab_start + V): with vocab_start > 0 the call is one shard of a larger
// vocabulary, lse is the whole vocabulary's, and only the shard holding a label adds its term.
//
// The vocabulary is walked in fixed steps of Vs rows.  Per step:
//   K3 bwd_dz     : logit tile recompute (same MFMA main loop and tiles as the forward) and
//                   dz rounded to bf16, written both token-major into a [T x Vs] workspace slab
//                   and vocabulary-major into a [Vs x Tp] slab (dz^T);
//   transpose     : W_step -> W_step^T [H x Vs] (a vocabulary-contiguous copy, so both gradient
//                   GEMMs read K-contiguous operands; h^T [H x Tp] is made once per call);
//   K5 grad_weight: grad_W[step rows] (+)= dz^T . h  (K = tokens, one chain per element, no split)
//   K4 grad_hidden: grad_h += dz . W_step           (K = vocabulary; the accumulator is loaded
//                   from grad_h so the chain simply continues across steps)
// No atomics anywhere; every output element is produced by exactly one lane.
#include "kernels.hpp"

namespace lmh {

// ---------------------------------------------------------------------------------------------
// K3: dz tiles
// ---------------------------------------------------------------------------------------------

// dz and dz^T are written once per step and next read by the gradient GEMMs after the whole dz
// launch; stores with the non-temporal hint measured 0.8 % faster for the backward than plain
// ones (the gradient GEMM's fp32 C stores, re-read by the next step's accumulation, were slower
// with it).
__device__ __forceinline__ void st_dz(__bf16* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

constexpr int DZ_PITCH = WAVE_M * 2 + 16;  // bytes per staged token row (padded against conflicts)

// dz of a wavefront's tile part: the lane's four consecutive entries 16 m + 4 g4 + (0..3) of token
// n * 16 + j, rounded to bf16 and staged token-major in LDS at wl.  dz = g (onehot - p) is formed as
// fmaf(-g, p, label ? g : 0); without an entropy gradient the exponent is one fmaf,
// z log2(e) - lse log2(e).  The label test compares the label's offset from the lane's entry 0
// with the entry's constant offset 16 m + i (a label outside the call's rows gives a negative
// offset).  Unless FULL, entries past the call's rows and tokens past T are zeros.
template <class Cfg, bool SCALED, bool EGRAD, bool FULL>
__device__ __forceinline__ void dz_stage(const f32x4 (&acc)[MSUB][Cfg::NSUB], const float* __restrict__ grad,
                                         const float* __restrict__ lse, const int* __restrict__ labels,
                                         const float* __restrict__ grad_entropy, const float* __restrict__ entropy,
                                         float temperature, int T, int V, int vocab_start, int vs0, int wv, int tok0,
                                         char* wl) {
  const int lane = threadIdx.x & 63;
  const int j = acc_col(lane);
  const int g4 = lane >> 4;
#pragma unroll
  for (int n = 0; n < Cfg::NSUB; ++n) {
    const int tok = tok0 + n * MFMA_MN + j;
    const bool tok_ok = FULL || tok < T;
    float g = tok_ok ? grad[tok] : 0.f;
    const float L = tok_ok ? lse[tok] : 0.f;
    // the label as a weight row of this call (-1 when another shard's or out of range)
    const int yg = tok_ok ? labels[tok] : -1;
    const int y = yg >= vocab_start && yg - vocab_start < V ? yg - vocab_start : -1;
    const int yl = y - (vs0 + wv + 4 * g4);  // label offset from the lane's entry 0
    float ge = 0.f, He = 0.f;
    if (EGRAD) {
      ge = tok_ok ? grad_entropy[tok] : 0.f;
      He = tok_ok ? entropy[tok] : 0.f;
    }
    if (SCALED) {  // the 1/tau of the chain rule, folded into the per-token factors
      g = g / temperature;
      ge = ge / temperature;
    }
    const float lL = L * LOG2E;
#pragma unroll
    for (int m = 0; m < MSUB; ++m) {
      f32x4 dv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float z = SCALED ? acc[m][n][i] / temperature : acc[m][n][i];
        float p, lp = 0.f;
        if (EGRAD) {
          lp = z - L;
          p = __builtin_amdgcn_exp2f(lp * LOG2E);
        } else {
          p = __builtin_amdgcn_exp2f(__builtin_fmaf(z, LOG2E, -lL));
        }
        float d = __builtin_fmaf(-g, p, yl == m * MFMA_MN + i ? g : 0.f);
        if (EGRAD) d = d - ge * (p * (lp + He));
        if (!FULL) {
          const int v = vs0 + wv + m * MFMA_MN + acc_row(i, lane);
          d = v < V && tok_ok ? d : 0.f;
        }
        dv[i] = d;
      }
      *reinterpret_cast<bf16x4*>(wl + (n * MFMA_MN + j) * DZ_PITCH + (m * MFMA_MN + 4 * g4) * 2) =
          __builtin_convertvector(dv, bf16x4);
    }
  }
}

// With a temperature tau the logits are z / tau and the logit gradient carries 1/tau; with an
// entropy gradient gE the term -gE p (log p + H) is added (log p = z / tau - lse), as in the
// forward definition (verl PR #8026 review on the temperature order; the entropy gradient that
// SkyRL PR #1765 leaves unwired).
template <class Cfg, bool SCALED, bool EGRAD>
__global__ __launch_bounds__(Cfg::NTHREADS) void bwd_dz_kernel(
    const __bf16* __restrict__ hidden, const __bf16* __restrict__ weight, const int* __restrict__ labels,
    const float* __restrict__ grad, const float* __restrict__ lse, const float* __restrict__ grad_entropy,
    const float* __restrict__ entropy, float temperature, int T, int H, int V, int vocab_start, int vs0, int Vc,
    int Vs, int n_mt, int n_nt, __bf16* __restrict__ dz, __bf16* __restrict__ dzt, int ldt,
    int* __restrict__ gemm_sched) {
  loop_placement_pad<4 + 2 * SCALED + EGRAD>();
  // the gradient GEMM that follows this launch claims its tiles from these counters; the previous
  // step's GEMM has finished before this launch starts
  if (blockIdx.x == 0 && threadIdx.x < BWD_SCHED_WORDS) gemm_sched[threadIdx.x] = 0;
  constexpr int STAGE_OUT = Cfg::NWAVES * Cfg::WAVE_N * DZ_PITCH;
  constexpr int LDS = PingPong<Cfg>::LDS_BYTES > STAGE_OUT ? PingPong<Cfg>::LDS_BYTES : STAGE_OUT;
  __shared__ __attribute__((aligned(1024))) char lds[LDS];
  int mt, nt;
  tile_coords<8>(blockIdx.x, gridDim.x, n_mt, n_nt, mt, nt);
  const int v0 = mt * Cfg::TM;  // local vocabulary row inside the step
  const int t0 = nt * Cfg::TN;
  f32x4 acc[MSUB][Cfg::NSUB];
#pragma unroll
  for (int m = 0; m < MSUB; ++m)
#pragma unroll
    for (int n = 0; n < Cfg::NSUB; ++n) acc[m][n] = (f32x4)(0.0f);
  tile_mainloop_pingpong<Cfg>(weight + (int64_t)(vs0 + v0) * H, H, min(Cfg::TM, Vc - v0), hidden + (int64_t)t0 * H,
                              H, min(Cfg::TN, T - t0), H, lds, acc);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave % Cfg::WM, wn = wave / Cfg::WM;
  const int g4 = lane >> 4;
  const int wv = v0 + wm * WAVE_M;             // local column of this wavefront's first entry
  const int tok0 = t0 + wn * Cfg::WAVE_N;
  char* wl = lds + wave * Cfg::WAVE_N * DZ_PITCH;

  // dz of the lane's entries, staged token-major in LDS (see dz_stage); a wavefront whose 128
  // rows and WAVE_N tokens all exist (every one but the tail tiles') skips the range tests
  const bool full = __builtin_amdgcn_readfirstlane(vs0 + wv + WAVE_M <= V && tok0 + Cfg::WAVE_N <= T);
  if (full)
    dz_stage<Cfg, SCALED, EGRAD, true>(acc, grad, lse, labels, grad_entropy, entropy, temperature, T, V, vocab_start,
                                       vs0, wv, tok0, wl);
  else
    dz_stage<Cfg, SCALED, EGRAD, false>(acc, grad, lse, labels, grad_entropy, entropy, temperature, T, V,
                                        vocab_start, vs0, wv, tok0, wl);
  __syncthreads();
  // copy the wavefront's [WAVE_N tokens x 128 entries] block out, 16 bytes per lane
  constexpr int CHUNKS = Cfg::WAVE_N * (WAVE_M / 8);
#pragma unroll
  for (int i = 0; i < CHUNKS / 64; ++i) {
    const int q = lane + 64 * i;
    const int row = q / (WAVE_M / 8);
    const int c = q % (WAVE_M / 8);
    const int tok = tok0 + row;
    const u32x4 v = *reinterpret_cast<const u32x4*>(wl + row * DZ_PITCH + c * 16);
    if (tok < T) st_dz(dz + (int64_t)tok * Vs + wv + c * 8, v);
  }
  // dz^T: the same staged block read by transposing LDS reads.  A 16-lane group takes a job of
  // 16 entries x 8 tokens: lane 4 e + q of the group addresses token rows 8 tb + e and 8 tb + 4 + e
  // at entries 16 vb + 4 q .. + 3, and lane i receives entry 16 vb + i of the 8 tokens, one
  // 16-byte run of a dz^T row.  Tokens past T within a written run are zeros.
  {
    constexpr int TB = Cfg::WAVE_N / 8, JOBS = (WAVE_M / 16) * TB;
    const int jj = lane & 15;
    const uint32_t a0 = lds_addr(wl) + (jj >> 2) * DZ_PITCH + (jj & 3) * 8;
#pragma unroll
    for (int it = 0; it < JOBS / 4; ++it) {
      const int job = it * 4 + g4;
      const int vb = job / TB, tb = job % TB;
      const uint32_t a = a0 + 8 * tb * DZ_PITCH + 32 * vb;
      const s16x4 lo = ds_read_tr16(a);
      const s16x4 hi = ds_read_tr16(a + 4 * DZ_PITCH);
      const int tok = tok0 + 8 * tb;
      if (tok < T)
        st_dz(dzt + (int64_t)(wv + 16 * vb + jj) * ldt + tok,
              __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7)));
    }
  }
}

// ---------------------------------------------------------------------------------------------
// transposes: dst[c][r] = src[r][c] for r < R, 0 for R <= r < Rp; c < C (C % 8 == 0)
// ---------------------------------------------------------------------------------------------

constexpr int TR_TILE = 64;

__global__ __launch_bounds__(256) void transpose_pad_kernel(const __bf16* __restrict__ src, int64_t lds_, int R,
                                                            int C, __bf16* __restrict__ dst, int64_t ldd, int Rp) {
  __shared__ unsigned short tile[TR_TILE][TR_TILE + 2];
  const int r0 = blockIdx.x * TR_TILE;
  const int c0 = blockIdx.y * TR_TILE;
  const int tid = threadIdx.x;
  const unsigned short* s16 = reinterpret_cast<const unsigned short*>(src);
  // load: 64 rows x 8 chunks of 8 elements, 2 chunks per thread
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = tid + 256 * i;
    const int rr = q >> 3, cc = (q & 7) * 8;
    const int r = r0 + rr, c = c0 + cc;
    u32x4 v = (u32x4)(0u);
    if (r < R && c < C) v = *reinterpret_cast<const u32x4*>(s16 + (int64_t)r * lds_ + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[rr][cc + 2 * e] = (unsigned short)(v[e] & 0xffffu);
      tile[rr][cc + 2 * e + 1] = (unsigned short)(v[e] >> 16);
    }
  }
  __syncthreads();
  unsigned short* d16 = reinterpret_cast<unsigned short*>(dst);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = tid + 256 * i;
    const int cc = q >> 3, rr = (q & 7) * 8;
    const int c = c0 + cc, r = r0 + rr;
    if (c >= C || r >= Rp) continue;
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[e] = (unsigned)tile[rr + 2 * e][cc] | ((unsigned)tile[rr + 2 * e + 1][cc] << 16);
    *reinterpret_cast<u32x4*>(d16 + (int64_t)c * ldd + r) = v;
  }
}

static void launch_transpose(const __bf16* src, int64_t ld_src, int R, int C, __bf16* dst, int64_t ld_dst, int Rp,
                             hipStream_t stream) {
  dim3 grid((Rp + TR_TILE - 1) / TR_TILE, (C + TR_TILE - 1) / TR_TILE);
  hipLaunchKernelGGL(transpose_pad_kernel, grid, dim3(256), 0, stream, src, ld_src, R, C, dst, ld_dst, Rp);
}

// ---------------------------------------------------------------------------------------------
// K4 / K5: C[M x N] fp32 = (accumulate ? C : 0) + A[M x K] . B[N x K]^T, two problems per launch
// ---------------------------------------------------------------------------------------------

struct GemmProblem {
  const __bf16* A;
  int64_t lda;
  int M;
  const __bf16* B;
  int64_t ldb;
  int N;
  int K;
  float* C;
  int64_t ldc;
  int accumulate;
  int n_mt, n_nt;
};

// C element (row, col) of the wavefront's accumulator m, n, i: row = m0 + lane_row + 16 m + i,
// col = n0 + lane_col + 16 n.  The per-lane parts are hidden from the optimizer so that it keeps
// one offset per lane instead of hoisting 128 of them out of the persistent tile loop.
template <class Cfg>
__device__ __forceinline__ void c_lane_coords(int& lane_row, int& lane_col) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  lane_row = (wave % Cfg::WM) * WAVE_M + acc_row(0, lane);
  lane_col = (wave / Cfg::WM) * Cfg::WAVE_N + acc_col(lane);
  asm volatile("" : "+v"(lane_row), "+v"(lane_col));
}

// The accumulator starts at C when accumulating, so the MFMA chain continues across calls.
template <class Cfg>
__device__ __forceinline__ void gemm_acc_init(const GemmProblem& p, int m0, int n0, f32x4 (&acc)[MSUB][Cfg::NSUB]) {
  if (!p.accumulate) {
#pragma unroll
    for (int m = 0; m < MSUB; ++m)
#pragma unroll
      for (int n = 0; n < Cfg::NSUB; ++n) acc[m][n] = (f32x4)(0.0f);
    return;
  }
  int lane_row, lane_col;
  c_lane_coords<Cfg>(lane_row, lane_col);
  const float* c = p.C + (int64_t)m0 * p.ldc + n0;
  const int lo = lane_row * (int)p.ldc + lane_col;
  if (m0 + Cfg::TM <= p.M && n0 + Cfg::TN <= p.N) {
#pragma unroll
    for (int m = 0; m < MSUB; ++m)
#pragma unroll
      for (int n = 0; n < Cfg::NSUB; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[m][n][i] = c[lo + (m * MFMA_MN + i) * (int)p.ldc + n * MFMA_MN];
  } else {
#pragma unroll
    for (int m = 0; m < MSUB; ++m)
#pragma unroll
      for (int n = 0; n < Cfg::NSUB; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = m0 + lane_row + m * MFMA_MN + i < p.M && n0 + lane_col + n * MFMA_MN < p.N;
          acc[m][n][i] = ok ? c[lo + (m * MFMA_MN + i) * (int)p.ldc + n * MFMA_MN] : 0.f;
        }
  }
}

template <class Cfg>
__device__ __forceinline__ void gemm_acc_store(const GemmProblem& p, int m0, int n0,
                                               const f32x4 (&acc)[MSUB][Cfg::NSUB]) {
  int lane_row, lane_col;
  c_lane_coords<Cfg>(lane_row, lane_col);
  float* c = p.C + (int64_t)m0 * p.ldc + n0;
  const int lo = lane_row * (int)p.ldc + lane_col;
  if (m0 + Cfg::TM <= p.M && n0 + Cfg::TN <= p.N) {
#pragma unroll
    for (int m = 0; m < MSUB; ++m)
#pragma unroll
      for (int n = 0; n < Cfg::NSUB; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) c[lo + (m * MFMA_MN + i) * (int)p.ldc + n * MFMA_MN] = acc[m][n][i];
  } else {
#pragma unroll
    for (int m = 0; m < MSUB; ++m)
#pragma unroll
      for (int n = 0; n < Cfg::NSUB; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (m0 + lane_row + m * MFMA_MN + i < p.M && n0 + lane_col + n * MFMA_MN < p.N)
            c[lo + (m * MFMA_MN + i) * (int)p.ldc + n * MFMA_MN] = acc[m][n][i];
  }
}

// Tile grouping of the gradient GEMMs inside each XCD's range: groups of 4 m-tiles by all
// n-tiles ran the backward 0.5 % faster than groups of 8 (and 2, 3, 6 and 16 were slower); the
// dz launch keeps groups of 8, its fastest.
constexpr int GEMM_GROUP_M = 4;

// Persistent grid over both problems, one workgroup per CU, tiles from a TileQueue: problem 0's
// tiles are handed out first (the launcher puts the long-K problem there), so the short tiles
// fill the end.  As in the forward, the next tile's first loads are issued before the finished
// tile's results are stored, and the claim of the tile after next is read a tile later.
template <class Cfg>
__global__ __launch_bounds__(Cfg::NTHREADS) void gemm_tn_f32_persistent_kernel(GemmProblem p0, GemmProblem p1,
                                                                               int* __restrict__ sched) {
  loop_placement_pad<8>();
  __shared__ __attribute__((aligned(1024))) char lds[PingPong<Cfg>::LDS_BYTES];
  // tile numbers pass from thread 0 to the workgroup through the first word of B slot 1 (see the
  // forward's persistent kernel)
  int* const bc = reinterpret_cast<int*>(lds + PingPong<Cfg>::B_BASE + PingPong<Cfg>::SLOT);
  const int nt0 = p0.M > 0 ? p0.n_mt * p0.n_nt : 0;
  const int nt1 = p1.M > 0 ? p1.n_mt * p1.n_nt : 0;
  const TileQueue q{sched, nt0, nt1};
  const int xcd = blockIdx.x & 7;
  if (threadIdx.x == 0) bc[0] = q.resolve(xcd, q.claim(xcd));
  __syncthreads();
  int t = bc[0];
  if (t < 0) return;

  // tile t -> problem and origin
  auto locate = [&](int tile, bool& second, int& m0, int& n0) {
    second = tile >= nt0;
    const GemmProblem& p = second ? p1 : p0;
    int mt, nt;
    group_coords<GEMM_GROUP_M>(second ? tile - nt0 : tile, p.n_mt, p.n_nt, mt, nt);
    m0 = mt * Cfg::TM;
    n0 = nt * Cfg::TN;
  };
  auto start = [&](PingPong<Cfg>& pp, bool second, int m0, int n0) {
    const GemmProblem& p = second ? p1 : p0;
    pp.start(p.A + (int64_t)m0 * p.lda, p.lda, min(Cfg::TM, p.M - m0), p.B + (int64_t)n0 * p.ldb, p.ldb,
             min(Cfg::TN, p.N - n0), p.K);
  };

  PingPong<Cfg> pp(lds);
  bool second;
  int m0, n0;
  locate(t, second, m0, n0);
  start(pp, second, m0, n0);
  int claim = 0;
  if (threadIdx.x == 0) claim = q.claim(xcd);
  for (;;) {
    f32x4 acc[MSUB][Cfg::NSUB];
    gemm_acc_init<Cfg>(second ? p1 : p0, m0, n0, acc);
    // The accumulators are complete here (their loads waited for).  Without this the compiler
    // waits for them at their first MFMA inside the K loop, and those vmcnt waits, executed on
    // every step, also wait for the prefetching loads the step has just issued (5 % of the GEMM).
#pragma unroll
    for (int m = 0; m < MSUB; ++m)
#pragma unroll
      for (int n = 0; n < Cfg::NSUB; ++n) asm volatile("" : "+v"(acc[m][n]));
    pp.run(acc);
    if (threadIdx.x == 0) bc[0] = q.resolve(xcd, claim);
    __syncthreads();
    const int tn = bc[0];
    __builtin_amdgcn_sched_barrier(0);
    bool second_n = false;
    int m0n = 0, n0n = 0;
    if (tn >= 0) {
      locate(tn, second_n, m0n, n0n);
      start(pp, second_n, m0n, n0n);
      if (threadIdx.x == 0) claim = q.claim(xcd);
    }
    gemm_acc_store<Cfg>(second ? p1 : p0, m0, n0, acc);
    if (tn < 0) break;
    second = second_n;
    m0 = m0n;
    n0 = n0n;
  }
}

template <class Cfg>
static GemmProblem make_problem(const __bf16* A, int64_t lda, int M, const __bf16* B, int64_t ldb, int N, int K,
                                float* C, int64_t ldc, int accumulate) {
  GemmProblem p{A, lda, M, B, ldb, N, K, C, ldc, accumulate, (M + Cfg::TM - 1) / Cfg::TM, (N + Cfg::TN - 1) / Cfg::TN};
  return p;
}

// Launches one or two problems (M == 0: none) in a single persistent grid.
template <class Cfg>
static void launch_gemm_tn(const GemmProblem& p0, const GemmProblem& p1, int* sched, int cus, hipStream_t stream) {
  const int n0 = p0.M > 0 ? p0.n_mt * p0.n_nt : 0;
  const int n1 = p1.M > 0 ? p1.n_mt * p1.n_nt : 0;
  if (n0 + n1 == 0) return;
  hipLaunchKernelGGL(gemm_tn_f32_persistent_kernel<Cfg>, dim3(min(n0 + n1, cus)), dim3(Cfg::NTHREADS), 0, stream, p0,
                     p1, sched);
}

// ---------------------------------------------------------------------------------------------
// orchestration
// ---------------------------------------------------------------------------------------------

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

BwdLayout bwd_layout(int64_t T, int64_t H, int64_t V, int64_t step) {
  BwdLayout L{};
  L.T = (int)T;
  L.H = (int)H;
  L.V = (int)V;
  L.Tp = (int)((T + 63) / 64 * 64);
  const int64_t vr = (V + BWD_STEP_UNIT - 1) / BWD_STEP_UNIT * BWD_STEP_UNIT;
  L.Vs = (int)(vr < step ? vr : step);
  size_t off = 0;
  L.off_dz = off;
  off += align256((size_t)T * L.Vs * 2);
  L.off_dzt = off;
  off += align256((size_t)L.Vs * L.Tp * 2);
  L.off_wt = off;
  off += align256((size_t)H * L.Vs * 2);
  L.off_ht = off;
  off += align256((size_t)H * L.Tp * 2);
  L.nsteps = (int)((V + L.Vs - 1) / L.Vs);
  L.off_sched = off;
  off += align256((size_t)BWD_SCHED_WORDS * sizeof(int));
  L.total = off;
  return L;
}

// 256 x 256 tiles, 8 wavefronts (2 per SIMD), ping-pong main loop (160 KB of LDS)
using CfgDz = PipeCfg<2, 4, 4, 2, 64>;
using CfgGrad = PipeCfg<2, 4, 4, 2, 64>;

void launch_bwd(const BwdArgs& a, hipStream_t stream) {
  const BwdLayout& L = a.L;
  __bf16* dz = reinterpret_cast<__bf16*>(a.ws + L.off_dz);
  __bf16* dzt = reinterpret_cast<__bf16*>(a.ws + L.off_dzt);
  __bf16* wt = reinterpret_cast<__bf16*>(a.ws + L.off_wt);
  __bf16* ht = reinterpret_cast<__bf16*>(a.ws + L.off_ht);
  // tile counters of the gradient GEMM, zeroed by each step's dz launch
  int* gemm_sched = reinterpret_cast<int*>(a.ws + L.off_sched);
  if (!a.grad_hidden && !a.grad_weight) return;
  if (a.grad_weight) launch_transpose(a.hidden, L.H, L.T, L.H, ht, L.Tp, L.Tp, stream);

  for (int vs0 = 0; vs0 < L.V; vs0 += L.Vs) {
    const int Vc = L.V - vs0 < L.Vs ? L.V - vs0 : L.Vs;
    {
      const int n_mt = (Vc + CfgDz::TM - 1) / CfgDz::TM;
      const int n_nt = (L.T + CfgDz::TN - 1) / CfgDz::TN;
      const bool scaled = a.temperature != 1.0f, egrad = a.grad_entropy != nullptr;
      auto kern = scaled ? (egrad ? bwd_dz_kernel<CfgDz, true, true> : bwd_dz_kernel<CfgDz, true, false>)
                         : (egrad ? bwd_dz_kernel<CfgDz, false, true> : bwd_dz_kernel<CfgDz, false, false>);
      hipLaunchKernelGGL(kern, dim3(n_mt * n_nt), dim3(CfgDz::NTHREADS), 0, stream, a.hidden, a.weight, a.labels,
                         a.grad, a.lse, a.grad_entropy, a.entropy, a.temperature, L.T, L.H, L.V, a.vocab_start, vs0,
                         Vc, L.Vs, n_mt, n_nt, dz, dzt, L.Tp, gemm_sched);
    }
    // dz^T rows hold tokens up to T rounded up to 8 (zeros past T); the gradient GEMM reads no
    // 16-byte chunk that starts at or past T
    GemmProblem pw{}, ph{};
    if (a.grad_weight) {
      pw = make_problem<CfgGrad>(dzt, L.Tp, Vc, ht, L.Tp, L.H, L.T, a.grad_weight + (int64_t)vs0 * L.H, L.H,
                                 a.accumulate_gw);
    }
    if (a.grad_hidden) {
      launch_transpose(a.weight + (int64_t)vs0 * L.H, L.H, Vc, L.H, wt, L.Vs, (Vc + 63) / 64 * 64, stream);
      ph = make_problem<CfgGrad>(dz, L.Vs, L.T, wt, L.Vs, L.H, Vc, a.grad_hidden, L.H, vs0 > 0 ? 1 : 0);
    }
    // grad_hidden first: its tiles run K = Vs (four times the grad_weight tiles' K = T at the
    // benchmark sizes), and dispatching the long tiles first lets the short ones fill the tail
    launch_gemm_tn<CfgGrad>(ph, pw, gemm_sched, a.cus, stream);
  }
}

}  // namespace lmh
