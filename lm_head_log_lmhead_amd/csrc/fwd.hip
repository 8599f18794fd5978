// fwd.hip — forward kernels of the fused LM-head log-prob.
//
// K1 fwd_partials: the logit tile z = W_tile . h_tile^T (vocabulary on the MFMA M axis, tokens on
//    the N axis, so each lane holds 32 vocabulary entries of one token and the per-token softmax
//    reduction is mostly in-lane).  Its epilogue reduces every (token, 128-entry vocabulary
//    chunk) to one record {m, n, b, u}:
//        m = max z,  n = #{z == m},  b = sum_{z < m} exp(z - m),  u = sum exp(z - m) (z - m)
//    (and, when asked, q = sum exp(2 (z - m))) and stores the label's logit when the label falls
//    in the chunk.  Logits never leave the registers.  (SkyRL PR #1765 "[megatron] Triton backend
//    for fused LM-head log-prob": the vocab-tiled online softmax that never materializes per-chunk
//    logits, and the -inf masking of out-of-bounds vocabulary columns in the tail tile.)
//    With a temperature, every logit is first divided by it in fp32 (verl PR #8026
//    "batch-invariant actor forward and sampler log-prob formula", review on the temperature
//    order: fp32 logits divided by the fp32 temperature inside the chunk).
// K2 fwd_finalize: folds each row's records in a fixed order (64 fixed segments of consecutive
//    chunks, each folded in ascending order, then the 64 segment states merged in a fixed binary
//    tree — a function of V only) and writes logprob = (z_y - M) - log S, entropy = log S - U/S, lse = M + log S,
//    with log S = log N + log1p(B/N), and sum_p2 = Q / S^2.  (verl PR #8026, first review: fp32
//    log_softmax over the full vocabulary then gather, with entropy and sum_pi_squared of the same
//    softmax; SkyRL PR #1765, precision-policy commit: logprob 0 for an out-of-vocabulary label.)
#include <stdlib.h>

#include "kernels.hpp"

// Build-time tuning knobs (all choices give the same bits: the per-wavefront vocabulary extent
// and the MFMA chain are fixed).
// large-T tile: 256 x 256, 8 wavefronts, ping-pong main loop; XCD tile grouping
#ifndef LMH_GROUP_M
#define LMH_GROUP_M 4
#endif
// small-T tiles (T <= 32 and 32 < T <= 64): wavefront grid (WM, WN, NSUB), stages and K step of
// the spread main loop
#ifndef LMH_SMALL_NS
#define LMH_SMALL_NS 3
#endif
#ifndef LMH_SMALL_BK
#define LMH_SMALL_BK 128
#endif
#ifndef LMH_S64_NS
#define LMH_S64_NS 3
#endif
#ifndef LMH_S64_BK
#define LMH_S64_BK 128
#endif
#ifndef LMH_SMALL_SHAPE
#define LMH_SMALL_SHAPE 1, 2, 1
#endif
#ifndef LMH_S64_SHAPE
#define LMH_S64_SHAPE 1, 4, 1
#endif
// persistent large-T tile: tiles before the end of an XCD's range below which the next tile is
// claimed only when the current one finishes
#ifndef LMH_CLAIM_DEFER
#define LMH_CLAIM_DEFER 128
#endif
// mid-T tile (64 < T <= LMH_MID_MAX)
#ifndef LMH_MID_MAX
#define LMH_MID_MAX 128
#endif
#ifndef LMH_MID_SHAPE
#define LMH_MID_SHAPE 2, 2, 4
#endif
#ifndef LMH_MID_NS
#define LMH_MID_NS 3
#endif

namespace lmh {

// ---------------------------------------------------------------------------------------------
// K1: logit tiles + per-chunk records
// ---------------------------------------------------------------------------------------------

// Logits at vocabulary index >= V (tail tile only) are replaced by this sentinel: it is far
// below every real logit, so it never reaches the max, and exp2 of its shift underflows to 0, so
// it adds exactly zero to every sum (0 * d is -0 for finite d).
constexpr float MASKED_LOGIT = -1.0e30f;
constexpr float LN2 = 0.6931471805599453f;  // converts the shift sum from log2 units

// Options of the record epilogue, fixed per kernel instantiation.
template <bool SCALED_, bool P2_>
struct RecOpt {
  static constexpr bool SCALED = SCALED_;  // divide every logit by the temperature
  static constexpr bool P2 = P2_;          // also record q = sum exp(2 (z - m))
};

// Lane l holds, for each of its NSUB tokens (column l % 16 of an MFMA block), the 32 entries at
// wavefront rows 16 m + 4 (l / 16) + i; lanes l, l^16, l^32, l^48 together hold the token's 128.
// lw[n] is the label's offset from wave_v0 for token n * 16 + l % 16 (any value outside [0, 128)
// when the label is not in this chunk, out of vocabulary, or the token is past T).
template <int NSUB, bool TAIL, class Opt>
__device__ __forceinline__ void fwd_records(f32x4 (&acc)[MSUB][NSUB], int lane, int wave_v0, int tok0, int V,
                                            const int (&lw)[NSUB], const FwdArgs& a, int chunk) {
  const int j = acc_col(lane);
  const int g = lane >> 4;
  if (Opt::SCALED) {
    const float tau = a.temperature;
#pragma unroll
    for (int m = 0; m < MSUB; ++m)
#pragma unroll
      for (int n = 0; n < NSUB; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[m][n][i] = acc[m][n][i] / tau;
  }
  if (TAIL) {
#pragma unroll
    for (int m = 0; m < MSUB; ++m)
#pragma unroll
      for (int n = 0; n < NSUB; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (wave_v0 + m * MFMA_MN + acc_row(i, lane) >= V) acc[m][n][i] = MASKED_LOGIT;
  }
#pragma unroll
  for (int n = 0; n < NSUB; ++n) {
    const int tok = tok0 + n * MFMA_MN + j;
    const bool tok_ok = tok < a.T;

    // pass 1: chunk max over this lane's 32 entries, then across the four lanes of the token
    float mx = acc[0][n][0];
#pragma unroll
    for (int m = 0; m < MSUB; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, acc[m][n][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));

    // pass 2: count at the max, sum of exp below it, sum of exp * shift (fixed order: m, then i)
    int cnt = 0;
    float b = 0.f, u = 0.f, q = 0.f;
    // The exponent is formed as z log2(e) - m log2(e) with one fused multiply-add, and the shift is
    // summed in the same log2 units and converted once per chunk; entries equal to the max are
    // taken out of b, u (and counted in n) by the comparison z == m itself, so their rounding
    // residual in the fused shift never reaches the sums.
    const float mxl = mx * LOG2E;
#pragma unroll
    for (int m = 0; m < MSUB; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float z = acc[m][n][i];
        const float d2 = __builtin_fmaf(z, LOG2E, -mxl);
        const bool at_max = z == mx;
        const float e = at_max ? 0.f : __builtin_amdgcn_exp2f(d2);
        cnt += at_max;
        b += e;
        u = __builtin_fmaf(e, d2, u);
        if (Opt::P2) q = at_max ? q + 1.f : __builtin_fmaf(e, e, q);
      }
    u = u * LN2;

    // the four lanes' partial sums as (s0 + s1) + (s2 + s3): by commutativity of each addition,
    // every lane of the token ends with the same bits
    cnt += __shfl_xor(cnt, 16);
    b += __shfl_xor(b, 16);
    u += __shfl_xor(u, 16);
    cnt += __shfl_xor(cnt, 32);
    b += __shfl_xor(b, 32);
    u += __shfl_xor(u, 32);
    if (Opt::P2) {
      q += __shfl_xor(q, 16);
      q += __shfl_xor(q, 32);
    }

    // label logit: local index w sits in block w / 16, lane group (w % 16) / 4, register w % 4.
    // Few chunks hold a label, so the select runs behind a wavefront-uniform branch.
    const int w = lw[n];
    const bool mine = (unsigned)w < (unsigned)WAVE_M && ((w >> 2) & 3) == g;
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(mine) != 0, 0)) {
      const int idx = ((w >> 4) << 2) | (w & 3);
      float val = 0.f;
#pragma unroll
      for (int m = 0; m < MSUB; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) val = (idx == m * 4 + i) ? acc[m][n][i] : val;
      if (mine) a.zy[tok] = val;
    }
    if (g == 0 && tok_ok) {
      f32x4 v;
      v[0] = mx;
      // a chunk of NaN logits (max NaN, no entry equal to it) is counted once, so that the fold,
      // which skips records of count 0, carries its NaN into the row's outputs
      v[1] = mx == mx ? (float)cnt : 1.f;
      v[2] = b;
      v[3] = u;
      const size_t at = (size_t)chunk * (size_t)a.T + tok;
      a.rec[at] = v;
      if (Opt::P2) a.rec2[at] = q;
    }
  }
}

// The wavefront's labels as offsets from its first vocabulary row (see fwd_records); a label
// outside this call's rows [vocab_start, vocab_start + V) is not in any of its chunks.
template <int NSUB>
__device__ __forceinline__ void label_offsets(const int (&y)[NSUB], int wave_v0, const FwdArgs& a, int (&lw)[NSUB]) {
#pragma unroll
  for (int n = 0; n < NSUB; ++n) {
    // vocab_start + V <= vocab_total < 2^31, so neither difference overflows
    const bool in_rows = y[n] >= a.vocab_start && y[n] - a.vocab_start < a.V;
    lw[n] = in_rows ? y[n] - a.vocab_start - wave_v0 : -1;
  }
}

template <int NSUB>
__device__ __forceinline__ void load_labels(const int* __restrict__ labels, int tok0, int lane, int T, int (&y)[NSUB]) {
#pragma unroll
  for (int n = 0; n < NSUB; ++n) {
    const int tok = tok0 + n * MFMA_MN + acc_col(lane);
    y[n] = tok < T ? labels[tok] : -1;
  }
}

// Records of the wavefront's chunk of the tile at (v0, t0) (local weight rows); lw from
// label_offsets.
template <class Cfg, class Opt>
__device__ __forceinline__ void tile_records(f32x4 (&acc)[MSUB][Cfg::NSUB], int v0, int t0, const int (&lw)[Cfg::NSUB],
                                             const FwdArgs& a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave % Cfg::WM, wn = wave / Cfg::WM;
  const int wave_v0 = v0 + wm * WAVE_M;
  if (wave_v0 >= a.V) return;  // this wavefront's chunk lies wholly past the weight rows
  const int tok0 = t0 + wn * Cfg::WAVE_N;
  const int chunk = (a.vocab_start + wave_v0) / WAVE_M;
  // the chunk's first token tile marks whether its squared-sum records exist
  if (t0 == 0 && wn == 0 && lane == 0) a.p2ok[chunk] = Opt::P2 ? 1 : 0;
  if (wave_v0 + WAVE_M <= a.V)
    fwd_records<Cfg::NSUB, false, Opt>(acc, lane, wave_v0, tok0, a.V, lw, a, chunk);
  else
    fwd_records<Cfg::NSUB, true, Opt>(acc, lane, wave_v0, tok0, a.V, lw, a, chunk);
}

template <class Cfg, class Opt>
__global__ __launch_bounds__(Cfg::NTHREADS) void fwd_partials_kernel(FwdArgs a, int n_mt, int n_nt) {
  __shared__ __attribute__((aligned(1024))) char lds[Cfg::LDS_BYTES];
  int mt, nt;
  tile_coords<LMH_GROUP_M>(blockIdx.x, gridDim.x, n_mt, n_nt, mt, nt);
  const int v0 = mt * Cfg::TM;
  const int t0 = nt * Cfg::TN;
  f32x4 acc[MSUB][Cfg::NSUB];
#pragma unroll
  for (int m = 0; m < MSUB; ++m)
#pragma unroll
    for (int n = 0; n < Cfg::NSUB; ++n) acc[m][n] = (f32x4)(0.0f);
  const __bf16* A = a.weight + (int64_t)v0 * a.H;
  const __bf16* B = a.hidden + (int64_t)t0 * a.H;
  const int rowsA = min(Cfg::TM, a.V - v0), rowsB = min(Cfg::TN, a.T - t0);
  static_assert(Cfg::LOOP == LOOP_SPREAD, "one-tile-per-workgroup grid: spread main loop");
  tile_mainloop_spread<Cfg>(A, a.H, rowsA, B, a.H, rowsB, a.H, lds, acc);
  const int wave = threadIdx.x >> 6;
  int y[Cfg::NSUB], lw[Cfg::NSUB];
  load_labels(a.labels, t0 + (wave / Cfg::WM) * Cfg::WAVE_N, threadIdx.x & 63, a.T, y);
  label_offsets(y, v0 + (wave % Cfg::WM) * WAVE_M, a, lw);
  tile_records<Cfg, Opt>(acc, v0, t0, lw, a);
}

// Persistent form for the ping-pong tile: one workgroup per CU.
//
// Tiles are handed out by a TileQueue over per-XCD counters in the workspace.  A workgroup on XCD
// x takes the next tile of x's contiguous tile range (so the workgroups of an XCD work on
// neighbouring tiles together, sharing A and B rows in that XCD's L2); once x's range is used up
// it takes tiles from the other XCDs' ranges.  XCDs do not run at the same speed, and a static
// split leaves the fastest idle at the end.  The counters decide only which workgroup computes a
// tile, never what it computes: every tile's records are the same bits whoever computes them.
//
// The claim of the tile after next is issued during the current tile's epilogue and read after
// the next tile's K loop, so its latency hides behind that loop.  The next tile's first loads are
// issued before the finished tile's records are computed, so their latency hides behind that VALU
// work, and no workgroup launch separates the tiles.

__global__ void fwd_sched_reset_kernel(int* __restrict__ sched) {
  if (threadIdx.x < SCHED_WORDS) sched[threadIdx.x] = 0;
}

template <class Cfg, class Opt>
__global__ __launch_bounds__(Cfg::NTHREADS) void fwd_partials_persistent_kernel(FwdArgs a, int n_mt, int n_nt) {
  loop_placement_pad<2 * Opt::SCALED + Opt::P2>();
  __shared__ __attribute__((aligned(1024))) char lds[Cfg::LDS_BYTES];
  // Tile numbers are passed from thread 0 to the workgroup through the first word of B slot 1,
  // which no load writes between the end of one K loop and the first barrier of the next.
  int* const bc = reinterpret_cast<int*>(lds + PingPong<Cfg>::B_BASE + PingPong<Cfg>::SLOT);
  const TileQueue q{a.sched, n_mt * n_nt, 0};
  const int xcd = blockIdx.x & 7;
  const int wm = (threadIdx.x >> 6) % Cfg::WM;
  const int wn = (threadIdx.x >> 6) / Cfg::WM;
  const int lane = threadIdx.x & 63;
  const int H = a.H;

  if (threadIdx.x == 0) bc[0] = q.resolve(xcd, q.claim(xcd));
  __syncthreads();
  int L = bc[0];
  if (L < 0) return;

  PingPong<Cfg> pp(lds);
  int mt, nt;
  group_coords<LMH_GROUP_M>(L, n_mt, n_nt, mt, nt);
  int v0 = mt * Cfg::TM, t0 = nt * Cfg::TN;
  pp.start(a.weight + (int64_t)v0 * H, H, min(Cfg::TM, a.V - v0), a.hidden + (int64_t)t0 * H, H,
           min(Cfg::TN, a.T - t0), H);
  // Thread 0: raw counter value of the next tile's claim on this XCD's range, or -1 when it has
  // not been taken yet.  A claim is taken a tile ahead while the XCD's range still has more than
  // LMH_CLAIM_DEFER tiles past the current one; nearer the end it is taken only when the tile
  // finishes, so the last tiles go to the workgroups that are free first.
  int own_start, own_count;
  xcd_range(xcd, n_mt * n_nt, own_start, own_count);
  int claim = 0;
  if (threadIdx.x == 0) claim = q.claim(xcd);
  for (;;) {
    int y[Cfg::NSUB];
    load_labels(a.labels, t0 + wn * Cfg::WAVE_N, lane, a.T, y);
    f32x4 acc[MSUB][Cfg::NSUB];
#pragma unroll
    for (int m = 0; m < MSUB; ++m)
#pragma unroll
      for (int n = 0; n < Cfg::NSUB; ++n) acc[m][n] = (f32x4)(0.0f);
    pp.run(acc);
    // The labels are consumed here, before the next tile's loads go out: the compiler's wait for
    // them then covers nothing else.  The empty asm pins the offsets here; left free, the compiler
    // sank them below the next tile's loads, and its wait for the labels then also waited for
    // those loads before the records could start.
    int lw[Cfg::NSUB];
    label_offsets(y, v0 + wm * WAVE_M, a, lw);
#pragma unroll
    for (int n = 0; n < Cfg::NSUB; ++n) asm volatile("" : "+v"(lw[n]));
    if (threadIdx.x == 0) {
      if (claim < 0) claim = q.claim(xcd);   // a deferred claim: its latency is exposed here
      bc[0] = q.resolve(xcd, claim);
    }
    __syncthreads();
    const int Ln = bc[0];
    __builtin_amdgcn_sched_barrier(0);
    int v0n = 0, t0n = 0;
    if (Ln >= 0) {
      group_coords<LMH_GROUP_M>(Ln, n_mt, n_nt, mt, nt);
      v0n = mt * Cfg::TM;
      t0n = nt * Cfg::TN;
      pp.start(a.weight + (int64_t)v0n * H, H, min(Cfg::TM, a.V - v0n), a.hidden + (int64_t)t0n * H, H,
               min(Cfg::TN, a.T - t0n), H);
      if (threadIdx.x == 0) claim = claim + LMH_CLAIM_DEFER < own_count ? q.claim(xcd) : -1;
    }
    tile_records<Cfg, Opt>(acc, v0, t0, lw, a);
    if (Ln < 0) break;
    L = Ln;
    v0 = v0n;
    t0 = t0n;
  }
}

// K-split form for launches of few tile rounds (one workgroup per CU).
//
// With few tiles per CU the dynamic queue leaves a partly empty last round: at T = 256 and
// V = 152064, 594 tiles on 256 CUs are 2.32 rounds, and a third of the CUs run a third tile while
// the rest idle.  Here the K steps of all tiles, in tile order, are cut into one contiguous range
// per workgroup of equal length, so every workgroup has the same number of steps.  A range starts
// inside a tile (its "tail": steps kb .. S-1), covers whole tiles, and ends inside another (its
// "head": steps 0 .. ke-1), whose tail is the next workgroup's first part.  A workgroup computes
// its head first and hands the accumulators to the next workgroup through the workspace; it
// computes its own tail last, continuing the accumulators the previous workgroup handed over.
// The chain of every output element is the same as in one piece: the same MFMAs over the same
// k slices in ascending order, the fp32 accumulators stored and loaded exactly in between.
//
// Workgroup numbers come from a counter taken at start, so the workgroup a tail waits for took
// its number earlier and is running; it computes its head before anything else, so every wait
// ends.  The hand-over uses coherent (sc1) stores and loads, which the XCDs' separate L2 caches
// serve consistently: the writer's stores complete before it sets the flag, and the reader loads
// the accumulators only after it has seen the flag.  The counter and flags are zeroed, and the
// ranges written, by fwd_sk_reset_kernel before the launch.

// Zeroes the counter and the flags of G workgroups and writes each workgroup's range of the U K
// steps (S per tile): [U g / G, U (g + 1) / G) as {tail tile, tail's first step, head tile, head's
// end step}.
__global__ void fwd_sk_reset_kernel(int* __restrict__ sync, int G, int64_t U, int S) {
  for (int i = threadIdx.x; i <= G; i += blockDim.x) sync[i] = 0;
  for (int g = threadIdx.x; g < G; g += blockDim.x) {
    const int64_t b = U * g / G, e = U * (g + 1) / G;
    int4 r;
    r.x = (int)(b / S);
    r.y = (int)(b % S);
    r.z = (int)(e / S);
    r.w = (int)(e % S);
    reinterpret_cast<int4*>(sync + SK_BOUNDS_WORD)[g] = r;
  }
}

struct SkPiece {
  int L, k0, k1;  // tile and its K steps [k0, k1)
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t sk_slot(const FwdArgs& a, int g) {
  return __builtin_amdgcn_make_buffer_rsrc(a.sk_acc + (size_t)g * (SK_SLOT_BYTES / 16), 0, (int)SK_SLOT_BYTES,
                                          0x00020000);
}
constexpr int SC1 = 16;  // cache policy of the hand-over: coherent across the XCDs

template <class Cfg, class Opt>
__global__ __launch_bounds__(Cfg::NTHREADS) void fwd_partials_sk_kernel(FwdArgs a, int n_mt, int n_nt, int spin_limit) {
  loop_placement_pad<9 + 2 * Opt::SCALED + Opt::P2>();
  __shared__ __attribute__((aligned(1024))) char lds[Cfg::LDS_BYTES];
  int* const bc = reinterpret_cast<int*>(lds + PingPong<Cfg>::B_BASE + PingPong<Cfg>::SLOT);
  const int tid = threadIdx.x;
  const int wm = (tid >> 6) % Cfg::WM;
  const int wn = (tid >> 6) / Cfg::WM;
  const int lane = tid & 63;
  const int H = a.H;
  const int S = (H + Cfg::BK - 1) / Cfg::BK;  // K steps of a tile

  if (tid == 0) bc[0] = atomicAdd(a.sk_sync, 1);
  __syncthreads();
  const int g = bc[0];
  // This workgroup's steps (e - b >= S of them): a tail of tile tb from step kb (if kb > 0), whole
  // tiles, a head of tile te up to step ke (if ke > 0), as written by fwd_sk_reset_kernel.
  const int4 rb = reinterpret_cast<const int4*>(a.sk_sync + SK_BOUNDS_WORD)[g];
  const int tb = __builtin_amdgcn_readfirstlane(rb.x), kb = __builtin_amdgcn_readfirstlane(rb.y);
  const int te = __builtin_amdgcn_readfirstlane(rb.z), ke = __builtin_amdgcn_readfirstlane(rb.w);
  const int np = (ke > 0) + (te - tb - (kb > 0)) + (kb > 0);
  // piece i in order: the head (the next workgroup waits for it), whole tiles, the tail
  auto piece = [&](int i) -> SkPiece {
    const int first_full = tb + (kb > 0);
    if (ke > 0) {
      if (i == 0) return SkPiece{te, 0, ke};
      --i;
    }
    if (i < te - first_full) return SkPiece{first_full + i, 0, S};
    return SkPiece{tb, kb, S};
  };

  PingPong<Cfg, true> pp(lds);
  int v0 = 0, t0 = 0;
  auto start = [&](const SkPiece& p, int& pv0, int& pt0) {
    int mt, nt;
    group_coords<LMH_GROUP_M>(p.L, n_mt, n_nt, mt, nt);
    pv0 = mt * Cfg::TM;
    pt0 = nt * Cfg::TN;
    const int kofs = p.k0 * Cfg::BK;
    pp.start(a.weight + (int64_t)pv0 * H + kofs, H, min(Cfg::TM, a.V - pv0), a.hidden + (int64_t)pt0 * H + kofs, H,
             min(Cfg::TN, a.T - pt0), min(H - kofs, (p.k1 - p.k0) * Cfg::BK));
  };
  SkPiece cur = piece(0);
  start(cur, v0, t0);
  bool flag_due = false;  // the head's accumulator stores are out; its flag goes up after the next K loop
  for (int i = 0;; ++i) {
    int y[Cfg::NSUB];
    load_labels(a.labels, t0 + wn * Cfg::WAVE_N, lane, a.T, y);
    f32x4 acc[MSUB][Cfg::NSUB];
    if (cur.k0 > 0) {
      // a tail: continue the accumulators of the previous workgroup's head
      if (tid == 0) {
        const int* flag = a.sk_sync + g;   // flag of workgroup g - 1
        int seen = 0;
        for (int spin = 0; spin < spin_limit; ++spin) {
          if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
            seen = 1;
            break;
          }
          __builtin_amdgcn_s_sleep(4);
        }
        bc[1] = seen;  // B slot 1, which this piece's first loads leave free
      }
      __syncthreads();
      const bool handed = __builtin_amdgcn_readfirstlane(bc[1]) != 0;
      const __amdgpu_buffer_rsrc_t slot = sk_slot(a, g - 1);
      // one offset register (the accumulator index goes in soffset), computed here from an opaque
      // thread index so the compiler does not keep it live across the K loops
      int voff = threadIdx.x;
      asm volatile("" : "+v"(voff));
      voff *= 16;
#pragma unroll
      for (int m = 0; m < MSUB; ++m)
#pragma unroll
        for (int n = 0; n < Cfg::NSUB; ++n)
          acc[m][n] = __builtin_amdgcn_raw_buffer_load_b128(slot, voff, (m * Cfg::NSUB + n) * Cfg::NTHREADS * 16, SC1);
      // wait for the accumulators here rather than at their first MFMA inside the K loop
#pragma unroll
      for (int m = 0; m < MSUB; ++m)
#pragma unroll
        for (int n = 0; n < Cfg::NSUB; ++n) asm volatile("" : "+v"(acc[m][n]));
      if (!handed) {
        // the wait ran out: poison the tile so its records, and the rows' outputs, are NaN
#pragma unroll
        for (int m = 0; m < MSUB; ++m)
#pragma unroll
          for (int n = 0; n < Cfg::NSUB; ++n) acc[m][n] = (f32x4)(__builtin_nanf(""));
      }
    } else {
#pragma unroll
      for (int m = 0; m < MSUB; ++m)
#pragma unroll
        for (int n = 0; n < Cfg::NSUB; ++n) acc[m][n] = (f32x4)(0.0f);
    }
    pp.run(acc);
    // run() returns after every wavefront has waited for all its memory operations (vmcnt 0) and
    // passed the loop's last barrier, so the head's accumulator stores issued before it are done
    if (flag_due && tid == 0) __hip_atomic_store(a.sk_sync + 1 + g, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    flag_due = false;
    const bool last = i + 1 == np;
    if (cur.k1 < S) {
      // a head: hand the accumulators to the next workgroup (a head is never the last piece)
      const __amdgpu_buffer_rsrc_t slot = sk_slot(a, g);
      int voff = threadIdx.x;
      asm volatile("" : "+v"(voff));
      voff *= 16;
#pragma unroll
      for (int m = 0; m < MSUB; ++m)
#pragma unroll
        for (int n = 0; n < Cfg::NSUB; ++n)
          __builtin_amdgcn_raw_buffer_store_b128(acc[m][n], slot, voff, (m * Cfg::NSUB + n) * Cfg::NTHREADS * 16, SC1);
      cur = piece(i + 1);
      if (cur.k0 > 0) {
        // the next piece is this workgroup's tail, which may wait for the previous workgroup: raise
        // the flag now, so no chain of waits forms
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0) __hip_atomic_store(a.sk_sync + 1 + g, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        flag_due = true;
      }
      start(cur, v0, t0);
      continue;
    }
    int lw[Cfg::NSUB];
    label_offsets(y, v0 + wm * WAVE_M, a, lw);
#pragma unroll
    for (int n = 0; n < Cfg::NSUB; ++n) asm volatile("" : "+v"(lw[n]));
    __builtin_amdgcn_sched_barrier(0);
    // the next piece's first loads go out before this tile's records are computed (run() returns
    // with every slot free in every wavefront)
    SkPiece nxt = cur;
    int v0n = v0, t0n = t0;
    if (!last) {
      nxt = piece(i + 1);
      start(nxt, v0n, t0n);
    }
    tile_records<Cfg, Opt>(acc, v0, t0, lw, a);
    if (last) break;
    cur = nxt;
    v0 = v0n;
    t0 = t0n;
  }
}

// ---------------------------------------------------------------------------------------------
// K2: fixed-order fold of the records and the final outputs
// ---------------------------------------------------------------------------------------------

struct Rec {
  float m, n, b, u, q;
};

// Merge record r into state s (both relative to their own max).  Empty records (n == 0) are the
// identity.  The three cases keep b, u and q relative to the larger max, so nothing below the
// max is ever added to the count n.  With P2 false, q is carried as 0 and not computed.
template <bool P2>
__device__ __forceinline__ Rec fold(Rec s, Rec r) {
  if (r.n == 0.f) return s;
  if (s.n == 0.f) return r;
  if (r.m > s.m) {
    const float dm = s.m - r.m;
    const float a = __builtin_amdgcn_exp2f(dm * LOG2E);
    const float sn = s.b + s.n;
    Rec o;
    o.m = r.m;
    o.n = r.n;
    o.b = __builtin_fmaf(sn, a, r.b);
    o.u = __builtin_fmaf(__builtin_fmaf(dm, sn, s.u), a, r.u);
    o.q = P2 ? __builtin_fmaf(s.q, a * a, r.q) : 0.f;
    return o;
  }
  if (r.m == s.m) {
    s.n += r.n;
    s.b += r.b;
    s.u += r.u;
    if (P2) s.q += r.q;
    return s;
  }
  const float dm = r.m - s.m;
  const float a = __builtin_amdgcn_exp2f(dm * LOG2E);
  const float rn = r.b + r.n;
  s.b = __builtin_fmaf(rn, a, s.b);
  s.u = __builtin_fmaf(__builtin_fmaf(dm, rn, r.u), a, s.u);
  if (P2) s.q = __builtin_fmaf(r.q, a * a, s.q);
  return s;
}

// Outputs of row t from its folded state: log S = log N + log1p(B / N) keeps tiny entropies
// relatively exact; the log-prob is (z_y - M) - log S, 0 for a label outside the vocabulary.
template <bool P2>
__device__ __forceinline__ void finalize_row(const FwdArgs& a, int t, const Rec& st) {
  const float logS = logf(st.n) + log1pf(st.b / st.n);
  const int y = a.labels[t];
  const bool in_vocab = y >= 0 && y < a.vocab_total;
  a.logprob[t] = in_vocab ? (a.zy[t] - st.m) - logS : 0.f;
  if (a.entropy) a.entropy[t] = logS - st.u / (st.n + st.b);
  if (a.lse) a.lse[t] = st.m + logS;
  if (P2) {
    const float S = st.n + st.b;
    a.sum_p2[t] = st.q / (S * S);
  }
}

constexpr int FIN_NSEG = 64;  // fixed number of fold segments per row

// A workgroup of FW wavefronts folds a block of TPW tokens at a time ((TPW, FW) = (8, 8), (16, 16)
// or (32, 16)).  Lane l of a wavefront serves token l % TPW and segment slot l / TPW, so a
// wavefront covers 64 / TPW segments of each of its tokens per pass and the FW wavefronts cover
// all 64 segments in 64 / (FW * 64 / TPW) passes (one, or two for (32, 16)).  The block size grows
// with T so that the blocks cover the CUs (256 of them at T = 2048, 4096 and 8192) while a
// segment's loads stay whole 128-byte lines.  Each segment is folded in ascending chunk order, its
// records loaded in batches (one batch covers a segment of up to 20 chunks with one pass, i.e. V
// up to 163840); then the 64 segment states of a token are merged in a fixed binary tree inside one
// wavefront (lane s holds segment s; at level d = 1, 2, 4, ..., 32 lane s with s % 2d == 0 merges
// the state of lane s + d into its own), six dependent merges instead of a chain of 64.  Neither
// the spread of segments over lanes nor the batching changes any value; the order is a function
// of V only.
// Segment states of a row block in LDS, one array per field with rows padded to TPW + 1 words:
// the stores (consecutive lanes, consecutive tokens) and the tree's loads (consecutive lanes,
// consecutive segments of one token, TPW + 1 words apart) hit 64 different banks.
template <int TPW>
struct SegStates {
  float m[FIN_NSEG][TPW + 1], n[FIN_NSEG][TPW + 1], b[FIN_NSEG][TPW + 1], u[FIN_NSEG][TPW + 1],
      q[FIN_NSEG][TPW + 1];
  __device__ __forceinline__ void put(int sg, int t, const Rec& r, bool p2) {
    m[sg][t] = r.m;
    n[sg][t] = r.n;
    b[sg][t] = r.b;
    u[sg][t] = r.u;
    if (p2) q[sg][t] = r.q;
  }
  __device__ __forceinline__ Rec get(int sg, int t, bool p2) const {
    return Rec{m[sg][t], n[sg][t], b[sg][t], u[sg][t], p2 ? q[sg][t] : 0.f};
  }
};

template <bool P2, int TPW, int FW>
__device__ __forceinline__ void fold_row_block(const FwdArgs& a, int n_c, int blk, SegStates<TPW>& part) {
  static_assert(FIN_NSEG == 64, "one segment state per lane in the tree");
  constexpr int LPT = 64 / TPW;                      // segment slots per wavefront and pass
  constexpr int PASSES = FIN_NSEG / (FW * LPT);
  static_assert(PASSES >= 1 && PASSES * FW * LPT == FIN_NSEG, "segment slots");
  constexpr int BATCH = 20 / PASSES;                 // records per segment loaded before folding
  const int T = a.T;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int tl = lane % TPW;
  const int t = blk * TPW + tl;
  const bool t_ok = t < T;
  int sg[PASSES], lo[PASSES], len[PASSES];
  Rec seg[PASSES];
  int maxlen = 0;
#pragma unroll
  for (int j = 0; j < PASSES; ++j) {
    sg[j] = (j * FW + w) * LPT + lane / TPW;
    lo[j] = (int)((int64_t)sg[j] * n_c / FIN_NSEG);
    len[j] = (int)((int64_t)(sg[j] + 1) * n_c / FIN_NSEG) - lo[j];
    maxlen = max(maxlen, len[j]);
    seg[j] = Rec{-__builtin_inff(), 0.f, 0.f, 0.f, 0.f};
  }
  // Each segment is folded in ascending chunk order; the loads of a batch are all issued first.
  for (int b = 0; b < maxlen; b += BATCH) {
    f32x4 r[PASSES][BATCH];
    float r2[PASSES][BATCH];
#pragma unroll
    for (int j = 0; j < PASSES; ++j)
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        const int c = b + i;
        const bool ok = t_ok && c < len[j];
        const size_t at = (size_t)(lo[j] + c) * (size_t)T + t;
        r[j][i] = ok ? a.rec[at] : (f32x4)(0.f);
        // a chunk whose partials ran without squared sums gives NaN, which the fold carries to
        // the row's sum_p2
        r2[j][i] = (P2 && ok) ? (a.p2ok[lo[j] + c] ? a.rec2[at] : __builtin_nanf("")) : 0.f;
      }
#pragma unroll
    for (int j = 0; j < PASSES; ++j)
#pragma unroll
      for (int i = 0; i < BATCH; ++i)
        seg[j] = fold<P2>(seg[j], Rec{r[j][i][0], r[j][i][1], r[j][i][2], r[j][i][3], r2[j][i]});
  }
#pragma unroll
  for (int j = 0; j < PASSES; ++j) part.put(sg[j], tl, seg[j], P2);
  __syncthreads();
  // wavefront w merges the segment states of tokens w, w + 16, ... of the workgroup
  for (int k = w; k < TPW; k += FW) {
    const int tt = blk * TPW + k;
    if (tt >= T) break;  // k is the same in every lane
    Rec st = part.get(lane, k, P2);
#pragma unroll
    for (int d = 1; d < FIN_NSEG; d *= 2) {
      Rec o;
      o.m = __shfl_down(st.m, d);
      o.n = __shfl_down(st.n, d);
      o.b = __shfl_down(st.b, d);
      o.u = __shfl_down(st.u, d);
      o.q = P2 ? __shfl_down(st.q, d) : 0.f;
      const Rec f = fold<P2>(st, o);
      if ((lane & (2 * d - 1)) == 0) st = f;
    }
    if (lane == 0) finalize_row<P2>(a, tt, st);
  }
}

// Grid-stride over the row blocks, so that the grid stays bounded for any T.
constexpr int FIN_MAX_GRID = 1 << 16;

template <bool P2, int TPW, int FW>
__global__ __launch_bounds__(64 * FW) void fwd_finalize_kernel(FwdArgs a, int n_c, int nblk) {
  __shared__ SegStates<TPW> part;
  for (int blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    fold_row_block<P2, TPW, FW>(a, n_c, blk, part);
    __syncthreads();  // the next block's segment states overwrite part
  }
}

// Small T: one wavefront per token, lane s folding segment s (the lane layout of the tree above),
// so the T rows' folds spread over T wavefronts instead of the few workgroups of
// fwd_finalize_kernel (one workgroup, one CU, at T <= 16).  Same segments, same ascending order
// inside a segment, same tree: the same bits.
constexpr int FINW_WAVES = 4;  // wavefronts (tokens) per workgroup

template <bool P2>
__global__ __launch_bounds__(64 * FINW_WAVES) void fwd_finalize_wave_kernel(FwdArgs a, int n_c) {
  constexpr int BATCH = 20;  // one batch covers a segment of V <= 163840
  const int T = a.T;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * FINW_WAVES + (threadIdx.x >> 6);
  if (t >= T) return;  // the whole wavefront
  const int lo = (int)((int64_t)lane * n_c / FIN_NSEG);
  const int len = (int)((int64_t)(lane + 1) * n_c / FIN_NSEG) - lo;
  Rec st{-__builtin_inff(), 0.f, 0.f, 0.f, 0.f};
  for (int b = 0; b < len; b += BATCH) {
    f32x4 r[BATCH];
    float r2[BATCH];
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int c = b + i;
      const bool ok = c < len;
      const size_t at = (size_t)(lo + c) * (size_t)T + t;
      r[i] = ok ? a.rec[at] : (f32x4)(0.f);
      r2[i] = (P2 && ok) ? (a.p2ok[lo + c] ? a.rec2[at] : __builtin_nanf("")) : 0.f;
    }
#pragma unroll
    for (int i = 0; i < BATCH; ++i) st = fold<P2>(st, Rec{r[i][0], r[i][1], r[i][2], r[i][3], r2[i]});
  }
#pragma unroll
  for (int d = 1; d < FIN_NSEG; d *= 2) {
    Rec o;
    o.m = __shfl_down(st.m, d);
    o.n = __shfl_down(st.n, d);
    o.b = __shfl_down(st.b, d);
    o.u = __shfl_down(st.u, d);
    o.q = P2 ? __shfl_down(st.q, d) : 0.f;
    const Rec f = fold<P2>(st, o);
    if ((lane & (2 * d - 1)) == 0) st = f;
  }
  if (lane == 0) finalize_row<P2>(a, t, st);
}

// ---------------------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------------------

template <class Cfg, class Opt>
static void launch_partials_opt(const FwdArgs& a, hipStream_t stream) {
  const int n_mt = (a.V + Cfg::TM - 1) / Cfg::TM;
  const int n_nt = (a.T + Cfg::TN - 1) / Cfg::TN;
  if constexpr (Cfg::LOOP == LOOP_PINGPONG) {
    // one workgroup per CU (the tile takes all of a CU's LDS)
    const int ntiles = n_mt * n_nt;
    if (a.sk_acc && fwd_sk_wanted(a.T, a.V, a.cus)) {
      const int G = min(ntiles, min(a.cus, SK_MAX_WG));
      const int S = (a.H + Cfg::BK - 1) / Cfg::BK;
      hipLaunchKernelGGL(fwd_sk_reset_kernel, dim3(1), dim3(256), 0, stream, a.sk_sync, G, (int64_t)ntiles * S, S);
      hipLaunchKernelGGL((fwd_partials_sk_kernel<Cfg, Opt>), dim3(G), dim3(Cfg::NTHREADS), 0, stream, a, n_mt, n_nt,
                         sk_spin_limit());
      return;
    }
    hipLaunchKernelGGL(fwd_sched_reset_kernel, dim3(1), dim3(64), 0, stream, a.sched);
    hipLaunchKernelGGL((fwd_partials_persistent_kernel<Cfg, Opt>), dim3(min(ntiles, a.cus)), dim3(Cfg::NTHREADS), 0,
                       stream, a, n_mt, n_nt);
  } else {
    hipLaunchKernelGGL((fwd_partials_kernel<Cfg, Opt>), dim3(n_mt * n_nt), dim3(Cfg::NTHREADS), 0, stream, a, n_mt,
                       n_nt);
  }
}

template <class Cfg>
static void launch_partials_cfg(const FwdArgs& a, hipStream_t stream) {
  const bool scaled = a.temperature != 1.0f;
  if (scaled && a.want_p2)
    launch_partials_opt<Cfg, RecOpt<true, true>>(a, stream);
  else if (scaled)
    launch_partials_opt<Cfg, RecOpt<true, false>>(a, stream);
  else if (a.want_p2)
    launch_partials_opt<Cfg, RecOpt<false, true>>(a, stream);
  else
    launch_partials_opt<Cfg, RecOpt<false, false>>(a, stream);
}

// Tile configurations, chosen by T.  Each has a 128-entry vocabulary extent per wavefront and the
// same MFMA chain, so all give the same bits.
template <class P, int LOOP_>
struct FwdCfg : P {
  static constexpr int LOOP = LOOP_;
  // the ping-pong loop keeps three A slots and two B slots of one K step each
  static constexpr int LDS_BYTES = LOOP_ == LOOP_PINGPONG ? 5 * 256 * P::ROW : P::LDS_BYTES;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};
// T > 128: 256 vocab x 256 tokens, 8 wavefronts (2 per SIMD) in two groups that alternate between
// loads and MFMAs, K = 64 steps, three A slots and two B slots (160 KB of LDS), persistent grid.
// Its MFMA rate is the highest of the tiles, and from T = 192 up it is the fastest even where many
// of its token columns are empty.
using CfgBig = FwdCfg<PipeCfg<2, 4, 4, 2, 64>, LOOP_PINGPONG>;
// T <= 64 is HBM-bound: the time is the weight stream, so these tiles are sized for streaming.
// They cover 128 vocabulary rows (one wavefront's extent), so the 1188 tiles of V = 152064 give
// 4.6 tiles per CU and the last round of tiles leaves few CUs idle (256-row tiles gave 2.3 per CU
// and ran 10 % longer); one workgroup per CU holds enough loads in flight.
// T <= 32: 128 vocab x 32 tokens, 2 wavefronts (16 tokens each), three stages of K = 128 with the
// loads spread between the MFMAs (120 KB of LDS).  A K step of 128 reads 256 contiguous bytes of
// each weight row: 0.7-1.5 % faster at T = 16 and 32 than five stages of K = 64 (four stages of
// K = 128 were slower).
using CfgSmall = FwdCfg<PipeCfg<LMH_SMALL_SHAPE, LMH_SMALL_NS, LMH_SMALL_BK>, LOOP_SPREAD>;
// 32 < T <= 64: 128 vocab x 64 tokens, 4 wavefronts (16 tokens each), three stages of K = 128
// (144 KB of LDS, one workgroup per CU): 0.5 % faster at T = 48 and 64 than three stages of K = 64
// with two workgroups per CU, which had been 1.5 % faster than four stages of K = 64.
using CfgS64 = FwdCfg<PipeCfg<LMH_S64_SHAPE, LMH_S64_NS, LMH_S64_BK>, LOOP_SPREAD>;

// 64 < T <= 128: 256 vocab x 128 tokens, 4 wavefronts, three stages of K = 64 (144 KB of LDS).
// Against the 256 x 256 persistent tile it wins by 13 % at T = 96 and 128 and loses from T = 192.
using CfgMid = FwdCfg<PipeCfg<LMH_MID_SHAPE, LMH_MID_NS, 64>, LOOP_SPREAD>;

bool fwd_sk_wanted(int64_t T, int64_t V, int cus) {
  // One token tile only: with two or more, consecutive K ranges run a vocabulary tile's token tiles
  // one after another on one workgroup instead of side by side on one XCD, and the weight is read
  // from memory once per token tile (measured 17-27 % slower at T = 384 .. 1024).  Below T = 192
  // the tile's steps are short enough that the hand-overs cost what the balance gains (measured:
  // 3 % slower at T = 129, even at T = 160, 4 % faster at T = 200, 9 % at T = 256).
  if (T < LMH_SK_MIN_T || T > 256) return false;
  const int64_t ntiles = (V + 255) / 256;
  const int64_t G = min(cus, SK_MAX_WG);
  return ntiles > G && ntiles < (int64_t)LMH_SK_MAX_ROUNDS * G;
}

int sk_spin_limit() {
  const char* e = getenv("LMH_SK_SPIN_LIMIT");
  if (!e) return SK_SPIN_LIMIT;
  char* end = nullptr;
  const long v = strtol(e, &end, 10);
  if (end == e) return SK_SPIN_LIMIT;  // not a number: the default bound
  return v <= 0 ? 0 : v < SK_SPIN_LIMIT ? (int)v : SK_SPIN_LIMIT;
}

void launch_fwd_partials(const FwdArgs& a, hipStream_t stream) {
  if (a.T <= 32)
    launch_partials_cfg<CfgSmall>(a, stream);
  else if (a.T <= 64)
    launch_partials_cfg<CfgS64>(a, stream);
  else if (a.T <= LMH_MID_MAX)
    launch_partials_cfg<CfgMid>(a, stream);
  else
    launch_partials_cfg<CfgBig>(a, stream);
}

template <int TPW, int FW>
static void launch_finalize_tpw(const FwdArgs& a, int n_c, hipStream_t stream) {
  const int nblk = (a.T + TPW - 1) / TPW;
  const dim3 grid(min(nblk, FIN_MAX_GRID));
  if (a.sum_p2)
    hipLaunchKernelGGL((fwd_finalize_kernel<true, TPW, FW>), grid, dim3(64 * FW), 0, stream, a, n_c, nblk);
  else
    hipLaunchKernelGGL((fwd_finalize_kernel<false, TPW, FW>), grid, dim3(64 * FW), 0, stream, a, n_c, nblk);
}

#ifndef LMH_FINW_MAX_T
#define LMH_FINW_MAX_T 512
#endif

void launch_fwd_finalize(const FwdArgs& a, hipStream_t stream) {
  const int n_c = (a.vocab_total + WAVE_M - 1) / WAVE_M;
  if (a.T <= LMH_FINW_MAX_T) {
    const dim3 grid((a.T + FINW_WAVES - 1) / FINW_WAVES);
    if (a.sum_p2)
      hipLaunchKernelGGL(fwd_finalize_wave_kernel<true>, grid, dim3(64 * FINW_WAVES), 0, stream, a, n_c);
    else
      hipLaunchKernelGGL(fwd_finalize_wave_kernel<false>, grid, dim3(64 * FINW_WAVES), 0, stream, a, n_c);
    return;
  }
  // row blocks of TPW tokens on FW wavefronts: enough blocks to cover the CUs (256 at T = 2048,
  // 4096 and 8192), the segment loads of a block one 128-byte line per segment or more
  if (a.T < 4096)
    launch_finalize_tpw<8, 8>(a, n_c, stream);
  else if (a.T < 8192)
    launch_finalize_tpw<16, 16>(a, n_c, stream);
  else
    launch_finalize_tpw<32, 16>(a, n_c, stream);
}

}  // namespace lmh
