// kernels.hpp — internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tile_gemm.hpp"

namespace lmh {

// Vocabulary width of one forward record (one wavefront's M extent).
constexpr int VOCAB_CHUNK = WAVE_M;
// Vocabulary rows per backward step: the widest (fastest) step; a smaller workspace takes the
// widest multiple of BWD_STEP_UNIT that fits.  No result depends on it bit-wise: grad_hidden's MFMA
// chain continues across steps and step bounds are multiples of the K slice, grad_weight's chain
// runs over tokens.
#ifndef LMH_BWD_STEP
#define LMH_BWD_STEP 65536
#endif
constexpr int BWD_VOCAB_STEP = LMH_BWD_STEP;
constexpr int BWD_STEP_UNIT = 256;
// Tile counters of the backward's persistent gradient GEMM (one per XCD), zeroed before each
// step's GEMM by that step's dz launch.
constexpr int BWD_SCHED_WORDS = 16;

// Words of the forward workspace used by the large-T tile scheduler (one counter per XCD).
constexpr int SCHED_WORDS = 16;

// K-split schedule of the large-T tile for launches of few tile rounds: at most SK_MAX_WG
// workgroups, each with one accumulator slot of a whole 256 x 256 fp32 tile in the workspace, and
// a word array [0] = workgroup counter, [1 + g] = flag "workgroup g's accumulators are stored",
// [SK_BOUNDS_WORD + 4 g ..] = workgroup g's range of K steps.
constexpr int SK_MAX_WG = 256;
constexpr size_t SK_SLOT_BYTES = 256 * 256 * 4;
constexpr int SK_BOUNDS_WORD = 260;  // 16-byte aligned, past the flags
constexpr int SK_SYNC_WORDS = SK_BOUNDS_WORD + 4 * SK_MAX_WG;
// A tail's wait for the previous workgroup ends by construction; the bound (polls of the flag)
// only keeps a broken invariant from hanging the device.  A tail that gives up continues NaN
// accumulators instead, so the call's outputs are NaN rather than wrong.
constexpr int SK_SPIN_LIMIT = 1 << 22;
// SK_SPIN_LIMIT, or the smaller bound the environment variable LMH_SK_SPIN_LIMIT sets (read per
// launch; 0 makes every tail give up at once, which is how the tests take that path).
int sk_spin_limit();
#ifndef LMH_SK_MAX_ROUNDS
#define LMH_SK_MAX_ROUNDS 4
#endif
#ifndef LMH_SK_MIN_T
#define LMH_SK_MIN_T 192
#endif
// Whether the forward of T tokens over V weight rows runs the K-split schedule when the workspace
// has room for it: one token tile of the large-T tile (LMH_SK_MIN_T <= T <= 256), and more
// vocabulary tiles than workgroups but fewer than LMH_SK_MAX_ROUNDS per workgroup.
bool fwd_sk_wanted(int64_t T, int64_t V, int cus);

struct FwdArgs {
  const __bf16* hidden;
  const __bf16* weight;
  const int* labels;
  int T, H, V;        // V: weight rows of this call
  int vocab_start;    // vocabulary id of weight row 0 (a multiple of VOCAB_CHUNK)
  int vocab_total;    // vocabulary the records and the fold cover (vocab_start + V <= vocab_total)
  float temperature;  // the logits are divided by it before the softmax (1: no division)
  int want_p2;        // also record sum exp(2 (z - max)) per chunk
  f32x4* rec;         // [n_c][T] records, n_c = ceil(vocab_total / VOCAB_CHUNK)
  float* rec2;        // [n_c][T] sum of exp(2 (z - max)) per chunk
  float* zy;          // [T] label logits (divided by the temperature)
  int* sched;         // [SCHED_WORDS] tile counters, reset by the partials launch
  int* p2ok;          // [n_c] 1 if the chunk's rec2 was written by the last partials run over it
  f32x4* sk_acc;      // [SK_MAX_WG] accumulator slots of the K-split schedule, or null (not used)
  int* sk_sync;       // [SK_SYNC_WORDS] its workgroup counter and flags
  float* logprob;
  float* entropy;
  float* lse;
  float* sum_p2;
  int cus;            // compute units of the device (persistent grids)
};

void launch_fwd_partials(const FwdArgs& a, hipStream_t stream);
void launch_fwd_finalize(const FwdArgs& a, hipStream_t stream);

struct BwdLayout {
  int T, H, V;
  int Tp;      // T rounded up to 64 (pitch of the transposed token-major buffers)
  int Vs;      // vocabulary rows per step: min(step, V rounded up to BWD_STEP_UNIT)
  int nsteps;  // ceil(V / Vs)
  size_t off_dz, off_dzt, off_wt, off_ht, off_sched, total;
};

// Workspace layout for a step of `step` vocabulary rows (a multiple of BWD_STEP_UNIT, at most
// BWD_VOCAB_STEP); total grows with the step.
BwdLayout bwd_layout(int64_t T, int64_t H, int64_t V, int64_t step);

struct BwdArgs {
  const __bf16* hidden;
  const __bf16* weight;
  const int* labels;
  const float* grad;          // [T] upstream gradient of the log-probs
  const float* lse;           // [T] of the logits divided by the temperature
  const float* grad_entropy;  // [T] upstream gradient of the entropies, or null
  const float* entropy;       // [T] forward entropies (needed with grad_entropy)
  float temperature;
  int vocab_start;            // vocabulary id of weight row 0 (labels are vocabulary ids)
  float* grad_hidden;
  float* grad_weight;
  int accumulate_gw;
  char* ws;
  BwdLayout L;
  int cus;      // compute units of the device (persistent grids)
};

void launch_bwd(const BwdArgs& a, hipStream_t stream);

}  // namespace lmh
