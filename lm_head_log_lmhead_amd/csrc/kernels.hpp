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
