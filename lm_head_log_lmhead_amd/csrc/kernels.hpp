// kernels.hpp — internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tile_gemm.hpp"

namespace lmh {

// Vocabulary width of one forward record (one wavefront's M extent).
constexpr int VOCAB_CHUNK = WAVE_M;
// Vocabulary rows per backward step (a multiple of the 256-row tile and of the K step).
// grad_hidden does not depend on it bit-wise: each step continues the previous step's MFMA
// accumulation chain.
constexpr int BWD_VOCAB_STEP = 16384;

// Words of the forward workspace used by the large-T tile scheduler (one counter per XCD).
constexpr int SCHED_WORDS = 16;

struct FwdArgs {
  const __bf16* hidden;
  const __bf16* weight;
  const int* labels;
  int T, H, V;
  f32x4* rec;   // [n_c][T] records
  float* zy;    // [T] label logits
  int* sched;   // [SCHED_WORDS] tile counters, reset by the partials launch
  float* logprob;
  float* entropy;
  float* lse;
  int cus;      // compute units of the device (persistent grids)
};

void launch_fwd_partials(const FwdArgs& a, hipStream_t stream);
void launch_fwd_finalize(const FwdArgs& a, hipStream_t stream);

struct BwdLayout {
  int T, H, V;
  int Tp;      // T rounded up to 64 (pitch of the transposed token-major buffers)
  int Vs;      // vocabulary rows per step: min(BWD_VOCAB_STEP, V rounded up to 256)
  int nsteps;  // ceil(V / Vs)
  size_t off_dz, off_dzt, off_wt, off_ht, off_sched, total;
};

BwdLayout bwd_layout(int64_t T, int64_t H, int64_t V);

struct BwdArgs {
  const __bf16* hidden;
  const __bf16* weight;
  const int* labels;
  const float* grad;
  const float* lse;
  float* grad_hidden;
  float* grad_weight;
  int accumulate_gw;
  char* ws;
  BwdLayout L;
  int cus;      // compute units of the device (persistent grids)
};

void launch_bwd(const BwdArgs& a, hipStream_t stream);

}  // namespace lmh
