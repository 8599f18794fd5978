// api.hip — the C ABI (include/lmhead_logprob.h): host-side validation, workspace carving and
// launch.  Every check runs before the first launch; a failed check launches nothing.
#include "lmhead_logprob.h"

#include <math.h>
#include <string.h>

#include <atomic>

#include "kernels.hpp"

// Workspace of lmhead_logprob_fwd_noalloc: one array per device, alive until the process ends.
// In host code `scratch` names a host-side stand-in, not the device memory: the device address is
// looked up with hipGetSymbolAddress (scratch_for_current_device below) and only that address is
// handed to kernels.
static __device__ __align__(256) char scratch[LMH_NOALLOC_SCRATCH_BYTES];

namespace {

using lmh::FwdArgs;

constexpr int64_t MAX_H = 1 << 20;
// Exclusive bounds on V (also vocab_start + V of a shard) and T.  The kernels index vocabulary rows
// and tokens with 32-bit ints, including indices rounded up to a whole tile (256) or a whole
// backward step (65536 rows), so both stay 2^16 below 2^31.
constexpr int64_t MAX_V = (int64_t(1) << 31) - (int64_t(1) << 16);
constexpr int64_t MAX_T = (int64_t(1) << 31) - (int64_t(1) << 16);
// backward: token-major transposed operands are read through 32-bit buffer offsets (256 rows x T)
constexpr int64_t MAX_T_BWD = int64_t(1) << 22;

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Sizes: returns LMH_OK, or the error for the first violated rule.
lmh_status_t check_sizes(int64_t T, int64_t H, int64_t V) {
  if (T < 0 || H <= 0 || V <= 0) return LMH_ERR_INVALID_ARG;
  if (H % 8 != 0 || H > MAX_H || V >= MAX_V || T >= MAX_T) return LMH_ERR_UNSUPPORTED;
  // At most 2^36 (row, chunk) records (1.1 TB of workspace, beyond any one device's memory), so
  // every derived size fits its type: the large-T tile count (about records / 512 < 2^28) is
  // a 32-bit int in the kernels, record offsets are 64-bit.
  const int64_t n_c = (V + lmh::VOCAB_CHUNK - 1) / lmh::VOCAB_CHUNK;
  if (T > 0 && n_c > (int64_t(1) << 36) / T) return LMH_ERR_UNSUPPORTED;
  return LMH_OK;
}

struct FwdWs {
  size_t rec_off, rec2_off, zy_off, sched_off, p2ok_off, total;
  size_t sk_sync_off, sk_acc_off, total_sk;
};

// Forward workspace for a vocabulary of V rows: records and squared-sum records for every
// 128-row chunk, label logits, tile counters, and one flag per chunk telling whether its
// squared-sum records were written (total bytes: the least every forward call accepts).  Past
// that, the K-split schedule's counter, flags and accumulator slots (total_sk); a partials call
// whose workspace holds them runs that schedule where it applies.
FwdWs fwd_ws(int64_t T, int64_t V) {
  const int64_t n_c = (V + lmh::VOCAB_CHUNK - 1) / lmh::VOCAB_CHUNK;
  FwdWs w;
  w.rec_off = 0;
  w.rec2_off = align256((size_t)n_c * (size_t)T * 16);
  w.zy_off = w.rec2_off + align256((size_t)n_c * (size_t)T * 4);
  w.sched_off = w.zy_off + align256((size_t)T * 4);
  w.p2ok_off = w.sched_off + align256(lmh::SCHED_WORDS * sizeof(int));
  w.total = w.p2ok_off + align256((size_t)n_c * sizeof(int));
  w.sk_sync_off = w.total;
  w.sk_acc_off = w.sk_sync_off + align256(lmh::SK_SYNC_WORDS * sizeof(int));
  w.total_sk = w.sk_acc_off + (size_t)lmh::SK_MAX_WG * lmh::SK_SLOT_BYTES;
  return w;
}

// The workspace size that gives the fastest schedule (the K-split one where it applies on a
// device of SK_MAX_WG compute units).
size_t fwd_ws_fast(int64_t T, int64_t V) {
  const FwdWs w = fwd_ws(T, V);
  return lmh::fwd_sk_wanted(T, V, lmh::SK_MAX_WG) ? w.total_sk : w.total;
}

lmh_status_t check_inputs(const void* hidden, const void* weight, const int32_t* labels) {
  if (!hidden || !weight || !labels) return LMH_ERR_INVALID_ARG;
  if (!aligned(hidden, 16) || !aligned(weight, 16) || !aligned(labels, 4)) return LMH_ERR_UNSUPPORTED;
  return LMH_OK;
}

lmh_status_t check_ws(const void* ws, size_t bytes, size_t need) {
  if (bytes < need) return LMH_ERR_WORKSPACE_TOO_SMALL;
  if (need > 0 && !ws) return LMH_ERR_INVALID_ARG;
  if (ws && !aligned(ws, 256)) return LMH_ERR_UNSUPPORTED;
  return LMH_OK;
}

lmh_status_t check_out(const float* p, bool required) {
  if (!p) return required ? LMH_ERR_INVALID_ARG : LMH_OK;
  return aligned(p, 4) ? LMH_OK : LMH_ERR_UNSUPPORTED;
}

lmh_status_t check_in(const float* p) {
  if (!p) return LMH_ERR_INVALID_ARG;
  return aligned(p, 4) ? LMH_OK : LMH_ERR_UNSUPPORTED;
}

lmh_status_t check_temperature(float t) { return (isfinite(t) && t > 0.0f) ? LMH_OK : LMH_ERR_INVALID_ARG; }

lmh_status_t launched() { return hipGetLastError() == hipSuccess ? LMH_OK : LMH_ERR_HIP; }

// Compute units of the current device (the large-T grids have one workgroup per CU).
lmh_status_t device_cus(int& cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LMH_ERR_HIP;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return LMH_ERR_HIP;
  if (cus < 8) cus = 8;
  return LMH_OK;
}

FwdArgs make_fwd_args(const void* hidden, const void* weight, const int32_t* labels, int64_t T, int64_t H,
                      int64_t V, int64_t vocab_start, int64_t vocab_total, float temperature, int want_p2,
                      float* logprob, float* entropy, float* lse, float* sum_p2, void* workspace,
                      size_t workspace_bytes) {
  const FwdWs w = fwd_ws(T, vocab_total);
  char* ws = static_cast<char*>(workspace);
  FwdArgs a;
  a.hidden = static_cast<const __bf16*>(hidden);
  a.weight = static_cast<const __bf16*>(weight);
  a.labels = labels;
  a.T = (int)T;
  a.H = (int)H;
  a.V = (int)V;
  a.vocab_start = (int)vocab_start;
  a.vocab_total = (int)vocab_total;
  a.temperature = temperature;
  a.want_p2 = want_p2;
  a.rec = reinterpret_cast<lmh::f32x4*>(ws + w.rec_off);
  a.rec2 = reinterpret_cast<float*>(ws + w.rec2_off);
  a.zy = reinterpret_cast<float*>(ws + w.zy_off);
  a.sched = reinterpret_cast<int*>(ws + w.sched_off);
  a.p2ok = reinterpret_cast<int*>(ws + w.p2ok_off);
  const bool sk_room = workspace_bytes >= w.total_sk;
  a.sk_sync = sk_room ? reinterpret_cast<int*>(ws + w.sk_sync_off) : nullptr;
  a.sk_acc = sk_room ? reinterpret_cast<lmh::f32x4*>(ws + w.sk_acc_off) : nullptr;
  a.logprob = logprob;
  a.entropy = entropy;
  a.lse = lse;
  a.sum_p2 = sum_p2;
  a.cus = 0;
  return a;
}

#define LMH_TRY(expr)                      \
  do {                                     \
    const lmh_status_t s_ = (expr);        \
    if (s_ != LMH_OK) return s_;           \
  } while (0)

// The weight rows of a call are the vocabulary ids [vocab_start, vocab_start + V) of a
// vocabulary of vocab_total; shards start on a chunk and all but the last cover whole chunks.
lmh_status_t check_shard(int64_t V, int64_t vocab_start, int64_t vocab_total) {
  if (V <= 0 || vocab_start < 0 || vocab_total <= 0) return LMH_ERR_INVALID_ARG;
  if (vocab_start > vocab_total - V) return LMH_ERR_INVALID_ARG;  // vocab_start + V > vocab_total, without overflow
  if (vocab_start % lmh::VOCAB_CHUNK != 0) return LMH_ERR_UNSUPPORTED;
  if (V % lmh::VOCAB_CHUNK != 0 && vocab_start + V != vocab_total) return LMH_ERR_UNSUPPORTED;
  return LMH_OK;
}

lmh_status_t fwd_partials_impl(const void* hidden, const void* weight, const int32_t* labels, int64_t T, int64_t H,
                               int64_t V, float temperature, int64_t vocab_start, int64_t vocab_total,
                               int want_sum_p2, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  LMH_TRY(check_sizes(T, H, vocab_total));
  LMH_TRY(check_shard(V, vocab_start, vocab_total));
  if (want_sum_p2 != 0 && want_sum_p2 != 1) return LMH_ERR_INVALID_ARG;
  LMH_TRY(check_temperature(temperature));
  if (T == 0) return LMH_OK;
  LMH_TRY(check_inputs(hidden, weight, labels));
  LMH_TRY(check_ws(workspace, workspace_bytes, fwd_ws(T, vocab_total).total));
  FwdArgs a = make_fwd_args(hidden, weight, labels, T, H, V, vocab_start, vocab_total, temperature, want_sum_p2,
                            nullptr, nullptr, nullptr, nullptr, workspace, workspace_bytes);
  LMH_TRY(device_cus(a.cus));
  (void)hipGetLastError();  // clear any stale error so the check after launching sees only ours
  lmh::launch_fwd_partials(a, stream);
  return launched();
}

lmh_status_t fwd_finalize_impl(const int32_t* labels, int64_t T, int64_t H, int64_t V, float* logprob,
                               float* entropy, float* lse, float* sum_p2, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  LMH_TRY(check_sizes(T, H, V));
  if (T == 0) return LMH_OK;
  if (!labels) return LMH_ERR_INVALID_ARG;
  if (!aligned(labels, 4)) return LMH_ERR_UNSUPPORTED;
  LMH_TRY(check_out(logprob, true));
  LMH_TRY(check_out(entropy, false));
  LMH_TRY(check_out(lse, false));
  LMH_TRY(check_out(sum_p2, false));
  LMH_TRY(check_ws(workspace, workspace_bytes, fwd_ws(T, V).total));
  (void)hipGetLastError();
  lmh::launch_fwd_finalize(
      make_fwd_args(nullptr, nullptr, labels, T, H, V, 0, V, 1.0f, sum_p2 != nullptr, logprob, entropy, lse, sum_p2,
                    workspace, workspace_bytes),
      stream);
  return launched();
}

lmh_status_t fwd_impl(const void* hidden, const void* weight, const int32_t* labels, int64_t T, int64_t H, int64_t V,
                      float temperature, float* logprob, float* entropy, float* lse, float* sum_p2, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  LMH_TRY(check_sizes(T, H, V));
  LMH_TRY(check_temperature(temperature));
  if (T == 0) return LMH_OK;
  LMH_TRY(check_inputs(hidden, weight, labels));
  LMH_TRY(check_out(logprob, true));
  LMH_TRY(check_out(entropy, false));
  LMH_TRY(check_out(lse, false));
  LMH_TRY(check_out(sum_p2, false));
  LMH_TRY(check_ws(workspace, workspace_bytes, fwd_ws(T, V).total));
  FwdArgs a = make_fwd_args(hidden, weight, labels, T, H, V, 0, V, temperature, sum_p2 != nullptr, logprob, entropy,
                            lse, sum_p2, workspace, workspace_bytes);
  LMH_TRY(device_cus(a.cus));
  (void)hipGetLastError();
  lmh::launch_fwd_partials(a, stream);
  if (hipGetLastError() != hipSuccess) return LMH_ERR_HIP;
  lmh::launch_fwd_finalize(a, stream);
  return launched();
}

// Rounds of dz tiles (256 x 256, one per CU at a time) the backward runs with a step of `step`
// vocabulary rows: the measure of time used to pick among the steps that fit a workspace.
int64_t bwd_dz_rounds(int64_t T, int64_t V, int64_t step, int cus) {
  const int64_t nt = (T + 255) / 256;
  const int64_t full = V / step, rest = V % step;
  const int64_t per_step = ((step + 255) / 256 * nt + cus - 1) / cus;
  return full * per_step + (rest ? ((rest + 255) / 256 * nt + cus - 1) / cus : 0);
}

// The backward's layout for a workspace of `bytes`: the widest vocabulary step (a multiple of
// BWD_STEP_UNIT, at most BWD_VOCAB_STEP) whose buffers fit when that is the fastest schedule's;
// otherwise, among the steps that fit down to half the widest, the one with the fewest rounds of
// dz tiles on `cus` compute units (a step whose tiles fill the last round of every step beats a
// slightly wider one that leaves it nearly empty).  False if not even the narrowest step fits.
// The layout's total grows with the step, so the widest fit is found by bisection.  No result
// depends on the step.
bool bwd_choose_layout(int64_t T, int64_t H, int64_t V, size_t bytes, int cus, lmh::BwdLayout& L) {
  L = lmh::bwd_layout(T, H, V, lmh::BWD_VOCAB_STEP);
  if (L.total <= bytes) return true;
  constexpr int64_t U = lmh::BWD_STEP_UNIT;
  int64_t lo = 1, hi = lmh::BWD_VOCAB_STEP / U;  // in units of BWD_STEP_UNIT
  if (lmh::bwd_layout(T, H, V, lo * U).total > bytes) return false;
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) / 2;
    if (lmh::bwd_layout(T, H, V, mid * U).total <= bytes)
      lo = mid;
    else
      hi = mid - 1;
  }
  int64_t best = lo;
  for (int64_t u = lo - 1; u >= 1 && 2 * u >= lo; --u)
    if (bwd_dz_rounds(T, V, u * U, cus) < bwd_dz_rounds(T, V, best * U, cus)) best = u;
  L = lmh::bwd_layout(T, H, V, best * U);
  return true;
}

lmh_status_t bwd_impl(const void* hidden, const void* weight, const int32_t* labels, int64_t T, int64_t H, int64_t V,
                      float temperature, int64_t vocab_start, const float* grad_logprob, const float* lse,
                      const float* grad_entropy, const float* entropy, float* grad_hidden, float* grad_weight,
                      int accumulate_grad_weight, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  LMH_TRY(check_sizes(T, H, V));
  if (accumulate_grad_weight != 0 && accumulate_grad_weight != 1) return LMH_ERR_INVALID_ARG;
  LMH_TRY(check_temperature(temperature));
  if (vocab_start < 0 || vocab_start >= MAX_V - V) return LMH_ERR_INVALID_ARG;  // V < MAX_V checked above
  if (T >= MAX_T_BWD) return LMH_ERR_UNSUPPORTED;
  if (T == 0) return LMH_OK;  // no rows: nothing is launched and the gradient buffers are untouched
  LMH_TRY(check_inputs(hidden, weight, labels));
  LMH_TRY(check_in(grad_logprob));
  LMH_TRY(check_in(lse));
  if (grad_entropy) {
    LMH_TRY(check_in(grad_entropy));
    LMH_TRY(check_in(entropy));
  }
  LMH_TRY(check_out(grad_hidden, false));
  LMH_TRY(check_out(grad_weight, false));
  // any workspace down to the narrowest step's is accepted (the step is chosen below)
  LMH_TRY(check_ws(workspace, workspace_bytes, lmh::bwd_layout(T, H, V, lmh::BWD_STEP_UNIT).total));
  if (!grad_hidden && !grad_weight) return LMH_OK;
  lmh::BwdArgs a;
  LMH_TRY(device_cus(a.cus));
  lmh::BwdLayout L;
  if (!bwd_choose_layout(T, H, V, workspace_bytes, a.cus, L)) return LMH_ERR_WORKSPACE_TOO_SMALL;
  (void)hipGetLastError();
  a.hidden = static_cast<const __bf16*>(hidden);
  a.weight = static_cast<const __bf16*>(weight);
  a.labels = labels;
  a.grad = grad_logprob;
  a.lse = lse;
  a.grad_entropy = grad_entropy;
  a.entropy = grad_entropy ? entropy : nullptr;
  a.temperature = temperature;
  a.vocab_start = (int)vocab_start;
  a.grad_hidden = grad_hidden;
  a.grad_weight = grad_weight;
  a.accumulate_gw = accumulate_grad_weight;
  a.ws = static_cast<char*>(workspace);
  a.L = L;
  lmh::launch_bwd(a, stream);
  return launched();
}

// Device address of `scratch` on the current device, looked up on the first call made on that
// device and kept (the lookup is idempotent, so racing first calls store the same value).
constexpr int MAX_DEVICES = 256;
std::atomic<void*> scratch_ptr[MAX_DEVICES];

lmh_status_t scratch_for_current_device(void*& ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LMH_ERR_HIP;
  if (dev < 0 || dev >= MAX_DEVICES) return LMH_ERR_UNSUPPORTED;
  void* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LMH_ERR_HIP;
    scratch_ptr[dev].store(p, std::memory_order_release);
  }
  ptr = p;
  return LMH_OK;
}

}  // namespace

extern "C" {

lmh_status_t lmhead_logprob_fwd_noalloc(const void* hidden, const void* weight, const int32_t* labels, int64_t T,
                                        int64_t H, int64_t V, float* logprob, float* entropy, float* lse,
                                        hipStream_t stream) {
  LMH_TRY(check_sizes(T, H, V));
  if (T == 0) return LMH_OK;
  LMH_TRY(check_inputs(hidden, weight, labels));
  LMH_TRY(check_out(logprob, true));
  LMH_TRY(check_out(entropy, false));
  LMH_TRY(check_out(lse, false));
  const size_t need = fwd_ws(T, V).total;
  if (need > (size_t)LMH_NOALLOC_SCRATCH_BYTES) return LMH_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  LMH_TRY(scratch_for_current_device(ws));
  // the tile counters (and the K-split schedule's counter and flags) in the scratch are reset by a
  // kernel inside the call, and every other word the call reads is written by it first, so the
  // previous call's contents do not matter
  return fwd_impl(hidden, weight, labels, T, H, V, 1.0f, logprob, entropy, lse, nullptr, ws,
                  (size_t)LMH_NOALLOC_SCRATCH_BYTES, stream);
}

size_t lmhead_logprob_fwd_workspace_size(int64_t T, int64_t H, int64_t V) {
  if (check_sizes(T, H, V) != LMH_OK) return 0;
  return fwd_ws_fast(T, V);
}

size_t lmhead_logprob_fwd_workspace_size_min(int64_t T, int64_t H, int64_t V) {
  if (check_sizes(T, H, V) != LMH_OK) return 0;
  return fwd_ws(T, V).total;
}

lmh_status_t lmhead_logprob_fwd_partials(const void* hidden, const void* weight, const int32_t* labels, int64_t T,
                                         int64_t H, int64_t V, void* workspace, size_t workspace_bytes,
                                         hipStream_t stream) {
  return fwd_partials_impl(hidden, weight, labels, T, H, V, 1.0f, 0, V, 0, workspace, workspace_bytes, stream);
}

lmh_status_t lmhead_logprob_fwd_partials_ex(const void* hidden, const void* weight, const int32_t* labels, int64_t T,
                                            int64_t H, int64_t V, float temperature, int64_t vocab_start,
                                            int64_t vocab_total, int want_sum_p2, void* workspace,
                                            size_t workspace_bytes, hipStream_t stream) {
  return fwd_partials_impl(hidden, weight, labels, T, H, V, temperature, vocab_start, vocab_total, want_sum_p2,
                           workspace, workspace_bytes, stream);
}

lmh_status_t lmhead_logprob_fwd_finalize(const int32_t* labels, int64_t T, int64_t H, int64_t V, float* logprob,
                                         float* entropy, float* lse, void* workspace, size_t workspace_bytes,
                                         hipStream_t stream) {
  return fwd_finalize_impl(labels, T, H, V, logprob, entropy, lse, nullptr, workspace, workspace_bytes, stream);
}

lmh_status_t lmhead_logprob_fwd_finalize_ex(const int32_t* labels, int64_t T, int64_t H, int64_t V, float* logprob,
                                            float* entropy, float* lse, float* sum_p2, void* workspace,
                                            size_t workspace_bytes, hipStream_t stream) {
  return fwd_finalize_impl(labels, T, H, V, logprob, entropy, lse, sum_p2, workspace, workspace_bytes, stream);
}

lmh_status_t lmhead_logprob_fwd(const void* hidden, const void* weight, const int32_t* labels, int64_t T, int64_t H,
                                int64_t V, float* logprob, float* entropy, float* lse, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  return fwd_impl(hidden, weight, labels, T, H, V, 1.0f, logprob, entropy, lse, nullptr, workspace, workspace_bytes,
                  stream);
}

lmh_status_t lmhead_logprob_fwd_ex(const void* hidden, const void* weight, const int32_t* labels, int64_t T,
                                   int64_t H, int64_t V, float temperature, float* logprob, float* entropy,
                                   float* lse, float* sum_p2, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  return fwd_impl(hidden, weight, labels, T, H, V, temperature, logprob, entropy, lse, sum_p2, workspace,
                  workspace_bytes, stream);
}

size_t lmhead_logprob_bwd_workspace_size(int64_t T, int64_t H, int64_t V) {
  if (check_sizes(T, H, V) != LMH_OK) return 0;
  return lmh::bwd_layout(T, H, V, lmh::BWD_VOCAB_STEP).total;
}

size_t lmhead_logprob_bwd_workspace_size_step(int64_t T, int64_t H, int64_t V, int64_t step) {
  if (check_sizes(T, H, V) != LMH_OK || step <= 0) return 0;
  if (step > lmh::BWD_VOCAB_STEP) step = lmh::BWD_VOCAB_STEP;  // clamped first: no overflow rounding up
  step = (step + lmh::BWD_STEP_UNIT - 1) / lmh::BWD_STEP_UNIT * lmh::BWD_STEP_UNIT;
  return lmh::bwd_layout(T, H, V, step).total;
}

lmh_status_t lmhead_logprob_bwd(const void* hidden, const void* weight, const int32_t* labels, int64_t T, int64_t H,
                                int64_t V, const float* grad_logprob, const float* lse, float* grad_hidden,
                                float* grad_weight, int accumulate_grad_weight, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  return bwd_impl(hidden, weight, labels, T, H, V, 1.0f, 0, grad_logprob, lse, nullptr, nullptr, grad_hidden,
                  grad_weight, accumulate_grad_weight, workspace, workspace_bytes, stream);
}

lmh_status_t lmhead_logprob_bwd_ex(const void* hidden, const void* weight, const int32_t* labels, int64_t T,
                                   int64_t H, int64_t V, float temperature, int64_t vocab_start,
                                   const float* grad_logprob, const float* lse, const float* grad_entropy,
                                   const float* entropy, float* grad_hidden, float* grad_weight,
                                   int accumulate_grad_weight, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  return bwd_impl(hidden, weight, labels, T, H, V, temperature, vocab_start, grad_logprob, lse, grad_entropy, entropy,
                  grad_hidden, grad_weight, accumulate_grad_weight, workspace, workspace_bytes, stream);
}

const char* lmhead_status_string(lmh_status_t s) {
  // A C caller may pass any int; its bytes are read as an int, not as the enum (whose C++ range
  // covers only the listed codes).
  int code;
  memcpy(&code, &s, sizeof code);
  switch (code) {
    case LMH_OK: return "ok";
    case LMH_ERR_INVALID_ARG: return "invalid argument (null required pointer, non-positive size or temperature)";
    case LMH_ERR_UNSUPPORTED: return "unsupported (H % 8 != 0, a size limit, a misaligned pointer or shard)";
    case LMH_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case LMH_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

}  // extern "C"
