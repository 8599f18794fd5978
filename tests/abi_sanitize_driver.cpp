// Host-side driver for the sanitizer build of the C ABI (tests/test_abi_sanitize.py).  It calls
// every entry point with sizes at and past the documented bounds and with null, misaligned and
// fake (never dereferenced) pointers, and checks the documented statuses.  On a host without a GPU
// a call whose arguments all validate stops at the device query and returns LMH_ERR_HIP; with a
// GPU visible those calls are skipped.  Built with -fsanitize=address,undefined on the host side,
// so any out-of-range access or signed overflow in the validation and workspace arithmetic aborts.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "lmhead_logprob.h"

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

// Fake device addresses: aligned, never dereferenced on the host.
static void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }
static float* F(uintptr_t a) { return reinterpret_cast<float*>(a); }
static const int32_t* I(uintptr_t a) { return reinterpret_cast<const int32_t*>(a); }

int main(int argc, char** argv) {
  const bool have_gpu = argc > 1 && argv[1][0] == '1';
  const int64_t B31 = int64_t(1) << 31, B16 = int64_t(1) << 16;
  const int64_t Ts[] = {-1, 0, 1, 63, 64, 257, (1 << 22) - 1, 1 << 22, B31 - B16 - 1, B31 - B16, B31, INT64_MAX};
  const int64_t Hs[] = {-8, 0, 8, 12, 4096, 1 << 20, (1 << 20) + 8, INT64_MAX - 7};
  const int64_t Vs[] = {-1, 0, 1, 2, 128, 129, 152064, B31 - B16 - 1, B31 - B16, B31, int64_t(1) << 40, INT64_MAX};
  const size_t BIG = SIZE_MAX / 2;
  for (int64_t T : Ts)
    for (int64_t H : Hs)
      for (int64_t V : Vs) {
        const size_t fw = lmhead_logprob_fwd_workspace_size(T, H, V);
        const size_t fw_min = lmhead_logprob_fwd_workspace_size_min(T, H, V);
        const size_t bw = lmhead_logprob_bwd_workspace_size(T, H, V);
        const bool sizes_ok = T >= 0 && T < B31 - B16 && H >= 8 && H % 8 == 0 && H <= (1 << 20) && V >= 1 &&
                              V < B31 - B16 && (T == 0 || (V + 127) / 128 <= (int64_t(1) << 36) / T);
        EXPECT((fw > 0) == sizes_ok);
        EXPECT((fw_min > 0) == sizes_ok && fw_min <= fw);
        EXPECT((bw > 0) == sizes_ok);
        if (sizes_ok) {
          EXPECT(fw % 256 == 0 && bw % 256 == 0);
          size_t prev = 0;
          for (int64_t step = 256; step <= 65536; step *= 4) {
            const size_t s = lmhead_logprob_bwd_workspace_size_step(T, H, V, step);
            EXPECT(s >= prev && s <= bw);  // equal once the step covers V
            prev = s;
          }
          EXPECT(lmhead_logprob_bwd_workspace_size_step(T, H, V, 0) == 0);
          EXPECT(lmhead_logprob_bwd_workspace_size_step(T, H, V, INT64_MAX) == bw);
        }
        // forward: a too-small workspace is refused before the device is touched
        const lmh_status_t s_small = lmhead_logprob_fwd(P(0x1000), P(0x2000), I(0x3000), T, H, V, F(0x4000),
                                                        nullptr, nullptr, P(0x10000), 0, nullptr);
        if (!sizes_ok)
          EXPECT(s_small == LMH_ERR_INVALID_ARG || s_small == LMH_ERR_UNSUPPORTED);
        else if (T == 0)
          EXPECT(s_small == LMH_OK);
        else
          EXPECT(s_small == LMH_ERR_WORKSPACE_TOO_SMALL);
        if (!have_gpu && sizes_ok && T > 0) {
          EXPECT(lmhead_logprob_fwd(P(0x1000), P(0x2000), I(0x3000), T, H, V, F(0x4000), F(0x5000), F(0x6000),
                                    P(0x10000), BIG, nullptr) == LMH_ERR_HIP);
          EXPECT(lmhead_logprob_bwd(P(0x1000), P(0x2000), I(0x3000), T, H, V, F(0x4000), F(0x5000), F(0x6000),
                                    F(0x7000), 0, P(0x10000), BIG, nullptr) ==
                 (T >= (1 << 22) ? LMH_ERR_UNSUPPORTED : LMH_ERR_HIP));
          const lmh_status_t na = lmhead_logprob_fwd_noalloc(P(0x1000), P(0x2000), I(0x3000), T, H, V, F(0x4000),
                                                             nullptr, nullptr, nullptr);
          EXPECT(na == (fw_min <= LMH_NOALLOC_SCRATCH_BYTES ? LMH_ERR_HIP : LMH_ERR_WORKSPACE_TOO_SMALL));
        }
        // the smallest forward workspace passes validation; one byte less does not
        if (sizes_ok && T > 0 && !have_gpu) {
          EXPECT(lmhead_logprob_fwd(P(0x1000), P(0x2000), I(0x3000), T, H, V, F(0x4000), nullptr, nullptr,
                                    P(0x10000), fw_min - 1, nullptr) == LMH_ERR_WORKSPACE_TOO_SMALL);
          EXPECT(lmhead_logprob_fwd(P(0x1000), P(0x2000), I(0x3000), T, H, V, F(0x4000), nullptr, nullptr,
                                    P(0x10000), fw_min, nullptr) == LMH_ERR_HIP);
        }
        // the narrowest backward step's workspace passes validation; one byte less does not
        if (sizes_ok && T > 0 && T < (1 << 22)) {
          const size_t least = lmhead_logprob_bwd_workspace_size_step(T, H, V, 256);
          EXPECT(lmhead_logprob_bwd(P(0x1000), P(0x2000), I(0x3000), T, H, V, F(0x4000), F(0x5000), nullptr,
                                    nullptr, 0, P(0x10000), least - 1, nullptr) == LMH_ERR_WORKSPACE_TOO_SMALL);
          EXPECT(lmhead_logprob_bwd(P(0x1000), P(0x2000), I(0x3000), T, H, V, F(0x4000), F(0x5000), nullptr,
                                    nullptr, 0, P(0x10000), least, nullptr) == LMH_OK);
        }
      }
  // argument rules of the extended entry points
  const float bad_tau[] = {0.0f, -1.0f, __builtin_nanf(""), __builtin_inff()};
  for (float t : bad_tau) {
    EXPECT(lmhead_logprob_fwd_ex(P(0x1000), P(0x2000), I(0x3000), 4, 8, 10, t, F(0x4000), nullptr, nullptr,
                                 nullptr, P(0x10000), BIG, nullptr) == LMH_ERR_INVALID_ARG);
    EXPECT(lmhead_logprob_bwd_ex(P(0x1000), P(0x2000), I(0x3000), 4, 8, 10, t, 0, F(0x4000), F(0x5000), nullptr,
                                 nullptr, nullptr, nullptr, 0, P(0x10000), BIG, nullptr) == LMH_ERR_INVALID_ARG);
  }
  const int64_t starts[] = {-128, 0, 64, 128, B31 - B16 - 10, B31, INT64_MAX - 5};
  for (int64_t vs : starts)
    for (int64_t vt : {int64_t(10), int64_t(1024), B31 - B16 - 1, B31, INT64_MAX}) {
      const lmh_status_t s = lmhead_logprob_fwd_partials_ex(P(0x1000), P(0x2000), I(0x3000), 4, 8, 128, 1.0f, vs,
                                                            vt, 0, P(0x10000), 0, nullptr);
      EXPECT(s != LMH_OK && s != LMH_ERR_HIP);
      const lmh_status_t b = lmhead_logprob_bwd_ex(P(0x1000), P(0x2000), I(0x3000), 4, 8, 10, 1.0f, vs, F(0x4000),
                                                   F(0x5000), nullptr, nullptr, nullptr, nullptr, 0, P(0x10000),
                                                   BIG, nullptr);
      EXPECT(b == ((vs >= 0 && vs < B31 - B16 - 10) ? LMH_OK : LMH_ERR_INVALID_ARG));
    }
  EXPECT(lmhead_logprob_fwd(P(0x1008), P(0x2000), I(0x3000), 4, 8, 10, F(0x4000), nullptr, nullptr, P(0x10000),
                            BIG, nullptr) == LMH_ERR_UNSUPPORTED);
  EXPECT(lmhead_logprob_fwd(nullptr, P(0x2000), I(0x3000), 4, 8, 10, F(0x4000), nullptr, nullptr, P(0x10000),
                            BIG, nullptr) == LMH_ERR_INVALID_ARG);
  EXPECT(lmhead_logprob_fwd_finalize(I(0x3000), 4, 8, 10, F(0x4000), F(0x5002), nullptr, P(0x10000), BIG,
                                     nullptr) == LMH_ERR_UNSUPPORTED);
  for (int s = -1; s < 7; ++s) EXPECT(lmhead_status_string(static_cast<lmh_status_t>(s)) != nullptr);
  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("abi sanitize driver ok\n");
  return 0;
}
