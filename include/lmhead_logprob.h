/*
 * lmhead_logprob.h — C ABI of the fused LM-head log-prob for AMD Instinct MI355X (gfx950).
 *
 * What it computes.  For every token row t of hidden[T,H] and the LM-head weight[V,H]:
 *   z_t      = hidden_t . weight^T                    (fp32 logits over the whole vocabulary,
 *                                                      accumulated from bf16 products; never
 *                                                      written to memory)
 *   lse_t    = log sum_j exp(z_tj)
 *   logprob_t = z_t,y_t - lse_t, written as (z_y - max) - log(sum exp(z - max)), i.e. the fp32
 *              log-softmax over the full vocabulary gathered at the label
 *              (verl PR #8026 "batch-invariant actor forward and sampler log-prob formula",
 *              first review: the sampler formula, fp32 log_softmax then gather, and the note that
 *              per-row or chunked evaluation gives the same value as one big log_softmax);
 *   entropy_t = -sum_j p_tj log p_tj of the same softmax (metric only, no gradient;
 *              SkyRL PR #1765 "[megatron] Triton backend for fused LM-head log-prob",
 *              maintainer review and PR summary: entropy stays no-grad).
 * The [T,V] logits are never materialized: the projection is folded into a vocabulary-tiled
 * online softmax (SkyRL PR #1765, design commit and PR summary).
 *
 * Labels outside [0, V) (for example -100 ignore ids) give logprob 0; their entropy is computed
 * as usual, and their backward keeps only the -softmax term, dz = -g * p (SkyRL PR #1765,
 * precision-policy commit on the out-of-vocab gradient).
 *
 * Batch invariance.  Each row's outputs are bitwise identical whatever T, the row's position in
 * the batch, or how the caller splits the rows into calls.  The per-row arithmetic is one fixed
 * sequence: one MFMA instruction shape and one K order over H, a per-row reduction inside a
 * fixed 128-column vocabulary chunk, and a fold of the chunk records in an order that depends on
 * V only.  No value is combined by atomics and nothing splits H or V by T; the only atomic
 * operations are the persistent kernels' tile and workgroup counters and the K-split hand-over's
 * flags, which choose the workgroup that computes a tile or part of one, never what it computes or
 * in which order (a K-split tile's fp32 accumulators pass between workgroups exactly, continuing
 * the same chain).  (Megatron-LM PR #5897
 * "Batch-invariant train/inference logprob parity", commit message: a row's output must not
 * change with the total row count.)
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers owned by the caller.  The library never allocates, frees or
 *    synchronizes, and holds no mutable global state except the allocation-free forward's
 *    per-device scratch array (see lmhead_logprob_fwd_noalloc); it is thread-safe.
 *  - Work is enqueued on `stream` and the call returns; outputs are valid when the stream reaches
 *    that point.  `stream` may be NULL (the default stream).
 *  - Arguments are validated on the host before anything is launched.  On failure the status is
 *    returned and nothing is launched.  T == 0 returns LMH_OK and launches nothing.
 *  - Layouts: hidden bf16 [T,H] row-major contiguous; weight bf16 [V,H] row-major contiguous;
 *    labels int32 [T]; all per-row outputs fp32 [T]; gradients fp32 row-major contiguous.
 *  - Requirements: H % 8 == 0, 8 <= H <= 1048576, 1 <= V < 2^31 - 2^16, 0 <= T < 2^31 - 2^16 and
 *    T * ceil(V / 128) <= 2^36 (the forward's records; LMH_ERR_UNSUPPORTED otherwise); hidden and
 *    weight 16-byte aligned; labels, per-row arrays and gradients 4-byte aligned; workspace
 *    256-byte aligned.  Non-finite inputs give undefined outputs (no error).
 *  - No C++ exception crosses the ABI.  There is no silent fallback: an unsupported request is
 *    an error code.
 */
#ifndef LMHEAD_LOGPROB_H
#define LMHEAD_LOGPROB_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#if defined(_WIN32)
#define LMH_API
#else
#define LMH_API __attribute__((visibility("default")))
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LMH_OK = 0,
  LMH_ERR_INVALID_ARG = 1,          /* null required pointer, negative or zero size           */
  LMH_ERR_UNSUPPORTED = 2,          /* H % 8 != 0, size limits, misaligned pointer              */
  LMH_ERR_WORKSPACE_TOO_SMALL = 3,  /* workspace_bytes below the smallest accepted size          */
  LMH_ERR_HIP = 4                   /* a kernel launch failed (hipGetLastError after launching) */
} lmh_status_t;

/* Bytes of workspace for the fastest lmhead_logprob_fwd (also the stage entry points below).
 * Returns 0 for invalid sizes.  The workspace holds one 20-byte record per (row, 128-column
 * vocabulary chunk), one float per row, 256 bytes of tile-scheduler counters and one int per
 * chunk.  Where the call has one 256-token tile and few 256-row vocabulary tiles per compute unit
 * (192 <= T <= 256 and 256 < ceil(V / 256) < 1024, e.g. T = 256 at V = 152064) it also holds
 * 64 MiB of accumulator slots and 5 KiB of flags, with which the partials stage splits the tiles'
 * K loops evenly over the compute units (same bits as without); a workgroup that continues
 * another's accumulators waits for them with a bounded poll (2^22 polls; the environment variable
 * LMH_SK_SPIN_LIMIT can only lower the bound), and a wait that runs out, which the launch's order
 * of workgroups rules out, makes the call's outputs NaN instead of wrong.  The initial contents do
 * not matter.
 * Calls that may run concurrently need separate workspaces. */
LMH_API size_t lmhead_logprob_fwd_workspace_size(int64_t T, int64_t H, int64_t V);

/* The smallest forward workspace the calls accept: lmhead_logprob_fwd_workspace_size without the
 * accumulator slots and flags (equal to it where those do not apply).  Any workspace_bytes from
 * this size up is accepted; below lmhead_logprob_fwd_workspace_size the partials stage runs
 * without the K split (the same bits, more time at few tiles per compute unit). */
LMH_API size_t lmhead_logprob_fwd_workspace_size_min(int64_t T, int64_t H, int64_t V);

/* Forward.  logprob is required; entropy and lse may be NULL (not computed / not written).
 * lse is what lmhead_logprob_bwd needs later. */
LMH_API lmh_status_t lmhead_logprob_fwd(const void* hidden, const void* weight, const int32_t* labels,
                                        int64_t T, int64_t H, int64_t V,
                                        float* logprob, float* entropy, float* lse,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The forward as its two stages (lmhead_logprob_fwd is exactly these two calls in order):
 *  1. _partials runs the vocabulary-tiled logit GEMM and writes, into the workspace, one record
 *     per (row, vocabulary chunk): (chunk max, count of logits equal to it, sum of exp(z - max)
 *     over logits below it, sum of exp(z - max)(z - max)) plus the label's logit.
 *  2. _finalize folds each row's records in a fixed order and writes the outputs.
 * The workspace contents between the stages are private to the library. */
LMH_API lmh_status_t lmhead_logprob_fwd_partials(const void* hidden, const void* weight, const int32_t* labels,
                                                 int64_t T, int64_t H, int64_t V,
                                                 void* workspace, size_t workspace_bytes, hipStream_t stream);
LMH_API lmh_status_t lmhead_logprob_fwd_finalize(const int32_t* labels, int64_t T, int64_t H, int64_t V,
                                                 float* logprob, float* entropy, float* lse,
                                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace for lmhead_logprob_bwd's fastest schedule.  Returns 0 for invalid sizes.
 * The backward walks the vocabulary in steps; per step it keeps dz in bf16 twice (token-major and
 * vocabulary-major, 4 * T bytes per vocabulary row) and the step's weight rows transposed, plus the
 * transposed hidden once (2 * H * T bytes).  The fastest step is 65536 rows (about 1.8 GB at
 * T = 4096, H = 5120).  A smaller workspace is accepted down to the size for a 256-row step
 * (lmhead_logprob_bwd_workspace_size_step(T, H, V, 256)): the call then takes a step, a multiple
 * of 256 rows whose buffers fit the bytes given (the widest, or one down to half as wide that
 * keeps the compute units busier).  The results are the same bits for every step width. */
LMH_API size_t lmhead_logprob_bwd_workspace_size(int64_t T, int64_t H, int64_t V);

/* Bytes of workspace the backward needs with a vocabulary step of `step` rows (rounded up to a
 * multiple of 256, at most 65536).  Returns 0 for invalid sizes or step <= 0. */
LMH_API size_t lmhead_logprob_bwd_workspace_size_step(int64_t T, int64_t H, int64_t V, int64_t step);

/* Backward of sum_t grad_logprob_t * logprob_t (entropy has no gradient).
 * dz_tj = g_t * ([j == y_t] - exp(z_tj - lse_t)), the logits being recomputed (SkyRL PR #1765:
 * design commit, recompute the per-chunk logits in backward; streaming-backward commit, the
 * -p*g term plus the label term).  dz is rounded to bf16 before the two gradient GEMMs.
 *   grad_hidden [T,H] fp32 = dz . weight   (written, or NULL to skip)
 *   grad_weight [V,H] fp32 = dz^T . hidden (overwritten if accumulate_grad_weight == 0, else
 *                                            added to; NULL to skip)
 * lse must be the lse[T] written by lmhead_logprob_fwd for the same inputs.  The backward also
 * needs T < 2^22 (LMH_ERR_UNSUPPORTED otherwise).  T == 0 leaves the gradient buffers untouched.
 * grad_hidden is bitwise invariant to how rows are split across calls.  grad_weight is
 * deterministic; splitting the rows at multiples of 64 and accumulating the parts in order with
 * accumulate_grad_weight = 1 reproduces one call bit for bit. */
LMH_API lmh_status_t lmhead_logprob_bwd(const void* hidden, const void* weight, const int32_t* labels,
                                        int64_t T, int64_t H, int64_t V,
                                        const float* grad_logprob, const float* lse,
                                        float* grad_hidden, float* grad_weight, int accumulate_grad_weight,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- Extended entry points -------------------------------------------------------------------
 *
 * Temperature.  `temperature` (fp32, finite, > 0; otherwise LMH_ERR_INVALID_ARG) divides every
 * fp32 logit before the softmax, so logprob, entropy, lse and sum_p2 are those of
 * softmax(z / temperature), and the backward carries the chain-rule factor 1/temperature.  The
 * division is an fp32 IEEE division of the fp32 logit by the caller's fp32 temperature — never
 * by a bf16-rounded temperature (verl PR #8026 "batch-invariant actor forward and sampler
 * log-prob formula", review on the temperature order: dividing bf16 logits by a temperature cast
 * to bf16 changes every token; the sampler divides fp32 logits by the fp32 temperature).
 * temperature == 1 gives exactly the bits of the plain entry points.
 *
 * sum_p2 [T] (or NULL): sum_j p_tj^2 of the same softmax, fp32 (verl PR #8026, first review:
 * sum_pi_squared is computed next to the entropy from the same logits).
 *
 * Entropy gradient: grad_entropy [T] (or NULL) is the upstream gradient of the entropies; the
 * logit gradient then also carries -grad_entropy_t * p_tj * (log p_tj + entropy_t), with
 * entropy [T] the forward's entropy output for the same inputs and temperature (required when
 * grad_entropy is given).  The pages leave this gradient unwired (SkyRL PR #1765 "[megatron]
 * Triton backend for fused LM-head log-prob", PR summary); it is the derivative of the entropy
 * definition above.
 */
LMH_API lmh_status_t lmhead_logprob_fwd_ex(const void* hidden, const void* weight, const int32_t* labels,
                                           int64_t T, int64_t H, int64_t V, float temperature,
                                           float* logprob, float* entropy, float* lse, float* sum_p2,
                                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Partials stage over one vocabulary shard.  The weight rows given (`weight` [V,H]) are the
 * vocabulary ids [vocab_start, vocab_start + V) of a vocabulary of vocab_total ids; the
 * workspace is sized for vocab_total (lmhead_logprob_fwd_workspace_size(T, H, vocab_total)) and
 * this call writes the records of its own 128-row chunks only, plus the label logit of every row
 * whose label falls in its rows.  Running the shards of a vocabulary in any order into one
 * workspace, then lmhead_logprob_fwd_finalize_ex with vocab_total, gives the bits of one call on
 * the whole weight.  A tensor-parallel caller exchanges the record rows of its shard instead (the
 * vocabulary-sharded layout of SkyRL PR #1765: each rank holds a slice of the LM head and only
 * the owner of a label contributes its logit).  Requirements: vocab_start a multiple of 128;
 * vocab_start + V <= vocab_total (LMH_ERR_INVALID_ARG otherwise); V a multiple of 128 unless the
 * shard ends at vocab_total (LMH_ERR_UNSUPPORTED otherwise).  want_sum_p2 (0 or 1) records what
 * sum_p2 needs; finalize asked for sum_p2 after a shard was run without it writes NaN to sum_p2
 * (the workspace keeps one flag per 128-row chunk saying whether its squared sums were recorded). */
LMH_API lmh_status_t lmhead_logprob_fwd_partials_ex(const void* hidden, const void* weight, const int32_t* labels,
                                                    int64_t T, int64_t H, int64_t V, float temperature,
                                                    int64_t vocab_start, int64_t vocab_total, int want_sum_p2,
                                                    void* workspace, size_t workspace_bytes, hipStream_t stream);
LMH_API lmh_status_t lmhead_logprob_fwd_finalize_ex(const int32_t* labels, int64_t T, int64_t H, int64_t V,
                                                    float* logprob, float* entropy, float* lse, float* sum_p2,
                                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Backward with a temperature and an optional entropy gradient (see above); lse is the one the
 * forward wrote with the same temperature.  grad_logprob is required (pass zeros when only the
 * entropy carries a gradient).
 * Vocabulary shard: the weight rows given are the vocabulary ids [vocab_start, vocab_start + V)
 * and lse (and entropy) are those of the whole vocabulary, as lmhead_logprob_fwd_finalize_ex
 * writes them after all shards.  The label term is added only where the label lies in these rows
 * (on the other shards the row keeps -p g, the out-of-range rule: SkyRL PR #1765, only the owner
 * of a label contributes it).  grad_weight [V,H] receives the shard's rows, bitwise equal to those
 * rows of a call on the whole weight; grad_hidden [T,H] receives this shard's share, dz[:, rows] .
 * weight, which the caller adds over the shards (tensor-parallel: the all-reduce of grad_hidden).
 * vocab_start = 0 is the whole vocabulary.  vocab_start < 0 or vocab_start + V >= 2^31 - 2^16
 * gives LMH_ERR_INVALID_ARG. */
LMH_API lmh_status_t lmhead_logprob_bwd_ex(const void* hidden, const void* weight, const int32_t* labels,
                                           int64_t T, int64_t H, int64_t V, float temperature,
                                           int64_t vocab_start, const float* grad_logprob, const float* lse,
                                           const float* grad_entropy, const float* entropy,
                                           float* grad_hidden, float* grad_weight, int accumulate_grad_weight,
                                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- Allocation-free forward ---------------------------------------------------------------
 *
 * For callers that cannot allocate device memory or pass a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments and results as
 * lmhead_logprob_fwd (the same kernels, so the same bits) without the workspace: the library
 * keeps one built-in scratch array of LMH_NOALLOC_SCRATCH_BYTES per device, which each device
 * holds until the process ends.  The call makes no allocation of any kind.
 * Limit: lmhead_logprob_fwd_workspace_size_min(T, H, V) <= LMH_NOALLOC_SCRATCH_BYTES (20 bytes per
 * row and 128-row vocabulary chunk, about T * ceil(V / 128) <= 3.3e6, e.g. T <= 2823 at
 * V = 152064); larger calls return LMH_ERR_WORKSPACE_TOO_SMALL with nothing launched.
 * Every call on a device uses that device's one array: calls that may overlap on one device (on
 * different streams, or from different host threads without ordering) race and give undefined
 * results; calls ordered on one stream are safe.  The first call on a device looks up the array's
 * device address (hipGetSymbolAddress) and keeps it; the device is the current one. */
#define LMH_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
LMH_API lmh_status_t lmhead_logprob_fwd_noalloc(const void* hidden, const void* weight, const int32_t* labels,
                                                int64_t T, int64_t H, int64_t V,
                                                float* logprob, float* entropy, float* lse, hipStream_t stream);

/* Static English text for a status code (never NULL). */
LMH_API const char* lmhead_status_string(lmh_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* LMHEAD_LOGPROB_H */
