/*
 * libdllm_commit -- the per-step commit of masked (absorbing-state) diffusion-LM
 * decoding, for AMD Instinct MI355X (gfx950).
 *
 * One decoding step of a masked diffusion LM runs the model over the canvas,
 * proposes a token for every position, and commits a subset of the proposals
 * (mlx-arsenal research note "dLLM block decoding", section "The pattern").
 * This library is that commit: the token statistics of the logits and the
 * commit rules, as pure functions; the model and the decode loop stay with the
 * caller (same section: "the loop stays with the caller").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Return value: DLLM_OK (0) or a negative DLLM_ERR_* code.  On error nothing
 *    is launched and no output is touched; dllm_last_error() returns a message
 *    naming the offending argument (per calling thread).
 *  - Memory: every array is caller-owned, contiguous, row-major DEVICE memory,
 *    except where an argument says HOST.  The library never allocates, frees
 *    or synchronizes; it keeps no state between calls except the workspace the
 *    caller passes to dllm_token_stats.
 *  - Streams: work is enqueued on `stream` (0 = the null stream); results are
 *    valid once the stream has reached that point.
 *  - Shapes: B batch rows of L positions; position (b, l) is element b*L + l of
 *    every (B, L) array.  B = 0 or L = 0 returns DLLM_OK with no launch.
 *  - Masks are uint8: input masks treat any nonzero byte as true; output masks
 *    are written as 0 or 1 for every position.
 *  - Scores are float32.  A NaN score counts as the worst possible score: -inf
 *    for a confidence, +inf for an entropy.  -0.0 and +0.0 are equal.
 *  - Rankings are stable: equal scores order by lower position ("Deviations
 *    from the references": sorting is stable, the forced token is the first
 *    maximal one).
 *  - A batch row may hold at most DLLM_MAX_L positions for the ranking rules
 *    (threshold, topk, factor, entropy_bound); longer rows return
 *    DLLM_ERR_UNSUPPORTED.
 *  - dllm_token_stats / dllm_commit_step take at most (2^32 - 1) / 1024 = 4194303
 *    positions B * L per call (one workgroup per position or slice of a
 *    position); more return DLLM_ERR_UNSUPPORTED.
 */
#ifndef DLLM_COMMIT_H
#define DLLM_COMMIT_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  DLLM_OK = 0,
  DLLM_ERR_ARG = -1,          /* bad pointer, size, parameter or combination  */
  DLLM_ERR_DTYPE = -2,        /* unknown logits dtype                         */
  DLLM_ERR_SHAPE = -3,        /* workspace too small for the shape            */
  DLLM_ERR_HIP = -4,          /* a HIP call or kernel launch failed           */
  DLLM_ERR_UNSUPPORTED = -5   /* a size beyond what the library implements    */
};

enum { DLLM_F32 = 0, DLLM_BF16 = 1 };

#define DLLM_MAX_L 4096
#define DLLM_MAX_SUPPRESS 64
/* bytes of the library-owned workspace of dllm_commit_step_static, per GPU */
#define DLLM_STATIC_SCRATCH_BYTES (1u << 20)

enum {
  DLLM_RULE_THRESHOLD = 1,
  DLLM_RULE_TOPK = 2,
  DLLM_RULE_FACTOR = 3,
  DLLM_RULE_ENTROPY_BOUND = 4,
  DLLM_RULE_EDIT = 5
};

/* The confidence a fused THRESHOLD / TOPK / FACTOR rule ranks by (mojo-dllm
 * "The GPU path", row statistics paragraph: LLaDA and maskgit_plus use p,
 * topk_margin p minus the runner-up's probability, Dream the negative
 * entropy). */
enum {
  DLLM_SCORE_PROB = 0,          /* prob */
  DLLM_SCORE_MARGIN = 1,        /* margin (the margin output must be given) */
  DLLM_SCORE_NEG_ENTROPY = 2    /* -entropy */
};

/* One commit rule run inside dllm_token_stats on the statistics it has just
 * computed (same launch).  The result is identical to calling the matching
 * dllm_transfer_* function on dllm_token_stats' outputs.
 *   kind    DLLM_RULE_*.
 *   mask    (B, L) uint8: the candidates (for EDIT: the editable positions).
 *   out     (B, L) uint8: the commit mask (for EDIT: the edit mask); must not
 *           alias any other array of the call.
 *   param   tau (THRESHOLD), f (FACTOR), gamma (ENTROPY_BOUND), tau_edit (EDIT);
 *           ignored for TOPK.  Must not be NaN.
 *   strict  THRESHOLD only: 0 -> conf >= tau, 1 -> conf > tau.
 *   k       TOPK only: (B,) int32 quotas.
 *   tokens  EDIT only: (B, L) int32 current canvas.
 *   score   THRESHOLD / FACTOR / TOPK: DLLM_SCORE_* (0 = prob); must be 0 for
 *           the other kinds.
 *   taus    THRESHOLD only: (B,) float64 DEVICE, one threshold per batch row
 *           (used in place of param), or NULL.  The entries are read by the
 *           kernel and must not be NaN (a NaN entry passes no candidate, so its
 *           row commits only the forced one).  Per-row threshold schedules:
 *           mlxcel "Block Diffusion", "LLaDA-2 Block Unmasking".
 * THRESHOLD / FACTOR / TOPK rank by the score (prob by default), ENTROPY_BOUND
 * by entropy, EDIT uses x0, prob and tokens.  Zero-fill the struct before
 * setting its fields. */
typedef struct {
  int kind;
  const uint8_t *mask;
  uint8_t *out;
  double param;
  int strict;
  const int32_t *k;
  const int32_t *tokens;
  int score;
  const double *taus;
} dllm_rule;

/* Optional outputs and options of dllm_token_stats / dllm_commit_step.
 *   margin   (B, L) float32 DEVICE output, or NULL: p_(1) - p_(2) of the
 *            softmax over the unsuppressed ids, the topk_margin confidence
 *            (mojo-dllm "The GPU path": p minus the runner-up's probability,
 *            the runner-up being the largest logit at any index but the first
 *            maximal one; a tie gives 0, one unsuppressed id gives 1), whatever
 *            x0 is.
 *   argmax   (B, L) int32 DEVICE output, or NULL: the first index of the
 *            largest logit, also when x0 is sampled (the DiffusionGemma loop of
 *            mlx-arsenal "Uniform-noise decoding (DiffusionGemma)" keeps both
 *            the argmax canvas and a categorical sample).
 *   stats_temperature  0 (none) or Ts > 0, finite: prob, entropy and margin
 *            are those of softmax(logits / Ts) (that loop measures entropy on
 *            the temperature-scaled logits); x0 and argmax do not depend on
 *            it.  With temperature = Ts too, x0 is a categorical sample of
 *            softmax(logits / Ts).
 * Zero-fill the struct before setting its fields. */
typedef struct {
  float *margin;
  int32_t *argmax;
  float stats_temperature;
} dllm_stats_extra;

/* ---------------------------------------------------------------------------
 * dllm_token_stats -- per position: the proposed token x0, its probability and
 * the entropy of the position's distribution (mlx-arsenal "dLLM block
 * decoding", "What mlx-arsenal ships", token_stats row: float32, NaN-safe,
 * greedy or Gumbel-max sampling with an explicit key, suppress_ids).
 *
 *   logits       (B, L, V) DEVICE, dtype DLLM_F32 or DLLM_BF16; the logits of
 *                position (b, l) start at element (b*L + l) * row_stride.
 *   row_stride   elements between consecutive positions, >= V.
 *   temperature  0 -> greedy: x0 is the first index of the largest logit.
 *                > 0 -> Gumbel-max: x0 is the first index of the largest
 *                logit/temperature + g, g = -log(-log u) with u drawn by
 *                Philox4x32-10 (Salmon et al., SC'11) under key (seed low 32,
 *                seed high 32) at counter (v/4, l, b, step), word v%4, and
 *                u = ((word >> 9) + 0.5) * 2^-23.  Must be finite and >= 0.
 *   seed, step   the noise key and the per-step counter word; step < 2^32.
 *                Ignored when temperature == 0.
 *   suppress_ids HOST array of n_suppress distinct ids in [0, V) removed before
 *                the softmax; n_suppress <= DLLM_MAX_SUPPRESS and < V; may be
 *                NULL when n_suppress == 0.
 *   x0           (B, L) int32 DEVICE output.
 *   prob         (B, L) float32 DEVICE output: softmax(logits)[x0], untempered.
 *   entropy      (B, L) float32 DEVICE output: -sum p log p of softmax(logits)
 *                over the unsuppressed ids (natural log), untempered.
 *   extra        HOST struct of optional outputs and options, or NULL (all
 *                off): see dllm_stats_extra.
 *   rules        HOST array of n_rules (0..2) rules fused into the same launch,
 *                or NULL.  At most one rule of each kind.
 *   workspace    DEVICE scratch of at least dllm_token_stats_workspace_size()
 *                bytes for this shape, zero-filled by the caller before its
 *                first use; every successful call leaves it zero-filled again,
 *                so it can be reused by later calls on the same stream.  Two
 *                calls in flight at once must not share a workspace.
 *
 * NaN safety: a NaN logit counts as -inf.  A position whose unsuppressed
 * logits are all -inf is uniform over the unsuppressed ids; a position with
 * +inf logits is uniform over its +inf ids.  No output is ever NaN.
 * -------------------------------------------------------------------------*/
int dllm_token_stats(const void *logits, int dtype, int64_t B, int64_t L,
                     int64_t V, int64_t row_stride, float temperature,
                     uint64_t seed, uint64_t step,
                     const int32_t *suppress_ids, int n_suppress,
                     int32_t *x0, float *prob, float *entropy,
                     const dllm_stats_extra *extra,
                     const dllm_rule *rules, int n_rules,
                     void *workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* Bytes of workspace dllm_token_stats needs for this shape on the current
 * device (a pure function of the arguments and the device).  Returns 0 on bad
 * arguments. */
size_t dllm_token_stats_workspace_size(int dtype, int64_t B, int64_t L,
                                       int64_t V);

/* ---------------------------------------------------------------------------
 * dllm_commit_step: one step of the decoding loops, in one launch.
 *
 * The loops of mlx-arsenal "dLLM block decoding" (the block loop of section
 * "The pattern" and the loop of section "Token editing (LLaDA2.1)") do, per
 * step: statistics, a commit rule over the masked candidates, an edit rule
 * over the committed positions of the block, then x <- where(commit | edit,
 * x0, x), and test on the host whether a mask is left and whether anything
 * was edited.  mojo-dllm ("Why the runtime looks different", few rows need
 * logits) computes logits only for the candidate rows.  This call does all of
 * it on the device:
 *   - exactly dllm_token_stats with the same rules (at most one ranking rule
 *     and at most one edit rule), on the same workspace;
 *   - with skip_rows != 0, a position that is in no rule's mask is not read:
 *     its x0, prob and entropy are left as they were (its logits may be
 *     anything), and its edit output is 0;
 *   - with tokens != NULL, tokens[b, l] = x0[b, l] wherever the ranking rule
 *     committed or the edit rule edited; other tokens are left as they were;
 *   - with counts != NULL, counts[2b] = candidates of the ranking rule left
 *     uncommitted in batch row b (0 without one) and counts[2b + 1] =
 *     positions edited in batch row b.  counts may be device memory or
 *     host-pinned memory mapped into the device's address space (then
 *     readable on the host once the stream has passed this call).
 *
 *   tokens  (B, L) int32 DEVICE, read and written (the edit rule's current
 *           tokens: an edit rule's own tokens pointer must be NULL or this).
 *   counts  (B, 2) int32, written.
 * tokens and counts must not alias any other array of the call.
 * Errors: as dllm_token_stats, plus DLLM_ERR_ARG for a NULL canvas, two
 * ranking rules, or aliasing.
 * -------------------------------------------------------------------------*/
typedef struct {
  int32_t *tokens;   /* (B, L) canvas updated in place, or NULL */
  int32_t *counts;   /* (B, 2) left / edited per batch row, or NULL */
  int skip_rows;     /* nonzero: rows in no rule's mask are not read */
} dllm_canvas;

int dllm_commit_step(const void *logits, int dtype, int64_t B, int64_t L,
                     int64_t V, int64_t row_stride, float temperature,
                     uint64_t seed, uint64_t step,
                     const int32_t *suppress_ids, int n_suppress,
                     int32_t *x0, float *prob, float *entropy,
                     const dllm_stats_extra *extra,
                     const dllm_rule *rules, int n_rules,
                     const dllm_canvas *canvas,
                     void *workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* dllm_commit_step with no workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops and
 * harnesses that forbid hipMalloc).  It allocates nothing: the counters and
 * split-row partials live in a library-owned device array of
 * DLLM_STATIC_SCRATCH_BYTES on each GPU, part of the library's code object
 * and held until the process ends.  Arguments, layouts and errors are those
 * of dllm_commit_step, plus DLLM_ERR_UNSUPPORTED when the shape needs more
 * than DLLM_STATIC_SCRATCH_BYTES (the need is
 * dllm_token_stats_workspace_size(dtype, B, L, V)), checked before anything
 * is launched.  Every call on one GPU shares that GPU's array: calls that can
 * overlap (issued on two streams, or from two host threads without ordering)
 * race and give wrong results; calls on one stream are ordered and safe.
 * Each call leaves the array zero-filled, which the next call needs; the
 * first call on a device also clears it once, with one small kernel on
 * `stream`. */
int dllm_commit_step_static(const void *logits, int dtype, int64_t B, int64_t L,
                            int64_t V, int64_t row_stride, float temperature,
                            uint64_t seed, uint64_t step,
                            const int32_t *suppress_ids, int n_suppress,
                            int32_t *x0, float *prob, float *entropy,
                            const dllm_stats_extra *extra,
                            const dllm_rule *rules, int n_rules,
                            const dllm_canvas *canvas, hipStream_t stream);

/* threshold_transfer ("What mlx-arsenal ships", threshold_transfer row; mlxcel
 * "Block Diffusion", "LLaDA-2 Block Unmasking"): per batch row, commit every
 * candidate with conf >= tau (conf > tau when strict != 0); if no candidate
 * passes, commit exactly one, the first candidate of maximal confidence.
 * conf (B, L) float32, cand (B, L) uint8, commit (B, L) uint8 out.  tau not NaN. */
int dllm_transfer_threshold(const float *conf, const uint8_t *cand, int64_t B,
                            int64_t L, double tau, int strict, uint8_t *commit,
                            hipStream_t stream);

/* dllm_transfer_threshold with one threshold per batch row: taus (B,) float64
 * DEVICE, taus[b] in place of tau for row b (mlxcel "Block Diffusion",
 * "LLaDA-2 Block Unmasking": per-row thresholds, e.g. rows at different steps
 * of a decaying schedule).  The entries must not be NaN (not checked: a NaN
 * entry passes no candidate and its row commits only the forced one). */
int dllm_transfer_threshold_rows(const float *conf, const uint8_t *cand, const double *taus,
                                 int64_t B, int64_t L, int strict, uint8_t *commit,
                                 hipStream_t stream);

/* The linearly decaying confidence threshold (mlxcel "Block Diffusion",
 * "LLaDA-2 Block Unmasking": an initial and a floor threshold, 0.95 by
 * default, with an optional linear decay): *out = max(tau_floor, tau_initial -
 * decay * step), computed in double on the host.  step >= 0; no argument may
 * be NaN.  Returns DLLM_ERR_ARG otherwise. */
int dllm_decaying_threshold(double tau_initial, double tau_floor, double decay, int64_t step,
                            double *out);

/* topk_transfer (topk_transfer row; mojo-dllm "The loop LLaDA uses"): commit
 * the k[b] most confident candidates of batch row b.  k (B,) int32 DEVICE;
 * k[b] <= 0 commits nothing, k[b] >= #candidates commits all of them. */
int dllm_transfer_topk(const float *conf, const uint8_t *cand, const int32_t *k,
                       int64_t B, int64_t L, uint8_t *commit,
                       hipStream_t stream);

/* factor_transfer (factor_transfer row; "Deviations": no off-by-one): sort the
 * candidates by decreasing confidence c_(0) >= c_(1) >= ...; commit the longest
 * prefix on which (i + 1) * (1 - c_(i)) <= f, evaluated exactly, and at least
 * one candidate.  f not NaN. */
int dllm_transfer_factor(const float *conf, const uint8_t *cand, int64_t B,
                         int64_t L, double f, uint8_t *commit,
                         hipStream_t stream);

/* entropy_bound_transfer (entropy_bound_transfer row; mlxcel "Samplers and
 * Reveal Policies": at least one accepted): sort the candidates by increasing
 * entropy H_(0) <= H_(1) <= ...; commit the longest prefix on which the
 * exclusive sum sum_{j<i} H_(j) <= gamma, evaluated exactly, and at least one
 * candidate.  gamma not NaN. */
int dllm_transfer_entropy_bound(const float *entropy, const uint8_t *cand,
                                int64_t B, int64_t L, double gamma,
                                uint8_t *commit, hipStream_t stream);

/* edit_transfer (edit_transfer row; "Token editing (LLaDA2.1)"): edit[b, l] =
 * editable[b, l] && x0[b, l] != tokens[b, l] && prob[b, l] > tau_edit (strict;
 * nothing is forced).  tau_edit not NaN. */
int dllm_transfer_edit(const int32_t *x0, const float *prob,
                       const int32_t *tokens, const uint8_t *editable,
                       int64_t B, int64_t L, double tau_edit, uint8_t *edit,
                       hipStream_t stream);

/* transfer_schedule (transfer_schedule row; mojo-dllm "The loop LLaDA uses":
 * masked positions spread over the steps evenly): schedule[b, s] =
 * n/steps + (s < n % steps ? 1 : 0) with n = max(n_masked[b], 0).
 * n_masked (B,) int32 DEVICE, schedule (B, steps) int32 DEVICE out, steps >= 1. */
int dllm_transfer_schedule(const int32_t *n_masked, int64_t B, int32_t steps,
                           int32_t *schedule, hipStream_t stream);

/* block_ranges (block_ranges row: prompt-relative or absolute-aligned; the
 * aligned loop of "Token editing (LLaDA2.1)"): the [start, end) blocks covering
 * the generation region [prompt_len, prompt_len + gen_len).  align == 0: blocks
 * start at prompt_len; align != 0: blocks are aligned on multiples of
 * block_len, the first one starting at floor(prompt_len / block_len) *
 * block_len.  The last block ends at prompt_len + gen_len; gen_len == 0 gives
 * no block.  HOST only.  Writes min(count, cap) pairs to out[2i], out[2i+1]
 * (out may be NULL when cap == 0) and returns the number of blocks, or a
 * negative DLLM_ERR_* code. */
int64_t dllm_block_ranges(int64_t prompt_len, int64_t gen_len,
                          int64_t block_len, int align, int64_t *out,
                          int64_t cap);

/* block_causal_mask (mlx_arsenal.attention.block_causal_mask: bidirectional
 * inside a block, causal across blocks, aligned on absolute positions;
 * "Mask conventions": additive, 0 attend, -inf blocked): out[q, k] = 0.0f if
 * k / block_len <= q / block_len, else -inf.  out (L, L) float32 DEVICE. */
int dllm_block_causal_mask(int64_t L, int64_t block_len, float *out,
                           hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Uniform-noise decoding (mlx-arsenal "dLLM block decoding", function table
 * row linear_temperature / uniform_canvas / renoise / StableConfidentStopping,
 * and the loop of "Uniform-noise decoding (DiffusionGemma)"; mlxcel "Block
 * Diffusion", "DiffusionGemma Canvas Denoising").  One step of that loop is a
 * dllm_token_stats launch with temperature = stats_temperature = T (x0 the
 * categorical sample, extra->argmax the argmax canvas, entropy of the scaled
 * logits) and a fused entropy_bound rule over every position, then
 * dllm_uniform_canvas + dllm_renoise for the new canvas and
 * dllm_stable_confident_stop for the per-row stop.
 * -------------------------------------------------------------------------*/

/* linear_temperature: *out = t_min + (t_max - t_min) * remaining / num_steps
 * (the temperature falls linearly with the remaining steps: t_max when
 * remaining = num_steps).  0 <= remaining <= num_steps, num_steps >= 1.
 * Host only. */
int dllm_linear_temperature(int remaining, int num_steps, double t_min,
                            double t_max, double *out);

/* uniform_canvas: out[b, l] uniform on [0, V): with w the four words of
 * Philox4x32-10 (key = seed low 32, seed high 32) at counter
 * (l, b, 0xFFFFFFFF, draw) and x = w0 + 2^32 w1, out = floor(x V / 2^64)
 * (bias at most V / 2^64).  draw < 2^32 picks an independent canvas (the
 * sampling noise of dllm_token_stats never uses counter word 2 = 0xFFFFFFFF).
 * out (B, L) int32 DEVICE; V in [1, 2^31). */
int dllm_uniform_canvas(int32_t *out, int64_t B, int64_t L, int64_t V,
                        uint64_t seed, uint64_t draw, hipStream_t stream);

/* renoise: out = where(accepted, sample, noise).  sample, noise, out (B, L)
 * int32 DEVICE (out may be sample or noise); accepted (B, L) uint8. */
int dllm_renoise(const int32_t *sample, const uint8_t *accepted,
                 const int32_t *noise, int64_t B, int64_t L, int32_t *out,
                 hipStream_t stream);

/* StableConfidentStopping: per batch row, stable_steps[b] counts the
 * consecutive calls whose argmax row equals the previous call's (0 on the
 * first call, first != 0); the row is confident when the mean of its L
 * entropies is at most confidence_threshold (sum <= c L in the extended
 * reals, finite terms summed exactly: a NaN, or +inf with -inf, is never
 * confident; a +inf term only for c = +inf; a -inf term always; L = 0
 * compares 0 with 0); done[b] |= (stable_steps[b] >=
 * stability_threshold && confident).  prev_argmax (B, L) int32 and
 * stable_steps (B,) int32 are the caller's state, updated in place; done (B,)
 * uint8 in/out.  stability_threshold >= 0, confidence_threshold not NaN. */
int dllm_stable_confident_stop(const int32_t *argmax, const float *entropy,
                               int64_t B, int64_t L, int stability_threshold,
                               double confidence_threshold, int first,
                               int32_t *prev_argmax, int32_t *stable_steps,
                               uint8_t *done, hipStream_t stream);

/* Measurement helper, not a step of the commit: the stage timestamps of the
 * last dllm_token_stats / dllm_commit_step launch (of either launch shape)
 * in a library built with stage timestamps (libdllm_commit_stages.so, built by
 * `python -m commit_step_amd.build --stages`; the product library returns
 * DLLM_ERR_UNSUPPORTED).  Thread 0 of each of the first 4096 workgroups
 * records the device's 100 MHz real-time counter at 16 stage slots: start,
 * stream end, slice counted, row merged, published, batch row counted, batch
 * row done, row skipped, finalized, stores drained, rule inputs loaded,
 * candidates ranked, 4 unused; dst[16 g + k] is workgroup g's stage k, 0 where
 * it did not pass that stage.  clear != 0: zero the records (call before the
 * launch); clear == 0: copy them into dst (HOST, n >= 16 * 4096).
 * Synchronous. */
int dllm_stage_timestamps(uint64_t *dst, size_t n, int clear);

/* Measurement helper, not a step of the commit: a plain streaming read of
 * `bytes` bytes at `buf` (DEVICE, 16-byte aligned, bytes a positive multiple
 * of 16) with the logit pass's 16-byte non-temporal loads, workgroup g reading
 * the g-th of `workgroups` equal contiguous chunks with `threads` (256 or 512)
 * threads.  It writes nothing but, in the rare case that a lane's xor of the
 * words it read equals 0x9E3779B9, sets bit 0 of *sink (DEVICE uint32).
 * Timing it over the logit buffers gives the read ceiling the logit pass is
 * compared with. */
int dllm_read_probe(const void *buf, int64_t bytes, int64_t workgroups, int threads,
                    uint32_t *sink, hipStream_t stream);

/* Message describing the last error returned on the calling thread ("" if
 * none). */
const char *dllm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DLLM_COMMIT_H */
