// dllm_token_stats and dllm_commit_step: host side (validation, workspace,
// launch plan) and the plain statistics kernels.  The kernels themselves are
// in token_stats_dev.h.
#include <stdarg.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "token_stats_dev.h"

namespace dllm {

// ---------------------------------------------------------------- host side

namespace {

Plan make_plan(int dtype, int64_t rows, int64_t V, int64_t row_stride, const void *logits) {
  const int esz = dtype == DLLM_BF16 ? 2 : 4;
  const int vecn = 16 / esz;
  Plan p;
  p.vec = ((uintptr_t)logits % 16 == 0) && ((row_stride * esz) % 16 == 0) && (V % vecn == 0);
  // Rows that are not all 16-byte aligned or not a whole number of 16-byte
  // loads: stream each slice's aligned body with 16-byte loads and its head
  // and tail by element.
  p.split = !p.vec && ((uintptr_t)logits % esz == 0);
  const int cus = device_cu_count();
  // Many rows -> 256-thread groups; a few long rows -> 512-thread groups
  // (measured best on the 256 x 262144 canvas, one row per CU: 8 waves with
  // one 16-byte-load chunk in flight each; more waves or slices per row
  // streamed slower).
  if (rows >= 4LL * cus || V < 16384) p.nt = 256;
  else p.nt = 512;
  p.slices = 1;
  const int64_t wgs = rows;
  if (wgs < cus && V >= 8192) {
    int64_t s = (cus + rows - 1) / rows;
    const int64_t min_slice = 4096;               // keep slices worth a launch
    s = std::min<int64_t>(s, std::max<int64_t>(1, V / min_slice));
    s = std::min<int64_t>(s, kMaxSlices);
    p.slices = (int)std::max<int64_t>(1, s);
  }
  int64_t sl = (V + p.slices - 1) / p.slices;
  sl = (sl + 7) / 8 * 8;
  p.slice_len = sl;
  p.slices = (int)((V + sl - 1) / sl);
  return p;
}

// Workspace: batch-row counters [B], edit counts [B], then for split rows the
// row counters [B*L] and the partials [B*L*slices], each region 256-byte aligned.
size_t workspace_bytes_for(int64_t B, int64_t L, int slices) {
  size_t bytes = 2 * (((size_t)B * 4 + 255) / 256 * 256);
  if (slices > 1) {
    bytes += ((size_t)B * L * 4 + 255) / 256 * 256;
    bytes += (size_t)B * L * slices * sizeof(Partial);
  }
  return bytes;
}

// Dispatch on the plan's (threads, loads per chunk).
template <typename T>
int launch_plan(const Plan &p, const StatsArgs &a, int64_t rows, bool sample, size_t smem,
                hipStream_t s, const char *who) {
  constexpr int U0 = ElemT<T>::U;
  if (p.nt == 512) return launch_f<T, 512, U0, false>(p, a, rows, sample, smem, s, who);
  return launch_f<T, 256, U0, false>(p, a, rows, sample, smem, s, who);
}

}  // namespace

// Host helper shared with the transfer entry points: validates a rule and
// fills its device view.
int prepare_rule(const dllm_rule &r, RuleDev &d, int64_t B, int64_t L, const char *who);

}  // namespace dllm

using namespace dllm;

#ifdef DLLM_STAGE_TIMESTAMPS
namespace dllm {
DLLM_STAGE_COPY_IMPL(stage_ts_copy_plain)
}  // namespace dllm
#endif

extern "C" int dllm_stage_timestamps(uint64_t *dst, size_t n, int clear) {
#ifdef DLLM_STAGE_TIMESTAMPS
  const size_t slots = (size_t)kStageWorkgroups * kStages;
  if (clear) {
    if (stage_ts_copy_plain(nullptr, true) != hipSuccess ||
        stage_ts_copy_full(nullptr, true) != hipSuccess)
      return fail(DLLM_ERR_HIP, "dllm_stage_timestamps: clearing failed");
    return ok();
  }
  if (!dst || n < slots)
    return fail(DLLM_ERR_ARG, "dllm_stage_timestamps: dst needs %zu slots", slots);
  static uint64_t other[(size_t)kStageWorkgroups * kStages];
  if (stage_ts_copy_plain(dst, false) != hipSuccess ||
      stage_ts_copy_full(other, false) != hipSuccess)
    return fail(DLLM_ERR_HIP, "dllm_stage_timestamps: copy failed");
  for (size_t i = 0; i < slots; ++i)           // one of the two kernel families ran
    if (other[i]) dst[i] = other[i];
  return ok();
#else
  (void)dst; (void)n; (void)clear;
  return fail(DLLM_ERR_UNSUPPORTED,
              "dllm_stage_timestamps: the library was built without stage timestamps");
#endif
}

extern "C" size_t dllm_token_stats_workspace_size(int dtype, int64_t B, int64_t L, int64_t V) {
  if ((dtype != DLLM_F32 && dtype != DLLM_BF16) || B < 0 || L < 0 || V < 1) return 0;
  const Plan p = make_plan(dtype, B * L, V, V, nullptr);
  return workspace_bytes_for(B, L, p.slices);
}

namespace {

// Both entry points: validation, workspace layout and the launch.  `canvas`
// is NULL for dllm_token_stats.
int stats_step(const char *who, const void *logits, int dtype, int64_t B, int64_t L, int64_t V,
               int64_t row_stride, float temperature, uint64_t seed, uint64_t step,
               const int32_t *suppress_ids, int n_suppress, int32_t *x0, float *prob,
               float *entropy, const dllm_stats_extra *extra, const dllm_rule *rules,
               int n_rules, const dllm_canvas *canvas,
               void *workspace, size_t workspace_bytes, hipStream_t stream) {
  if (dtype != DLLM_F32 && dtype != DLLM_BF16)
    return fail(DLLM_ERR_DTYPE, "%s: dtype %d is neither DLLM_F32 nor DLLM_BF16", who, dtype);
  if (B < 0 || L < 0) return fail(DLLM_ERR_ARG, "%s: B and L must be >= 0", who);
  if (V < 1 || V > 0x7fffffffLL)
    return fail(DLLM_ERR_ARG, "%s: V = %lld must be in [1, 2^31)", who, (long long)V);
  if (row_stride < V) return fail(DLLM_ERR_ARG, "%s: row_stride < V", who);
  if (!(temperature >= 0.0f) || temperature == __builtin_inff())
    return fail(DLLM_ERR_ARG, "%s: temperature must be finite and >= 0", who);
  if (step > 0xffffffffull) return fail(DLLM_ERR_ARG, "%s: step must be < 2^32", who);
  if (n_suppress < 0 || n_suppress > DLLM_MAX_SUPPRESS)
    return fail(DLLM_ERR_ARG, "%s: n_suppress must be in [0, %d]", who, DLLM_MAX_SUPPRESS);
  if (n_suppress > 0 && !suppress_ids)
    return fail(DLLM_ERR_ARG, "%s: suppress_ids is NULL", who);
  if (n_rules < 0 || n_rules > kMaxRules || (n_rules > 0 && !rules))
    return fail(DLLM_ERR_ARG, "%s: n_rules must be 0..%d with a rules array", who, kMaxRules);
  if (B == 0 || L == 0) return ok();
  if (!logits || !x0 || !prob || !entropy)
    return fail(DLLM_ERR_ARG, "%s: logits, x0, prob and entropy must be non-NULL", who);
  float *margin = extra ? extra->margin : nullptr;
  int32_t *argmax = extra ? extra->argmax : nullptr;
  float stats_t = extra ? extra->stats_temperature : 0.0f;
  if (stats_t == 0.0f) stats_t = 1.0f;
  if (!(stats_t > 0.0f) || stats_t == __builtin_inff())
    return fail(DLLM_ERR_ARG, "%s: stats_temperature must be 0 (none) or finite and > 0", who);

  StatsArgs a;
  memset(&a, 0, sizeof(a));
  // suppress ids: sorted, distinct, in range, not every id
  for (int i = 0; i < n_suppress; ++i) {
    const int32_t s = suppress_ids[i];
    if (s < 0 || s >= V)
      return fail(DLLM_ERR_ARG, "%s: suppress id %d is outside [0, V)", who, s);
    int j = i;
    while (j > 0 && a.suppress[j - 1] > s) { a.suppress[j] = a.suppress[j - 1]; --j; }
    a.suppress[j] = s;
  }
  for (int i = 1; i < n_suppress; ++i)
    if (a.suppress[i] == a.suppress[i - 1])
      return fail(DLLM_ERR_ARG, "%s: suppress id %d appears twice", who, a.suppress[i]);
  if (n_suppress >= V) return fail(DLLM_ERR_ARG, "%s: every id is suppressed", who);
  int first_allowed = 0;
  for (int i = 0; i < n_suppress && a.suppress[i] == first_allowed; ++i) ++first_allowed;

  // rules
  bool seen[6] = {false, false, false, false, false, false};
  const void *outs[kMaxRules] = {nullptr, nullptr};
  for (int i = 0; i < n_rules; ++i) {
    const dllm_rule &r = rules[i];
    if (r.kind < DLLM_RULE_THRESHOLD || r.kind > DLLM_RULE_EDIT)
      return fail(DLLM_ERR_ARG, "%s: rules[%d].kind = %d is not a DLLM_RULE_*", who, i, r.kind);
    if (seen[r.kind]) return fail(DLLM_ERR_ARG, "%s: rule kind %d appears twice", who, r.kind);
    seen[r.kind] = true;
    outs[i] = r.out;
    if (r.out == (const void *)x0 || r.out == (const void *)prob || r.out == (const void *)entropy ||
        (margin && r.out == (const void *)margin) || (argmax && r.out == (const void *)argmax) ||
        r.out == (const void *)r.mask || r.out == (const void *)logits ||
        (r.taus && r.out == (const void *)r.taus))
      return fail(DLLM_ERR_ARG, "%s: rules[%d].out aliases another array", who, i);
    if (r.taus && r.kind != DLLM_RULE_THRESHOLD)
      return fail(DLLM_ERR_ARG, "%s: only the threshold rule takes per-row thresholds", who);
    if (r.kind == DLLM_RULE_EDIT) {
      const bool canvas_tokens = canvas && canvas->tokens;
      if (!r.mask || !r.out || (!r.tokens && !canvas_tokens))
        return fail(DLLM_ERR_ARG, "%s: edit rule needs mask, out and tokens", who);
      if (canvas_tokens && r.tokens && r.tokens != canvas->tokens)
        return fail(DLLM_ERR_ARG, "%s: the edit rule's tokens must be the canvas", who);
      if (r.param != r.param) return fail(DLLM_ERR_ARG, "%s: tau_edit is NaN", who);
      a.has_edit = 1;
      a.edit_mask = r.mask;
      a.edit_out = r.out;
      a.edit_tokens = r.tokens ? r.tokens : canvas->tokens;
      a.edit_tau = r.param;
    } else {
      if (L > DLLM_MAX_L)
        return fail(DLLM_ERR_UNSUPPORTED, "%s: L = %lld exceeds DLLM_MAX_L = %d", who,
                    (long long)L, DLLM_MAX_L);
      const int rc = prepare_rule(r, a.rank_rules[a.n_rank_rules], B, L, who);
      if (rc != DLLM_OK) return rc;
      if (r.score == DLLM_SCORE_MARGIN && !margin)
        return fail(DLLM_ERR_ARG, "%s: a rule ranks by margin but the margin output is NULL", who);
      ++a.n_rank_rules;
    }
  }
  if (n_rules == 2 && outs[0] == outs[1])
    return fail(DLLM_ERR_ARG, "%s: the two rules share an output", who);
  if (canvas) {
    if (a.n_rank_rules > 1)
      return fail(DLLM_ERR_ARG, "%s: a canvas step takes at most one ranking rule", who);
    const void *arrays[] = {logits, x0, prob, entropy, margin, argmax, outs[0], outs[1]};
    for (const void *q : arrays)
      if (q && (q == (const void *)canvas->tokens || q == (const void *)canvas->counts))
        return fail(DLLM_ERR_ARG, "%s: canvas tokens or counts alias another array", who);
    if (canvas->tokens && (const void *)canvas->tokens == (const void *)canvas->counts)
      return fail(DLLM_ERR_ARG, "%s: canvas tokens and counts alias", who);
    a.canvas = canvas->tokens;
    a.counts = canvas->counts;
    a.skip_rows = canvas->skip_rows ? 1 : 0;
  }
  a.need_batch = (a.n_rank_rules > 0 || a.counts) ? 1 : 0;

  const int64_t rows = B * L;
  if (B > 0x7fffffffLL || L > 0x7fffffffLL || rows > (int64_t)(0xffffffffu / 1024u))
    return fail(DLLM_ERR_UNSUPPORTED, "%s: B * L = %lld positions exceeds the launch limit of %u", who,
                (long long)rows, 0xffffffffu / 1024u);
  const Plan p = make_plan(dtype, rows, V, row_stride, logits);
  const size_t need = workspace_bytes_for(B, L, p.slices);
  if (!workspace) return fail(DLLM_ERR_ARG, "%s: workspace is NULL", who);
  if (workspace_bytes < need)
    return fail(DLLM_ERR_SHAPE, "%s: workspace has %zu bytes, this shape needs %zu", who,
                workspace_bytes, need);
  if ((uintptr_t)workspace % 16)
    return fail(DLLM_ERR_ARG, "%s: workspace must be 16-byte aligned", who);

  unsigned char *ws = static_cast<unsigned char *>(workspace);
  a.batch_count = reinterpret_cast<uint32_t *>(ws);
  size_t off = ((size_t)B * 4 + 255) / 256 * 256;
  a.edit_count = reinterpret_cast<uint32_t *>(ws + off);
  off += ((size_t)B * 4 + 255) / 256 * 256;
  if (p.slices > 1) {
    a.row_count = reinterpret_cast<uint32_t *>(ws + off);
    off += ((size_t)rows * 4 + 255) / 256 * 256;
    a.partials = reinterpret_cast<Partial *>(ws + off);
  }
  a.logits = logits;
  a.row_stride = row_stride;
  a.V = V;
  a.L = L;
  a.slice_len = p.slice_len;
  a.slices = p.slices;
  a.inv_temp = temperature > 0.0f ? (float)(1.4426950408889634 / (double)temperature) : 0.0f;
  a.key0 = (uint32_t)(seed & 0xffffffffu);
  a.key1 = (uint32_t)(seed >> 32);
  a.step = (uint32_t)step;
  a.n_suppress = n_suppress;
  a.first_allowed = first_allowed;
  a.x0 = x0;
  a.prob = prob;
  a.entropy = entropy;
  a.margin = margin;
  a.argmax = argmax;
  a.c2 = (float)(1.4426950408889634 / (double)stats_t);
  const bool sample = temperature > 0.0f;
  size_t smem = a.n_rank_rules ? rule_smem_bytes((int)L, p.nt) : 0;
  if (p.slices > 1) smem = std::max(smem, (size_t)p.slices * sizeof(Partial));
  if (a.skip_rows || a.margin) return launch_full(dtype, p, a, rows, sample, smem, stream, who);
  if (dtype == DLLM_BF16) return launch_plan<uint16_t>(p, a, rows, sample, smem, stream, who);
  return launch_plan<float>(p, a, rows, sample, smem, stream, who);
}

}  // namespace

extern "C" int dllm_token_stats(const void *logits, int dtype, int64_t B, int64_t L, int64_t V,
                                int64_t row_stride, float temperature, uint64_t seed,
                                uint64_t step, const int32_t *suppress_ids, int n_suppress,
                                int32_t *x0, float *prob, float *entropy,
                                const dllm_stats_extra *extra, const dllm_rule *rules,
                                int n_rules, void *workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  return stats_step("dllm_token_stats", logits, dtype, B, L, V, row_stride, temperature, seed,
                    step, suppress_ids, n_suppress, x0, prob, entropy, extra, rules, n_rules,
                    nullptr, workspace, workspace_bytes, stream);
}

extern "C" int dllm_commit_step(const void *logits, int dtype, int64_t B, int64_t L, int64_t V,
                                int64_t row_stride, float temperature, uint64_t seed,
                                uint64_t step, const int32_t *suppress_ids, int n_suppress,
                                int32_t *x0, float *prob, float *entropy,
                                const dllm_stats_extra *extra, const dllm_rule *rules,
                                int n_rules, const dllm_canvas *canvas, void *workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  if (!canvas) return fail(DLLM_ERR_ARG, "dllm_commit_step: canvas is NULL");
  return stats_step("dllm_commit_step", logits, dtype, B, L, V, row_stride, temperature, seed,
                    step, suppress_ids, n_suppress, x0, prob, entropy, extra, rules, n_rules,
                    canvas, workspace, workspace_bytes, stream);
}

namespace dllm {
namespace {

// The workspace of dllm_commit_step_static: one array on each GPU, part of the
// code object (zero-initialised static storage).  In host code this name is a
// host-side stand-in, not the device address: kernels get the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[DLLM_STATIC_SCRATCH_BYTES];

__global__ void clear_scratch_kernel(uint4 *p, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

struct ScratchSlot {
  void *ptr = nullptr;    // device address of `scratch` on this device
  bool cleared = false;
};
std::mutex g_scratch_mu;
ScratchSlot g_scratch[64];

// The current device's scratch address.  Once per device: the symbol lookup
// (with that device current) and one clearing kernel on `stream`.
int static_scratch(hipStream_t stream, void **out, const char *who) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return fail(DLLM_ERR_HIP, "%s: no current device", who);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchSlot &slot = g_scratch[dev];
  if (!slot.ptr) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(DLLM_ERR_HIP, "%s: hipGetSymbolAddress(scratch) failed: %s", who,
                  hipGetErrorString(e));
    slot.ptr = p;
  }
  if (!slot.cleared) {
    clear_scratch_kernel<<<dim3(256), dim3(256), 0, stream>>>(static_cast<uint4 *>(slot.ptr),
                                                              DLLM_STATIC_SCRATCH_BYTES / 16);
    const int rc = check_launch(who);
    if (rc != DLLM_OK) return rc;
    slot.cleared = true;
  }
  *out = slot.ptr;
  return DLLM_OK;
}

}  // namespace
}  // namespace dllm

extern "C" int dllm_commit_step_static(const void *logits, int dtype, int64_t B, int64_t L,
                                       int64_t V, int64_t row_stride, float temperature,
                                       uint64_t seed, uint64_t step,
                                       const int32_t *suppress_ids, int n_suppress, int32_t *x0,
                                       float *prob, float *entropy,
                                       const dllm_stats_extra *extra, const dllm_rule *rules,
                                       int n_rules, const dllm_canvas *canvas,
                                       hipStream_t stream) {
  const char *who = "dllm_commit_step_static";
  if (!canvas) return fail(DLLM_ERR_ARG, "%s: canvas is NULL", who);
  const size_t need = dllm_token_stats_workspace_size(dtype, B, L, V);
  if (need > DLLM_STATIC_SCRATCH_BYTES)
    return fail(DLLM_ERR_UNSUPPORTED,
                "%s: this shape needs %zu bytes of workspace, more than the %u of the static "
                "scratch array; call dllm_commit_step with a workspace", who, need,
                (unsigned)DLLM_STATIC_SCRATCH_BYTES);
  void *ws = nullptr;
  const int rc = static_scratch(stream, &ws, who);
  if (rc != DLLM_OK) return rc;
  return stats_step(who, logits, dtype, B, L, V, row_stride, temperature, seed, step,
                    suppress_ids, n_suppress, x0, prob, entropy, extra, rules, n_rules, canvas,
                    ws, DLLM_STATIC_SCRATCH_BYTES, stream);
}
