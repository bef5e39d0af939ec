// The commit rules as standalone calls, the per-step schedule, the block
// helpers, and the library's error plumbing.
//
// Rules: mlx-arsenal research note "dLLM block decoding", "What mlx-arsenal
// ships" (one function-table row per rule) and "Deviations from the
// references"; mlxcel "Block Diffusion", "LLaDA-2 Block Unmasking" and
// "Samplers and Reveal Policies".  Each ranking rule runs one workgroup per
// batch row (rules_dev.h); edit, schedule and the mask are elementwise.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "common.h"
#include <mutex>
#include <unordered_map>

#include "rules_dev.h"

namespace dllm {

// ---------------------------------------------------------------- errors

static thread_local char g_err[512];

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = 0;
  return DLLM_OK;
}

int check_launch(const char *what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DLLM_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

int check_lds(const void *kernel, size_t dynamic_lds, const char *who) {
  static std::mutex mu;
  static std::unordered_map<const void *, size_t> static_lds;
  static int limit[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return fail(DLLM_ERR_HIP, "%s: no current device", who);
  size_t fixed = 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = static_lds.find(kernel);
    if (it == static_lds.end()) {
      hipFuncAttributes attr;
      if (hipFuncGetAttributes(&attr, kernel) != hipSuccess)
        return fail(DLLM_ERR_HIP, "%s: cannot query the kernel's LDS size", who);
      it = static_lds.emplace(kernel, attr.sharedSizeBytes).first;
    }
    fixed = it->second;
    if (limit[dev] == 0) {
      int n = 0;
      if (hipDeviceGetAttribute(&n, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
          n <= 0)
        return fail(DLLM_ERR_HIP, "%s: cannot query the device's LDS size", who);
      limit[dev] = n;
    }
  }
  if (fixed + dynamic_lds > (size_t)limit[dev])
    return fail(DLLM_ERR_UNSUPPORTED,
                "%s: the launch needs %zu bytes of LDS (%zu static + %zu dynamic), more than the "
                "device's %d per workgroup", who, fixed + dynamic_lds, fixed, dynamic_lds, limit[dev]);
  return DLLM_OK;
}

int device_cu_count() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// floor(g * 2^149) as a 320-bit two's complement number (|g| < 2^141).
static Fx fixed_floor_of_double(double g) {
  Fx r;
  fx_zero(r);
  if (g == 0.0) return r;
  int e = 0;
  const double fr = frexp(fabs(g), &e);                  // |g| = fr * 2^e, fr in [0.5, 1)
  const uint64_t mant = (uint64_t)ldexp(fr, 53);         // |g| = mant * 2^(e - 53)
  const int sh = e - 53 + 149;                           // |g| * 2^149 = mant * 2^sh
  const bool neg = g < 0.0;
  if (sh >= 0) {
    const int limb = sh >> 6, off = sh & 63;
    r.w[limb] = mant << off;
    if (off > 0 && limb < 4) r.w[limb + 1] = mant >> (64 - off);
    if (neg) fx_negate(r);
  } else {
    const int s = -sh;
    const uint64_t q = s >= 64 ? 0 : (mant >> s);
    const bool rem = s >= 64 ? true : ((mant & ((1ull << s) - 1)) != 0);
    r.w[0] = q;
    if (neg) {                                           // floor(-x) = -ceil(x)
      r.w[0] = q + (rem ? 1 : 0);
      fx_negate(r);
    }
  }
  return r;
}

int prepare_rule(const dllm_rule &r, RuleDev &d, int64_t B, int64_t L, const char *who) {
  (void)B;
  (void)L;
  memset(&d, 0, sizeof d);
  d.kind = r.kind;
  d.strict = r.strict ? 1 : 0;
  d.mask = r.mask;
  d.out = r.out;
  d.k = r.k;
  d.tokens = r.tokens;
  d.taus = r.taus;
  d.param = r.param;
  d.score = r.score;
  d.negate = r.score == DLLM_SCORE_NEG_ENTROPY ? 1 : 0;
  if (!r.mask || !r.out) return fail(DLLM_ERR_ARG, "%s: rule mask and out must be non-NULL", who);
  if (r.score < DLLM_SCORE_PROB || r.score > DLLM_SCORE_NEG_ENTROPY)
    return fail(DLLM_ERR_ARG, "%s: rule score %d is not a DLLM_SCORE_*", who, r.score);
  if (r.score != DLLM_SCORE_PROB && r.kind != DLLM_RULE_THRESHOLD && r.kind != DLLM_RULE_TOPK &&
      r.kind != DLLM_RULE_FACTOR)
    return fail(DLLM_ERR_ARG, "%s: only threshold, topk and factor take another score", who);
  if (r.taus && r.kind != DLLM_RULE_THRESHOLD)
    return fail(DLLM_ERR_ARG, "%s: only the threshold rule takes per-row thresholds", who);
  if (r.taus && (const void *)r.taus == (const void *)r.out)
    return fail(DLLM_ERR_ARG, "%s: the output aliases the thresholds", who);
  if (r.kind == DLLM_RULE_TOPK) {
    if (!r.k) return fail(DLLM_ERR_ARG, "%s: topk needs the k array", who);
    return DLLM_OK;
  }
  if (r.param != r.param) return fail(DLLM_ERR_ARG, "%s: the rule parameter is NaN", who);
  if (r.kind == DLLM_RULE_ENTROPY_BOUND) {
    const double g = r.param;
    d.gamma_is_pos_inf = (g == INFINITY);
    if (g >= 0x1p141) d.gamma_class = 1;
    else if (g <= -0x1p141) d.gamma_class = 2;
    else { d.gamma_class = 0; d.gamma_fx = fixed_floor_of_double(g); }
  }
  return DLLM_OK;
}

// ---------------------------------------------------------------- kernels

template <int NT>
__global__ __launch_bounds__(NT) void batch_rule_kernel(RuleDev r, int L, const float *conf,
                                                        const float *ent) {
  extern __shared__ __align__(16) unsigned char smem[];
  run_batch_rule<true>(r, (int)blockIdx.x, L, conf, ent, smem, CommitSink{nullptr, nullptr}, NT);
}

// The standalone threshold rule: one wave per batch row, four rows per
// workgroup.  It needs no ranking, so the pass count and the forced first
// maximal candidate are wave reductions; no LDS and no barrier.  Same decision
// as the fused routine (rule_threshold).
__global__ __launch_bounds__(256) void threshold_rows_kernel(RuleDev r, int64_t B, int L,
                                                            const float *conf) {
  const int lane = threadIdx.x & 63;
  const int64_t b = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= B) return;                           // whole waves only
  const float *c_row = conf + b * L;
  const uint8_t *m_row = r.mask + b * L;
  uint8_t *o_row = r.out + b * L;
  const double tau = r.taus ? r.taus[b] : r.param;
  int pass = 0;
  uint64_t best = kSentinel;
  // Eight positions per lane at a time, every load issued before any is used
  // (a lane past the row reads its first position, the value unused): one
  // memory round trip per block, not two per position.
  constexpr int CH = 8;
  for (int l0 = 0; l0 < L; l0 += 64 * CH) {
    float cvs[CH];
    uint32_t ms[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int l = l0 + j * 64 + lane;
      const int lc = l < L ? l : 0;
      cvs[j] = c_row[lc];
      ms[j] = m_row[lc];
    }
    // every use below depends on this empty asm, so no use (and no wait for
    // its load) is scheduled between the loads
#pragma unroll
    for (int j = 0; j < CH; ++j) asm volatile("" : "+v"(cvs[j]), "+v"(ms[j]));
    // branch-free use of the loaded values (a branch around a use lets the
    // compiler sink the load into it, one round trip again)
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int l = l0 + j * 64 + lane;
      const bool in_row = l < L;
      const bool cand = in_row && ms[j] != 0;
      const float c = conf_sanitized(r.negate ? -cvs[j] : cvs[j]);
      const double cd = (double)c;
      const bool v = cand && (r.strict ? (cd > tau) : (cd >= tau));
      pass += v ? 1 : 0;
      const uint64_t key = cand ? (((uint64_t)conf_key(c) << 32) | (uint32_t)l) : kSentinel;
      best = key < best ? key : best;
      if (in_row) o_row[l] = v ? 1 : 0;
    }
  }
  pass = wave_sum_i(pass);
  best = wave_min_u64(best);
  if (lane == 0 && pass == 0 && best != kSentinel) o_row[(uint32_t)best] = 1;
}

__global__ void edit_kernel(const int32_t *x0, const float *prob, const int32_t *tokens,
                            const uint8_t *editable, int64_t n, double tau, uint8_t *edit) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    edit[i] = edit_decision(editable[i], x0[i], tokens[i], prob[i], tau);
}

__global__ void schedule_kernel(const int32_t *n_masked, int64_t B, int32_t steps, int32_t *out) {
  const int64_t total = B * steps;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = i / steps;
    const int32_t s = (int32_t)(i - b * steps);
    const int32_t n = max(n_masked[b], 0);
    out[i] = n / steps + (s < n % steps ? 1 : 0);
  }
}

// One workgroup per query row q; keys k < (q/bl + 1) * bl attend (0), the
// rest are blocked (-inf).  16-byte stores when the row is 16-byte aligned.
__global__ __launch_bounds__(256) void block_mask_kernel(int64_t L, int64_t bl, float *out,
                                                         int vec_ok) {
  const int64_t q = blockIdx.x;
  const int64_t keep = min(L, (q / bl + 1) * bl);
  float *row = out + q * L;
  const float ninf = -__builtin_inff();
  if (vec_ok) {
    float4 *row4 = reinterpret_cast<float4 *>(row);
    for (int64_t j = threadIdx.x; j < L / 4; j += blockDim.x) {
      const int64_t k = 4 * j;
      float4 v;
      v.x = k < keep ? 0.f : ninf;
      v.y = k + 1 < keep ? 0.f : ninf;
      v.z = k + 2 < keep ? 0.f : ninf;
      v.w = k + 3 < keep ? 0.f : ninf;
      row4[j] = v;
    }
  } else {
    for (int64_t k = threadIdx.x; k < L; k += blockDim.x) row[k] = k < keep ? 0.f : ninf;
  }
}

static unsigned grid_for(int64_t n, int block) {
  int64_t g = (n + block - 1) / block;
  if (g > 65535 * 16) g = 65535 * 16;
  return (unsigned)(g < 1 ? 1 : g);
}

static int launch_batch_rule(const dllm_rule &rule, int64_t B, int64_t L, const float *scores,
                             hipStream_t s, const char *who) {
  if (B < 0 || L < 0) return fail(DLLM_ERR_ARG, "%s: B and L must be >= 0", who);
  if (B == 0 || L == 0) return ok();
  if (!scores) return fail(DLLM_ERR_ARG, "%s: the score array is NULL", who);
  if (B > 0x7fffffffLL) return fail(DLLM_ERR_UNSUPPORTED, "%s: B too large", who);
  if (L > DLLM_MAX_L)
    return fail(DLLM_ERR_UNSUPPORTED, "%s: L = %lld exceeds DLLM_MAX_L = %d", who, (long long)L,
                DLLM_MAX_L);
  RuleDev d;
  const int rc = prepare_rule(rule, d, B, L, who);
  if (rc != DLLM_OK) return rc;
  if ((const void *)rule.out == (const void *)scores || (const void *)rule.out == (const void *)rule.mask)
    return fail(DLLM_ERR_ARG, "%s: the output aliases an input", who);
  if (d.kind == DLLM_RULE_THRESHOLD) {
    if (B > (int64_t)(0xffffffffu / 64u))
      return fail(DLLM_ERR_UNSUPPORTED, "%s: B = %lld batch rows exceeds the launch limit", who, (long long)B);
    threshold_rows_kernel<<<dim3((unsigned)((B + 3) / 4)), dim3(256), 0, s>>>(d, B, (int)L, scores);
    return check_launch(who);
  }
  // one position per thread (the short-row paths) up to 1024 positions
  const int np = rule_pow2((int)L);
  const int nt = np > 512 ? 1024 : (np > 256 ? 512 : 256);
  if (B > (int64_t)(0xffffffffu / (unsigned)nt))
    return fail(DLLM_ERR_UNSUPPORTED, "%s: B = %lld batch rows exceeds the launch limit", who, (long long)B);
  const size_t smem = rule_smem_bytes((int)L, nt);
  const void *kern = nt == 1024 ? (const void *)&batch_rule_kernel<1024>
                     : nt == 512 ? (const void *)&batch_rule_kernel<512>
                                 : (const void *)&batch_rule_kernel<256>;
  const int lds = check_lds(kern, smem, who);
  if (lds != DLLM_OK) return lds;
  if (nt == 1024)
    batch_rule_kernel<1024><<<dim3((unsigned)B), dim3(1024), smem, s>>>(d, (int)L, scores, scores);
  else if (nt == 512)
    batch_rule_kernel<512><<<dim3((unsigned)B), dim3(512), smem, s>>>(d, (int)L, scores, scores);
  else
    batch_rule_kernel<256><<<dim3((unsigned)B), dim3(256), smem, s>>>(d, (int)L, scores, scores);
  return check_launch(who);
}

}  // namespace dllm

using namespace dllm;

extern "C" const char *dllm_last_error(void) { return g_err; }

extern "C" int dllm_transfer_threshold(const float *conf, const uint8_t *cand, int64_t B, int64_t L,
                                       double tau, int strict, uint8_t *commit, hipStream_t stream) {
  dllm_rule r;
  memset(&r, 0, sizeof r);
  r.kind = DLLM_RULE_THRESHOLD;
  r.mask = cand;
  r.out = commit;
  r.param = tau;
  r.strict = strict;
  return launch_batch_rule(r, B, L, conf, stream, "dllm_transfer_threshold");
}

extern "C" int dllm_transfer_threshold_rows(const float *conf, const uint8_t *cand,
                                            const double *taus, int64_t B, int64_t L, int strict,
                                            uint8_t *commit, hipStream_t stream) {
  if (!taus && B > 0 && L > 0)
    return fail(DLLM_ERR_ARG, "dllm_transfer_threshold_rows: taus must be non-NULL");
  dllm_rule r;
  memset(&r, 0, sizeof r);
  r.kind = DLLM_RULE_THRESHOLD;
  r.mask = cand;
  r.out = commit;
  r.taus = taus;
  r.strict = strict;
  return launch_batch_rule(r, B, L, conf, stream, "dllm_transfer_threshold_rows");
}

extern "C" int dllm_decaying_threshold(double tau_initial, double tau_floor, double decay,
                                       int64_t step, double *out) {
  if (!out) return fail(DLLM_ERR_ARG, "dllm_decaying_threshold: out must be non-NULL");
  if (tau_initial != tau_initial || tau_floor != tau_floor || decay != decay)
    return fail(DLLM_ERR_ARG, "dllm_decaying_threshold: an argument is NaN");
  if (step < 0) return fail(DLLM_ERR_ARG, "dllm_decaying_threshold: step must be >= 0");
  const double t = tau_initial - decay * (double)step;
  *out = t > tau_floor ? t : tau_floor;
  return DLLM_OK;
}

extern "C" int dllm_transfer_topk(const float *conf, const uint8_t *cand, const int32_t *k,
                                  int64_t B, int64_t L, uint8_t *commit, hipStream_t stream) {
  dllm_rule r;
  memset(&r, 0, sizeof r);
  r.kind = DLLM_RULE_TOPK;
  r.mask = cand;
  r.out = commit;
  r.k = k;
  return launch_batch_rule(r, B, L, conf, stream, "dllm_transfer_topk");
}

extern "C" int dllm_transfer_factor(const float *conf, const uint8_t *cand, int64_t B, int64_t L,
                                    double f, uint8_t *commit, hipStream_t stream) {
  dllm_rule r;
  memset(&r, 0, sizeof r);
  r.kind = DLLM_RULE_FACTOR;
  r.mask = cand;
  r.out = commit;
  r.param = f;
  return launch_batch_rule(r, B, L, conf, stream, "dllm_transfer_factor");
}

extern "C" int dllm_transfer_entropy_bound(const float *entropy, const uint8_t *cand, int64_t B,
                                           int64_t L, double gamma, uint8_t *commit,
                                           hipStream_t stream) {
  dllm_rule r;
  memset(&r, 0, sizeof r);
  r.kind = DLLM_RULE_ENTROPY_BOUND;
  r.mask = cand;
  r.out = commit;
  r.param = gamma;
  return launch_batch_rule(r, B, L, entropy, stream, "dllm_transfer_entropy_bound");
}

extern "C" int dllm_transfer_edit(const int32_t *x0, const float *prob, const int32_t *tokens,
                                  const uint8_t *editable, int64_t B, int64_t L, double tau_edit,
                                  uint8_t *edit, hipStream_t stream) {
  const char *who = "dllm_transfer_edit";
  if (B < 0 || L < 0) return fail(DLLM_ERR_ARG, "%s: B and L must be >= 0", who);
  if (tau_edit != tau_edit) return fail(DLLM_ERR_ARG, "%s: tau_edit is NaN", who);
  if (B == 0 || L == 0) return ok();
  if (!x0 || !prob || !tokens || !editable || !edit)
    return fail(DLLM_ERR_ARG, "%s: every array must be non-NULL", who);
  const int64_t n = B * L;
  edit_kernel<<<dim3(grid_for(n, 256)), dim3(256), 0, stream>>>(x0, prob, tokens, editable, n,
                                                              tau_edit, edit);
  return check_launch(who);
}

extern "C" int dllm_transfer_schedule(const int32_t *n_masked, int64_t B, int32_t steps,
                                      int32_t *schedule, hipStream_t stream) {
  const char *who = "dllm_transfer_schedule";
  if (B < 0) return fail(DLLM_ERR_ARG, "%s: B must be >= 0", who);
  if (steps < 1) return fail(DLLM_ERR_ARG, "%s: steps = %d must be >= 1", who, steps);
  if (B == 0) return ok();
  if (!n_masked || !schedule) return fail(DLLM_ERR_ARG, "%s: arrays must be non-NULL", who);
  schedule_kernel<<<dim3(grid_for(B * steps, 256)), dim3(256), 0, stream>>>(n_masked, B, steps,
                                                                         schedule);
  return check_launch(who);
}

extern "C" int64_t dllm_block_ranges(int64_t prompt_len, int64_t gen_len, int64_t block_len,
                                     int align, int64_t *out, int64_t cap) {
  const char *who = "dllm_block_ranges";
  if (prompt_len < 0 || gen_len < 0 || block_len < 1)
    return fail(DLLM_ERR_ARG, "%s: need prompt_len >= 0, gen_len >= 0, block_len >= 1", who);
  if (cap < 0 || (cap > 0 && !out)) return fail(DLLM_ERR_ARG, "%s: bad out / cap", who);
  if (prompt_len > INT64_MAX - gen_len) return fail(DLLM_ERR_ARG, "%s: region overflows", who);
  ok();
  if (gen_len == 0) return 0;
  const int64_t end_all = prompt_len + gen_len;
  const int64_t first = align ? (prompt_len / block_len) * block_len : prompt_len;
  const int64_t count = (end_all - first + block_len - 1) / block_len;
  for (int64_t i = 0; i < count && i < cap; ++i) {
    const int64_t s = first + i * block_len;
    out[2 * i] = s;
    out[2 * i + 1] = (end_all - s > block_len) ? s + block_len : end_all;
  }
  return count;
}

extern "C" int dllm_block_causal_mask(int64_t L, int64_t block_len, float *out, hipStream_t stream) {
  const char *who = "dllm_block_causal_mask";
  if (L < 0 || block_len < 1) return fail(DLLM_ERR_ARG, "%s: need L >= 0 and block_len >= 1", who);
  if (L == 0) return ok();
  if (!out) return fail(DLLM_ERR_ARG, "%s: out is NULL", who);
  if (L > (int64_t)(0xffffffffu / 256u)) return fail(DLLM_ERR_UNSUPPORTED, "%s: L too large", who);
  const int vec_ok = (L % 4 == 0) && ((uintptr_t)out % 16 == 0);
  block_mask_kernel<<<dim3((unsigned)L), dim3(256), 0, stream>>>(L, block_len, out, vec_ok);
  return check_launch(who);
}
