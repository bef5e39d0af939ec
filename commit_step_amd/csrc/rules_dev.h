// Commit rules over one batch row, run by one workgroup (any multiple of 64
// threads).  Shared by the standalone dllm_transfer_* kernels and by the fused
// path of dllm_token_stats, where the last workgroup to finish a batch row runs
// them on the statistics the whole launch has just written.
//
// Rankings: every candidate gets a 64-bit key (order-preserving float bits in
// the high word, position in the low word) and a workgroup bitonic sort in LDS
// orders them; equal scores therefore keep the lower position first (stable
// order, "Deviations from the references").  Non-candidates get the all-ones
// key and sort last.
#pragma once

#include "common.h"

namespace dllm {

constexpr uint64_t kSentinel = ~0ull;
constexpr int kScanThreads = 256;

// Host-prepared view of one rule.
struct RuleDev {
  int kind;
  int strict;
  const uint8_t *mask;
  uint8_t *out;
  const int32_t *k;
  const int32_t *tokens;
  double param;
  // ENTROPY_BOUND: floor(gamma * 2^149) as a signed fixed-point number, and
  // how to compare a finite sum with gamma: 0 = use gamma_fx, 1 = always <=
  // (gamma >= 2^141 or +inf), 2 = never <= (gamma <= -2^141 or -inf).
  Fx gamma_fx;
  int gamma_class;
  int gamma_is_pos_inf;
};

__host__ __device__ inline int rule_pow2(int L) {
  int n = 64;
  while (n < L) n <<= 1;
  return n;
}

// LDS bytes the rule routines need for a batch row of L positions.
__host__ __device__ inline size_t rule_smem_bytes(int L) {
  const size_t keys = (size_t)rule_pow2(L) * 8;
  const size_t bytes = ((size_t)L + 15) & ~(size_t)15;
  return keys + bytes + kScanThreads * sizeof(Fx) + 64;
}

struct RuleSmem {
  uint64_t *keys;     // [Np]
  uint8_t *commit;    // [L]
  Fx *scan;           // [kScanThreads]
  int *misc;          // [16]
};

__device__ inline RuleSmem rule_smem(unsigned char *base, int L) {
  RuleSmem s;
  const int Np = rule_pow2(L);
  s.keys = reinterpret_cast<uint64_t *>(base);
  s.commit = base + (size_t)Np * 8;
  s.scan = reinterpret_cast<Fx *>(base + (size_t)Np * 8 + (((size_t)L + 15) & ~(size_t)15));
  s.misc = reinterpret_cast<int *>(s.scan + kScanThreads);
  return s;
}

// Bitonic sort of Np keys, ascending.
__device__ inline void block_bitonic_sort(uint64_t *keys, int Np) {
  const int tid = threadIdx.x, nt = blockDim.x;
  for (int k = 2; k <= Np; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < (Np >> 1); i += nt) {
        const int lo = ((i & ~(j - 1)) << 1) | (i & (j - 1));
        const int hi = lo | j;
        const bool asc = (lo & k) == 0;
        const uint64_t a = keys[lo], b = keys[hi];
        if ((a > b) == asc) {
          keys[lo] = b;
          keys[hi] = a;
        }
      }
      __syncthreads();
    }
  }
}

// (i + 1) * (1 - c) <= f, exactly: (i+1)*c is exact in float64 (a 24-bit
// mantissa times an integer below 2^13), the difference (i+1) - (i+1)*c is
// kept as an unevaluated sum s + e (two-sum), and s + e <= f is decided from s
// and the sign of e.
__device__ inline bool factor_holds(int i, float c, double f) {
  const uint32_t u = __float_as_uint(c);
  if (!bits_finite(u)) {                       // c = +inf -> -inf product, -inf -> +inf
    const bool prod_neg_inf = !(u & 0x80000000u);
    return prod_neg_inf ? true : (f == __builtin_inf());
  }
  if (f == __builtin_inf()) return true;
  if (f == -__builtin_inf()) return false;
  const double a = (double)(i + 1);
  const double b = a * (double)c;
  const double s = a - b;
  const double bb = s - a;
  const double e = (a - (s - bb)) + (-b - bb);
  return s < f || (s == f && e <= 0.0);
}

// Write the batch row's commit bytes from LDS to global memory.
__device__ inline void write_commit(const RuleSmem &sm, uint8_t *out_row, int L) {
  for (int l = threadIdx.x; l < L; l += blockDim.x) out_row[l] = sm.commit[l];
}

// threshold: no ranking needed.
__device__ inline void rule_threshold(const RuleDev &r, int b, int L, const float *conf,
                                      const RuleSmem &sm) {
  const int tid = threadIdx.x, nt = blockDim.x;
  uint64_t *best = reinterpret_cast<uint64_t *>(sm.misc);    // misc[0..1]
  int *n_pass = sm.misc + 2;
  if (tid == 0) { *best = kSentinel; *n_pass = 0; }
  __syncthreads();
  const float *c_row = conf + (int64_t)b * L;
  const uint8_t *m_row = r.mask + (int64_t)b * L;
  int my_pass = 0;
  uint64_t my_best = kSentinel;
  for (int l = tid; l < L; l += nt) {
    uint8_t v = 0;
    if (m_row[l]) {
      const float c = conf_sanitized(c_row[l]);
      const double cd = (double)c;
      v = (r.strict ? (cd > r.param) : (cd >= r.param)) ? 1 : 0;
      my_pass += v;
      const uint64_t key = ((uint64_t)conf_key(c) << 32) | (uint32_t)l;
      my_best = key < my_best ? key : my_best;
    }
    sm.commit[l] = v;
  }
  if (my_pass) atomicAdd(n_pass, my_pass);
  if (my_best != kSentinel) atomicMin(reinterpret_cast<unsigned long long *>(best),
                                      (unsigned long long)my_best);
  __syncthreads();
  if (tid == 0 && *n_pass == 0 && *best != kSentinel) sm.commit[(uint32_t)*best] = 1;
  __syncthreads();
  write_commit(sm, r.out + (int64_t)b * L, L);
}

// Load the candidates' ranking keys and sort them; returns the candidate count.
__device__ inline int load_and_sort(const RuleDev &r, int b, int L, const float *score,
                                    bool by_entropy, const RuleSmem &sm) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int Np = rule_pow2(L);
  int *n_cand = sm.misc + 4;
  if (tid == 0) *n_cand = 0;
  __syncthreads();
  const float *s_row = score + (int64_t)b * L;
  const uint8_t *m_row = r.mask + (int64_t)b * L;
  int mine = 0;
  for (int i = tid; i < Np; i += nt) {
    uint64_t key = kSentinel;
    if (i < L) {
      if (m_row[i]) {
        const uint32_t hk = by_entropy ? ent_key(s_row[i]) : conf_key(s_row[i]);
        key = ((uint64_t)hk << 32) | (uint32_t)i;
        ++mine;
      }
      sm.commit[i] = 0;
    }
    sm.keys[i] = key;
  }
  if (mine) atomicAdd(n_cand, mine);
  __syncthreads();
  block_bitonic_sort(sm.keys, Np);
  return *n_cand;
}

// Commit the first n keys of the sorted order.
__device__ inline void commit_prefix(const RuleDev &r, int b, int L, int n, const RuleSmem &sm) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) sm.commit[(uint32_t)sm.keys[i]] = 1;
  __syncthreads();
  write_commit(sm, r.out + (int64_t)b * L, L);
}

__device__ inline void rule_topk(const RuleDev &r, int b, int L, const float *conf,
                                 const RuleSmem &sm) {
  const int nc = load_and_sort(r, b, L, conf, false, sm);
  int k = r.k[b];
  k = k < 0 ? 0 : (k > nc ? nc : k);
  commit_prefix(r, b, L, k, sm);
}

__device__ inline void rule_factor(const RuleDev &r, int b, int L, const float *conf,
                                   const RuleSmem &sm) {
  const int nc = load_and_sort(r, b, L, conf, false, sm);
  int *first_fail = sm.misc + 6;
  if (threadIdx.x == 0) *first_fail = nc;
  __syncthreads();
  for (int i = threadIdx.x; i < nc; i += blockDim.x) {
    const float c = conf_from_key((uint32_t)(sm.keys[i] >> 32));
    if (!factor_holds(i, c, r.param)) atomicMin(first_fail, i);
  }
  __syncthreads();
  const int n = nc ? max(*first_fail, 1) : 0;
  commit_prefix(r, b, L, n, sm);
}

// Does the exclusive prefix sum S_i (finite part `fin`, plus the -inf / +inf
// entries among the first i sorted candidates) satisfy S_i <= gamma?
__device__ inline bool ent_prefix_ok(const RuleDev &r, const Fx &fin, int n_neg, int n_pos) {
  if (n_neg && n_pos) return false;
  if (n_pos) return r.gamma_is_pos_inf != 0;
  if (n_neg) return true;
  if (r.gamma_class == 1) return true;
  if (r.gamma_class == 2) return false;
  return fx_le(fin, r.gamma_fx);
}

__device__ inline void rule_entropy_bound(const RuleDev &r, int b, int L, const float *ent,
                                          const RuleSmem &sm) {
  const int nc = load_and_sort(r, b, L, ent, true, sm);
  const int tid = threadIdx.x;
  int *first_fail = sm.misc + 6;
  int *n_neg_all = sm.misc + 7;
  int *n_pos_all = sm.misc + 8;
  if (tid == 0) { *first_fail = nc; *n_neg_all = 0; *n_pos_all = 0; }
  __syncthreads();
  // Sorted ascending: the -inf entropies come first and the +inf ones last.
  for (int i = tid; i < nc; i += blockDim.x) {
    const uint32_t u = __float_as_uint(ent_from_key((uint32_t)(sm.keys[i] >> 32)));
    if (u == 0xff800000u) atomicAdd(n_neg_all, 1);
    if (u == 0x7f800000u) atomicAdd(n_pos_all, 1);
  }
  // Each of the first kScanThreads threads owns one contiguous segment.
  const int seg = (nc + kScanThreads - 1) / kScanThreads;
  const int lo = tid * seg, hi = min(lo + seg, nc);
  Fx local;
  fx_zero(local);
  if (tid < kScanThreads) {
    for (int i = lo; i < hi; ++i) {
      const uint32_t u = __float_as_uint(ent_from_key((uint32_t)(sm.keys[i] >> 32)));
      if (bits_finite(u)) fx_add(local, fx_from_f32_bits(u));
    }
    sm.scan[tid] = local;
  }
  __syncthreads();
  // Inclusive scan of the segment totals (Hillis-Steele; integer adds, so the
  // order does not change the result).
  for (int off = 1; off < kScanThreads; off <<= 1) {
    Fx add;
    fx_zero(add);
    if (tid < kScanThreads && tid >= off) add = sm.scan[tid - off];
    __syncthreads();
    if (tid < kScanThreads && tid >= off) fx_add(sm.scan[tid], add);
    __syncthreads();
  }
  if (tid < kScanThreads && lo < hi) {
    Fx s;
    fx_zero(s);
    if (tid > 0) s = sm.scan[tid - 1];
    const int neg_all = *n_neg_all, pos_all = *n_pos_all;
    for (int i = lo; i < hi; ++i) {
      const int n_neg = min(i, neg_all);
      const int n_pos = max(0, i - (nc - pos_all));
      if (!ent_prefix_ok(r, s, n_neg, n_pos)) {
        atomicMin(first_fail, i);
        break;
      }
      const uint32_t u = __float_as_uint(ent_from_key((uint32_t)(sm.keys[i] >> 32)));
      if (bits_finite(u)) fx_add(s, fx_from_f32_bits(u));
    }
  }
  __syncthreads();
  const int n = nc ? max(*first_fail, 1) : 0;
  commit_prefix(r, b, L, n, sm);
}

// Runs a ranking rule on batch row b.  Every thread of the workgroup must call
// it.  `conf` is the confidence (prob) array and `ent` the entropy array.
__device__ inline void run_batch_rule(const RuleDev &r, int b, int L, const float *conf,
                                      const float *ent, unsigned char *smem) {
  const RuleSmem sm = rule_smem(smem, L);
  switch (r.kind) {
    case DLLM_RULE_THRESHOLD: rule_threshold(r, b, L, conf, sm); break;
    case DLLM_RULE_TOPK: rule_topk(r, b, L, conf, sm); break;
    case DLLM_RULE_FACTOR: rule_factor(r, b, L, conf, sm); break;
    case DLLM_RULE_ENTROPY_BOUND: rule_entropy_bound(r, b, L, ent, sm); break;
    default: break;
  }
  __syncthreads();
}

__device__ __forceinline__ uint8_t edit_decision(uint8_t editable, int32_t x0, int32_t tok,
                                                 float p, double tau_edit) {
  return (editable && x0 != tok && (double)conf_sanitized(p) > tau_edit) ? 1 : 0;
}

}  // namespace dllm
