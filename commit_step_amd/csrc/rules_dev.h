// Commit rules over one batch row, run by one workgroup.  Shared by the
// standalone dllm_transfer_* kernels and by the fused path of
// dllm_token_stats, where the last workgroup to finish a batch row runs them on
// the statistics the launch has just written.
//
// Rankings: every candidate gets a 64-bit key (order-preserving float bits in
// the high word, position in the low word), so ascending key order is the
// stable order of "Deviations from the references" (equal scores: lower
// position first), and the rank of a candidate (the number of candidate keys
// below its own) is its index in the sorted order.
//   * Short rows (L <= blockDim.x, one position per thread): the candidates are
//     compacted into an LDS list and each rank is an all-pairs count over it
//     with broadcast reads: one dependent phase, no sorting network.  For
//     entropy_bound only candidates with H <= gamma can be followed by another
//     committed candidate (entropies are >= 0), so ranks and prefix sums run
//     over that subset plus the smallest entropy above gamma.
//   * Long rows, and entropy rows with negative or non-finite entropies, use a
//     workgroup bitonic sort in LDS.
// The score arrays are read with agent-scope atomic loads (coherent across
// XCDs), because in the fused path they were written moments before by other
// workgroups of the same launch.
#pragma once

#include "common.h"

namespace dllm {

constexpr uint64_t kSentinel = ~0ull;

// Host-prepared view of one rule.
struct RuleDev {
  int kind;
  int strict;
  int score;           // fused ranking rules: which statistic is the confidence
  int negate;          // confidence = -score array (Dream's negative entropy)
  const uint8_t *mask;
  uint8_t *out;
  const int32_t *k;
  const int32_t *tokens;
  const double *taus;  // THRESHOLD: per-row thresholds in place of param, or null
  double param;
  // ENTROPY_BOUND, exact comparison of a finite sum with gamma: floor(gamma *
  // 2^149) as a signed fixed-point number, and 0 = use gamma_fx, 1 = always <=
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

// LDS bytes the rule routines need for a batch row of L positions run by nt
// threads.
__host__ __device__ inline size_t rule_smem_bytes(int L, int nt) {
  const size_t Np = (size_t)rule_pow2(L);
  const size_t lists = Np * 20 + (size_t)nt * 12;   // short rows (lists, x0 per position)
  const size_t keys = Np * 8;                        // sorting network
  return (((lists > keys ? lists : keys) + 7) & ~(size_t)7) + 512;
}

struct RuleSmem {
  uint64_t *keys;     // [Np] sorted keys (long rows) / compacted list (short rows)
  double *hs;         // [Np] values matching the list (short rows)
  double *part_sum;   // [nt]
  int *part_cnt;      // [nt]
  int32_t *x0s;       // [Np] x0 of every position (short rows with a canvas)
  int *misc;          // [128]
  int nt;             // threads of the workgroup (a compile-time constant at every caller)
};

__device__ inline RuleSmem rule_smem(unsigned char *base, int L, int nt_) {
  RuleSmem s;
  s.nt = nt_;
  const size_t Np = (size_t)rule_pow2(L), nt = (size_t)nt_;
  s.keys = reinterpret_cast<uint64_t *>(base);
  s.hs = reinterpret_cast<double *>(base + Np * 8);
  s.part_sum = reinterpret_cast<double *>(base + Np * 16);
  s.part_cnt = reinterpret_cast<int *>(base + Np * 16 + nt * 8);
  s.x0s = reinterpret_cast<int32_t *>(base + Np * 16 + nt * 12);
  const size_t lists = Np * 20 + nt * 12;
  const size_t top = lists > Np * 8 ? lists : Np * 8;
  s.misc = reinterpret_cast<int *>(base + ((top + 7) & ~(size_t)7));
  return s;
}

__device__ __forceinline__ float load_coherent(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t load_coherent_i32(const int32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Where a rank rule's commits go besides its mask: inside the canvas step,
// x0 is written into the batch row's canvas at every committed position as
// the rule decides it (no second pass over the mask).  Both pointers are the
// batch row's own (position l at [l]); canvas is null outside the canvas step.
struct CommitSink {
  int32_t *canvas;
  const int32_t *x0;      // published by this launch: read with coherent loads
};

// Candidates of the batch row and how many the rule committed (thread 0).
struct RuleCount {
  int nc;
  int committed;
};

// A ranking rule's confidence from its score array (negated for a negative
// entropy; NaN stays NaN and counts as -inf).
__device__ __forceinline__ float rule_conf(const RuleDev &r, const float *p) {
  const float v = load_coherent(p);
  return r.negate ? -v : v;
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

// Does S_i <= gamma hold, given [finite part of S_i <= gamma] and the number
// of -inf / +inf entropies among the first i sorted candidates?
__device__ __forceinline__ bool ent_prefix_ok(const RuleDev &r, bool finite_le, int n_neg,
                                              int n_pos) {
  if (n_neg && n_pos) return false;
  if (n_pos) return r.gamma_is_pos_inf != 0;
  if (n_neg) return true;
  if (r.gamma_class == 1) return true;
  if (r.gamma_class == 2) return false;
  return finite_le;
}

// Exact first index i at which the prefix sum sum_{j<i} h[j] of finite,
// non-negative float32 values (in sorted order, in LDS) exceeds gamma; n if
// none.  One thread walks the list in fixed point: the rare path taken when a
// float64 prefix lands within its rounding bound of gamma.
__device__ inline int exact_first_fail(const RuleDev &r, const float *h, int n, int *slot) {
  if (threadIdx.x == 0) {
    Fx s;
    fx_zero(s);
    int upto = n;
    for (int i = 0; i < n; ++i) {
      if (!fx_le(s, r.gamma_fx)) { upto = i; break; }
      fx_add(s, fx_from_f32_bits(__float_as_uint(h[i])));
    }
    *slot = upto;
  }
  __syncthreads();
  const int v = *slot;
  __syncthreads();
  return v;
}

// ---------------------------------------------------------------- short rows
// One position per thread.  Per-wave counts and minima go through LDS slots,
// one slot per wave (misc ints [0,16) [16,32) [32,48) [48,64), 64-bit slots
// from int 64 on), so no slot needs clearing first and every phase ends in a
// single barrier.

__device__ __forceinline__ int lane_prefix(uint64_t m) {   // set bits below this lane
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

// Number of list entries in [j0, j1) below q and, with VALS, the sum of their
// values.  The bounds are wave-uniform, so every lane reads the same entries
// (broadcast LDS reads); four entries per step, two accumulators.
template <bool VALS>
__device__ __forceinline__ void count_below(uint64_t q, const uint64_t *keys, const double *vals,
                                            int j0, int j1, int &cnt, double &sum) {
  int c0 = 0, c1 = 0;
  double s0 = 0.0, s1 = 0.0;
  int j = j0;
  for (; j + 8 <= j1; j += 8) {
    uint64_t kk[8];
    double vv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      kk[u] = keys[j + u];
      if constexpr (VALS) vv[u] = vals[j + u];
    }
#pragma unroll
    for (int u = 0; u < 8; u += 2) {
      const bool la = kk[u] < q, lb = kk[u + 1] < q;
      c0 += (int)la;
      c1 += (int)lb;
      if constexpr (VALS) {
        s0 += la ? vv[u] : 0.0;
        s1 += lb ? vv[u + 1] : 0.0;
      }
    }
  }
  for (; j + 4 <= j1; j += 4) {
    const uint64_t k0 = keys[j], k1 = keys[j + 1], k2 = keys[j + 2], k3 = keys[j + 3];
    const bool l0 = k0 < q, l1 = k1 < q, l2 = k2 < q, l3 = k3 < q;
    c0 += (int)l0 + (int)l2;
    c1 += (int)l1 + (int)l3;
    if constexpr (VALS) {
      const double v0 = vals[j], v1 = vals[j + 1], v2 = vals[j + 2], v3 = vals[j + 3];
      s0 += l0 ? v0 : 0.0;
      s1 += l1 ? v1 : 0.0;
      s0 += l2 ? v2 : 0.0;
      s1 += l3 ? v3 : 0.0;
    }
  }
  for (; j < j1; ++j) {
    const bool lt = keys[j] < q;
    c0 += (int)lt;
    if constexpr (VALS) s0 += lt ? vals[j] : 0.0;
  }
  cnt = c0 + c1;
  sum = s0 + s1;
}

// Ranks against list[0, n) of nq queries: query i is list[i] for i < n0 and
// `extra` for i == n0 < nq.  G = blockDim.x / P threads share a query (P a
// power of two >= max(nq, 64), so each wave works on one part of the list);
// the owner, thread i < P, returns the count, the value sum and its query.
// Transposed ranks of up to 64 QPL queries: each wave scans a 1/nw share of
// the list for QPL queries per lane (query lane + 64 u), so every key read
// serves QPL comparisons.  The per-wave counts and sums meet in LDS atomics on
// part_cnt / part_sum, which the caller zeroed before its compaction barrier
// (both hold at least 64 QPL entries: one per thread of the workgroup).
// Counts are exact; the float64 sums then add in any order, which the
// callers' error bound already allows for.
template <bool VALS, int QPL>
__device__ inline int transposed_rank(int nq, int n0, uint64_t extra, const uint64_t *list, int n,
                                      const double *vals, const RuleSmem &sm, double &sum,
                                      uint64_t &query) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, nw = sm.nt >> 6;
  const int per = (n + nw - 1) / nw;
  const int j0 = min(wave * per, n), j1 = min(j0 + per, n);
  uint64_t qk[QPL];
  int c[QPL];
  double sq[QPL];
#pragma unroll
  for (int u = 0; u < QPL; ++u) {
    const int i = lane + 64 * u;
    qk[u] = i < n0 ? list[i] : (i < nq ? extra : 0ull);   // 0: no key lies below
    c[u] = 0;
    sq[u] = 0.0;
  }
  int j = j0;
  for (; j + 4 <= j1; j += 4) {
    uint64_t k[4];
    double v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      k[e] = list[j + e];
      if constexpr (VALS) v[e] = vals[j + e];
    }
#pragma unroll
    for (int u = 0; u < QPL; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool lt = k[e] < qk[u];
        c[u] += (int)lt;
        if constexpr (VALS) sq[u] += lt ? v[e] : 0.0;
      }
  }
  for (; j < j1; ++j) {
    const uint64_t k = list[j];
#pragma unroll
    for (int u = 0; u < QPL; ++u) {
      const bool lt = k < qk[u];
      c[u] += (int)lt;
      if constexpr (VALS) sq[u] += lt ? vals[j] : 0.0;
    }
  }
#pragma unroll
  for (int u = 0; u < QPL; ++u) {
    const int i = lane + 64 * u;
    if (i < nq) {
      if (c[u]) atomicAdd(&sm.part_cnt[i], c[u]);
      if (VALS && sq[u] != 0.0) atomicAdd(&sm.part_sum[i], sq[u]);
    }
  }
  __syncthreads();
  query = t < n0 ? list[t] : (t < nq ? extra : kSentinel);
  sum = (VALS && t < nq) ? sm.part_sum[t] : 0.0;
  return t < nq ? sm.part_cnt[t] : 0;
}

// WIDE: also the transposed form for up to 512 queries (eight per lane); only
// the standalone rule kernels take it, since a second inlined copy of the
// transposed loop makes the fused kernels copy their argument block to scratch.
template <bool VALS, bool WIDE = false>
__device__ inline int block_rank(int nq, int n0, uint64_t extra, const uint64_t *list, int n,
                                 const double *vals, const RuleSmem &sm, int P, double &sum,
                                 uint64_t &query) {
  if (nq <= 256) return transposed_rank<VALS, 4>(nq, n0, extra, list, n, vals, sm, sum, query);
  if constexpr (WIDE)
    if (nq <= 512 && sm.nt >= 512)
      return transposed_rank<VALS, 8>(nq, n0, extra, list, n, vals, sm, sum, query);
  const int t = threadIdx.x, G = sm.nt / P, part = t / P, i = t - part * P;
  const int per = (n + G - 1) / G;
  const int j0 = min(part * per, n), j1 = min(j0 + per, n);
  const uint64_t q = i < n0 ? list[i] : (i < nq ? extra : kSentinel);
  int cnt = 0;
  double s = 0.0;
  if (i < nq) count_below<VALS>(q, list, vals, j0, j1, cnt, s);
  if (G > 1) {
    if (part > 0 && i < nq) {
      sm.part_cnt[t] = cnt;
      if (VALS) sm.part_sum[t] = s;
    }
    __syncthreads();
    if (part == 0 && i < nq)
      for (int g = 1; g < G; ++g) {
        cnt += sm.part_cnt[g * P + i];
        if (VALS) s += sm.part_sum[g * P + i];
      }
  }
  sum = s;
  query = q;
  return cnt;
}

__device__ __forceinline__ int owners_for(int n, int nt) {
  int P = 64;
  while (P < n) P <<= 1;
  return P < nt ? P : nt;
}

// Sum over the waves' slots, and the part of it from waves below `wave`.
__device__ __forceinline__ int slots_sum(const int *slots, int nw, int wave, int *below) {
  int tot = 0, lo = 0;
  for (int w = 0; w < nw; ++w) {
    const int c = slots[w];
    lo += w < wave ? c : 0;
    tot += c;
  }
  if (below) *below = lo;
  return tot;
}

// topk / factor on a short row.
template <bool WIDE = false>
__device__ inline RuleCount short_rank_rule(const RuleDev &r, int b, int L, const float *conf,
                                            const RuleSmem &sm, const CommitSink &sk) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, nw = sm.nt >> 6;
  const uint8_t *m_row = r.mask + (int64_t)b * L;
  uint8_t *o_row = r.out + (int64_t)b * L;
  // Score, token and mask are loaded by every thread, whatever the mask
  // says (threads past the row read its first position, their values
  // unused), with no branch between the loads: one memory round trip, not
  // one per load.
  const bool in_row = t < L;
  const int tt = in_row ? t : 0;
  const float cv0 = rule_conf(r, conf + (int64_t)b * L + tt);
  const int32_t xv = sk.canvas ? load_coherent_i32(sk.x0 + tt) : 0;
  const uint8_t mv = m_row[tt];
  const int kq = r.kind == DLLM_RULE_TOPK ? r.k[b] : 0;     // in flight with the row's loads
  const float cv = in_row ? cv0 : 0.f;
  if (sk.canvas && in_row) sm.x0s[t] = xv;
  const bool cand = in_row && mv;
  const float c = cand ? conf_sanitized(cv) : 0.f;
  const uint64_t key = cand ? (((uint64_t)conf_key(c) << 32) | (uint32_t)t) : kSentinel;
  int *wcnt = sm.misc, *wfail = sm.misc + 32;
  sm.part_cnt[t] = 0;                         // for the transposed ranks
  const uint64_t m = __builtin_amdgcn_ballot_w64(cand);
  if (lane == 0) wcnt[wave] = __builtin_popcountll(m);
  __syncthreads();
  int off;
  const int n = slots_sum(wcnt, nw, wave, &off);
  if (cand) sm.keys[off + lane_prefix(m)] = key;
  __syncthreads();
  if (n <= 64) {
    // One wave ranks every candidate and finds the first failure; the other
    // waves only clear their own non-candidates, so no further barrier.
    if (t < L && !cand) o_row[t] = 0;
    if (wave != 0) return RuleCount{n, 0};
    const bool own = lane < n;
    const uint64_t qk = own ? sm.keys[lane] : kSentinel;
    int rk = 0;
    double unused1;
    int nc1;
    if (r.kind == DLLM_RULE_TOPK) {
      nc1 = kq < 0 ? 0 : (kq > n ? n : kq);
      // a quota of none, all or one needs no all-pairs ranks: the single
      // commit of a quota of one is the smallest key (the most confident)
      if (nc1 == 1) {
        const uint64_t best = wave_min_u64(qk);      // every lane takes part in the reduction
        rk = (own && qk == best) ? 0 : 1;
      }
      else if (nc1 == 0 || nc1 == n) rk = 0;
      else if (own) count_below<false>(qk, sm.keys, nullptr, 0, n, rk, unused1);
      if (nc1 == 0) rk = 1;
    } else {
      if (own) count_below<false>(qk, sm.keys, nullptr, 0, n, rk, unused1);
      const bool fails = own && !factor_holds(rk, conf_from_key((uint32_t)(qk >> 32)), r.param);
      const int first = wave_min_i(fails ? rk : 0x7fffffff);
      nc1 = n ? max(first < n ? first : n, 1) : 0;
    }
    if (own) {
      const bool c1 = rk < nc1;
      o_row[(uint32_t)qk] = c1 ? 1 : 0;
      if (c1 && sk.canvas) sk.canvas[(uint32_t)qk] = sm.x0s[(uint32_t)qk];
    }
    return RuleCount{n, nc1};
  }
  const int P = owners_for(n, sm.nt);
  double unused;
  uint64_t q;
  const int rank = block_rank<false, WIDE>(n, n, kSentinel, sm.keys, n, nullptr, sm, P, unused, q);
  const bool owner = t < n;     // thread t < n owns query t
  int n_commit;
  if (r.kind == DLLM_RULE_TOPK) {
    n_commit = kq < 0 ? 0 : (kq > n ? n : kq);
  } else {
    const bool fails = owner && !factor_holds(rank, conf_from_key((uint32_t)(q >> 32)), r.param);
    const int wmin = wave_min_i(fails ? rank : 0x7fffffff);
    if (lane == 0) wfail[wave] = wmin;
    __syncthreads();
    int first = 0x7fffffff;
    for (int w = 0; w < nw; ++w) first = min(first, wfail[w]);
    n_commit = n ? max(first < n ? first : n, 1) : 0;
  }
  if (owner) {
    const bool c1 = rank < n_commit;
    o_row[(uint32_t)q] = c1 ? 1 : 0;
    if (c1 && sk.canvas) sk.canvas[(uint32_t)q] = sm.x0s[(uint32_t)q];
  }
  if (t < L && !cand) o_row[t] = 0;
  return RuleCount{n, n_commit};
}

// entropy_bound on a short row.  Returns false (nothing written, every thread
// alike) when a candidate entropy is negative or not finite, or the subset
// H <= gamma is too large for the all-pairs pass; the caller then takes the
// sorted path.  Entropies being >= 0, only candidates with H <= gamma can be
// followed by another committed one, so ranks and prefix sums run over that
// subset F plus the smallest key above gamma.
template <bool WIDE = false>
__device__ inline bool short_entropy_rule(const RuleDev &r, int b, int L, const float *ent,
                                          const RuleSmem &sm, const CommitSink &sk,
                                          RuleCount &rc) {
  const int t = threadIdx.x, nt = sm.nt, lane = t & 63, wave = t >> 6, nw = nt >> 6;
  const uint8_t *m_row = r.mask + (int64_t)b * L;
  uint8_t *o_row = r.out + (int64_t)b * L;
  // entropy, token and mask in one round trip (as in short_rank_rule)
  const bool in_row = t < L;
  const int tt = in_row ? t : 0;
  const float hv0 = load_coherent(ent + (int64_t)b * L + tt);
  const int32_t xv = sk.canvas ? load_coherent_i32(sk.x0 + tt) : 0;
  const uint8_t mv = m_row[tt];
  const float hv = in_row ? hv0 : 0.f;
  if (sk.canvas && in_row) sm.x0s[t] = xv;
  const bool cand = in_row && mv;
  const float h = cand ? hv : 0.f;
  const uint32_t u = __float_as_uint(h);
  const bool bad = cand && u != 0x80000000u && (!bits_finite(u) || (u & 0x80000000u) != 0);
  const uint64_t key = cand ? (((uint64_t)ent_key(h) << 32) | (uint32_t)t) : kSentinel;
  const bool in_f = cand && (double)h <= r.param;
  const bool above = cand && !in_f;
  int *wF = sm.misc, *wA = sm.misc + 16, *wFail = sm.misc + 32, *wUnc = sm.misc + 48;
  uint64_t *wNext = reinterpret_cast<uint64_t *>(sm.misc + 64);
  int *slot = sm.misc + 100;
  sm.part_cnt[t] = 0;                         // for the transposed ranks
  sm.part_sum[t] = 0.0;
  const uint64_t mF = __builtin_amdgcn_ballot_w64(in_f);
  const uint64_t mA = __builtin_amdgcn_ballot_w64(above);
  const bool wbad = __builtin_amdgcn_ballot_w64(bad) != 0;
  const uint64_t wnext = wave_min_u64(above ? key : kSentinel);
  if (lane == 0) {
    wF[wave] = __builtin_popcountll(mF);
    wA[wave] = __builtin_popcountll(mA) | (wbad ? 0x100000 : 0);
    wNext[wave] = wnext;
  }
  __syncthreads();
  int offF, nA = 0, anybad = 0;
  const int nF = slots_sum(wF, nw, wave, &offF);
  uint64_t nxt = kSentinel;
  for (int w = 0; w < nw; ++w) {
    nA += wA[w] & 0xfffff;
    anybad |= wA[w] >> 20;
    nxt = wNext[w] < nxt ? wNext[w] : nxt;
  }
  DLLM_STAGE(kStageRuleLoaded);
  if (anybad || nF + 1 > nt || nF > 1024) return false;
  const int nc = nF + nA;
  if (in_f) {
    const int pos = offF + lane_prefix(mF);
    sm.keys[pos] = key;
    sm.hs[pos] = (double)h;
  }
  __syncthreads();
  // queries: every key of F, then the smallest key above gamma (index nF)
  const bool has_next = nxt != kSentinel;
  const int nq = nF + (has_next ? 1 : 0);
  if (nq <= 64) {
    // Up to 64 queries, lane q of every wave holding query q: wave w compares
    // it with F's keys w, w + nw, ..., and the waves' counts and partial sums
    // meet in LDS (atomic adds; the sum's order varies, but a prefix within
    // its rounding bound of gamma is decided exactly below, so the decisions
    // do not).  Then wave 0 decides, and the other waves are done.
    if (above && key != nxt) o_row[t] = 0;
    if (t < L && !cand) o_row[t] = 0;
    rc = RuleCount{nc, 0};
    const bool lv = lane < nq;
    const uint64_t qk = lane < nF ? sm.keys[lane] : (lv ? nxt : kSentinel);
    {
      int c = 0;
      double sq = 0.0;
      for (int i = wave; i < nF; i += nw) {
        const bool lt = sm.keys[i] < qk;
        c += lt ? 1 : 0;
        sq += lt ? sm.hs[i] : 0.0;
      }
      if (lv && c) {
        atomicAdd(&sm.part_cnt[lane], c);
        atomicAdd(&sm.part_sum[lane], sq);
      }
    }
    __syncthreads();
    if (wave != 0) return true;
    const int rk = lv ? sm.part_cnt[lane] : 0;
    const double Sq = lv ? sm.part_sum[lane] : 0.0;
    const double err1 = (double)(nF + 64) * 0x1p-52 * Sq;
    const bool unc = lv && r.gamma_class == 0 && err1 != 0.0 && fabs(Sq - r.param) <= err1;
    const bool fl = lv && !ent_prefix_ok(r, Sq <= r.param, 0, 0);
    int first1 = wave_min_i(fl ? rk : 0x7fffffff);
    if (__builtin_amdgcn_ballot_w64(unc) != 0) {
      // rare: decide the prefixes exactly, walking the queries in rank order
      // (every lane runs the same wave-uniform walk)
      const uint32_t hbits = __float_as_uint(ent_from_key((uint32_t)(qk >> 32)));
      Fx acc;
      fx_zero(acc);
      int upto = nq;
      for (int i = 0; i < nq; ++i) {
        if (!fx_le(acc, r.gamma_fx)) { upto = i; break; }
        const uint64_t who = __builtin_amdgcn_ballot_w64(lv && rk == i);
        const uint32_t hb = __builtin_amdgcn_readlane(hbits, (int)__builtin_ctzll(who));
        fx_add(acc, fx_from_f32_bits(hb));
      }
      first1 = upto < nq ? upto : 0x7fffffff;
    }
    const int ns1 = first1 != 0x7fffffff ? first1 : min(nF + 1, nc);
    const int ncm1 = nc ? max(ns1, 1) : 0;
    DLLM_STAGE(kStageRuleRanked);
    if (lv) {
      const bool c1 = rk < ncm1;
      o_row[(uint32_t)qk] = c1 ? 1 : 0;
      if (c1 && sk.canvas) sk.canvas[(uint32_t)qk] = sm.x0s[(uint32_t)qk];
    }
    rc = RuleCount{nc, ncm1};
    return true;
  }
  const int P = owners_for(nq, nt);
  double S;
  uint64_t q;
  const int rank = block_rank<true, WIDE>(nq, nF, nxt, sm.keys, nF, sm.hs, sm, P, S, q);
  const bool live = t < nq;     // thread t < nq owns query t
  // Entropies are >= 0, so sum |h| = S: |S - exact| <= (terms + 64) 2^-53 S
  // whatever the summation order.
  const double err = (double)(nF + 64) * 0x1p-52 * S;
  const bool uncertain = live && r.gamma_class == 0 && err != 0.0 && fabs(S - r.param) <= err;
  const bool fails = live && !ent_prefix_ok(r, S <= r.param, 0, 0);
  const int wmin = wave_min_i(fails ? rank : 0x7fffffff);
  const bool wunc = __builtin_amdgcn_ballot_w64(uncertain) != 0;
  if (lane == 0) {
    wFail[wave] = wmin;
    wUnc[wave] = wunc ? 1 : 0;
  }
  __syncthreads();
  int first = 0x7fffffff, anyunc = 0;
  for (int w = 0; w < nw; ++w) {
    first = min(first, wFail[w]);
    anyunc |= wUnc[w];
  }
  if (anyunc) {
    // rare: decide the prefixes exactly, in rank order
    float *hsorted = reinterpret_cast<float *>(sm.part_cnt);
    if (live) hsorted[rank] = ent_from_key((uint32_t)(q >> 32));
    __syncthreads();
    const int upto = exact_first_fail(r, hsorted, nq, slot);
    first = upto < nq ? upto : 0x7fffffff;
  }
  // No failure up to the smallest entropy above gamma: the candidate after it
  // fails (its prefix holds an entropy above gamma), or the row ends.
  const int n_star = first != 0x7fffffff ? first : min(nF + 1, nc);
  const int n_commit = nc ? max(n_star, 1) : 0;
  if (live) {
    const bool c1 = rank < n_commit;
    o_row[(uint32_t)q] = c1 ? 1 : 0;
    if (c1 && sk.canvas) sk.canvas[(uint32_t)q] = sm.x0s[(uint32_t)q];
  }
  if (above && key != nxt) o_row[t] = 0;
  if (t < L && !cand) o_row[t] = 0;
  rc = RuleCount{nc, n_commit};
  return true;
}

// ---------------------------------------------------------------- long rows

// Plain LDS bitonic sort of Np keys, ascending.
__device__ inline void block_sort_lds(uint64_t *keys, int Np, int nt) {
  const int tid = threadIdx.x;
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

// Sorted candidate keys of batch row b in sm.keys[0..nc); returns nc.
__device__ inline int sort_candidates(const RuleDev &r, int b, int L, const float *score,
                                      bool by_entropy, const RuleSmem &sm) {
  const int tid = threadIdx.x, nt = sm.nt;
  const int Np = rule_pow2(L);
  const float *s_row = score + (int64_t)b * L;
  const uint8_t *m_row = r.mask + (int64_t)b * L;
  int *cnt = sm.misc + 4;
  if (tid == 0) *cnt = 0;
  __syncthreads();
  int mine = 0;
  for (int i = tid; i < Np; i += nt) {
    uint64_t key = kSentinel;
    const float v = i < L ? (by_entropy ? load_coherent(s_row + i) : rule_conf(r, s_row + i)) : 0.f;
    if (i < L && m_row[i]) {
      const uint32_t hk = by_entropy ? ent_key(v) : conf_key(v);
      key = ((uint64_t)hk << 32) | (uint32_t)i;
      ++mine;
    }
    sm.keys[i] = key;
  }
  if (mine) atomicAdd(cnt, mine);
  __syncthreads();
  const int nc = *cnt;
  block_sort_lds(sm.keys, Np, nt);
  return nc;
}

// Commit the first n of the nc sorted candidates; zero every other position.
__device__ inline RuleCount commit_sorted(const RuleDev &r, int b, int L, int n, int nc,
                                          const RuleSmem &sm, const CommitSink &sk) {
  uint8_t *o_row = r.out + (int64_t)b * L;
  const uint8_t *m_row = r.mask + (int64_t)b * L;
  for (int i = threadIdx.x; i < nc; i += sm.nt) {
    const uint32_t pos = (uint32_t)sm.keys[i];
    o_row[pos] = i < n ? 1 : 0;
    if (i < n && sk.canvas) sk.canvas[pos] = load_coherent_i32(sk.x0 + pos);
  }
  for (int l = threadIdx.x; l < L; l += sm.nt)
    if (!m_row[l]) o_row[l] = 0;
  return RuleCount{nc, n};
}

__device__ inline RuleCount long_rank_rule(const RuleDev &r, int b, int L, const float *conf,
                                           const RuleSmem &sm, const CommitSink &sk) {
  const int nc = sort_candidates(r, b, L, conf, false, sm);
  int n;
  if (r.kind == DLLM_RULE_TOPK) {
    const int k = r.k[b];
    n = k < 0 ? 0 : (k > nc ? nc : k);
  } else {
    int *first_fail = sm.misc + 6;
    if (threadIdx.x == 0) *first_fail = nc;
    __syncthreads();
    for (int i = threadIdx.x; i < nc; i += sm.nt)
      if (!factor_holds(i, conf_from_key((uint32_t)(sm.keys[i] >> 32)), r.param))
        atomicMin(first_fail, i);
    __syncthreads();
    n = nc ? max(*first_fail, 1) : 0;
  }
  return commit_sorted(r, b, L, n, nc, sm, sk);
}

// entropy_bound on the sorted candidates, for any entropies (NaN counts as
// +inf): exact sequential walk in fixed point by one thread.
__device__ inline RuleCount long_entropy_rule(const RuleDev &r, int b, int L, const float *ent,
                                              const RuleSmem &sm, const CommitSink &sk) {
  const int nc = sort_candidates(r, b, L, ent, true, sm);
  int *first_fail = sm.misc + 6;
  if (threadIdx.x == 0) {
    int n_neg_all = 0, n_pos_all = 0;
    for (int i = 0; i < nc; ++i) {
      const uint32_t u = __float_as_uint(ent_from_key((uint32_t)(sm.keys[i] >> 32)));
      n_neg_all += u == 0xff800000u;
      n_pos_all += u == 0x7f800000u;
    }
    Fx s;
    fx_zero(s);
    int ff = nc;
    for (int i = 0; i < nc; ++i) {
      const int n_neg = min(i, n_neg_all), n_pos = max(0, i - (nc - n_pos_all));
      const bool fle = r.gamma_class == 0 ? fx_le(s, r.gamma_fx) : true;
      if (!ent_prefix_ok(r, fle, n_neg, n_pos)) { ff = i; break; }
      const uint32_t u = __float_as_uint(ent_from_key((uint32_t)(sm.keys[i] >> 32)));
      if (bits_finite(u)) fx_add(s, fx_from_f32_bits(u));
    }
    *first_fail = ff;
  }
  __syncthreads();
  const int n = nc ? max(*first_fail, 1) : 0;
  return commit_sorted(r, b, L, n, nc, sm, sk);
}

// threshold: no ranking needed.
__device__ inline RuleCount rule_threshold(const RuleDev &r, int b, int L, const float *conf,
                                           const RuleSmem &sm, const CommitSink &sk) {
  const int tid = threadIdx.x, nt = sm.nt;
  unsigned long long *best = reinterpret_cast<unsigned long long *>(sm.misc + 24);
  int *n_pass = sm.misc + 2;
  int *n_cand = sm.misc + 3;
  if (tid == 0) { *best = kSentinel; *n_pass = 0; *n_cand = 0; }
  __syncthreads();
  const float *c_row = conf + (int64_t)b * L;
  const uint8_t *m_row = r.mask + (int64_t)b * L;
  uint8_t *o_row = r.out + (int64_t)b * L;
  const double tau = r.taus ? r.taus[b] : r.param;
  int my_pass = 0, my_cand = 0;
  uint64_t my_best = kSentinel;
  for (int l = tid; l < L; l += nt) {
    uint8_t v = 0;
    const float cv = rule_conf(r, c_row + l);
    const int32_t xv = sk.canvas ? load_coherent_i32(sk.x0 + l) : 0;
    if (m_row[l]) {
      ++my_cand;
      const float c = conf_sanitized(cv);
      const double cd = (double)c;
      v = (r.strict ? (cd > tau) : (cd >= tau)) ? 1 : 0;
      my_pass += v;
      const uint64_t key = ((uint64_t)conf_key(c) << 32) | (uint32_t)l;
      my_best = key < my_best ? key : my_best;
    }
    o_row[l] = v;
    if (v && sk.canvas) sk.canvas[l] = xv;
  }
  if (my_pass) atomicAdd(n_pass, my_pass);
  if (my_cand) atomicAdd(n_cand, my_cand);
  if (my_best != kSentinel) atomicMin(best, (unsigned long long)my_best);
  __syncthreads();
  RuleCount rc{*n_cand, *n_pass};
  if (tid == 0 && *n_pass == 0 && *best != kSentinel) {
    const uint32_t pos = (uint32_t)*best;
    o_row[pos] = 1;
    if (sk.canvas) sk.canvas[pos] = load_coherent_i32(sk.x0 + pos);
    rc.committed = 1;
  }
  return rc;
}

// Runs a ranking rule on batch row b.  Every thread of the workgroup must call
// it.  `conf` is the confidence (prob) array and `ent` the entropy array.
// Returns the candidate and commit counts (valid in thread 0).
template <bool WIDE = false>
__device__ inline RuleCount run_batch_rule(const RuleDev &r, int b, int L, const float *conf,
                                           const float *ent, unsigned char *smem,
                                           const CommitSink &sk, int nt) {
  const RuleSmem sm = rule_smem(smem, L, nt);
  const bool short_row = L <= nt;
  RuleCount rc{0, 0};
  switch (r.kind) {
    case DLLM_RULE_THRESHOLD:
      rc = rule_threshold(r, b, L, conf, sm, sk);
      break;
    case DLLM_RULE_TOPK:
    case DLLM_RULE_FACTOR:
      if (short_row) rc = short_rank_rule<WIDE>(r, b, L, conf, sm, sk);
      else rc = long_rank_rule(r, b, L, conf, sm, sk);
      break;
    case DLLM_RULE_ENTROPY_BOUND: {
      const bool done = short_row && short_entropy_rule<WIDE>(r, b, L, ent, sm, sk, rc);
      if (!done) {
        __syncthreads();
        rc = long_entropy_rule(r, b, L, ent, sm, sk);
      }
      break;
    }
    default:
      break;
  }
  __syncthreads();
  return rc;
}

__device__ __forceinline__ uint8_t edit_decision(uint8_t editable, int32_t x0, int32_t tok,
                                                 float p, double tau_edit) {
  return (editable && x0 != tok && (double)conf_sanitized(p) > tau_edit) ? 1 : 0;
}

}  // namespace dllm
