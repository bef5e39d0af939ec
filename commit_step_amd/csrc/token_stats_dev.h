// Device side of dllm_token_stats / dllm_commit_step, shared by the two
// translation units that instantiate its kernels (token_stats.hip: the plain
// statistics launch; token_stats_full.hip: the canvas-step / margin variant),
// so the two halves compile in parallel.
//
// The kernel: one pass over (B, L, V) logits -> (x0, prob, entropy) per
// position, optionally followed, in the same launch, by the commit rules.
//
// What is computed: mlx-arsenal research note "dLLM block decoding", "What
// mlx-arsenal ships", token_stats row (proposed token, its probability and the
// entropy, float32, NaN-safe, greedy or Gumbel-max with an explicit key,
// suppress_ids removed before the softmax); mojo-dllm "The GPU path", row
// statistics paragraph (first index of the maximum; p = 1/z; the entropy from
// sum e^(x-m) and sum e^(x-m)(x-m)).
//
// Design for gfx950.  The step reads B*L*V logits once and does a few dozen
// operations per element, so it is bound by HBM bandwidth, with the vector ALU
// close behind for bf16; there is no dense contraction and no MFMA.
//   * Each workgroup streams one row (or a slice of one) with 16-byte loads;
//     consecutive lanes read consecutive 16 bytes, so every wave load is 1 KiB
//     contiguous.  The next chunk is loaded while the current one is reduced.
//   * One pass, where the page's device kernel makes two: the running maximum M
//     is shared by the 64 lanes of a wave (a DPP max per chunk), so a rise of M
//     is a rare, wave-uniform event.  Each lane accumulates, relative to M and
//     in base 2, z- = sum of 2^d over every element except one maximal element,
//     and S = sum 2^d d, d = (x - M) log2 e.  Keeping the maximal element out of
//     z- keeps log z = log1p(z-) accurate for peaked rows (z close to 1); it is
//     excluded exactly once, in the chunk where M rises.
//   * Wave partials (M, first index of M, z-, S) merge associatively through
//     LDS; a row split over several workgroups merges its slices through the
//     caller's workspace, in slice order, so results are bit-reproducible.
//   * prob = 1 / (1 + z-) (greedy) and H = log1p(z-) - ln2 * S / (1 + z-).
//   * Rows holding NaN or +inf, or whose unsuppressed logits are all -inf, are
//     detected after the pass and recomputed by a plain two-pass loop with the
//     exact limit semantics.
//   * Fused rules: the workgroup that finishes the last position of a batch row
//     (a counter in the workspace) runs the ranking rules on the statistics the
//     launch has just written; the edit rule is decided per position.
#pragma once

#include <stdarg.h>
#include <stddef.h>
#include <string.h>

#include <algorithm>

#include "common.h"
#include "rules_dev.h"

namespace dllm {

constexpr float kInf = __builtin_inff();
constexpr int kIdxNone = 0x7fffffff;
constexpr int kMaxRules = 2;
constexpr int kMaxSlices = 256;   // slices of one row (partials merged in LDS)



struct Partial {          // one row slice's statistics (workspace)
  float M;                // max of the slice (-inf: empty)
  int idx;                // first index of M
  float z;                // sum 2^((x-M)log2e) over the slice but one maximal element
  float S;                // sum 2^d d, d = (x-M)log2e
  float sb;               // sampled: best score x/T + g
  int ib;                 // sampled: its index
  float xb;               // sampled: its logit
  float R2;               // runner-up: largest logit but one maximal element (-inf: none)
};
static_assert(sizeof(Partial) == 32, "Partial is zeroed as two 16-byte words");
static_assert(offsetof(Partial, idx) == 4 && offsetof(Partial, S) == 12 &&
                  offsetof(Partial, ib) == 20 && offsetof(Partial, R2) == 28,
              "Partial moves as four (float, 32-bit) pairs");

// Publishing to other workgroups of the same launch, which may run on other
// XCDs (each with its own L2): values are written with agent-scope atomic
// stores (coherent at device level), the writer waits until they have
// completed, and only then counts itself in with a device-scope atomic; the
// reader, having seen the count, reads them with agent-scope atomic loads.
// This is the mechanism an agent-scope release/acquire uses for atomic data,
// without the writeback of the whole L2 that non-atomic data would need.
template <typename V>
__device__ __forceinline__ void store_coherent(V *p, V v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename V>
__device__ __forceinline__ V load_coh(const V *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores_complete() { __builtin_amdgcn_s_waitcnt(0); }

// A partial moves as four 64-bit coherent words (field pairs).
__device__ __forceinline__ uint64_t pack2(uint32_t lo, uint32_t hi) {
  return (uint64_t)lo | ((uint64_t)hi << 32);
}
__device__ __forceinline__ void store_partial(Partial *dst, const Partial &p) {
  uint64_t *w = reinterpret_cast<uint64_t *>(dst);
  store_coherent(&w[0], pack2(__float_as_uint(p.M), (uint32_t)p.idx));
  store_coherent(&w[1], pack2(__float_as_uint(p.z), __float_as_uint(p.S)));
  store_coherent(&w[2], pack2(__float_as_uint(p.sb), (uint32_t)p.ib));
  store_coherent(&w[3], pack2(__float_as_uint(p.xb), __float_as_uint(p.R2)));
}
__device__ __forceinline__ Partial load_partial(const Partial *src) {
  const uint64_t *w = reinterpret_cast<const uint64_t *>(src);
  const uint64_t w0 = load_coh(&w[0]), w1 = load_coh(&w[1]);
  const uint64_t w2 = load_coh(&w[2]), w3 = load_coh(&w[3]);
  Partial p;
  p.M = __uint_as_float((uint32_t)w0); p.idx = (int)(uint32_t)(w0 >> 32);
  p.z = __uint_as_float((uint32_t)w1); p.S = __uint_as_float((uint32_t)(w1 >> 32));
  p.sb = __uint_as_float((uint32_t)w2); p.ib = (int)(uint32_t)(w2 >> 32);
  p.xb = __uint_as_float((uint32_t)w3); p.R2 = __uint_as_float((uint32_t)(w3 >> 32));
  return p;
}

// Kernel arguments.  Every scalar a workgroup reads on its way through a row
// comes first, so it shares the first few 64-byte lines of the argument
// segment (each line a workgroup touches is a scalar-cache miss on its
// critical path); the suppress list and the rules follow.
struct StatsArgs {
  const void *logits;
  int64_t row_stride;
  int64_t V;
  int64_t L;
  int64_t slice_len;       // elements per slice (multiple of 8)
  int slices;
  int skip_rows;           // rows in no rule's mask are neither read nor written
  int need_batch;          // run the batch-row completion (rank rules or counts)
  int n_rank_rules;
  int has_edit;
  int n_suppress;
  int first_allowed;       // lowest id not suppressed
  float inv_temp;          // log2(e) / T: the Gumbel-max score in base-2 units
  uint32_t key0, key1, step;
  int32_t *x0;
  float *prob;
  float *entropy;
  float *margin;           // or NULL
  int32_t *argmax;         // greedy first argmax (also when sampling), or NULL
  float c2;                // log2 e / Ts: Ts the statistics temperature
  const uint8_t *edit_mask;
  uint8_t *edit_out;
  const int32_t *edit_tokens;
  double edit_tau;
  int32_t *canvas;         // (B, L) tokens, updated in place, or NULL (canvas step)
  int32_t *counts;         // (B, 2) candidates left uncommitted, positions edited; or NULL
  // workspace
  uint32_t *batch_count;   // [B]
  uint32_t *row_count;     // [B*L] (slices > 1)
  uint32_t *edit_count;    // [B] edits of the batch row (counts only)
  Partial *partials;       // [B*L*slices] (slices > 1)
  int32_t suppress[DLLM_MAX_SUPPRESS];   // sorted ascending
  RuleDev rank_rules[kMaxRules];
};

// Logits are read exactly once: 16-byte loads with the non-temporal hint, so
// the stream does not churn L2 and the Infinity Cache.
__device__ __forceinline__ uint4 load_stream(const uint4 *p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <typename T> struct ElemT;
template <> struct ElemT<uint16_t> {   // bf16 bit patterns
  static constexpr int VEC = 8;        // elements per 16-byte load
  static constexpr int U = 4;          // loads per lane per chunk
  __device__ static float at(const uint4 &v, int e) {
    const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
    return (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  }
  __device__ static float load1(const uint16_t *p) { return __uint_as_float((uint32_t)*p << 16); }
  __device__ static float widen1(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
};
template <> struct ElemT<float> {
  static constexpr int VEC = 4;
  static constexpr int U = 8;
  __device__ static float at(const uint4 &v, int e) {
    const uint32_t w = e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
    return __uint_as_float(w);
  }
  __device__ static float load1(const float *p) { return *p; }
  __device__ static float widen1(float f) { return f; }
};

// Wave-local running state.  Weights are taken against the reference
// R = RN(M log2 e): an element x weighs 2^(x log2e - R), its exponent one fma,
// so x log2 e is never rounded on its own.  The wave partial is converted to
// weights relative to M itself (2^((x - M) log2 e)) when the stream ends,
// using the exact residual M log2e - R.
struct WaveState {
  float c;       // log2 e / Ts: exponents are x c - R (Ts the statistics temperature)
  float M;       // wave-uniform running max
  float R;       // wave-uniform reference RN(M log2 e)
  int idx;       // wave-uniform first index of M
  float zx, Sx;  // wave-uniform: demoted maxima and ties of M, against R
  float z, S;    // per lane, against R
  float sb;      // per lane sampled best
  int ib;
  float xb;
  float m2;      // per lane: runner-up candidates (largest logit below the top one)
  float m2x;     // wave-uniform: demoted maxima, and M itself once it is tied
};

__device__ __forceinline__ float clamp_d(float d) {
  // d <= a tiny positive residual; below -200 (and -inf) the term 2^d is 0 in
  // float32.  An unsigned min on the bits maps every such d (and -inf) to -200
  // while leaving [-200, +inf) untouched, so 0 * -inf never arises.  NaN d
  // passes through.
  return __uint_as_float(min(__float_as_uint(d), 0xC3480000u));
}

// Process one chunk: every lane holds CH = U * VEC elements, element j of load
// k at index idx_of(k, j, lane).  A chunk that raises the wave maximum takes
// the rescaling path; every other chunk costs one fma, one clamp, one exp2,
// one add and one fma per element.
// Lowest index in the chunk of an element equal to v (some lane holds one):
// the first load k with a match, its lowest lane, that lane's lowest element.
template <int U, int VEC, typename IdxF>
__device__ __forceinline__ int first_index_of(const float (&x)[U * VEC], float v, IdxF idx_of) {
#pragma unroll
  for (int k = 0; k < U; ++k) {
    uint64_t m[VEC], lanes = 0;
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      m[j] = __builtin_amdgcn_ballot_w64(x[k * VEC + j] == v);
      lanes |= m[j];
    }
    if (lanes != 0) {
      const int ln = __builtin_ctzll(lanes);
      int jj = 0;
#pragma unroll
      for (int j = VEC - 1; j >= 0; --j)
        if ((m[j] >> ln) & 1ull) jj = j;
      return idx_of(k, jj, ln);
    }
  }
  return kIdxNone;
}

// ANY_ORDER: chunks may arrive in any index order, so a chunk that ties the
// maximum can still hold its first occurrence.  RUNNER_UP: also track the
// largest logit but one maximal element (for the margin).
template <int U, int VEC, bool ANY_ORDER, bool RUNNER_UP, typename IdxF>
__device__ __forceinline__ void chunk_update(WaveState &st, const float (&x)[U * VEC],
                                             IdxF idx_of) {
  constexpr int CH = U * VEC;
  float cm = x[0];
#pragma unroll
  for (int e = 1; e < CH; ++e) cm = fmaxf(cm, x[e]);
  if (__builtin_amdgcn_ballot_w64(cm > st.M) != 0) {
    // The wave maximum rises (about ln(#chunks) times per wave): rescale,
    // demote the old maximal element into the uniform extra sums, and exclude
    // the new maximal elements from z (one of them stays out; the others are
    // ties and re-enter through zx).  Counting and locating them runs on the
    // scalar unit from ballots.
    const float cmw = wave_max(cm);
    const float Rn = cmw * st.c;
    if (RUNNER_UP) st.m2x = fmaxf(st.m2x, st.M);   // the old maximum is now a runner-up
    if (st.M != -kInf) {
      const float delta = st.R - Rn;
      const float f = __builtin_amdgcn_exp2f(delta);
      st.S = f * fmaf(delta, st.z, st.S);
      st.z = st.z * f;
      const float e0 = fmaf(st.M, st.c, -st.R);        // exact residual
      const float w0 = __builtin_amdgcn_exp2f(e0);
      const float zx1 = st.zx + w0;
      st.Sx = f * fmaf(delta, zx1, fmaf(w0, e0, st.Sx));
      st.zx = zx1 * f;
    }
    st.M = cmw;
    st.R = Rn;
    int cnt = 0, first = kIdxNone;
    float m2c = -kInf;                               // this lane, maxima left out
#pragma unroll
    for (int k = 0; k < U; ++k) {
      uint64_t lanes = 0;
      uint64_t m[VEC];
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        const float xv = x[k * VEC + j];
        const bool eq = xv == cmw;
        m[j] = __builtin_amdgcn_ballot_w64(eq);
        cnt += __builtin_popcountll(m[j]);
        lanes |= m[j];
        const float d = clamp_d(fmaf(xv, st.c, -Rn));
        const float t = eq ? 0.0f : __builtin_amdgcn_exp2f(d);
        st.z += t;
        st.S = fmaf(t, d, st.S);
        if (RUNNER_UP) m2c = fmaxf(m2c, eq ? -kInf : xv);
      }
      if (first == kIdxNone && lanes != 0) {
        const int ln = __builtin_ctzll(lanes);
        int jj = 0;
#pragma unroll
        for (int j = VEC - 1; j >= 0; --j)
          if ((m[j] >> ln) & 1ull) jj = j;
        first = idx_of(k, jj, ln);
      }
    }
    st.idx = first;
    if (RUNNER_UP) {
      st.m2 = fmaxf(st.m2, m2c);
      if (cnt > 1) st.m2x = cmw;                     // a tie: the runner-up is the maximum
    }
    if (cnt > 1) {
      // ties of the new maximum weigh 2^e1 against R
      const float e1 = fmaf(cmw, st.c, -Rn);
      const float w1 = (float)(cnt - 1) * __builtin_amdgcn_exp2f(e1);
      st.zx += w1;
      st.Sx = fmaf(w1, e1, st.Sx);
    }
  } else if (st.M != -kInf) {
    if (RUNNER_UP) st.m2 = fmaxf(st.m2, cm);   // a tie here counts as runner-up
    const float nR = -st.R;
#pragma unroll
    for (int e = 0; e < CH; ++e) {
      const float d = clamp_d(fmaf(x[e], st.c, nR));
      const float t = __builtin_amdgcn_exp2f(d);
      st.z += t;
      st.S = fmaf(t, d, st.S);
    }
    if constexpr (ANY_ORDER) {
      if (__builtin_amdgcn_ballot_w64(cm == st.M) != 0)
        st.idx = min(st.idx, first_index_of<U, VEC>(x, st.M, idx_of));
    }
  }
}

// Wave sums against R -> weights relative to M (exact residual e = M log2e - R:
// 2^(x log2e - M log2e) = 2^(x log2e - R) 2^-e).  A reference that overflowed
// (|M| > 2^127 / log2 e) poisons z so the row takes the two-pass path.
__device__ __forceinline__ void to_max_relative(const WaveState &st, float &z, float &S) {
  if (st.M == -kInf) return;
  if (!bits_finite(__float_as_uint(st.R))) { z = __builtin_nanf(""); return; }
  const float e = fmaf(st.M, st.c, -st.R);
  const float g = __builtin_amdgcn_exp2f(-e);
  S = g * fmaf(-e, z, S);
  z = g * z;
}

// Merge partial b into a (a, b relative to their own maxima).
__device__ __forceinline__ void merge_partial(Partial &a, const Partial &b, float c) {
  if (b.M == -kInf) return;
  if (a.M == -kInf) {
    const float sb = a.sb; const int ib = a.ib; const float xb = a.xb;
    a = b;
    // sampling fields merge separately below
    a.sb = sb; a.ib = ib; a.xb = xb;
  } else {
    Partial w = a, o = b;
    if (b.M > a.M || (b.M == a.M && b.idx < a.idx)) { w = b; o = a; }
    const float delta = (o.M - w.M) * c;
    const float f = __builtin_amdgcn_exp2f(delta);
    const float zo = 1.0f + o.z;
    const float z = w.z + zo * f;
    const float S = w.S + f * fmaf(delta, zo, o.S);
    const float r2 = fmaxf(w.R2, o.M);     // the other part's maximum is a runner-up
    const float sb = a.sb; const int ib = a.ib; const float xb = a.xb;
    a = w;
    a.z = z;
    a.S = S;
    a.R2 = r2;
    a.sb = sb; a.ib = ib; a.xb = xb;
  }
}
__device__ __forceinline__ void merge_sample(Partial &a, const Partial &b) {
  if (b.sb > a.sb || (b.sb == a.sb && b.ib < a.ib)) { a.sb = b.sb; a.ib = b.ib; a.xb = b.xb; }
}

__device__ __forceinline__ Partial empty_partial() {
  Partial p;
  p.M = -kInf; p.idx = kIdxNone; p.z = 0.f; p.S = 0.f;
  p.sb = -kInf; p.ib = kIdxNone; p.xb = -kInf; p.R2 = -kInf;
  return p;
}

// Butterfly merge over the partials of lanes [0, n) of a wave (n a power of
// two, at most 64): log2(n) rounds instead of n - 1 dependent merges.  Both
// merges give the same bits whichever side a partial is on, so every lane of
// the group ends with the same, launch-independent result.
template <bool SAMPLE>
__device__ __forceinline__ Partial butterfly_merge(Partial q, int n, float c) {
  for (int off = 1; off < n; off <<= 1) {
    Partial o;
    o.M = __shfl_xor(q.M, off);
    o.idx = __shfl_xor(q.idx, off);
    o.z = __shfl_xor(q.z, off);
    o.S = __shfl_xor(q.S, off);
    o.R2 = __shfl_xor(q.R2, off);
    if constexpr (SAMPLE) {
      o.sb = __shfl_xor(q.sb, off);
      o.ib = __shfl_xor(q.ib, off);
      o.xb = __shfl_xor(q.xb, off);
    } else {
      o.sb = -kInf; o.ib = kIdxNone; o.xb = -kInf;
    }
    merge_partial(q, o, c);
    if constexpr (SAMPLE) merge_sample(q, o);
  }
  return q;
}

__device__ __forceinline__ bool is_suppressed(const StatsArgs &a, int64_t v) {
  for (int i = 0; i < a.n_suppress; ++i)
    if (a.suppress[i] == v) return true;
  return false;
}

__device__ __forceinline__ float gumbel_at(const StatsArgs &a, uint32_t b, uint32_t l, int64_t v) {
  const Philox4 p = philox4x32_10((uint32_t)(v >> 2), l, b, a.step, a.key0, a.key1);
  const int j = (int)(v & 3);       // a select, not an indexed load (no scratch)
  return gumbel2_from_word(j == 0 ? p.w[0] : j == 1 ? p.w[1] : j == 2 ? p.w[2] : p.w[3]);
}

// The group of four whose best score the lane kept (st.ib its first index):
// reload its logits (the sweep read them in whole 16-byte loads, so all four
// lie in the row), suppress as the sweep did, rescore with the same operations
// (the same bits), and keep the first element that reaches the group's best.
template <typename T>
__device__ __forceinline__ void recover_group_best(const StatsArgs &a, const T *row, uint32_t b,
                                                   uint32_t l, WaveState &st) {
  if (st.ib == kIdxNone) return;
  const int vq = st.ib;
  float xr[4];
  if constexpr (sizeof(T) == 2) {
    const uint2 w = *reinterpret_cast<const uint2 *>(row + vq);
    xr[0] = __uint_as_float(w.x << 16); xr[1] = __uint_as_float(w.x & 0xffff0000u);
    xr[2] = __uint_as_float(w.y << 16); xr[3] = __uint_as_float(w.y & 0xffff0000u);
  } else {
    const uint4 w = *reinterpret_cast<const uint4 *>(row + vq);
    xr[0] = __uint_as_float(w.x); xr[1] = __uint_as_float(w.y);
    xr[2] = __uint_as_float(w.z); xr[3] = __uint_as_float(w.w);
  }
  for (int i = 0; i < a.n_suppress; ++i) {
    const int d = a.suppress[i] - vq;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (d == j) xr[j] = -kInf;
  }
  const Philox4 p = philox4x32_10((uint32_t)vq >> 2, l, b, a.step, a.key0, a.key1);
  int jb = 0;
  float xb = xr[0];
#pragma unroll
  for (int j = 3; j >= 0; --j) {
    const float sc = fmaf(xr[j], a.inv_temp, gumbel2_from_word(p.w[j]));
    if (sc == st.sb) { jb = j; xb = xr[j]; }
  }
  st.ib = vq + jb;
  st.xb = xb;
}

// The span of VEC elements whose best score the lane kept on a split row
// (st.ib the span's first index; its four-element generator groups start r =
// st.ib & 3 elements before it): reload it (a whole 16-byte load of the
// slice's aligned body), suppress and rescore exactly as the sweep did (the
// same bits), and keep the first element that reaches the span's best.
template <typename T>
__device__ __forceinline__ void recover_span_best(const StatsArgs &a, const T *row, uint32_t b,
                                                  uint32_t l, WaveState &st) {
  using E = ElemT<T>;
  constexpr int VEC = E::VEC;
  constexpr int NG = VEC / 4 + 1;
  if (st.ib == kIdxNone) return;
  const int v0 = st.ib, r = v0 & 3;
  const uint4 w = *reinterpret_cast<const uint4 *>(row + v0);
  float xr[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) xr[e] = E::at(w, e);
  for (int i = 0; i < a.n_suppress; ++i) {
    const int d = a.suppress[i] - v0;
#pragma unroll
    for (int j = 0; j < VEC; ++j)
      if (d == j) xr[j] = -kInf;
  }
  uint32_t wd[4 * NG];
#pragma unroll
  for (int q = 0; q < NG; ++q) {
    const Philox4 p = philox4x32_10((uint32_t)(v0 >> 2) + q, l, b, a.step, a.key0, a.key1);
#pragma unroll
    for (int j = 0; j < 4; ++j) wd[4 * q + j] = p.w[j];
  }
  int jb = 0;
  float xb = xr[0];
#pragma unroll
  for (int j = VEC - 1; j >= 0; --j) {
    const uint32_t wj = r == 0 ? wd[j] : r == 1 ? wd[j + 1] : r == 2 ? wd[j + 2] : wd[j + 3];
    const float sc = fmaf(xr[j], a.inv_temp, gumbel2_from_word(wj));
    if (sc == st.sb) { jb = j; xb = xr[j]; }
  }
  st.ib = v0 + jb;
  st.xb = xb;
}

// The greedy pass reads the output pointers (x0, prob, entropy, ...: one
// line of the argument block) first when it publishes the row; loading one of
// them while the first logit loads are in flight puts that line in the scalar
// cache, so publication does not wait on the miss.  The sampled pass reads the
// same line for its generator key at the start.
template <bool SAMPLE>
__device__ __forceinline__ void touch_publish_args(const StatsArgs &a) {
  if constexpr (!SAMPLE) asm volatile("" ::"s"(a.x0));
}

// Stream [lo, hi) of one row.  VECLOAD: 16-byte loads (row start 16-byte
// aligned, lo/hi multiples of VEC).  Full workgroup iterations run without
// bounds checks, with the next iteration's loads in flight while the current
// one is reduced; one masked iteration finishes the slice.  The workgroup's
// partial lands in *out (valid in thread 0).
// FULL: the canvas-step / margin variant (row skipping, runner-up tracking);
// the plain statistics launch compiles without either.
// SPLIT (rows that are not 16-byte aligned, VECLOAD): the slice's
// 16-byte-aligned body [blo, bhi) streams with 16-byte loads, and its head
// [lo, blo) and tail [bhi, hi), fewer than VEC elements each, are read one
// element per lane by wave 0 at the end, as one more chunk in any index order.
// A sampled body load starts r = blo & 3 elements into a generator group, so
// it draws from VEC / 4 + 1 groups (VEC / 4 when r is 0) and keeps the best
// score of its whole span (recover_span_best finds the element).
template <typename T, int NT, int UV, bool SAMPLE, bool VECLOAD, bool FULL, bool SPLIT>
__device__ void stream_slice(const StatsArgs &a, const T *row, int64_t lo, int64_t hi,
                             uint32_t b, uint32_t l, Partial *wave_parts, Partial *out) {
  static_assert(!SPLIT || VECLOAD, "SPLIT: 16-byte-load kernels only");
  using E = ElemT<T>;
  constexpr int VEC = VECLOAD ? E::VEC : 1;
  constexpr int U = VECLOAD ? UV : 8;
  constexpr int CH = VEC * U;
  constexpr int STEP = NT * CH;                 // elements per workgroup iteration
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  WaveState st;
  st.c = a.c2;
  st.M = -kInf; st.R = -kInf; st.idx = kIdxNone; st.zx = 0.f; st.Sx = 0.f; st.z = 0.f; st.S = 0.f;
  st.sb = -kInf; st.ib = kIdxNone; st.xb = -kInf; st.m2 = -kInf; st.m2x = -kInf;
  // Every row sweeps its iterations in index order.  (Starting each row at a
  // row-dependent iteration, to keep rows that lie 512 KiB apart off the
  // same HBM channels at the same time, measured 0.2 us slower on the 256-row
  // canvas once the loads were non-temporal.)
  int sp = 0;          // next suppress id not below the current iteration
  // SPLIT and SAMPLE: all-ones masks for bits 1 and 0 of blo & 3, held in
  // vector registers the compiler cannot see through, so that the word
  // choices below are bitwise merges (a select on them became a dynamically
  // indexed array in scratch memory, a uniform one a chain of branches)
  uint32_t m2 = 0u, m1 = 0u;

  auto process = [&](float (&x)[CH], int64_t base) {
    // suppress ids inside this iteration (rare, workgroup-uniform test); the
    // bases ascend
    while (sp < a.n_suppress && a.suppress[sp] < base) ++sp;
    if (sp < a.n_suppress && a.suppress[sp] < base + STEP) {
      for (int q = sp; q < a.n_suppress && a.suppress[q] < base + STEP; ++q) {
        // element (k, thread, e) of the iteration holds base + (k NT + thread) VEC + e;
        // the owner and slot are uniform, so x stays in registers
        const int off = (int)(a.suppress[q] - base);
        const int ks = off / (NT * VEC), rs = off - ks * (NT * VEC);
        const int owner = rs / VEC, es = rs - owner * VEC;
        if (tid == owner) {
#pragma unroll
          for (int k = 0; k < U; ++k)
#pragma unroll
            for (int e = 0; e < VEC; ++e)
              if (k == ks && e == es) x[k * VEC + e] = -kInf;
        }
      }
    }
    if constexpr (SAMPLE) {
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const int64_t v0 = base + (int64_t)(k * NT + tid) * VEC;
        if constexpr (SPLIT) {
          // the span v0 .. v0 + VEC - 1 starts r = blo & 3 words into group
          // v0 >> 2 (the same r for the whole slice: every body load starts
          // at blo plus a multiple of VEC); element j takes word r + j of the
          // groups' words in a row, merged in two steps (r & 2, then r & 1)
          constexpr int NG = VEC / 4 + 1;
          uint32_t wd[4 * NG];
#pragma unroll
          for (int q = 0; q < NG; ++q) {
            const Philox4 p =
                philox4x32_10((uint32_t)(v0 >> 2) + q, l, b, a.step, a.key0, a.key1);
#pragma unroll
            for (int j = 0; j < 4; ++j) wd[4 * q + j] = p.w[j];
          }
          uint32_t wt[4 * NG - 2];
#pragma unroll
          for (int i = 0; i < 4 * NG - 2; ++i) wt[i] = (wd[i + 2] & m2) | (wd[i] & ~m2);
          float gm = -kInf;
#pragma unroll
          for (int j = 0; j < VEC; ++j) {
            const uint32_t wj = (wt[j + 1] & m1) | (wt[j] & ~m1);
            gm = fmaxf(gm, fmaf(x[k * VEC + j], a.inv_temp, gumbel2_from_word(wj)));
          }
          if (gm > st.sb) { st.sb = gm; st.ib = (int)v0; }
        } else if constexpr (VEC >= 4) {
          // One generator call scores a group of four: only the group's best
          // score and the group's first index are kept (strictly greater
          // keeps the earlier group on ties); the element and its logit are
          // recovered once, when the stream ends (recover_group_best).
#pragma unroll
          for (int q = 0; q < VEC / 4; ++q) {
            const int64_t vq = v0 + 4 * q;
            const Philox4 p = philox4x32_10((uint32_t)(vq >> 2), l, b, a.step, a.key0, a.key1);
            float sc[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
              sc[j] = fmaf(x[k * VEC + 4 * q + j], a.inv_temp, gumbel2_from_word(p.w[j]));
            const float gm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
            if (gm > st.sb) { st.sb = gm; st.ib = (int)vq; }
          }
        } else {
          const float xv = x[k];
          if (v0 < hi) {
            const float sc = fmaf(xv, a.inv_temp, gumbel_at(a, b, l, v0));
            if (sc > st.sb) { st.sb = sc; st.ib = (int)v0; st.xb = xv; }
          }
        }
      }
    }
    chunk_update<U, VEC, false, FULL>(st, x, [&](int k, int j, int ln) -> int {
      return (int)(base + (int64_t)(k * NT + wave * 64 + ln) * VEC + j);
    });
  };

  float x[CH];
  if constexpr (VECLOAD) {
    constexpr int64_t ITER = STEP / VEC;          // uint4 per workgroup iteration
    int64_t blo = lo, bhi = hi;                   // the 16-byte-load body
    if constexpr (SPLIT) {
      const uint32_t mis = (uint32_t)reinterpret_cast<uintptr_t>(row + lo) & 15u;
      blo = min(lo + (int64_t)(((16u - mis) & 15u) / sizeof(T)), hi);
      bhi = blo + (hi - blo) / VEC * VEC;
      if constexpr (SAMPLE) {
        m2 = (blo & 2) ? ~0u : 0u;
        m1 = (blo & 1) ? ~0u : 0u;
        asm volatile("" : "+v"(m2), "+v"(m1));
      }
    }
    const int64_t n_full = (bhi - blo) / STEP;
    const uint4 *p = reinterpret_cast<const uint4 *>(row + blo) + tid;
    // Two register buffers in turn: the loads of iteration i + 1 are in flight
    // while iteration i is reduced, and no buffer is ever copied.
    auto load = [&](uint4 (&r)[U], int64_t it) {
      const uint4 *q = p + it * ITER;
#pragma unroll
      for (int k = 0; k < U; ++k) r[k] = load_stream(q + k * NT);
    };
    auto run = [&](const uint4 (&r)[U], int64_t it) {
#pragma unroll
      for (int k = 0; k < U; ++k)
#pragma unroll
        for (int e = 0; e < VEC; ++e) x[k * VEC + e] = E::at(r[k], e);
      process(x, blo + it * STEP);
    };
    if (n_full > 0) {
      uint4 ba[U], bb[U];
      load(ba, 0);
      touch_publish_args<SAMPLE>(a);
      int64_t it = 0;
      for (; it + 2 < n_full; it += 2) {
        load(bb, it + 1);
        run(ba, it);
        load(ba, it + 2);
        run(bb, it + 1);
      }
      if (it + 1 < n_full) {
        load(bb, it + 1);
        run(ba, it);
        run(bb, it + 1);
      } else {
        run(ba, it);
      }
    }
    const int64_t tb = blo + n_full * STEP;
    if (tb < bhi) {
      // The masked iteration issues all its loads before it uses any (a load
      // inside a divergent branch made the compiler wait for it there, one
      // round trip per slot): a slot that no lane needs is skipped on a
      // uniform branch, and a lane past the end reads the slice's first word
      // instead (in bounds, its value unused).
      uint4 r[U];
#pragma unroll
      for (int k = 0; k < U; ++k) {
        // a skipped slot keeps an unspecified value (an empty asm defines it
        // without an instruction); no lane reads it
        asm("" : "=v"(r[k].x), "=v"(r[k].y), "=v"(r[k].z), "=v"(r[k].w));
        if (tb + (int64_t)k * NT * VEC < bhi) {
          const int64_t v0 = tb + (int64_t)(k * NT + tid) * VEC;
          r[k] = load_stream(reinterpret_cast<const uint4 *>(row + (v0 < bhi ? v0 : blo)));
        }
      }
      touch_publish_args<SAMPLE>(a);
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const bool ok = tb + (int64_t)(k * NT + tid) * VEC < bhi;
#pragma unroll
        for (int e = 0; e < VEC; ++e) x[k * VEC + e] = ok ? E::at(r[k], e) : -kInf;
      }
      process(x, tb);
    }
    if constexpr (SPLIT) {
      if constexpr (SAMPLE) recover_span_best(a, row, b, l, st);
      // head and tail: lane j < nh holds element lo + j, lane nh + j element
      // bhi + j; in index order along the lanes
      const int nh = (int)(blo - lo), nq = (int)(hi - bhi);
      if (wave == 0 && nh + nq > 0) {
        const bool mine = lane < nh + nq;
        const int64_t v = lane < nh ? lo + lane : bhi + (lane - nh);
        float x1[1];
        x1[0] = -kInf;
        if (mine) {
          const float xv = E::load1(row + v);
          x1[0] = is_suppressed(a, v) ? -kInf : xv;
          if constexpr (SAMPLE) {
            // the lane's kept element (if any) lies in the body; a head
            // element comes before it and wins a tie
            const float sc = fmaf(x1[0], a.inv_temp, gumbel_at(a, b, l, v));
            if (sc > st.sb || (sc == st.sb && st.ib != kIdxNone && v < st.ib)) {
              st.sb = sc; st.ib = (int)v; st.xb = x1[0];
            }
          }
        }
        chunk_update<1, 1, true, FULL>(st, x1, [&](int, int, int ln) -> int {
          return (int)(ln < nh ? lo + ln : bhi + (ln - nh));
        });
      }
    }
  } else {
    // Rows without 16-byte alignment: one element per load, every load of an
    // iteration issued before any is used (a lane past the end reads the
    // slice's first element, its value unused), two register sets in turn.
    const int64_t n_it = (hi - lo + STEP - 1) / STEP;
    T ra[U], rb[U];
    auto ld = [&](T (&r)[U], int64_t it) {
      const int64_t base = lo + it * STEP;
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const int64_t v = base + (int64_t)(k * NT + tid);
        r[k] = row[v < hi ? v : lo];
      }
    };
    auto use = [&](const T (&r)[U], int64_t it) {
      const int64_t base = lo + it * STEP;
#pragma unroll
      for (int k = 0; k < U; ++k)
        x[k] = base + (int64_t)(k * NT + tid) < hi ? E::widen1(r[k]) : -kInf;
      process(x, base);
    };
    ld(ra, 0);
    int64_t it = 0;
    for (; it + 2 < n_it; it += 2) {
      ld(rb, it + 1);
      use(ra, it);
      ld(ra, it + 2);
      use(rb, it + 1);
    }
    if (it + 1 < n_it) {
      ld(rb, it + 1);
      use(ra, it);
      use(rb, it + 1);
    } else {
      use(ra, it);
    }
  }

  if constexpr (SAMPLE && VECLOAD && !SPLIT) recover_group_best(a, row, b, l, st);

  // Wave partial -> LDS.
  Partial p;
  p.M = st.M;
  p.idx = st.idx;
  p.z = wave_sum(st.z) + st.zx;
  p.S = wave_sum(st.S) + st.Sx;
  to_max_relative(st, p.z, p.S);
  p.sb = -kInf; p.ib = kIdxNone; p.xb = -kInf;
  p.R2 = FULL ? fmaxf(wave_max(st.m2), st.m2x) : -kInf;
  if constexpr (SAMPLE) {
    // first-best over the lanes: max score, lowest index on ties
    float sb = st.sb; int ib = st.ib; float xb = st.xb;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float osb = __shfl_xor(sb, off);
      const int oib = __shfl_xor(ib, off);
      const float oxb = __shfl_xor(xb, off);
      if (osb > sb || (osb == sb && oib < ib)) { sb = osb; ib = oib; xb = oxb; }
    }
    p.sb = sb; p.ib = ib; p.xb = xb;
  }
  if (lane == 0) wave_parts[wave] = p;
  __syncthreads();
  if (wave == 0) {
    constexpr int NW = NT / 64;
    const Partial acc =
        butterfly_merge<SAMPLE>(lane < NW ? wave_parts[lane] : empty_partial(), NW, a.c2);
    if (lane == 0) *out = acc;
  }
}

struct RowResult { int x0; float prob; float ent; float margin; int argmax; };

// Plain two-pass recomputation of a degenerate row (NaN, +inf, or no finite
// unsuppressed logit), with the limit semantics of the header.  Every thread
// of the workgroup calls it; the result is valid in thread 0.
template <typename T, int NT, bool SAMPLE>
__device__ RowResult slow_row(const StatsArgs &a, const T *row, uint32_t b, uint32_t l,
                              unsigned char *scratch) {
  using E = ElemT<T>;
  const int tid = threadIdx.x;
  float *fs = reinterpret_cast<float *>(scratch);          // [NT]
  int *is = reinterpret_cast<int *>(scratch) + NT;         // [NT]
  int *js = reinterpret_cast<int *>(scratch) + 2 * NT;     // [NT]
  float *gs = reinterpret_cast<float *>(scratch) + 3 * NT; // [NT]
  const int64_t V = a.V;
  // pass 1: max (NaN -> -inf), its first index, number and first index of +inf
  float m = -kInf; int im = kIdxNone; int ninf = 0; int iinf = kIdxNone;
  for (int64_t v = tid; v < V; v += NT) {
    if (is_suppressed(a, v)) continue;
    float x = E::load1(row + v);
    if (x != x) x = -kInf;
    if (x > m) { m = x; im = (int)v; }
    if (x == kInf) { ++ninf; if (iinf == kIdxNone) iinf = (int)v; }
  }
  fs[tid] = m; is[tid] = im; js[tid] = ninf; gs[tid] = __int_as_float(iinf);
  __syncthreads();
  __shared__ float s_m;
  __shared__ int s_im, s_ninf, s_iinf;
  if (tid == 0) {
    float M = -kInf; int IM = kIdxNone; int N = 0; int II = kIdxNone;
    for (int t = 0; t < NT; ++t) {
      if (fs[t] > M || (fs[t] == M && is[t] < IM)) { M = fs[t]; IM = is[t]; }
      N += js[t];
      II = min(II, __float_as_int(gs[t]));
    }
    s_m = M; s_im = IM; s_ninf = N; s_iinf = II;
  }
  __syncthreads();
  const float M = s_m;
  const int nA = (int)V - a.n_suppress;
  const bool finite = bits_finite(__float_as_uint(M));
  // pass 2: sums relative to M excluding the first maximal element (finite M),
  // the runner-up logit, and the sampled argmax over the relevant support.
  float z = 0.f, S = 0.f, sb = -kInf, xb = -kInf, r2 = -kInf; int ib = kIdxNone;
  for (int64_t v = tid; v < V; v += NT) {
    if (is_suppressed(a, v)) continue;
    float x = E::load1(row + v);
    if (x != x) x = -kInf;
    if (finite) {
      if (v != s_im) {
        r2 = fmaxf(r2, x);
        const float d = (x - M) * a.c2;
        const float t = __builtin_amdgcn_exp2f(d);
        z += t;
        if (t > 0.f) S = fmaf(t, d, S);
      }
      if (SAMPLE) {
        const float s = fmaf(x, a.inv_temp, gumbel_at(a, b, l, v));
        if (s > sb) { sb = s; ib = (int)v; xb = x; }
      }
    } else if (SAMPLE) {
      const bool in_support = (M == -kInf) ? true : (x == kInf);
      if (in_support) {
        const float g = gumbel_at(a, b, l, v);
        if (g > sb) { sb = g; ib = (int)v; xb = x; }
      }
    }
  }
  __syncthreads();
  fs[tid] = z; gs[tid] = S; is[tid] = ib; js[tid] = __float_as_int(sb);
  float *xs = reinterpret_cast<float *>(scratch) + 4 * NT;
  float *rs = reinterpret_cast<float *>(scratch) + 5 * NT;
  xs[tid] = xb;
  rs[tid] = r2;
  __syncthreads();
  RowResult r;
  r.x0 = 0; r.prob = 0.f; r.ent = 0.f; r.margin = 0.f; r.argmax = 0;
  if (tid == 0) {
    float Z = 0.f, SS = 0.f, SB = -kInf, XB = -kInf, R2 = -kInf; int IB = kIdxNone;
    for (int t = 0; t < NT; ++t) {
      Z += fs[t];
      SS += gs[t];
      R2 = fmaxf(R2, rs[t]);
      const float s = __int_as_float(js[t]);
      if (s > SB || (s == SB && is[t] < IB)) { SB = s; IB = is[t]; XB = xs[t]; }
    }
    if (finite) {
      r.ent = log1pf(Z) - kLn2 * SS / (1.0f + Z);
      r.margin = -expm1f((R2 - M) * a.c2 * kLn2) / (1.0f + Z);
      r.argmax = s_im;
      if (SAMPLE) {
        r.x0 = IB;
        r.prob = __builtin_amdgcn_exp2f((XB - M) * a.c2) / (1.0f + Z);
      } else {
        r.x0 = s_im;
        r.prob = 1.0f / (1.0f + Z);
      }
    } else if (M == -kInf) {
      r.x0 = SAMPLE ? IB : a.first_allowed;
      r.argmax = a.first_allowed;
      r.prob = 1.0f / (float)nA;
      r.ent = logf((float)nA);
      r.margin = nA == 1 ? 1.0f : 0.0f;
    } else {
      r.x0 = SAMPLE ? IB : s_iinf;
      r.argmax = s_iinf;
      r.prob = 1.0f / (float)s_ninf;
      r.ent = logf((float)s_ninf);
      r.margin = s_ninf == 1 ? 1.0f : 0.0f;
    }
  }
  return r;
}

// Does any fused rule look at this row?
__device__ __forceinline__ bool row_needed(const StatsArgs &a, int64_t row_id) {
  // every mask byte is loaded before any is tested (no short-circuit, whose
  // branch on a loaded byte would cost a round trip per mask)
  uint32_t need = a.has_edit ? a.edit_mask[row_id] : 0u;
#pragma unroll
  for (int r = 0; r < kMaxRules; ++r)
    need |= r < a.n_rank_rules ? a.rank_rules[r].mask[row_id] : 0u;
  return need != 0;
}

// log(1 + z) for finite z >= 0 in a few instructions: with u = RN(1 + z),
// log1p(z) = log(u) z / (u - 1), which keeps the relative accuracy of log(u)
// however small z is (D. Goldberg, "What every computer scientist should know
// about floating-point arithmetic", ACM Computing Surveys 23(1), 1991,
// Theorem 4); log(u) from the hardware base-2 logarithm (1 ulp) and the
// quotient from the hardware reciprocal (1 ulp): a few ulp in all.
__device__ __forceinline__ float log1p_nonneg(float z) {
  const float u = 1.0f + z;
  const float um1 = u - 1.0f;
  if (um1 == 0.0f) return z;
  return __builtin_amdgcn_logf(u) * kLn2 * (z * __builtin_amdgcn_rcpf(um1));
}

// The row's statistics from its merged partial; false for a degenerate row
// (NaN, +inf, no finite unsuppressed logit), which slow_row recomputes.  One
// thread runs this on the critical path after the slowest row's stream, so it
// uses the hardware reciprocal and logarithm (a few ulp) instead of the
// correctly rounded division and the library log1p (~150 dependent
// instructions).  z >= 0 and S <= 0 (every d <= 0), so H = log1p(z) - ln2 S /
// (1 + z) adds two non-negative terms and keeps their relative accuracy.
template <bool SAMPLE, bool FULL>
__device__ __forceinline__ bool finalize_partial(const Partial &p, float c, RowResult &res) {
  const bool ok = bits_finite(__float_as_uint(p.M)) && bits_finite(__float_as_uint(p.z)) &&
                  bits_finite(__float_as_uint(p.S)) &&
                  (!SAMPLE || (p.ib != kIdxNone && bits_finite(__float_as_uint(p.sb))));
  if (ok) {
    const float zf = 1.0f + p.z;
    const float rz = __builtin_amdgcn_rcpf(zf);
    res.ent = log1p_nonneg(p.z) - kLn2 * p.S * rz;
    // (1 - e^((runner-up - max)/Ts)) / z; only the FULL kernels track the runner-up
    res.margin = FULL ? -expm1f((p.R2 - p.M) * c * kLn2) * rz : 0.f;
    res.argmax = p.idx;
    if (SAMPLE) {
      res.x0 = p.ib;
      res.prob = __builtin_amdgcn_exp2f((p.xb - p.M) * c) * rz;
    } else {
      res.x0 = p.idx;
      res.prob = rz;
    }
  }
  return ok;
}

// Writes one row's statistics (coherent: the batch-row finisher and the
// rules read them) and decides its edit; returns 1 if the row was edited.
__device__ __forceinline__ int publish_row(const StatsArgs &a, int64_t row_id,
                                           const RowResult &res, uint8_t edit_m, int32_t edit_t) {
  store_coherent(&a.x0[row_id], res.x0);
  store_coherent(&a.prob[row_id], res.prob);
  store_coherent(&a.entropy[row_id], res.ent);
  if (a.margin) store_coherent(&a.margin[row_id], res.margin);
  if (a.argmax) a.argmax[row_id] = res.argmax;
  if (!a.has_edit) return 0;
  const uint8_t e = edit_decision(edit_m, res.x0, edit_t, res.prob, a.edit_tau);
  a.edit_out[row_id] = e;
  if (e && a.canvas) a.canvas[row_id] = res.x0;      // this row's own token
  return e;
}

// Counts of batch row b: candidates the rank rule left uncommitted and
// positions edited.  The rule has already written x0 into the canvas at the
// positions it committed.  edits < 0: the edit count is in the workspace.
__device__ inline void finish_counts(const StatsArgs &a, uint32_t b, int edits,
                                     const RuleCount &rc) {
  if (threadIdx.x != 0 || !a.counts) return;
  if (edits < 0) {
    edits = (int)load_coh(&a.edit_count[b]);
    a.edit_count[b] = 0u;        // leave the workspace zeroed
  }
  a.counts[2 * b] = a.n_rank_rules ? rc.nc - rc.committed : 0;
  a.counts[2 * b + 1] = edits;
}

// The batch row's statistics are all published: rank rules (the first one
// also updating the canvas), then the counts.
__device__ inline void complete_batch_row(const StatsArgs &a, uint32_t b, unsigned char *smem,
                                          int edits, int nt) {
  RuleCount rc0{0, 0};
  for (int r = 0; r < a.n_rank_rules; ++r) {
    const RuleDev &rule = a.rank_rules[r];
    const float *conf = rule.score == DLLM_SCORE_MARGIN        ? a.margin
                        : rule.score == DLLM_SCORE_NEG_ENTROPY ? a.entropy
                                                               : a.prob;
    const CommitSink sk{r == 0 && a.canvas ? a.canvas + (int64_t)b * a.L : nullptr,
                        a.x0 + (int64_t)b * a.L};
    const RuleCount rc = run_batch_rule(rule, (int)b, (int)a.L, conf, a.entropy, smem, sk, nt);
    if (r == 0) rc0 = rc;
  }
  finish_counts(a, b, edits, rc0);
  if (threadIdx.x == 0) a.batch_count[b] = 0u;   // leave the workspace zeroed
}

// Whole rows: after a row's statistics are published, count the row into its
// batch row; the workgroup that completes the batch row runs the rank rules on
// the statistics the launch has just written (coherent loads), then the canvas
// update and the counts.
__device__ inline void finish_row(const StatsArgs &a, uint32_t b, unsigned char *smem, int nt,
                                  uint32_t *batch_cnt) {
  __shared__ int s_last;
  const int tid = threadIdx.x;
  if (!a.need_batch) return;
  // Bring the argument fields that the batch-row completion reads into the
  // scalar cache now, all at once, while the row's stores drain: after tens of
  // microseconds of streaming they have left it, and the one workgroup that
  // completes the batch row would otherwise take several dependent
  // argument-load misses after its count returns (measured: 0.4-0.6 us).
  asm volatile("" ::"s"(a.L), "s"(a.n_rank_rules), "s"(a.x0), "s"(a.entropy), "s"(a.canvas),
               "s"(a.edit_count), "s"(a.rank_rules[0].mask), "s"(a.rank_rules[0].param),
               "s"(a.rank_rules[0].gamma_class));
  if (tid == 0) {
    wait_stores_complete();
    DLLM_STAGE(kStageStoresDrained);
    const uint32_t prev = atomicAdd(batch_cnt, 1u);
    s_last = (prev == (uint32_t)(a.L - 1));
    DLLM_STAGE(kStageBatchCounted);
  }
  __syncthreads();
  if (!s_last) return;
  complete_batch_row(a, b, smem, -1, nt);
  DLLM_STAGE(kStageBatchDone);
}

template <typename T, int NT, int UV, bool SAMPLE, bool VECLOAD, bool FULL, bool SPLIT>
__global__ __launch_bounds__(NT) void token_stats_kernel(StatsArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];   // slice partials, then the rules
  __shared__ Partial wave_parts[NT / 64];
  __shared__ Partial slice_parts_acc;
  __shared__ int s_flag;
  __shared__ __align__(16) unsigned char slow_scratch[6 * NT * 4];

  const int tid = threadIdx.x;
  DLLM_STAGE_SCOPE();
  DLLM_STAGE(kStageStart);
  // The argument fields the prologue needs, in one round of scalar loads (at
  // the launch's start they all miss the scalar cache, and dependent rounds
  // add up).
  asm volatile("" ::"s"(a.logits), "s"(a.row_stride), "s"(a.V), "s"(a.L), "s"(a.slice_len),
               "s"(a.slices), "s"(a.has_edit), "s"(a.c2));
  if constexpr (FULL)
    asm volatile("" ::"s"(a.skip_rows), "s"(a.n_rank_rules), "s"(a.rank_rules[0].mask));
  // 32-bit index arithmetic: the host limits a launch to fewer than 2^32
  // workgroups and L to below 2^31.
  const uint32_t wg = blockIdx.x;
  const uint32_t ns = (uint32_t)a.slices, nl = (uint32_t)a.L;
  const uint32_t row32 = ns == 1u ? wg : wg / ns;
  const int64_t row_id = row32;
  const int slice = (int)(wg - row32 * ns);
  const uint32_t b = row32 < nl ? 0u : row32 / nl, l = row32 - b * nl;
  const T *row = reinterpret_cast<const T *>(a.logits) + row_id * a.row_stride;
  const int64_t lo = (int64_t)slice * a.slice_len;
  const int64_t hi = min(lo + a.slice_len, a.V);

  // Candidate-row skipping: a row that no rule looks at is not read, and its
  // statistics are left as they were; an edit rule's output for it is 0.
  // Slice 0 still counts it into its batch row.
  if (FULL && a.skip_rows && !row_needed(a, row_id)) {
    if (slice != 0) return;
    if (tid == 0 && a.has_edit) a.edit_out[row_id] = 0;
    DLLM_STAGE(kStageSkipped);
    finish_row(a, b, smem, NT, a.batch_count + b);
    return;
  }

  // The edit rule's inputs for this row, loaded before the stream so that
  // their latency hides behind it (the tokens are read before any write of
  // this launch, as they would be at publication).
  uint8_t edit_m = 0;
  int32_t edit_t = 0;
  if (tid == 0 && a.has_edit) {
    edit_m = a.edit_mask[row_id];
    edit_t = a.edit_tokens[row_id];
  }

  stream_slice<T, NT, UV, SAMPLE, VECLOAD, FULL, SPLIT>(a, row, lo, hi, b, l, wave_parts,
                                                 &slice_parts_acc);
  DLLM_STAGE(kStageStreamEnd);

  // The hand-off counters' base addresses, loaded here (an empty asm that
  // uses them) so that these argument loads are not on the hand-off's
  // critical path once the stores have drained.
  asm volatile("" ::"s"(a.row_count), "s"(a.batch_count));
  uint32_t *row_cnt = a.row_count + row_id;    // used only with split rows
  uint32_t *batch_cnt = a.batch_count + b;

  // Split rows: publish the slice partial and count it on the row's own
  // counter (a counter per row keeps the atomics of a launch spread out); the
  // last slice to arrive fetches every slice's partial at once into LDS and
  // merges them in slice order.
  if (a.slices > 1) {
    Partial *parts = &a.partials[row_id * a.slices];
    if (tid == 0) {
      store_partial(&parts[slice], slice_parts_acc);
      wait_stores_complete();
      const uint32_t prev = atomicAdd(row_cnt, 1u);
      s_flag = (prev == (uint32_t)(a.slices - 1));
      DLLM_STAGE(kStageSliceCounted);
    }
    __syncthreads();
    if (!s_flag) return;
    Partial *lds = reinterpret_cast<Partial *>(smem);    // [slices], before the rules use it
    for (int s = tid; s < a.slices; s += NT) lds[s] = load_partial(&parts[s]);
    __syncthreads();
    if (tid < 64) {
      // lane l merges slices l, l + 64, ... in order, then a butterfly over
      // the lanes: a fixed order, so results are reproducible
      Partial acc = tid < a.slices ? lds[tid] : empty_partial();
      for (int s = tid + 64; s < a.slices; s += 64) {
        merge_partial(acc, lds[s], a.c2);
        if (SAMPLE) merge_sample(acc, lds[s]);
      }
      int n = 1;
      while (n < a.slices && n < 64) n <<= 1;
      acc = butterfly_merge<SAMPLE>(acc, n, a.c2);
      if (tid == 0) {
        slice_parts_acc = acc;
        *row_cnt = 0u;
      }
    }
    __syncthreads();
    DLLM_STAGE(kStageRowMerged);
  }

  // Finalize the row.
  __shared__ int s_slow;
  RowResult res;
  res.x0 = 0; res.prob = 0.f; res.ent = 0.f; res.margin = 0.f; res.argmax = 0;
  if (tid == 0) s_slow = !finalize_partial<SAMPLE, FULL>(slice_parts_acc, a.c2, res);
  DLLM_STAGE(kStageFinalized);
  __syncthreads();
  if (s_slow) res = slow_row<T, NT, SAMPLE>(a, row, b, l, slow_scratch);
  if (tid == 0 && publish_row(a, row_id, res, edit_m, edit_t) && a.counts)
    atomicAdd(&a.edit_count[b], 1u);
  DLLM_STAGE(kStagePublished);
  if (a.slices > 1) {
    Partial *parts = &a.partials[row_id * a.slices];
    for (int s = tid; s < a.slices; s += NT) {         // leave the records zero-filled
      uint4 *w = reinterpret_cast<uint4 *>(&parts[s]);
      w[0] = make_uint4(0u, 0u, 0u, 0u);
      w[1] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  finish_row(a, b, smem, NT, batch_cnt);
}

// ---------------------------------------------------------------- launch plan

struct Plan {
  int nt;
  int slices;
  int64_t slice_len;
  bool vec;        // 16-byte loads throughout (aligned rows)
  bool split;      // not aligned: a 16-byte-load body with an element head and tail (greedy)
};

// Launch of the plan's kernel, after checking that its LDS (static + smem
// dynamic bytes) fits the device; returns a DLLM status.
template <typename T, int NT, int UV, bool FULL>
int launch_f(const Plan &p, const StatsArgs &a, int64_t rows, bool sample, size_t smem,
             hipStream_t s, const char *who) {
  dim3 grid((unsigned)(rows * p.slices)), block(NT);
  void (*kern)(StatsArgs) =
      sample ? (p.vec ? token_stats_kernel<T, NT, UV, true, true, FULL, false>
                      : p.split ? token_stats_kernel<T, NT, UV, true, true, FULL, true>
                                : token_stats_kernel<T, NT, UV, true, false, FULL, false>)
             : (p.vec ? token_stats_kernel<T, NT, UV, false, true, FULL, false>
                      : p.split ? token_stats_kernel<T, NT, UV, false, true, FULL, true>
                                : token_stats_kernel<T, NT, UV, false, false, FULL, false>);
  const int lds = check_lds((const void *)kern, smem, who);
  if (lds != DLLM_OK) return lds;
  kern<<<grid, block, smem, s>>>(a);
  return check_launch(who);
}

// The FULL = true kernels, instantiated in token_stats_full.hip.
int launch_full(int dtype, const Plan &p, const StatsArgs &a, int64_t rows, bool sample,
                size_t smem, hipStream_t s, const char *who);

}  // namespace dllm
