// Shared host and device helpers of libdllm_commit (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dllm_commit.h"

namespace dllm {

// ---------------------------------------------------------------- host side

// Records a printf-style message for dllm_last_error() and returns `code`.
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the message; returns DLLM_OK.
int ok();
// DLLM_ERR_HIP with a message if the last launch failed, else DLLM_OK.
int check_launch(const char *what);
// Compute units of the current device (cached per device).
int device_cu_count();
// DLLM_ERR_UNSUPPORTED, with a message naming `who`, if a launch of `kernel`
// with `dynamic_lds` bytes of dynamic LDS would exceed the current device's
// LDS per workgroup (static size cached per kernel); a launch that asks for
// more makes the runtime abort the queue.  DLLM_ERR_HIP if the sizes cannot be
// queried; else DLLM_OK.
int check_lds(const void *kernel, size_t dynamic_lds, const char *who);

// Stage timestamps (an instrumented build only, -DDLLM_STAGE_TIMESTAMPS):
// thread 0 of each workgroup records the 100 MHz real-time counter when it
// reaches a stage of the step, in LDS (an LDS write adds no wait for memory
// to the step it measures), and copies the records to a device array of
// this translation unit when the kernel returns (the first kStageWorkgroups
// workgroups), which dllm_stage_timestamps copies out.  A kernel opts in with
// DLLM_STAGE_SCOPE() at its start.  In the product build these are empty.
constexpr int kStageWorkgroups = 4096;
constexpr int kStages = 16;
enum Stage {
  kStageStart = 0,         // first instruction
  kStageStreamEnd = 1,     // the slice streamed and its waves merged
  kStageSliceCounted = 2,  // split rows: the slice partial published and counted
  kStageRowMerged = 3,     // split rows, last slice: every slice merged
  kStagePublished = 4,     // the row's statistics written
  kStageBatchCounted = 5,  // the row counted into its batch row
  kStageBatchDone = 6,     // the completing workgroup: rules and counts done
  kStageSkipped = 7,       // canvas step: the row needed by no rule, not read
  kStageFinalized = 8,     // the row's statistics computed (before they are written)
  kStageStoresDrained = 9, // the row's stores complete, before its batch-row count
  kStageRuleLoaded = 10,   // the completing workgroup: the rule's inputs loaded
  kStageRuleRanked = 11,   // the completing workgroup: the candidates ranked
};
#ifdef DLLM_STAGE_TIMESTAMPS
static __device__ uint64_t stage_ts[kStageWorkgroups * kStages];
static __shared__ uint64_t stage_lds[kStages];
// The counter read waits for itself in the same asm block, and the memory
// clobber keeps the compiler from moving memory operations across a stage mark.
__device__ __forceinline__ uint64_t stage_clock() {
  uint64_t t;
  asm volatile("s_memrealtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(t) : : "memory");
  return t;
}
#define DLLM_STAGE(k)                                                                     \
  do {                                                                                    \
    if (threadIdx.x == 0) stage_lds[(k)] = stage_clock();                                 \
  } while (0)
struct StageFlush {
  __device__ StageFlush() {
    if (threadIdx.x == 0)
      for (int k = 0; k < kStages; ++k) stage_lds[k] = 0;
  }
  __device__ ~StageFlush() {
    // stages this workgroup did not pass keep their older records
    if (threadIdx.x == 0 && blockIdx.x < (unsigned)kStageWorkgroups)
      for (int k = 0; k < kStages; ++k)
        if (stage_lds[k]) stage_ts[blockIdx.x * kStages + k] = stage_lds[k];
  }
};
#define DLLM_STAGE_SCOPE() StageFlush stage_flush_
// Copies this translation unit's array to host memory (clear: zero it first
// instead); hipMemcpy*Symbol status.
hipError_t stage_ts_copy_full(uint64_t *dst, bool clear);
hipError_t stage_ts_copy_plain(uint64_t *dst, bool clear);
#define DLLM_STAGE_COPY_IMPL(name)                                                        \
  hipError_t name(uint64_t *dst, bool clear) {                                            \
    static uint64_t zeros[kStageWorkgroups * kStages];                                    \
    if (clear) return hipMemcpyToSymbol(HIP_SYMBOL(stage_ts), zeros, sizeof(zeros));      \
    return hipMemcpyFromSymbol(dst, HIP_SYMBOL(stage_ts), sizeof(zeros));                 \
  }
#else
#define DLLM_STAGE(k) do { } while (0)
#define DLLM_STAGE_SCOPE() do { } while (0)
#endif

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

// ---------------------------------------------------------------- wave64 reductions
// DPP patterns of the GFX9 family: quad_perm, row_half_mirror, row_mirror and the
// row broadcasts 15 / 31 combine all 64 lanes in six VALU steps; lane 63 ends up
// with the full result, which readlane makes wave-uniform.

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float old, float v) {
  return __int_as_float(dpp_i<CTRL, ROW_MASK>(__float_as_int(old), __float_as_int(v)));
}

constexpr int kQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;
constexpr int kRowBcast15 = 0x142;
constexpr int kRowBcast31 = 0x143;

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<kQuadSwap1>(v, v));
  v = fmaxf(v, dpp_f<kQuadSwap2>(v, v));
  v = fmaxf(v, dpp_f<kRowHalfMirror>(v, v));
  v = fmaxf(v, dpp_f<kRowMirror>(v, v));
  v = fmaxf(v, dpp_f<kRowBcast15, 0xA>(-__builtin_inff(), v));
  v = fmaxf(v, dpp_f<kRowBcast31, 0xC>(-__builtin_inff(), v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<kQuadSwap1>(v, v);
  v += dpp_f<kQuadSwap2>(v, v);
  v += dpp_f<kRowHalfMirror>(v, v);
  v += dpp_f<kRowMirror>(v, v);
  v += dpp_f<kRowBcast15, 0xA>(0.0f, v);
  v += dpp_f<kRowBcast31, 0xC>(0.0f, v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ int wave_sum_i(int v) {
  v += dpp_i<kQuadSwap1>(v, v);
  v += dpp_i<kQuadSwap2>(v, v);
  v += dpp_i<kRowHalfMirror>(v, v);
  v += dpp_i<kRowMirror>(v, v);
  v += dpp_i<kRowBcast15, 0xA>(0, v);
  v += dpp_i<kRowBcast31, 0xC>(0, v);
  return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ int wave_min_i(int v) {
  v = min(v, dpp_i<kQuadSwap1>(v, v));
  v = min(v, dpp_i<kQuadSwap2>(v, v));
  v = min(v, dpp_i<kRowHalfMirror>(v, v));
  v = min(v, dpp_i<kRowMirror>(v, v));
  v = min(v, dpp_i<kRowBcast15, 0xA>(0x7fffffff, v));
  v = min(v, dpp_i<kRowBcast31, 0xC>(0x7fffffff, v));
  return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  int x = (int)v;
  x = (int)min((uint32_t)x, (uint32_t)dpp_i<kQuadSwap1>(x, x));
  x = (int)min((uint32_t)x, (uint32_t)dpp_i<kQuadSwap2>(x, x));
  x = (int)min((uint32_t)x, (uint32_t)dpp_i<kRowHalfMirror>(x, x));
  x = (int)min((uint32_t)x, (uint32_t)dpp_i<kRowMirror>(x, x));
  x = (int)min((uint32_t)x, (uint32_t)dpp_i<kRowBcast15, 0xA>(-1, x));
  x = (int)min((uint32_t)x, (uint32_t)dpp_i<kRowBcast31, 0xC>(-1, x));
  return (uint32_t)__builtin_amdgcn_readlane(x, 63);
}

// Wave minimum of a 64-bit key: the high words first, then the low words of
// the lanes holding that high word.
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
  const uint32_t hi = wave_min_u32((uint32_t)(v >> 32));
  const uint32_t lo = wave_min_u32((uint32_t)(v >> 32) == hi ? (uint32_t)v : 0xffffffffu);
  return ((uint64_t)hi << 32) | lo;
}

// ---------------------------------------------------------------- float helpers

__device__ __host__ __forceinline__ bool bits_finite(uint32_t u) {
  return (u & 0x7f800000u) != 0x7f800000u;
}

// Order-preserving map of float32 bits to uint32 (ascending), after
// canonicalising -0 to +0.  NaN must have been replaced beforehand.
__device__ __forceinline__ uint32_t sortable_asc(uint32_t u) {
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint32_t unsortable_asc(uint32_t s) {
  return (s & 0x80000000u) ? (s & 0x7fffffffu) : ~s;
}

// A confidence ranks best-first: NaN counts as -inf.
__device__ __forceinline__ uint32_t conf_key(float c) {
  uint32_t u = __float_as_uint(c);
  if ((u & 0x7fffffffu) > 0x7f800000u) u = 0xff800000u;   // NaN -> -inf
  return ~sortable_asc(u);
}
__device__ __forceinline__ float conf_from_key(uint32_t k) {
  return __uint_as_float(unsortable_asc(~k));
}
// An entropy ranks lowest-first: NaN counts as +inf.
__device__ __forceinline__ uint32_t ent_key(float h) {
  uint32_t u = __float_as_uint(h);
  if ((u & 0x7fffffffu) > 0x7f800000u) u = 0x7f800000u;   // NaN -> +inf
  return sortable_asc(u);
}
__device__ __forceinline__ float ent_from_key(uint32_t k) {
  return __uint_as_float(unsortable_asc(k));
}
__device__ __forceinline__ float conf_sanitized(float c) {
  uint32_t u = __float_as_uint(c);
  return ((u & 0x7fffffffu) > 0x7f800000u) ? -__builtin_inff() : c;
}

// ---------------------------------------------------------------- Philox4x32-10
// J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel Random Numbers:
// As Easy as 1, 2, 3" (SC'11): ten rounds of two 32x32->64 products on the even
// counter words, xor-mixed with the odd words and the key, the key bumped by
// the Weyl constants after every round.
struct Philox4 { uint32_t w[4]; };

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    // each 32 x 32 -> 64-bit product in one instruction (both halves at once),
    // each three-way xor in one v_bitop3_b32 (truth table 0x96: odd parity)
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    c0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
    c1 = (uint32_t)p1;
    c2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    c3 = (uint32_t)p0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  Philox4 o;
  o.w[0] = c0; o.w[1] = c1; o.w[2] = c2; o.w[3] = c3;
  return o;
}

// Gumbel(0,1) draw from one Philox word, u = ((w >> 9) + 0.5) * 2^-23 (exact in
// float32), in base-2 units: returns -log2(-log2 u), which is log2(e) g + log2(ln 2)
// for the Gumbel draw g = -ln(-ln u).  With the logit scaled by log2(e) / T, the
// score x log2(e) / T - log2(-log2 u) is log2(e) (x / T + g) plus a constant: the
// same argmax as the Gumbel-max score, with two multiplies fewer per element.
// u is built without a conversion: one funnel shift puts the 23 word bits under
// the exponent of 1.0 (the float 1 + m 2^-23, m = w >> 9), and subtracting
// 1 - 2^-24 leaves (2m + 1) 2^-24, a 24-bit significand, so the difference is exact.
__device__ __forceinline__ float gumbel2_from_word(uint32_t w) {
  const float u = __uint_as_float(__builtin_amdgcn_alignbit(0x7fu, w, 9)) - 0x1.fffffep-1f;
  return -__builtin_amdgcn_logf(-__builtin_amdgcn_logf(u));   // -log2(-log2 u)
}

// ---------------------------------------------------------------- exact sums
// A float32 value is m * 2^(E) with a 24-bit integer m and E >= -149, so every
// finite float32, and every sum of up to 2^12 of them, is an integer multiple
// of 2^-149 below 2^290 in magnitude: five 64-bit limbs (two's complement) hold
// such sums exactly, and they add associatively.
struct Fx { uint64_t w[5]; };

__device__ __host__ __forceinline__ void fx_zero(Fx &a) {
  for (int i = 0; i < 5; ++i) a.w[i] = 0;
}
__device__ __host__ __forceinline__ void fx_add(Fx &a, const Fx &b) {
  uint64_t carry = 0;
  for (int i = 0; i < 5; ++i) {
    const uint64_t s = a.w[i] + b.w[i];
    const uint64_t c1 = s < a.w[i];
    const uint64_t t = s + carry;
    const uint64_t c2 = t < s;
    a.w[i] = t;
    carry = c1 | c2;
  }
}
__device__ __host__ __forceinline__ void fx_negate(Fx &a) {
  uint64_t carry = 1;
  for (int i = 0; i < 5; ++i) {
    const uint64_t t = ~a.w[i] + carry;
    carry = (carry && t == 0) ? 1 : 0;
    a.w[i] = t;
  }
}
// Signed a <= b.
__device__ __host__ __forceinline__ bool fx_le(const Fx &a, const Fx &b) {
  const int64_t ta = (int64_t)a.w[4], tb = (int64_t)b.w[4];
  if (ta != tb) return ta < tb;
  for (int i = 3; i >= 0; --i)
    if (a.w[i] != b.w[i]) return a.w[i] < b.w[i];
  return true;
}
// Exact fixed-point value of a finite float32 (units of 2^-149).
__device__ __host__ __forceinline__ Fx fx_from_f32_bits(uint32_t u) {
  Fx r;
  fx_zero(r);
  const uint32_t e = (u >> 23) & 0xffu, frac = u & 0x7fffffu;
  const uint64_t m = e ? (uint64_t)(frac | 0x800000u) : (uint64_t)frac;
  if (m == 0) return r;
  const int sh = (e ? (int)e : 1) - 1;              // 0 .. 253: value = m * 2^sh units
  // limb i holds bits [64 i, 64 i + 64): m shifted by sh - 64 i (constant i, so
  // every limb stays in a register)
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int s = sh - 64 * i;
    r.w[i] = (s >= 0 && s < 64) ? (m << s) : (s < 0 && s > -24) ? (m >> -s) : 0ull;
  }
  if (u & 0x80000000u) fx_negate(r);
  return r;
}

}  // namespace dllm
