// Uniform-noise decoding helpers: linear_temperature, uniform_canvas, renoise
// and the stable-and-confident stop (mlx-arsenal "dLLM block decoding",
// function table; the loop of "Uniform-noise decoding (DiffusionGemma)";
// mlxcel "Block Diffusion", "DiffusionGemma Canvas Denoising").  The
// statistics, the categorical sample and the entropy-bound acceptance of that
// loop are one dllm_token_stats launch (statistics temperature, argmax output,
// fused entropy_bound rule); these kernels are the rest of a step.  All are
// elementwise or one workgroup per batch row, far below the logit pass.
#include <math.h>
#include <string.h>

#include "common.h"

namespace dllm {

namespace {

constexpr uint32_t kCanvasStream = 0xFFFFFFFFu;

// Token v = floor(x V / 2^64) of the 64-bit word x = w0 + 2^32 w1 of
// Philox4x32-10 at counter (l, b, 0xFFFFFFFF, draw): uniform on [0, V) up to
// V / 2^64.  The counter word 2 is never a batch index of the sampling noise
// (counter (v/4, l, b, step)), so the streams do not meet.
__global__ void uniform_canvas_kernel(int32_t *out, int64_t B, int64_t L, uint32_t V,
                                      uint32_t k0, uint32_t k1, uint32_t draw) {
  const int64_t n = B * L;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t b = (uint32_t)(i / L), l = (uint32_t)(i - (int64_t)b * L);
    const Philox4 w = philox4x32_10(l, b, kCanvasStream, draw, k0, k1);
    const uint64_t x = (uint64_t)w.w[0] | ((uint64_t)w.w[1] << 32);
    out[i] = (int32_t)__umul64hi(x, (uint64_t)V);
  }
}

__global__ void renoise_kernel(const int32_t *sample, const uint8_t *accepted,
                               const int32_t *noise, int64_t n, int32_t *out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    out[i] = accepted[i] ? sample[i] : noise[i];
}

struct StopArgs {
  const int32_t *argmax;
  const float *entropy;
  int64_t L;
  int k;                 // stability threshold
  int first;             // no previous canvas yet
  int conf_class;        // a finite sum: 0 compare with thr, 1 always confident, 2 never
  int c_pinf;            // c = +inf (and L > 0): a +inf sum is confident too
  Fx thr;                // floor(c L 2^149)
  int32_t *prev;
  int32_t *count;
  uint8_t *done;
};

// One workgroup per batch row: is the argmax canvas the previous one, and is
// the sum of the entropies at most c L in the extended reals?  Finite terms
// are summed exactly (fixed point, units of 2^-149); a NaN term, or +inf and
// -inf together, leaves the sum undefined (not confident); +inf terms make it
// +inf (confident only for c = +inf), -inf terms -inf (confident).
template <int NT>
__global__ __launch_bounds__(NT) void stop_kernel(StopArgs a) {
  __shared__ Fx s_sum[NT];
  __shared__ int s_diff, s_nan, s_pinf, s_ninf;
  const int tid = threadIdx.x;
  const int64_t base = (int64_t)blockIdx.x * a.L;
  if (tid == 0) { s_diff = 0; s_nan = 0; s_pinf = 0; s_ninf = 0; }
  __syncthreads();
  Fx acc;
  fx_zero(acc);
  int diff = 0, nan = 0, pinf = 0, ninf = 0;
  for (int64_t l = tid; l < a.L; l += NT) {
    const int32_t am = a.argmax[base + l];
    if (!a.first && a.prev[base + l] != am) diff = 1;
    a.prev[base + l] = am;
    const uint32_t u = __float_as_uint(a.entropy[base + l]);
    if (bits_finite(u)) fx_add(acc, fx_from_f32_bits(u));
    else if (u & 0x007fffffu) nan = 1;
    else if (u >> 31) ninf = 1;
    else pinf = 1;
  }
  if (diff) s_diff = 1;
  if (nan) s_nan = 1;
  if (pinf) s_pinf = 1;
  if (ninf) s_ninf = 1;
  s_sum[tid] = acc;
  __syncthreads();
  if (tid == 0) {
    Fx tot = s_sum[0];
    for (int t = 1; t < NT; ++t) fx_add(tot, s_sum[t]);
    const bool same = !a.first && !s_diff;
    const int cnt = same ? a.count[blockIdx.x] + 1 : 0;
    a.count[blockIdx.x] = cnt;
    bool confident;
    if (s_nan || (s_pinf && s_ninf)) confident = false;
    else if (s_pinf) confident = a.c_pinf != 0;
    else if (s_ninf) confident = true;
    else confident = a.conf_class == 1 || (a.conf_class == 0 && fx_le(tot, a.thr));
    if (cnt >= a.k && confident) a.done[blockIdx.x] = 1;
  }
}

// floor(c * L * 2^149) as a signed 320-bit number, for |c| L < 2^170 (the
// product is mant L 2^(e-53) with mant < 2^53, L < 2^32: placed limb by limb,
// it stays below the sign bit, 2^319).
Fx fixed_floor_of_product(double c, uint32_t L) {
  Fx r;
  fx_zero(r);
  if (c == 0.0 || L == 0) return r;
  int e = 0;
  const double fr = frexp(fabs(c), &e);                   // |c| = fr 2^e, fr in [0.5, 1)
  const uint64_t mant = (uint64_t)ldexp(fr, 53);          // |c| = mant 2^(e - 53)
  const unsigned __int128 P = (unsigned __int128)mant * L; // < 2^85
  const int sh = e - 53 + 149;                            // |c| L 2^149 = P 2^sh
  const bool neg = c < 0.0;
  unsigned __int128 q;
  bool rem;
  if (sh >= 0) {
    // P 2^sh < 2^290: place it limb by limb
    for (int i = 0; i < 5; ++i) {
      const int s = sh - 64 * i;                          // bit of P at limb i's bit 0
      unsigned __int128 v;
      if (s >= 0) v = s >= 128 ? 0 : (P << s);
      else v = -s >= 128 ? 0 : (P >> -s);
      r.w[i] = (uint64_t)v;
    }
    if (neg) fx_negate(r);
    return r;
  }
  const int s = -sh;
  q = s >= 128 ? 0 : (P >> s);
  rem = s >= 128 ? (P != 0) : ((P & ((((unsigned __int128)1) << s) - 1)) != 0);
  if (neg && rem) q += 1;                                 // floor(-x) = -ceil(x)
  r.w[0] = (uint64_t)q;
  r.w[1] = (uint64_t)(q >> 64);
  if (neg) fx_negate(r);
  return r;
}

unsigned grid_for_n(int64_t n, int block) {
  int64_t g = (n + block - 1) / block;
  if (g > 65535 * 16) g = 65535 * 16;
  return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace
}  // namespace dllm

using namespace dllm;

extern "C" int dllm_linear_temperature(int remaining, int num_steps, double t_min, double t_max,
                                       double *out) {
  if (!out) return fail(DLLM_ERR_ARG, "dllm_linear_temperature: out is NULL");
  if (num_steps < 1 || remaining < 0 || remaining > num_steps)
    return fail(DLLM_ERR_ARG, "dllm_linear_temperature: need 0 <= remaining <= num_steps, "
                              "num_steps >= 1");
  if (!(t_min == t_min) || !(t_max == t_max))
    return fail(DLLM_ERR_ARG, "dllm_linear_temperature: t_min and t_max must not be NaN");
  *out = t_min + (t_max - t_min) * (double)remaining / (double)num_steps;
  return ok();
}

extern "C" int dllm_uniform_canvas(int32_t *out, int64_t B, int64_t L, int64_t V, uint64_t seed,
                                   uint64_t draw, hipStream_t stream) {
  const char *who = "dllm_uniform_canvas";
  if (B < 0 || L < 0) return fail(DLLM_ERR_ARG, "%s: B and L must be >= 0", who);
  if (V < 1 || V > 0x7fffffffLL) return fail(DLLM_ERR_ARG, "%s: V must be in [1, 2^31)", who);
  if (draw > 0xffffffffull) return fail(DLLM_ERR_ARG, "%s: draw must be < 2^32", who);
  if (B > 0xffffffffLL || L > 0xffffffffLL) return fail(DLLM_ERR_UNSUPPORTED, "%s: B or L too large", who);
  if (B == 0 || L == 0) return ok();
  if (!out) return fail(DLLM_ERR_ARG, "%s: out is NULL", who);
  uniform_canvas_kernel<<<grid_for_n(B * L, 256), 256, 0, stream>>>(
      out, B, L, (uint32_t)V, (uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32),
      (uint32_t)draw);
  return check_launch(who);
}

extern "C" int dllm_renoise(const int32_t *sample, const uint8_t *accepted, const int32_t *noise,
                            int64_t B, int64_t L, int32_t *out, hipStream_t stream) {
  const char *who = "dllm_renoise";
  if (B < 0 || L < 0) return fail(DLLM_ERR_ARG, "%s: B and L must be >= 0", who);
  if (B == 0 || L == 0) return ok();
  if (!sample || !accepted || !noise || !out)
    return fail(DLLM_ERR_ARG, "%s: sample, accepted, noise and out must be non-NULL", who);
  if ((const void *)out == (const void *)accepted)
    return fail(DLLM_ERR_ARG, "%s: out aliases accepted", who);
  renoise_kernel<<<grid_for_n(B * L, 256), 256, 0, stream>>>(sample, accepted, noise, B * L, out);
  return check_launch(who);
}

extern "C" int dllm_stable_confident_stop(const int32_t *argmax, const float *entropy, int64_t B,
                                          int64_t L, int stability_threshold,
                                          double confidence_threshold, int first,
                                          int32_t *prev_argmax, int32_t *stable_steps,
                                          uint8_t *done, hipStream_t stream) {
  const char *who = "dllm_stable_confident_stop";
  if (B < 0 || L < 0) return fail(DLLM_ERR_ARG, "%s: B and L must be >= 0", who);
  if (B > (int64_t)(0xffffffffu / 256u) || L > 0xffffffffLL)
    return fail(DLLM_ERR_UNSUPPORTED, "%s: B or L too large", who);
  if (stability_threshold < 0) return fail(DLLM_ERR_ARG, "%s: stability_threshold < 0", who);
  if (confidence_threshold != confidence_threshold)
    return fail(DLLM_ERR_ARG, "%s: confidence_threshold is NaN", who);
  if (B == 0) return ok();
  if (!argmax || !entropy || !prev_argmax || !stable_steps || !done)
    return fail(DLLM_ERR_ARG, "%s: every array must be non-NULL", who);
  if ((const void *)prev_argmax == (const void *)argmax)
    return fail(DLLM_ERR_ARG, "%s: prev_argmax aliases argmax", who);
  StopArgs a;
  memset(&a, 0, sizeof a);
  a.argmax = argmax;
  a.entropy = entropy;
  a.L = L;
  a.k = stability_threshold;
  a.first = first ? 1 : 0;
  a.prev = prev_argmax;
  a.count = stable_steps;
  a.done = done;
  // exact c L in fixed point; from |c L| >= 2^160 on, the comparison with a
  // finite sum is decided by the sign of c (L finite float32 values, each
  // below 2^128, sum to less than 2^160 in magnitude)
  const double mag = fabs(confidence_threshold) * (double)(L > 0 ? L : 1);
  if (confidence_threshold == 0.0 || L == 0) a.conf_class = 0;
  else if (mag >= 0x1p160 || confidence_threshold == INFINITY || confidence_threshold == -INFINITY)
    a.conf_class = confidence_threshold > 0 ? 1 : 2;
  a.c_pinf = (L > 0 && confidence_threshold == INFINITY) ? 1 : 0;
  if (a.conf_class == 0) a.thr = fixed_floor_of_product(confidence_threshold, (uint32_t)L);
  stop_kernel<256><<<dim3((unsigned)B), dim3(256), 0, stream>>>(a);
  return check_launch(who);
}
