// Read-bandwidth probe: a plain streaming read of a device buffer with the
// logit pass's 16-byte non-temporal loads and no arithmetic but one xor per
// word.  It gives the read ceiling that the logit pass is measured against,
// over the same buffers and, if asked, with the same decomposition (one
// contiguous chunk per workgroup).  It is a measurement helper, not a step of
// the commit.
#include "common.h"

namespace dllm {

namespace {

__device__ __forceinline__ uint4 probe_load(const uint4 *p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t fold(const uint4 &v) { return v.x ^ v.y ^ v.z ^ v.w; }

// Workgroup g reads the 16-byte words [g chunk, min((g + 1) chunk, n)): four
// loads per lane per iteration, two register sets in turn so that the next
// iteration's loads are in flight while the current one is folded.  A lane
// whose fold hits an arbitrary constant sets a flag, so the loads are live.
template <int NT>
__global__ __launch_bounds__(NT) void read_probe_kernel(const uint4 *p, int64_t n, int64_t chunk,
                                                        uint32_t *sink) {
  const int64_t lo = (int64_t)blockIdx.x * chunk;
  if (lo >= n) return;
  const int64_t len = min(chunk, n - lo);
  const uint4 *q = p + lo + threadIdx.x;
  constexpr int64_t IT = 4 * NT;
  const int64_t nit = len / IT;
  uint32_t acc = 0;
  uint4 ba[4], bb[4];
  auto ld = [&](uint4 (&r)[4], int64_t it) {
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = probe_load(q + it * IT + k * NT);
  };
  auto use = [&](const uint4 (&r)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) acc ^= fold(r[k]);
  };
  if (nit > 0) {
    ld(ba, 0);
    int64_t it = 0;
    for (; it + 2 < nit; it += 2) {
      ld(bb, it + 1);
      use(ba);
      ld(ba, it + 2);
      use(bb);
    }
    if (it + 1 < nit) {
      ld(bb, it + 1);
      use(ba);
      use(bb);
    } else {
      use(ba);
    }
  }
  for (int64_t j = nit * IT + threadIdx.x; j < len; j += NT) acc ^= fold(probe_load(p + lo + j));
  if (acc == 0x9E3779B9u) atomicOr(sink, 1u);
}

}  // namespace
}  // namespace dllm

using namespace dllm;

extern "C" int dllm_read_probe(const void *buf, int64_t bytes, int64_t workgroups, int threads,
                               uint32_t *sink, hipStream_t stream) {
  static const char *who = "dllm_read_probe";
  if (!buf || !sink) return fail(DLLM_ERR_ARG, "%s: buf or sink is NULL", who);
  if ((uintptr_t)buf % 16 != 0 || bytes <= 0 || bytes % 16 != 0)
    return fail(DLLM_ERR_ARG, "%s: buf must be 16-byte aligned and bytes a positive multiple of 16",
                who);
  if (workgroups < 1 || workgroups > 0x7fffffff)
    return fail(DLLM_ERR_ARG, "%s: workgroups = %lld is outside [1, 2^31)", who,
                (long long)workgroups);
  if (threads != 256 && threads != 512)
    return fail(DLLM_ERR_ARG, "%s: threads = %d (256 or 512)", who, threads);
  const int64_t n = bytes / 16;
  const int64_t chunk = (n + workgroups - 1) / workgroups;
  const uint4 *p = static_cast<const uint4 *>(buf);
  if (threads == 512)
    read_probe_kernel<512><<<dim3((unsigned)workgroups), dim3(512), 0, stream>>>(p, n, chunk, sink);
  else
    read_probe_kernel<256><<<dim3((unsigned)workgroups), dim3(256), 0, stream>>>(p, n, chunk, sink);
  return check_launch(who);
}
