// The canvas-step / margin variant of the statistics kernels (FULL = true:
// candidate-row skipping and runner-up tracking), instantiated apart so it
// compiles in parallel with token_stats.hip.
#include "token_stats_dev.h"

namespace dllm {

namespace {

template <typename T>
int launch_full_t(const Plan &p, const StatsArgs &a, int64_t rows, bool sample, size_t smem,
                  hipStream_t s, const char *who) {
  constexpr int U0 = ElemT<T>::U;
  if (p.nt == 512) return launch_f<T, 512, U0, true>(p, a, rows, sample, smem, s, who);
  return launch_f<T, 256, U0, true>(p, a, rows, sample, smem, s, who);
}

}  // namespace

#ifdef DLLM_STAGE_TIMESTAMPS
DLLM_STAGE_COPY_IMPL(stage_ts_copy_full)
#endif

int launch_full(int dtype, const Plan &p, const StatsArgs &a, int64_t rows, bool sample,
                size_t smem, hipStream_t s, const char *who) {
  if (dtype == DLLM_BF16) return launch_full_t<uint16_t>(p, a, rows, sample, smem, s, who);
  return launch_full_t<float>(p, a, rows, sample, smem, s, who);
}

}  // namespace dllm
