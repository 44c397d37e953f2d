// Engine clock probe: shader-clock cycles (s_memtime) over a window of the
// 100 MHz real-time counter (s_memrealtime), one working lane per workgroup,
// sleeping between reads. Measurement tooling beside the attention library;
// interface and semantics in include/miclock.h.
#include <hip/hip_runtime.h>

#include "miclock.h"

namespace {

__global__ void __launch_bounds__(64) clock_probe_kernel(uint64_t* __restrict__ out,
                                                         uint64_t warm, uint64_t window) {
  if (threadIdx.x != 0) return;
  const uint64_t entry = __builtin_amdgcn_s_memrealtime();
  while (__builtin_amdgcn_s_memrealtime() - entry < warm) __builtin_amdgcn_s_sleep(4);
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  uint64_t r1 = r0;
  while (r1 - r0 < window) {
    __builtin_amdgcn_s_sleep(4);
    r1 = __builtin_amdgcn_s_memrealtime();
  }
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  uint64_t* o = out + 4 * (int64_t)blockIdx.x;
  o[0] = c1 - c0;
  o[1] = r1 - r0;
  o[2] = r0;
  o[3] = entry;
}

}  // namespace

extern "C" int miclock_probe(uint64_t* out, int n_groups, uint64_t warm_ticks,
                             uint64_t window_ticks, void* stream) {
  if (out == nullptr) return 1;
  if (n_groups < 1 || n_groups > 1024 || warm_ticks > (1ull << 32) || window_ticks < 1 ||
      window_ticks > (1ull << 32))
    return 2;
  hipLaunchKernelGGL(clock_probe_kernel, dim3(n_groups), dim3(64), 0, (hipStream_t)stream, out,
                     warm_ticks, window_ticks);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}
