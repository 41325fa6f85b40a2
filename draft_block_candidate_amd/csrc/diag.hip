// Shader-clock probe: one wave reads the 100 MHz constant counter
// (s_memrealtime) and the shader clock counter (s_memtime) at the start and
// the end of a window of the constant counter, sleeping in between. Launched
// on a second stream beside a running kernel, it measures the shader clock
// that kernel runs at (the MI355X lowers it under sustained MFMA load).
// Diagnostic only: no step of the reranking path uses it.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

namespace ll {
namespace {

__global__ __launch_bounds__(64) void clock_probe_kernel(uint64_t* __restrict__ out, uint64_t window) {
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  uint64_t r = r0;
  // the constant counter only moves forward, so the loop ends after `window`
  // ticks (the host bounds it to one second)
  while (r - r0 < window) {
    __builtin_amdgcn_s_sleep(8);
    r = __builtin_amdgcn_s_memrealtime();
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) {
    out[0] = r - r0;
    out[1] = t1 - t0;
  }
}

}  // namespace

hipError_t launch_clock_probe(uint64_t* out, uint64_t window_ticks, hipStream_t stream) {
  hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0, stream, out, window_ticks);
  return hipGetLastError();
}

}  // namespace ll
