// Synthetic weight generation: a counter-based SplitMix64 stream per tensor.
//
// SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
// generators", OOPSLA 2014): state += 0x9E3779B97F4A7C15, then the variant-13
// mixer. splitmix64(x) below is the first output for state x. Element e of
// tensor t takes r = splitmix64(key_t + e) with key_t computed on the host.
#include "common.hpp"
#include "kernels.hpp"

namespace ll {

__device__ __forceinline__ uint64_t splitmix64_dev(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__global__ void weights_init_kernel(void* dst, uint64_t numel, uint64_t key, int kind, float scale) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t e = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; e < numel; e += stride) {
    const uint64_t r = splitmix64_dev(key + e);
    const int32_t u24 = (int32_t)(r >> 40);
    // 2u - 1 with u = u24 * 2^-24: an integer in [-2^24, 2^24) times 2^-24, exact.
    const float centred = (float)(2 * u24 - (1 << 24)) * 0x1p-24f;
    if (kind == 2) {
      ((float*)dst)[e] = __fadd_rn(1.0f, __fmul_rn(0.25f, centred));
    } else {
      const float w = __fmul_rn(centred, scale);
      if (kind == 0)
        ((uint16_t*)dst)[e] = (uint16_t)f32_to_bf16(w);
      else
        ((float*)dst)[e] = w;
    }
  }
}

hipError_t launch_weights_init(void* dst, uint64_t numel, uint64_t key, int kind, float scale,
                               hipStream_t stream) {
  if (numel == 0) return hipSuccess;
  uint64_t blocks = (numel + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(weights_init_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, dst, numel,
                     key, kind, scale);
  return hipGetLastError();
}

}  // namespace ll
