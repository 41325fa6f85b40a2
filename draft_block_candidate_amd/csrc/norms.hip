// RMSNorm of the fp32 residual stream before each sub-layer (LiLiCorr paper,
// Appendix A: pre-norm blocks with RMSNorm) for rows whose producing linear
// ran as whole tiles; the unit normalisation of the in/out vectors is in the
// heads linear's row kernel (gemm.hip).
#include "common.hpp"
#include "kernels.hpp"

namespace ll {
namespace {

// One wave per row. out = bf16((x * rstd) * gamma), rstd = 1/sqrt(mean(x^2) + eps).
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ x, int M, int H,
                                                      const float* __restrict__ gamma, float eps,
                                                      uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const float4* xr = (const float4*)(x + row * H);
  float ss = 0.f;
  for (int c4 = lane; c4 < H / 4; c4 += 64) {
    const float4 v = xr[c4];
    ss = fmaf(v.x, v.x, ss);
    ss = fmaf(v.y, v.y, ss);
    ss = fmaf(v.z, v.z, ss);
    ss = fmaf(v.w, v.w, ss);
  }
  ss = wave_sum(ss);
  const float rstd = 1.0f / __fsqrt_rn(ss / (float)H + eps);
  const float4* g4 = (const float4*)gamma;
  uint2* o2 = (uint2*)(out + row * H);
  for (int c4 = lane; c4 < H / 4; c4 += 64) {
    const float4 v = xr[c4], gv = g4[c4];
    o2[c4] = make_uint2(pack_bf16x2(v.x * rstd * gv.x, v.y * rstd * gv.y),
                        pack_bf16x2(v.z * rstd * gv.z, v.w * rstd * gv.w));
  }
}

// Same, with the row held in registers (one read of x) for H <= 64 * 4 * NV.
template <int NV>
__global__ __launch_bounds__(256) void rmsnorm_reg_kernel(const float* __restrict__ x, int M, int H,
                                                          const float* __restrict__ gamma, float eps,
                                                          uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const float4* xr = (const float4*)(x + row * H);
  const int n4 = H / 4;
  float4 v[NV];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c4 = lane + 64 * i;
    v[i] = c4 < n4 ? xr[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
    ss = fmaf(v[i].x, v[i].x, ss);
    ss = fmaf(v[i].y, v[i].y, ss);
    ss = fmaf(v[i].z, v[i].z, ss);
    ss = fmaf(v[i].w, v[i].w, ss);
  }
  ss = wave_sum(ss);
  const float rstd = 1.0f / __fsqrt_rn(ss / (float)H + eps);
  const float4* g4 = (const float4*)gamma;
  uint2* o2 = (uint2*)(out + row * H);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c4 = lane + 64 * i;
    if (c4 < n4) {
      const float4 gv = g4[c4];
      o2[c4] = make_uint2(pack_bf16x2(v[i].x * rstd * gv.x, v[i].y * rstd * gv.y),
                          pack_bf16x2(v[i].z * rstd * gv.z, v[i].w * rstd * gv.w));
    }
  }
}

}  // namespace

hipError_t launch_rmsnorm(const float* x, int M, int H, const float* gamma, float eps,
                          uint16_t* out, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  const dim3 grid((unsigned)((M + 3) / 4));
  if (H <= 1024)
    hipLaunchKernelGGL(rmsnorm_reg_kernel<4>, grid, dim3(256), 0, stream, x, M, H, gamma, eps, out);
  else if (H <= 2048)
    hipLaunchKernelGGL(rmsnorm_reg_kernel<8>, grid, dim3(256), 0, stream, x, M, H, gamma, eps, out);
  else
    hipLaunchKernelGGL(rmsnorm_kernel, grid, dim3(256), 0, stream, x, M, H, gamma, eps, out);
  return hipGetLastError();
}

}  // namespace ll
