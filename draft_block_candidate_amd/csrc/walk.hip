// Pair scores and the greedy commit.
//
// Pair scores (LiLiCorr paper, Eq. (1) and Section 3.5): for every adjacent
// slot pair, cos_s = out_{s-1} . in_s^T over unit vectors, one K x K product
// per pair. One wave per pair, 16 x 16 MFMA tiles over d_e.
//
// Greedy commit (Eq. (8); ties to the lower index as in the SGLang PR,
// "Why the custom kernels"): one wave per block, lane j scores candidate j.
// Only the walk is sequential, over slots.
#include "common.hpp"
#include "kernels.hpp"

namespace ll {
namespace {

__global__ __launch_bounds__(256) void pair_scores_kernel(const uint16_t* __restrict__ outv,
                                                          const uint16_t* __restrict__ inv, int N,
                                                          int B, int K, int de,
                                                          float* __restrict__ cos) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, c = lane & 15;
  const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= (int64_t)N * (B - 1)) return;
  const int64_t n = pair / (B - 1);
  const int s = (int)(pair - n * (B - 1)) + 1;
  const uint16_t* o = outv + ((n * B + s - 1) * K) * (int64_t)de;
  const uint16_t* in = inv + ((n * B + s) * K) * (int64_t)de;
  float* dst = cos + pair * K * K;
  const int tiles = (K + 15) / 16;
  for (int at = 0; at < tiles; ++at)
    for (int bt = 0; bt < tiles; ++bt) {
      const int a = at * 16 + c, b = bt * 16 + c;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      for (int k0 = 0; k0 < de; k0 += 32) {
        const u32x4_t af = a < K ? *(const u32x4_t*)(o + (int64_t)a * de + k0 + 8 * g)
                                 : u32x4_t{0, 0, 0, 0};
        const u32x4_t bf = b < K ? *(const u32x4_t*)(in + (int64_t)b * de + k0 + 8 * g)
                                 : u32x4_t{0, 0, 0, 0};
        acc = mfma16(af, bf, acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ra = at * 16 + 4 * g + i;
        if (ra < K && b < K) dst[ra * K + b] = acc[i];
      }
    }
}

__global__ __launch_bounds__(256) void greedy_walk_kernel(
    const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_logp,
    const float* __restrict__ cos, int N, int B, int K, float alpha, int use_logp,
    int32_t* __restrict__ out_tokens, float* __restrict__ score, float* __restrict__ gap) {
  const int lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const int64_t r0 = n * B;
  if (lane == 0) {
    out_tokens[r0] = topk_idx[r0 * K];
    if (score) score[r0] = topk_logp[r0 * K];
    if (gap) gap[r0] = 0.f;
  }
  int cprev = 0;
  for (int s = 1; s < B; ++s) {
    float z = -INFINITY;
    if (lane < K) {
      const float cs = cos[((n * (B - 1) + s - 1) * K + cprev) * K + lane];
      const float term = __fmul_rn(alpha, cs);
      z = use_logp ? __fadd_rn(topk_logp[(r0 + s) * K + lane], term) : term;
    }
    float bz = z;
    int bl = lane;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float oz = __shfl_xor(bz, off, 64);
      const int ol = __shfl_xor(bl, off, 64);
      if (oz > bz || (oz == bz && ol < bl)) {
        bz = oz;
        bl = ol;
      }
    }
    if (bl >= K) bl = 0;  // only reachable with non-finite scores; keeps every index in range
    const float second = wave_max(lane == bl ? -INFINITY : z);
    cprev = bl;
    if (lane == 0) {
      out_tokens[r0 + s] = topk_idx[(r0 + s) * K + bl];
      if (score) score[r0 + s] = bz;
      if (gap) gap[r0 + s] = K > 1 ? __fsub_rn(bz, second) : 0.f;
    }
  }
}

}  // namespace

hipError_t launch_pair_scores(const uint16_t* outv, const uint16_t* inv, int N, int B, int K,
                              int d_e, float* cos, hipStream_t stream) {
  const int64_t pairs = (int64_t)N * (B - 1);
  if (pairs <= 0) return hipSuccess;
  hipLaunchKernelGGL(pair_scores_kernel, dim3((unsigned)((pairs + 3) / 4)), dim3(256), 0, stream,
                     outv, inv, N, B, K, d_e, cos);
  return hipGetLastError();
}

hipError_t launch_greedy_walk(const int32_t* topk_idx, const float* topk_logp, const float* cos,
                              int N, int B, int K, float alpha, int use_logp, int32_t* out_tokens,
                              float* score, float* gap, hipStream_t stream) {
  hipLaunchKernelGGL(greedy_walk_kernel, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, stream,
                     topk_idx, topk_logp, cos, N, B, K, alpha, use_logp, out_tokens, score, gap);
  return hipGetLastError();
}

}  // namespace ll
