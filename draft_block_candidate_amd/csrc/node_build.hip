// Node construction for every candidate (LiLiCorr paper, Section 3.2 and
// Appendix A "Architecture"): the token's embedding row, the slot and rank
// table rows, and a two-layer network over five confidence scalars (log-prob,
// prob, gap to the slot's top log-prob, rank scaled to [0, 1], top-choice
// flag). This kernel computes the first (5 -> H) layer with SiLU and the table
// sum; the second layer is an MFMA GEMM whose epilogue adds the table sum.
#include "common.hpp"
#include "kernels.hpp"

namespace ll {
namespace {

// One block per token; each thread owns 4 consecutive columns.
__global__ __launch_bounds__(256) void node_build_kernel(
    const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_logp, int B, int K, int H, int V,
    const uint16_t* __restrict__ E, const uint16_t* __restrict__ S, const uint16_t* __restrict__ R,
    const uint16_t* __restrict__ w1, const float* __restrict__ b1, uint16_t* __restrict__ hid,
    float* __restrict__ xbase) {
  const int64_t t = blockIdx.x;
  const int64_t row = t / K;       // (block, slot)
  const int j = (int)(t - row * K);
  const int s = (int)(row % B);
  int64_t tok = topk_idx[t];
  if (tok < 0 || tok >= V) tok = 0;  // ids come from the top-K stage; never read outside E
  const float lp = topk_logp[t];
  const float lp0 = topk_logp[row * K];
  float f[5];
  f[0] = lp;
  f[1] = expf(lp);
  f[2] = __fsub_rn(lp, lp0);
  f[3] = K > 1 ? __fdiv_rn((float)j, (float)(K - 1)) : 0.f;
  f[4] = j == 0 ? 1.f : 0.f;
  const uint2* e4 = (const uint2*)(E + tok * H);
  const uint2* s4 = (const uint2*)(S + (int64_t)s * H);
  const uint2* r4 = (const uint2*)(R + (int64_t)j * H);
  for (int c4 = threadIdx.x; c4 < H / 4; c4 += blockDim.x) {
    const uint2 ev = e4[c4], sv = s4[c4], rv = r4[c4];
    float xb[4], hz[4];
    const uint32_t ew[2] = {ev.x, ev.y}, sw[2] = {sv.x, sv.y}, rw[2] = {rv.x, rv.y};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t sh = (q & 1) ? 16 : 0;
      const float a = bf16_to_f32((ew[q >> 1] >> sh) & 0xFFFF);
      const float b = bf16_to_f32((sw[q >> 1] >> sh) & 0xFFFF);
      const float c = bf16_to_f32((rw[q >> 1] >> sh) & 0xFFFF);
      xb[q] = __fadd_rn(__fadd_rn(a, b), c);
      const int col = c4 * 4 + q;
      const uint16_t* wr = w1 + (int64_t)col * 5;
      float z = 0.f;
#pragma unroll
      for (int i = 0; i < 5; ++i) z = fmaf(bf16_to_f32(wr[i]), f[i], z);
      hz[q] = silu(z + b1[col]);
    }
    ((float4*)(xbase + t * H))[c4] = make_float4(xb[0], xb[1], xb[2], xb[3]);
    ((uint2*)(hid + t * H))[c4] = make_uint2(pack_bf16x2(hz[0], hz[1]), pack_bf16x2(hz[2], hz[3]));
  }
}

}  // namespace

hipError_t launch_node_build(const int32_t* topk_idx, const float* topk_logp, int N, int B, int K,
                             int H, const uint16_t* E, const uint16_t* S, const uint16_t* R,
                             const uint16_t* conf_w1, const float* conf_b1, uint16_t* hid,
                             float* xbase, int V, hipStream_t stream) {
  const int64_t M = (int64_t)N * B * K;
  hipLaunchKernelGGL(node_build_kernel, dim3((unsigned)M), dim3(256), 0, stream, topk_idx,
                     topk_logp, B, K, H, V, E, S, R, conf_w1, conf_b1, hid, xbase);
  return hipGetLastError();
}

}  // namespace ll
