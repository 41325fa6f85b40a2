// Kernels of the paper's own head (LiLiCorr paper, Section 3.2 and Appendix A
// "Architecture") that the lattice head does not have; its products run on
// the MFMA linears of gemm.hip.
//   * the target's input-embedding rows of every drafted candidate, gathered
//     as the A operand of the embedding projection;
//   * RMSNorm of the bf16 target state before its projection;
//   * the fusion layer's input: the concatenation [node, t', node * t'];
//   * the anchor's out vector (unit-normalised) in slot 0 of the [N, B, K, d_e]
//     layout the pair scores read: every candidate row of slot 0 carries it
//     (slots 1..B-1 hold the lattice's out/in vectors, which the heads linear
//     stores there itself).
#include "common.hpp"
#include "kernels.hpp"

namespace ll {
namespace {

// One workgroup per drafted candidate: copy E_t[token] (H_t bf16) to row m.
// Lattice row m = (n, s - 1, j) for slot s >= 1 of block n.
__global__ __launch_bounds__(256) void gather_rows_kernel(const int32_t* __restrict__ topk_idx, int B,
                                                          int K, const uint16_t* __restrict__ table,
                                                          int Ht, int V, uint16_t* __restrict__ out) {
  const int64_t m = blockIdx.x;
  const int64_t per_block = (int64_t)(B - 1) * K;
  const int64_t n = m / per_block;
  const int64_t rest = m - n * per_block;           // (s - 1) K + j
  int64_t tok = topk_idx[(n * B) * K + K + rest];   // slot s = 1 + rest / K
  if (tok < 0 || tok >= V) tok = 0;                 // ids come from the top-K stage
  const uint4* src = (const uint4*)(table + tok * Ht);
  uint4* dst = (uint4*)(out + m * Ht);
  for (int c = threadIdx.x; c < Ht / 8; c += blockDim.x) dst[c] = src[c];
}

// One workgroup per row of bf16 x (H <= 8192): out = bf16((x * rstd) *
// gamma), rstd = 1 / sqrt(mean(x^2) + eps), the arithmetic of the fp32
// RMSNorm kernels. Each thread loads its (at most four) 8-element chunks once,
// all before the first is used.
__global__ __launch_bounds__(256) void rmsnorm_bf16_kernel(const uint16_t* __restrict__ x, int H,
                                                           const float* __restrict__ gamma, float eps,
                                                           uint16_t* __restrict__ out) {
  constexpr int NC = 4;
  __shared__ float s_red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const int h8 = H / 8;
  const uint4* xr = (const uint4*)(x + row * H);
  uint4 v[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) v[i] = xr[min(tid + 256 * i, h8 - 1)];   // clamped: unconditional
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    if (tid + 256 * i >= h8) continue;
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float a = bf16_to_f32(w[q] & 0xFFFF), b = bf16_to_f32(w[q] >> 16);
      ss = fmaf(a, a, ss);
      ss = fmaf(b, b, ss);
    }
  }
  ss = wave_sum(ss);
  if (lane == 0) s_red[wave] = ss;
  __syncthreads();
  const float tot = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
  const float rstd = 1.0f / __fsqrt_rn(tot / (float)H + eps);
  uint4* o = (uint4*)(out + row * H);
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = tid + 256 * i;
    if (c >= h8) continue;
    const float4 g0 = ((const float4*)gamma)[2 * c], g1 = ((const float4*)gamma)[2 * c + 1];
    const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    uint32_t r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      r[q] = pack_bf16x2(bf16_to_f32(w[q] & 0xFFFF) * rstd * g[2 * q],
                         bf16_to_f32(w[q] >> 16) * rstd * g[2 * q + 1]);
    o[c] = make_uint4(r[0], r[1], r[2], r[3]);
  }
}

// out[m] = [u[m], tb[n], bf16(u[m] * tb[n])] for lattice row m of block n,
// 8 bf16 (16 bytes) per thread step. The product of two bf16 values is exact
// in fp32, so its only rounding is the bf16 one.
__global__ __launch_bounds__(256) void concat_kernel(const uint16_t* __restrict__ u,
                                                     const uint16_t* __restrict__ tb, int64_t per_block,
                                                     int H, uint16_t* __restrict__ out) {
  const int64_t m = blockIdx.x;
  const int64_t n = m / per_block;
  const uint4* ur = (const uint4*)(u + m * H);
  const uint4* tr = (const uint4*)(tb + n * H);
  uint4* o = (uint4*)(out + m * 3 * H);
  const int h8 = H / 8;
  for (int c = threadIdx.x; c < h8; c += blockDim.x) {
    const uint4 a = ur[c], b = tr[c];
    uint4 p;
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
    uint32_t pw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      pw[i] = pack_bf16x2(bf16_to_f32(aw[i] & 0xFFFF) * bf16_to_f32(bw[i] & 0xFFFF),
                          bf16_to_f32(aw[i] >> 16) * bf16_to_f32(bw[i] >> 16));
    p.x = pw[0];
    p.y = pw[1];
    p.z = pw[2];
    p.w = pw[3];
    o[c] = a;
    o[h8 + c] = b;
    o[2 * h8 + c] = p;
  }
}

// One workgroup per block n: the anchor vector o_0 = bf16(a / max(|a|, 1e-12)),
// a = apre[n] (d_e <= 1024, so each thread keeps at most four elements),
// written to all K candidate rows of slot 0 in outv; the in rows of slot 0
// are zero.
__global__ __launch_bounds__(256) void anchor_rows_kernel(const float* __restrict__ apre, int B, int K,
                                                          int de, uint16_t* __restrict__ outv,
                                                          uint16_t* __restrict__ inv) {
  constexpr int NC = 4;
  __shared__ float s_red[4];
  const int64_t n = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* a = apre + n * de;
  float av[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) av[i] = a[min(tid + 256 * i, de - 1)];   // clamped: unconditional
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i)
    if (tid + 256 * i < de) ss = fmaf(av[i], av[i], ss);
  ss = wave_sum(ss);
  if (lane == 0) s_red[wave] = ss;
  __syncthreads();
  const float tot = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
  const float nr = fmaxf(__fsqrt_rn(tot), 1e-12f);
  uint16_t ov[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) ov[i] = (uint16_t)f32_to_bf16(__fdiv_rn(av[i], nr));
  const int64_t dst0 = (n * B * K) * (int64_t)de;
  for (int j = 0; j < K; ++j)
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int d = tid + 256 * i;
      if (d < de) {
        outv[dst0 + (int64_t)j * de + d] = ov[i];
        inv[dst0 + (int64_t)j * de + d] = 0;
      }
    }
}

}  // namespace

hipError_t launch_gather_rows(const int32_t* topk_idx, int N, int B, int K, const uint16_t* table,
                              int Ht, int V, uint16_t* out, hipStream_t stream) {
  const int64_t Mp = (int64_t)N * (B - 1) * K;
  if (Mp <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)Mp), dim3(256), 0, stream, topk_idx, B, K,
                     table, Ht, V, out);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_bf16(const uint16_t* x, int M, int H, const float* gamma, float eps,
                               uint16_t* out, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  if (H % 8 || H > 8192) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rmsnorm_bf16_kernel, dim3((unsigned)M), dim3(256), 0, stream, x, H, gamma, eps,
                     out);
  return hipGetLastError();
}

hipError_t launch_concat(const uint16_t* u, const uint16_t* tb, int N, int per_block, int H,
                         uint16_t* out, hipStream_t stream) {
  const int64_t Mp = (int64_t)N * per_block;
  if (Mp <= 0) return hipSuccess;
  hipLaunchKernelGGL(concat_kernel, dim3((unsigned)Mp), dim3(256), 0, stream, u, tb,
                     (int64_t)per_block, H, out);
  return hipGetLastError();
}

hipError_t launch_anchor_rows(const float* apre, int N, int B, int K, int de, uint16_t* outv,
                              uint16_t* inv, hipStream_t stream) {
  if (N <= 0) return hipSuccess;
  if (de > 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(anchor_rows_kernel, dim3((unsigned)N), dim3(256), 0, stream, apre, B, K, de,
                     outv, inv);
  return hipGetLastError();
}

}  // namespace ll
