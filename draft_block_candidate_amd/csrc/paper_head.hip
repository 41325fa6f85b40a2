// Kernels of the paper's own head (LiLiCorr paper, Section 3.2 and Appendix A
// "Architecture") that the lattice head does not have; its products run on
// the MFMA linears of gemm.hip.
//   * the target's input-embedding rows of every drafted candidate, gathered
//     as the A operand of the embedding projection;
//   * RMSNorm of the bf16 target state before its projection;
//   * the fusion layer's input: the concatenation [node, t', node * t'];
//   * the anchor's out vector (unit-normalised) and the [N, B, K, d_e] layout
//     the pair scores read: slot 0 carries the anchor vector in every candidate
//     row, slots 1..B-1 the lattice's out/in vectors.
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

// One wave per row of bf16 x: out = bf16((x * rstd) * gamma), rstd =
// 1 / sqrt(mean(x^2) + eps), the arithmetic of the fp32 RMSNorm kernels.
__global__ __launch_bounds__(256) void rmsnorm_bf16_kernel(const uint16_t* __restrict__ x, int M, int H,
                                                           const float* __restrict__ gamma, float eps,
                                                           uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const uint2* xr = (const uint2*)(x + row * H);
  float ss = 0.f;
  for (int c4 = lane; c4 < H / 4; c4 += 64) {
    const uint2 v = xr[c4];
    const float a = bf16_to_f32(v.x & 0xFFFF), b = bf16_to_f32(v.x >> 16);
    const float c = bf16_to_f32(v.y & 0xFFFF), d = bf16_to_f32(v.y >> 16);
    ss = fmaf(a, a, ss);
    ss = fmaf(b, b, ss);
    ss = fmaf(c, c, ss);
    ss = fmaf(d, d, ss);
  }
  ss = wave_sum(ss);
  const float rstd = 1.0f / __fsqrt_rn(ss / (float)H + eps);
  const float4* g4 = (const float4*)gamma;
  uint2* o2 = (uint2*)(out + row * H);
  for (int c4 = lane; c4 < H / 4; c4 += 64) {
    const uint2 v = xr[c4];
    const float4 g = g4[c4];
    o2[c4] = make_uint2(pack_bf16x2(bf16_to_f32(v.x & 0xFFFF) * rstd * g.x, bf16_to_f32(v.x >> 16) * rstd * g.y),
                        pack_bf16x2(bf16_to_f32(v.y & 0xFFFF) * rstd * g.z, bf16_to_f32(v.y >> 16) * rstd * g.w));
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

// One workgroup per (block n, slot s). Slot 0: the anchor vector
// o_0 = bf16(a / max(|a|, 1e-12)), a = apre[n], written to all K candidate rows
// of outv (the in rows are zero). Slots s >= 1: the K lattice rows of slot s.
__global__ __launch_bounds__(256) void assemble_kernel(const uint16_t* __restrict__ lat_out,
                                                       const uint16_t* __restrict__ lat_in,
                                                       const float* __restrict__ apre, int B, int K,
                                                       int de, uint16_t* __restrict__ outv,
                                                       uint16_t* __restrict__ inv) {
  __shared__ float s_red[4];
  const int64_t n = blockIdx.x / B;
  const int s = (int)(blockIdx.x - n * B);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t dst0 = ((n * B + s) * K) * (int64_t)de;
  if (s == 0) {
    const float* a = apre + n * de;
    float ss = 0.f;
    for (int d = tid; d < de; d += 256) ss = fmaf(a[d], a[d], ss);
    ss = wave_sum(ss);
    if (lane == 0) s_red[wave] = ss;
    __syncthreads();
    const float tot = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
    const float nr = fmaxf(__fsqrt_rn(tot), 1e-12f);
    for (int i = tid; i < K * de; i += 256) {
      const int d = i % de;
      outv[dst0 + i] = (uint16_t)f32_to_bf16(__fdiv_rn(a[d], nr));
      inv[dst0 + i] = 0;
    }
    return;
  }
  const int64_t src0 = ((n * (B - 1) + s - 1) * K) * (int64_t)de;
  const uint4* so = (const uint4*)(lat_out + src0);
  const uint4* si = (const uint4*)(lat_in + src0);
  uint4* d_o = (uint4*)(outv + dst0);
  uint4* d_i = (uint4*)(inv + dst0);
  for (int i = tid; i < K * de / 8; i += 256) {
    d_o[i] = so[i];
    d_i[i] = si[i];
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
  hipLaunchKernelGGL(rmsnorm_bf16_kernel, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, stream, x, M,
                     H, gamma, eps, out);
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

hipError_t launch_assemble(const uint16_t* lat_out, const uint16_t* lat_in, const float* apre, int N,
                           int B, int K, int de, uint16_t* outv, uint16_t* inv, hipStream_t stream) {
  hipLaunchKernelGGL(assemble_kernel, dim3((unsigned)((int64_t)N * B)), dim3(256), 0, stream,
                     lat_out, lat_in, apre, B, K, de, outv, inv);
  return hipGetLastError();
}

}  // namespace ll
