// Lattice attention (LiLiCorr paper, Section 3.2 and Appendix A: a
// bidirectional transformer over the whole candidate lattice of a block, with
// two per-head biases on the attention logits: one indexed by the signed slot
// distance between the two candidates, one for pairs in the same slot).
//
//   s_ij = q_i . k_j / sqrt(d_h) + Dist[slot_j - slot_i + 63] + Same [slot_i == slot_j]
//   p_ij = bf16(exp(s_ij - max_j s_ij)),  l_i = sum_j exp(s_ij - max_j s_ij)
//   o_i  = bf16(sum_j p_ij v_j / l_i)
//
// One workgroup per (query tile of 64, head, block); each wave owns 16
// queries. The lattice has at most 512 tokens, so a wave keeps its whole
// 16 x T score strip in registers: the row max is exact before any
// exponential (no online rescaling). Scores are computed transposed
// (S^T = K Q^T) so that each lane holds one query's column; that layout is
// directly the B operand of O^T = V^T P^T, the second MFMA product. V is
// staged through LDS transposed, 32 keys at a time.
#include "common.hpp"
#include "kernels.hpp"

namespace ll {
namespace {

constexpr int VT_STRIDE = 36;  // bf16 per transposed-V row (32 keys + pad, 8-byte aligned)

template <int TMAX, int DH>
__global__ __launch_bounds__(256) void attention_kernel(const uint16_t* __restrict__ qkv, int B,
                                                        int K, int H, const float* __restrict__ dist,
                                                        const float* __restrict__ same,
                                                        uint16_t* __restrict__ out) {
  constexpr int KT = TMAX / 16;   // 16-key tiles
  constexpr int KS = DH / 32;     // MFMA k-steps over d_h
  constexpr int DT = DH / 16;     // 16-wide d tiles of the output
  __shared__ float bias_tab[128];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[DH * VT_STRIDE];

  const int T = B * K;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int h = blockIdx.y;
  const int64_t n = blockIdx.z;
  const int64_t H3 = 3 * (int64_t)H;
  const uint16_t* blk = qkv + n * T * H3;
  const int q = blockIdx.x * 64 + wave * 16 + c;   // this lane's query
  const bool q_ok = q < T;
  const int slot_q = q_ok ? q / K : 0;

  if (tid < 127) bias_tab[tid] = dist[h * 127 + tid];
  const float same_h = same[h];
  __syncthreads();

  // Query fragment: B operand of S^T = K Q^T (column = query, k = d).
  u32x4_t qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qf[ks] = q_ok ? *(const u32x4_t*)(blk + (int64_t)q * H3 + h * DH + ks * 32 + 8 * g)
                  : u32x4_t{0, 0, 0, 0};

  // V chunk loader (32 keys x DH, 16 bytes per thread-slot); chunk 0 is issued
  // now so its latency overlaps the score computation.
  constexpr int VCH = (32 * DH / 8 + 255) / 256;
  u32x4_t vreg[VCH];
  auto load_v = [&](int ch) {
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int v = tid + 256 * i;
      const int key = v / (DH / 8), d8 = v % (DH / 8);
      const int kg = ch * 32 + key;
      vreg[i] = (v < 32 * DH / 8 && kg < T)
                    ? *(const u32x4_t*)(blk + (int64_t)kg * H3 + 2 * H + h * DH + d8 * 8)
                    : u32x4_t{0, 0, 0, 0};
    }
  };
  load_v(0);

  const float scale = 1.0f / __fsqrt_rn((float)DH);
  float s[KT][4];
  float mx = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    if (kt * 16 >= T) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s[kt][i] = -INFINITY;
      continue;
    }
    const int krow = kt * 16 + c;   // A operand row = key
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4_t kf = krow < T ? *(const u32x4_t*)(blk + (int64_t)krow * H3 + H + h * DH + ks * 32 + 8 * g)
                                  : u32x4_t{0, 0, 0, 0};
      acc = mfma16(kf, qf[ks], acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = kt * 16 + 4 * g + i;
      float v = -INFINITY;
      if (key < T) {
        const int slot_k = key / K;
        v = acc[i] * scale + bias_tab[slot_k - slot_q + 63];
        if (slot_k == slot_q) v += same_h;
      }
      s[kt][i] = v;
      mx = fmaxf(mx, v);
    }
  }
  // Row max over the 4 lane groups holding the same query.
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  float lsum = 0.f;
#pragma unroll
  for (int kt = 0; kt < KT; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = __expf(s[kt][i] - mx);
      s[kt][i] = p;
      lsum += p;
    }
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);

  f32x4_t oacc[DT];
#pragma unroll
  for (int d = 0; d < DT; ++d) oacc[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // P V over 32-key chunks. k-slot j of lane group g stands for key
  // 32*ch + 4g + j (j < 4) or 32*ch + 16 + 4g + (j - 4) (j >= 4).
  // V chunks are staged transposed in LDS; the next chunk's global loads are
  // in flight while the current chunk is multiplied.
  const int nch = (T + 31) / 32;
#pragma unroll
  for (int ch = 0; ch < KT / 2; ++ch) {
    if (ch >= nch) break;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int v = tid + 256 * i;
      if (v < 32 * DH / 8) {
        const int key = v / (DH / 8), d8 = v % (DH / 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          Vt[(d8 * 8 + 2 * e) * VT_STRIDE + key] = (uint16_t)(vreg[i][e] & 0xFFFF);
          Vt[(d8 * 8 + 2 * e + 1) * VT_STRIDE + key] = (uint16_t)(vreg[i][e] >> 16);
        }
      }
    }
    __syncthreads();
    if (ch + 1 < nch) load_v(ch + 1);
    u32x4_t pb;
    pb[0] = pack_bf16x2(s[2 * ch][0], s[2 * ch][1]);
    pb[1] = pack_bf16x2(s[2 * ch][2], s[2 * ch][3]);
    pb[2] = pack_bf16x2(s[2 * ch + 1][0], s[2 * ch + 1][1]);
    pb[3] = pack_bf16x2(s[2 * ch + 1][2], s[2 * ch + 1][3]);
#pragma unroll
    for (int d = 0; d < DT; ++d) {
      const uint16_t* vr = &Vt[(d * 16 + c) * VT_STRIDE];
      const u32x2_t lo = *(const u32x2_t*)(vr + 4 * g);
      const u32x2_t hi = *(const u32x2_t*)(vr + 16 + 4 * g);
      const u32x4_t va = {lo[0], lo[1], hi[0], hi[1]};
      oacc[d] = mfma16(va, pb, oacc[d]);
    }
  }

  if (q_ok) {
    const float inv = 1.0f / lsum;
    uint16_t* orow = out + (n * T + q) * (int64_t)H + h * DH;
#pragma unroll
    for (int d = 0; d < DT; ++d) {
      // oacc[d][i] = O[query q][d*16 + 4g + i]
      const uint32_t w0 = pack_bf16x2(oacc[d][0] * inv, oacc[d][1] * inv);
      const uint32_t w1 = pack_bf16x2(oacc[d][2] * inv, oacc[d][3] * inv);
      *(uint2*)(orow + d * 16 + 4 * g) = make_uint2(w0, w1);
    }
  }
}

template <int TMAX>
hipError_t launch_dh(int dh, const uint16_t* qkv, int N, int B, int K, int H, int heads,
                     const float* dist, const float* same, uint16_t* out, hipStream_t stream) {
  const int T = B * K;
  dim3 grid((unsigned)((T + 63) / 64), (unsigned)heads, (unsigned)N);
  if (dh == 32)
    hipLaunchKernelGGL((attention_kernel<TMAX, 32>), grid, dim3(256), 0, stream, qkv, B, K, H,
                       dist, same, out);
  else if (dh == 64)
    hipLaunchKernelGGL((attention_kernel<TMAX, 64>), grid, dim3(256), 0, stream, qkv, B, K, H,
                       dist, same, out);
  else
    hipLaunchKernelGGL((attention_kernel<TMAX, 128>), grid, dim3(256), 0, stream, qkv, B, K, H,
                       dist, same, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const uint16_t* qkv, int N, int B, int K, int H, int heads,
                            const float* dist, const float* same, uint16_t* out,
                            hipStream_t stream) {
  const int T = B * K, dh = H / heads;
  if (T <= 64) return launch_dh<64>(dh, qkv, N, B, K, H, heads, dist, same, out, stream);
  if (T <= 128) return launch_dh<128>(dh, qkv, N, B, K, H, heads, dist, same, out, stream);
  if (T <= 256) return launch_dh<256>(dh, qkv, N, B, K, H, heads, dist, same, out, stream);
  return launch_dh<512>(dh, qkv, N, B, K, H, heads, dist, same, out, stream);
}

}  // namespace ll
