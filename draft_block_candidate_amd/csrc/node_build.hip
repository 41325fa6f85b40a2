// Node construction for every candidate (LiLiCorr paper, Section 3.2 and
// Appendix A "Architecture"): the token's embedding row, the slot and rank
// table rows, and a two-layer network over five confidence scalars (log-prob,
// prob, gap to the slot's top log-prob, rank scaled to [0, 1], top-choice
// flag). This kernel computes the first (5 -> H) layer with SiLU and the table
// sum; the second layer is an MFMA GEMM whose epilogue adds the table sum.
#include "common.hpp"
#include "kernels.hpp"
#include "topk_merge.hpp"

namespace ll {
namespace {

// One block per TPB tokens; thread t owns the 4-column groups t, t + 256, ...
// (CG of them). The first-layer weights and biases of a thread's columns are
// loaded once per block and kept in registers; the tokens' embedding, slot
// and rank rows are all loaded before any is used.
// PAPER (the paper's own head): the tokens are the drafted candidates of slots
// 1..B-1 only, and the first term of the table sum is the slot's projected
// drafter hidden state ph[(n B + s) H ..] (fp32) instead of an E row; the
// target-embedding term is added by a later linear.
// WX = false (lattice head): only hid is written; the table sum is formed by
// the next linear's epilogue instead (NodeSource), so E, S and R are not read.
// MERGE (lattice head, one token per block, vocabulary rows split into P > 1
// chunks): the block's first wave merges its token's row from the chunk lists
// and (max, sum) pairs (part_*) itself, as the top-K merge kernel would, and
// the block writes its token's id and log-prob (and the row's lse from rank
// 0) to topk_idx / topk_logp, which are outputs here. This takes one launch
// out of the few-row step; every block of a row repeats the row's merge.
struct MergeSource {
  const float* part_val = nullptr;
  const int32_t* part_idx = nullptr;
  const float* part_ms = nullptr;
  int P = 1;
  float* lse = nullptr;   // optional
};

template <int CG, int TPB, bool PAPER, bool WX = true, bool MERGE = false>
__global__ __launch_bounds__(256) void node_build_kernel(
    const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_logp, int64_t M, int B,
    int K, int H, int V, const uint16_t* __restrict__ E, const float* __restrict__ ph,
    const uint16_t* __restrict__ S, const uint16_t* __restrict__ R, const uint16_t* __restrict__ w1,
    const float* __restrict__ b1, uint16_t* __restrict__ hid, float* __restrict__ xbase,
    uint64_t mk, uint64_t mb, uint64_t mb1, MergeSource ms = MergeSource{}) {
  static_assert(!MERGE || ((TPB == 1 || TPB == 8) && !PAPER && !WX), "in-block merge: lattice tokens of one row");
  const int tid = threadIdx.x, lane = tid & 63;
  // MERGE: the row's chunk entries (at most 64 lists of 64) and the merged
  // tokens (log-prob, the row's top log-prob, id). With TPB = 8 the launch
  // guarantees K % 8 == 0, so a block's eight tokens lie in one row.
  __shared__ float msv[MERGE ? 64 * 64 : 1];
  __shared__ int msi[MERGE ? 64 * 64 : 1];
  __shared__ float mres[TPB][3];
  if constexpr (MERGE) {
    const uint32_t t0 = (uint32_t)min((int64_t)blockIdx.x * TPB, M - 1);
    const uint32_t row = div_by(t0, mk);
    const int j0 = (int)(t0 - row * (uint32_t)K);
    if (tid < 64) {
      float rv, Mx, Sx;
      int ri;
      const float lse = merge_row_lists((int)row, K, ms.P, K, (int64_t)ms.P * K, 1, ms.P, ms.part_val,
                                        ms.part_idx, ms.part_ms, msv, msi, lane, rv, ri, Mx, Sx);
      const float lp0 = __fsub_rn(readlane_f(rv, 0), lse);
#pragma unroll
      for (int u = 0; u < TPB; ++u) {
        const int j = min(j0 + u, K - 1);
        const float lpj = __fsub_rn(readlane_f(rv, j), lse);
        const int idj = readlane_i(ri, j);
        if (lane == u) {
          const int64_t t = (int64_t)blockIdx.x * TPB + u;
          if (t < M) {
            ((int32_t*)topk_idx)[t] = idj;
            ((float*)topk_logp)[t] = lpj;
          }
          mres[u][0] = lpj;
          mres[u][1] = lp0;
          mres[u][2] = __int_as_float(idj);
        }
      }
      if (lane == 0 && j0 == 0 && ms.lse) ms.lse[row] = lse;
    }
    __syncthreads();
  }
  const int h4 = H / 4;
  // this thread's columns: w1 rows are 5 bf16 (10 bytes), so the 4 columns of
  // a group are 40 contiguous bytes
  float wv[CG][4][5], bv[CG][4];
#pragma unroll
  for (int g = 0; g < CG; ++g) {
    const int c4 = min(tid + 256 * g, h4 - 1);
    const uint2* wp = (const uint2*)(w1 + (int64_t)c4 * 20);
    uint32_t wr[10];
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const uint2 u = wp[i];
      wr[2 * i] = u.x;
      wr[2 * i + 1] = u.y;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const int h = q * 5 + i;   // bf16 index within the 20
        wv[g][q][i] = bf16_to_f32((wr[h >> 1] >> ((h & 1) * 16)) & 0xFFFF);
      }
    const float4 b = ((const float4*)b1)[c4];
    bv[g][0] = b.x; bv[g][1] = b.y; bv[g][2] = b.z; bv[g][3] = b.w;
  }
  // The block's tokens (clamped; the ones past M are computed, not stored).
  // Lane u works out token u's indices and features (slot and rank by the
  // exact multiply-shift division, M < 2^31), then every lane takes them by
  // readlane: the per-token work is done once per wave, not once per lane.
  int64_t tk[TPB];
  uint2 ev[TPB][CG], sv[TPB][CG], rv[TPB][CG];
  float4 pv[TPB][CG];
  float f[TPB][5];
  int tok_l, s_l, j_l, row_l;
  float fl[5];
  {
    const uint32_t t = (uint32_t)min((int64_t)blockIdx.x * TPB + min(lane, TPB - 1), M - 1);
    uint32_t row = div_by(t, mk);   // (block, slot)
    const int j = (int)(t - row * (uint32_t)K);
    if (PAPER) {                     // lattice row (n, s - 1) -> top-K row (n, s)
      const uint32_t n = div_by(row, mb1);
      row = n * (uint32_t)B + 1 + (row - n * (uint32_t)(B - 1));
    }
    const int s = (int)(row - div_by(row, mb) * (uint32_t)B);
    const int64_t ti = (int64_t)row * K + j;
    const int mu = min(lane, TPB - 1);   // MERGE: this lane's token of the block
    int tok = PAPER ? 0 : (MERGE ? __float_as_int(mres[mu][2]) : topk_idx[ti]);
    if (tok < 0 || tok >= V) tok = 0;  // ids come from the top-K stage; never read outside E
    const float lp = MERGE ? mres[mu][0] : topk_logp[ti];
    const float lp0 = MERGE ? mres[mu][1] : topk_logp[(int64_t)row * K];
    fl[0] = lp;
    fl[1] = expf(lp);
    fl[2] = __fsub_rn(lp, lp0);
    fl[3] = K > 1 ? __fdiv_rn((float)j, (float)(K - 1)) : 0.f;
    fl[4] = j == 0 ? 1.f : 0.f;
    tok_l = tok;
    s_l = s;
    j_l = j;
    row_l = (int)row;
  }
#pragma unroll
  for (int u = 0; u < TPB; ++u) {
    tk[u] = min((int64_t)blockIdx.x * TPB + u, M - 1);
    const int64_t tok = readlane_i(tok_l, u);
    const int s = readlane_i(s_l, u), j = readlane_i(j_l, u);
    const int64_t row = readlane_i(row_l, u);
#pragma unroll
    for (int i = 0; i < 5; ++i) f[u][i] = readlane_f(fl[i], u);
#pragma unroll
    for (int g = 0; g < CG; ++g) {
      if (!WX) break;
      const int c4 = min(tid + 256 * g, h4 - 1);
      if (PAPER)
        pv[u][g] = ((const float4*)(ph + row * H))[c4];
      else
        ev[u][g] = ((const uint2*)(E + tok * H))[c4];
      sv[u][g] = ((const uint2*)(S + (int64_t)s * H))[c4];
      rv[u][g] = ((const uint2*)(R + (int64_t)j * H))[c4];
    }
  }
#pragma unroll
  for (int u = 0; u < TPB; ++u) {
    const bool tok_ok = (int64_t)blockIdx.x * TPB + u < M;
#pragma unroll
    for (int g = 0; g < CG; ++g) {
      const int c4 = tid + 256 * g;
      const uint32_t ew[2] = {PAPER || !WX ? 0u : ev[u][g].x, PAPER || !WX ? 0u : ev[u][g].y},
                     sw[2] = {WX ? sv[u][g].x : 0u, WX ? sv[u][g].y : 0u},
                     rw[2] = {WX ? rv[u][g].x : 0u, WX ? rv[u][g].y : 0u};
      const float pw[4] = {PAPER && WX ? pv[u][g].x : 0.f, PAPER && WX ? pv[u][g].y : 0.f,
                           PAPER && WX ? pv[u][g].z : 0.f, PAPER && WX ? pv[u][g].w : 0.f};
      float xb[4], hz[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t sh = (q & 1) ? 16 : 0;
        const float a = PAPER ? pw[q] : bf16_to_f32((ew[q >> 1] >> sh) & 0xFFFF);
        const float b = bf16_to_f32((sw[q >> 1] >> sh) & 0xFFFF);
        const float c = bf16_to_f32((rw[q >> 1] >> sh) & 0xFFFF);
        xb[q] = __fadd_rn(__fadd_rn(a, b), c);
        float z = 0.f;
#pragma unroll
        for (int i = 0; i < 5; ++i) z = fmaf(wv[g][q][i], f[u][i], z);
        hz[q] = silu(z + bv[g][q]);
      }
      if (tok_ok && c4 < h4) {
        if (WX) ((float4*)(xbase + tk[u] * H))[c4] = make_float4(xb[0], xb[1], xb[2], xb[3]);
        ((uint2*)(hid + tk[u] * H))[c4] = make_uint2(pack_bf16x2(hz[0], hz[1]), pack_bf16x2(hz[2], hz[3]));
      }
    }
  }
}

}  // namespace

bool node_build_merges(int N, int B, int K, int H, int P) {
  const int64_t M = (int64_t)N * B * K;
  // One token per block below 4,096 tokens; above, eight tokens per block,
  // which is exactly one row at K = 8. Wider rows would make every block of a
  // row repeat a longer tournament (K = 32 at the entropy shape: node build
  // 38 -> 68 us against 8 us saved in the top-K stage).
  return P > 1 && P <= 64 && K <= 64 && B <= 64 && M < ((int64_t)1 << 31) &&
         (M < 4096 || (K == 8 && H <= 2048));
}

hipError_t launch_node_build_merge(const float* part_val, const int32_t* part_idx, const float* part_ms,
                                   int P, int32_t* topk_idx, float* topk_logp, float* lse, int N, int B,
                                   int K, int H, const uint16_t* conf_w1, const float* conf_b1,
                                   uint16_t* hid, int V, hipStream_t stream) {
  if (!node_build_merges(N, B, K, H, P)) return hipErrorInvalidValue;
  const int64_t M = (int64_t)N * B * K;
  const uint64_t mk = div_magic(K), mb = div_magic(B), mb1 = div_magic(1);
  MergeSource ms;
  ms.part_val = part_val;
  ms.part_idx = part_idx;
  ms.part_ms = part_ms;
  ms.P = P;
  ms.lse = lse;
#define LL_NBM(CG, TPB, grid)                                                                       \
  hipLaunchKernelGGL((node_build_kernel<CG, TPB, false, false, true>), grid, dim3(256), 0, stream,  \
                     topk_idx, topk_logp, M, B, K, H, V, nullptr, nullptr, nullptr, nullptr, conf_w1,  \
                     conf_b1, hid, nullptr, mk, mb, mb1, ms)
  if (M < 4096) {
    const dim3 grid((unsigned)M);
    if (H <= 1024)
      LL_NBM(1, 1, grid);
    else if (H <= 2048)
      LL_NBM(2, 1, grid);
    else
      LL_NBM(4, 1, grid);
  } else {   // K % 8 == 0: eight tokens of one row per block
    const dim3 grid8((unsigned)(M / 8));
    if (H <= 1024)
      LL_NBM(1, 8, grid8);
    else if (H <= 2048)
      LL_NBM(2, 8, grid8);
    else
      return hipErrorInvalidValue;   // the widest rows take four tokens per block
  }
#undef LL_NBM
  return hipGetLastError();
}

hipError_t launch_node_build(const int32_t* topk_idx, const float* topk_logp, int N, int B, int K,
                             int H, const uint16_t* E, const float* ph, const uint16_t* S,
                             const uint16_t* R, const uint16_t* conf_w1, const float* conf_b1,
                             uint16_t* hid, float* xbase, int V, hipStream_t stream) {
  const bool paper = ph != nullptr;
  const int64_t M = (int64_t)N * (paper ? B - 1 : B) * K;
  if (M <= 0) return hipSuccess;
  if (paper && !xbase) return hipErrorInvalidValue;
  if (M >= ((int64_t)1 << 31) || K > 64 || B > 64) return hipErrorInvalidValue;
  const uint64_t mk = div_magic(K), mb = div_magic(B), mb1 = div_magic(B > 1 ? B - 1 : 1);
#define LL_NB(CG, TPB, grid)                                                                     \
  do {                                                                                         \
    if (paper)                                                                                 \
      hipLaunchKernelGGL((node_build_kernel<CG, TPB, true>), grid, dim3(256), 0, stream,      \
                         topk_idx, topk_logp, M, B, K, H, V, E, ph, S, R, conf_w1, conf_b1,   \
                         hid, xbase, mk, mb, mb1);                                             \
    else if (xbase)                                                                            \
      hipLaunchKernelGGL((node_build_kernel<CG, TPB, false>), grid, dim3(256), 0, stream,     \
                         topk_idx, topk_logp, M, B, K, H, V, E, ph, S, R, conf_w1, conf_b1,   \
                         hid, xbase, mk, mb, mb1);                                             \
    else                                                                                       \
      hipLaunchKernelGGL((node_build_kernel<CG, TPB, false, false>), grid, dim3(256), 0,      \
                         stream, topk_idx, topk_logp, M, B, K, H, V, E, ph, S, R, conf_w1,    \
                         conf_b1, hid, xbase, mk, mb, mb1);                                    \
  } while (0)
  // few tokens: one per block (more blocks in flight); many: eight per block
  // (four for the widest rows, to bound the registers)
  if (M < 4096) {
    const dim3 grid((unsigned)M);
    if (H <= 1024)
      LL_NB(1, 1, grid);
    else if (H <= 2048)
      LL_NB(2, 1, grid);
    else
      LL_NB(4, 1, grid);
  } else {
    const dim3 grid8((unsigned)((M + 7) / 8)), grid4((unsigned)((M + 3) / 4));
    if (H <= 1024)
      LL_NB(1, 8, grid8);
    else if (H <= 2048)
      LL_NB(2, 8, grid8);
    else
      LL_NB(4, 4, grid4);
  }
#undef LL_NB
  return hipGetLastError();
}

}  // namespace ll
