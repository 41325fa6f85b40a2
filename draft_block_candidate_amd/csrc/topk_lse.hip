// Fused log-partition + exact top-K over vocabulary rows (one HBM pass).
//
// What it computes (LiLiCorr paper, Section 3.2 and Appendix A "Serving";
// SGLang PR "[Spec] Add LiLiCorr", section "Why the custom kernels"): for each
// row, lse = log sum_v exp(x_v) and the K entries ordered by (x desc, v asc),
// with logp = fl32(x - fl32(lse)).
//
// Design for gfx950 (the PR's Triton kernel pre-selects whole tiles; here the
// unit of work is one wave64 streaming a contiguous chunk of a row):
//  * each lane issues NV 16-byte non-temporal loads per iteration (coalesced:
//    64 lanes read 1 KiB contiguous per load);
//  * the log-partition is an online sum of exp2 terms against a lazily raised
//    per-lane reference max (raised only when a value exceeds it by 16), so
//    the common path is one fma + one v_exp_f32 + one add per element;
//  * the running top-K is a sorted list held one entry per lane (lane k holds
//    the k-th best key). An element can only enter if it beats entry K-1, the
//    wave-uniform threshold; the per-iteration test is one compare of each
//    lane's running max against it, so insertions (K ln(n/K) of them for n
//    streamed elements in random order) are the only slow path;
//  * the list is seeded from the first iteration by a 64-lane bitonic sort of
//    the lanes' best elements, so it starts at a tight threshold;
//  * chunks of one row are merged by a second kernel (one wave per row: a
//    K-step tournament over the chunks' sorted lists plus the log-sum-exp
//    combination of the chunks' (max, sum) pairs).
// Exactness: the streamed order is ascending in vocabulary index, so a value
// equal to the threshold never beats it in the fast test; everything that
// reaches the slow path is compared on the full (value, index) key.
#include <cmath>

#include "common.hpp"
#include "kernels.hpp"
#include "layout.hpp"

namespace ll {
namespace {

constexpr float kL2E = 1.4426950408889634f;
constexpr float kLazy = 16.0f;      // reference max may lag the true max by this much
constexpr float kMInit = -1e30f;
constexpr int kInvalid = 0x7fffffff;

__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ int readlane_i(int v, int l) { return __builtin_amdgcn_readlane(v, l); }

__device__ __forceinline__ bool key_gt(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

struct State {
  float m_ref, s;   // per lane: reference max and sum of exp(x - m_ref)
  float lv;         // list entry of this lane (lanes >= K hold -inf)
  int li;
  float th_v;       // wave-uniform threshold = list entry K-1
  int th_i;
};

__device__ __forceinline__ void list_insert(State& st, float cv, int ci, int K, int lane) {
  const bool better = (lane < K) && key_gt(st.lv, st.li, cv, ci);
  const int pos = __popcll(__ballot(better));
  const float upv = __shfl_up(st.lv, 1, 64);
  const int upi = __shfl_up(st.li, 1, 64);
  if (lane == pos) {
    st.lv = cv;
    st.li = ci;
  } else if (lane > pos && lane < K) {
    st.lv = upv;
    st.li = upi;
  }
  st.th_v = readlane_f(st.lv, K - 1);
  st.th_i = readlane_i(st.li, K - 1);
}

// Offer one element slot of every lane to the list (exact key compare).
__device__ __forceinline__ void offer(State& st, float x, int id, bool allowed, int K, int lane) {
  uint64_t mask = __ballot(allowed && key_gt(x, id, st.th_v, st.th_i));
  while (mask) {
    const int l = __ffsll((long long)mask) - 1;
    mask &= mask - 1;
    const float cv = readlane_f(x, l);
    const int ci = readlane_i(id, l);
    if (key_gt(cv, ci, st.th_v, st.th_i)) list_insert(st, cv, ci, K, lane);
  }
}

template <int NV, int EPV>
__device__ __forceinline__ void lse_update(State& st, const float (&x)[NV][EPV]) {
  float lm = x[0][0];
#pragma unroll
  for (int u = 0; u < NV; ++u)
#pragma unroll
    for (int e = 0; e < EPV; ++e) lm = fmaxf(lm, x[u][e]);
  if (__any(lm > st.m_ref + kLazy)) {
    const float nm = lm > st.m_ref + kLazy ? lm : st.m_ref;
    st.s *= __builtin_amdgcn_exp2f((st.m_ref - nm) * kL2E);
    st.m_ref = nm;
  }
  const float c = st.m_ref * kL2E;
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    float t = 0.f;
#pragma unroll
    for (int e = 0; e < EPV; ++e) t += __builtin_amdgcn_exp2f(fmaf(x[u][e], kL2E, -c));
    st.s += t;
  }
}

// Element (u, e) of a lane has row-local index base + u*64*EPV + lane*LS + e.
template <int NV, int EPV, int LS>
__device__ __forceinline__ int elem_idx(int base, int u, int e, int lane, float x) {
  return x == -INFINITY ? kInvalid : base + u * 64 * EPV + lane * LS + e;
}

// Exact pass over a group: every element that beats the threshold is offered.
template <int NV, int EPV, int LS>
__device__ __forceinline__ void group_exact(State& st, const float (&x)[NV][EPV], int base, int excl, int K,
                            int lane) {
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    float vm = x[u][0];
#pragma unroll
    for (int e = 1; e < EPV; ++e) vm = fmaxf(vm, x[u][e]);
    if (!__any(vm >= st.th_v)) continue;
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      const int id = elem_idx<NV, EPV, LS>(base, u, e, lane, x[u][e]);
      offer(st, x[u][e], id, id != excl, K, lane);
    }
  }
}

// Seed the list from a group: sort the 64 lanes' best elements (bitonic,
// descending by key), keep the first K, then offer the rest of the group.
template <int NV, int EPV, int LS>
__device__ __forceinline__ void group_seed(State& st, const float (&x)[NV][EPV], int base, int K, int lane) {
  float bv = -INFINITY;
  int bi = kInvalid;
#pragma unroll
  for (int u = 0; u < NV; ++u)
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      const int id = elem_idx<NV, EPV, LS>(base, u, e, lane, x[u][e]);
      if (key_gt(x[u][e], id, bv, bi)) {
        bv = x[u][e];
        bi = id;
      }
    }
  float sv = bv;
  int si = bi;
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const float ov = __shfl_xor(sv, j, 64);
      const int oi = __shfl_xor(si, j, 64);
      const bool keep_better = ((lane & j) == 0) == ((lane & k) == 0);
      const bool mine_better = key_gt(sv, si, ov, oi);
      if (keep_better != mine_better) {
        sv = ov;
        si = oi;
      }
    }
  }
  st.lv = lane < K ? sv : -INFINITY;
  st.li = lane < K ? si : kInvalid;
  st.th_v = readlane_f(st.lv, K - 1);
  st.th_i = readlane_i(st.li, K - 1);
  group_exact<NV, EPV, LS>(st, x, base, bi, K, lane);
}

template <int DT>
__device__ __forceinline__ float load_scalar(const void* p, int64_t i) {
  if (DT == 1) return bf16_to_f32(((const uint16_t*)p)[i]);
  return ((const float*)p)[i];
}

template <int EPV>
__device__ __forceinline__ void unpack(const u32x4_t& w, float (&x)[EPV]) {
  if constexpr (EPV == 8) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      x[2 * d] = __uint_as_float(w[d] << 16);
      x[2 * d + 1] = __uint_as_float(w[d] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int d = 0; d < 4; ++d) x[d] = __uint_as_float(w[d]);
  }
}

// One wave per (row, chunk). DT: 0 = fp32 logits, 1 = bf16 logits.
template <int DT, int NV>
__global__ __launch_bounds__(256) void topk_partial_kernel(const void* __restrict__ logits,
                                                           int rows, int V, int K, int P,
                                                           float* __restrict__ part_val,
                                                           int32_t* __restrict__ part_idx,
                                                           float* __restrict__ part_ms) {
  constexpr int EPV = DT == 1 ? 8 : 4;
  const int lane = threadIdx.x & 63;
  const int g = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int row = g / P, unit = g - (g / P) * P;
  if (row >= rows) return;

  const int64_t rs = (int64_t)row * V, re = rs + V;
  int64_t a0 = (rs + EPV - 1) / EPV * EPV, a1 = re / EPV * EPV;
  if (a1 <= a0) {  // no whole aligned vector: the row is all head
    a0 = re;
    a1 = re;
  }
  const int64_t nv = (a1 - a0) / EPV;
  const int64_t cv = (nv + P - 1) / P;
  const int64_t vb = min(nv, (int64_t)unit * cv), ve = min(nv, vb + cv);
  const u32x4_t* vbase = (const u32x4_t*)logits + a0 / EPV;
  const int head_len = (int)(a0 - rs), tail_len = (int)(re - a1);

  State st;
  st.m_ref = kMInit;
  st.s = 0.f;
  st.lv = -INFINITY;
  st.li = kInvalid;
  st.th_v = -INFINITY;
  st.th_i = kInvalid;
  bool seeded = false;

  // Head: elements before the first aligned vector (owned by chunk 0). It is
  // merged in after the list is seeded, with exact compares.
  auto do_edge = [&](int64_t start, int len) {
    float xe[1][EPV];
#pragma unroll
    for (int e = 0; e < EPV; ++e) xe[0][e] = -INFINITY;
    if (lane < len) xe[0][0] = load_scalar<DT>(logits, start + lane);
    lse_update<1, EPV>(st, xe);
    if (!seeded) {
      group_seed<1, EPV, 1>(st, xe, (int)(start - rs), K, lane);
      seeded = true;
    } else {
      group_exact<1, EPV, 1>(st, xe, (int)(start - rs), -1, K, lane);
    }
  };

  bool head_pending = unit == 0 && head_len > 0;
  for (int64_t v = vb; v < ve; v += 64 * NV) {
    float x[NV][EPV];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int64_t vi = v + u * 64 + lane;
      if (vi < ve) {
        const u32x4_t w = __builtin_nontemporal_load(vbase + vi);
        unpack<EPV>(w, x[u]);
      } else {
#pragma unroll
        for (int e = 0; e < EPV; ++e) x[u][e] = -INFINITY;
      }
    }
    const int base = (int)(a0 - rs + v * EPV);
    lse_update<NV, EPV>(st, x);
    if (!seeded) {
      group_seed<NV, EPV, EPV>(st, x, base, K, lane);
      seeded = true;
    } else {
      float lm = x[0][0];
#pragma unroll
      for (int u = 0; u < NV; ++u)
#pragma unroll
        for (int e = 0; e < EPV; ++e) lm = fmaxf(lm, x[u][e]);
      if (__any(lm > st.th_v)) group_exact<NV, EPV, EPV>(st, x, base, -1, K, lane);
    }
    if (head_pending) {
      do_edge(rs, head_len);
      head_pending = false;
    }
  }
  if (head_pending) do_edge(rs, head_len);
  if (unit == P - 1 && tail_len > 0) do_edge(a1, tail_len);

  // Chunk outputs: sorted list and (reference max, sum) of the wave.
  const int64_t o = (int64_t)row * P + unit;
  if (lane < K) {
    part_val[o * K + lane] = st.lv;
    part_idx[o * K + lane] = st.li;
  }
  const float M = wave_max(st.m_ref);
  const float S = wave_sum(st.s * __builtin_amdgcn_exp2f((st.m_ref - M) * kL2E));
  if (lane == 0) {
    part_ms[2 * o] = M;
    part_ms[2 * o + 1] = S;
  }
}

// One wave per row: combine the P chunk lists (tournament) and (max, sum)
// pairs. The row's P * K partial entries are staged in LDS first, so each of
// the K tournament steps reads the winner's next entry from LDS.
__global__ __launch_bounds__(64) void topk_merge_kernel(int rows, int K, int P,
                                                        const float* __restrict__ part_val,
                                                        const int32_t* __restrict__ part_idx,
                                                        const float* __restrict__ part_ms,
                                                        int32_t* __restrict__ topk_idx,
                                                        float* __restrict__ topk_logp,
                                                        float* __restrict__ lse_out) {
  extern __shared__ float sm[];
  float* sv = sm;                       // [P K]
  int* si = (int*)(sm + P * K);         // [P K]
  const int lane = threadIdx.x;
  const int row = blockIdx.x;
  const int64_t rbase = (int64_t)row * P * K;
  for (int i = lane; i < P * K; i += 64) {
    sv[i] = part_val[rbase + i];
    si[i] = part_idx[rbase + i];
  }
  float m = kMInit, s = 0.f;
  if (lane < P) {
    m = part_ms[2 * ((int64_t)row * P + lane)];
    s = part_ms[2 * ((int64_t)row * P + lane) + 1];
  }
  const float M = wave_max(m);
  const float S = wave_sum(s * __builtin_amdgcn_exp2f((m - M) * kL2E));
  const float lse = M + logf(S);
  __syncthreads();
  float hv = -INFINITY;
  int hi = kInvalid, hp = 0;
  if (lane < P) {
    hv = sv[lane * K];
    hi = si[lane * K];
  }
  float rv = -INFINITY;
  int ri = kInvalid;
  for (int k = 0; k < K; ++k) {
    // wave argmax of the heads by (value desc, index asc); keys are unique
    float bv = hv;
    int bi = hi, bl = lane;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      const int ol = __shfl_xor(bl, off, 64);
      if (key_gt(ov, oi, bv, bi) || (ov == bv && oi == bi && ol < bl)) {
        bv = ov;
        bi = oi;
        bl = ol;
      }
    }
    if (lane == k) {
      rv = bv;
      ri = bi;
    }
    if (lane == bl && lane < P) {
      ++hp;
      if (hp < K) {
        hv = sv[lane * K + hp];
        hi = si[lane * K + hp];
      } else {
        hv = -INFINITY;
        hi = kInvalid;
      }
    }
  }
  if (lane < K) {
    topk_idx[(int64_t)row * K + lane] = ri;
    topk_logp[(int64_t)row * K + lane] = __fsub_rn(rv, lse);
  }
  if (lse_out != nullptr && lane == 0) lse_out[row] = lse;
}

}  // namespace

hipError_t launch_topk_lse(const void* logits, int rows, int V, int K, int dtype, float* part_val,
                           int32_t* part_idx, float* part_ms, int32_t* topk_idx, float* topk_logp,
                           float* lse, hipStream_t stream) {
  const int P = topk_chunks_per_row(rows, V);
  const int64_t waves = (int64_t)rows * P;
  const unsigned blocks = (unsigned)((waves + 3) / 4);
  if (dtype == 1)
    hipLaunchKernelGGL((topk_partial_kernel<1, 4>), dim3(blocks), dim3(256), 0, stream, logits,
                       rows, V, K, P, part_val, part_idx, part_ms);
  else
    hipLaunchKernelGGL((topk_partial_kernel<0, 4>), dim3(blocks), dim3(256), 0, stream, logits,
                       rows, V, K, P, part_val, part_idx, part_ms);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)rows), dim3(64), (size_t)P * K * 8, stream,
                     rows, K, P, part_val, part_idx, part_ms, topk_idx, topk_logp, lse);
  return hipGetLastError();
}

}  // namespace ll
