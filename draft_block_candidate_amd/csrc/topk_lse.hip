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
  // wave_shr:1 (DPP): every lane receives the entry of the lane below it
  const float upv = dpp_f<0x138, 0xf>(st.lv, st.lv);
  const int upi = dpp_i<0x138, 0xf>(st.li, st.li);
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

template <int DT>
__device__ __forceinline__ float load_scalar(const void* p, int64_t i) {
  if (DT == 1) return bf16_to_f32(((const uint16_t*)p)[i]);
  return ((const float*)p)[i];
}

// Element e of a packed 16-byte vector.
template <int EPV>
__device__ __forceinline__ float elem(const u32x4_t& w, int e) {
  if constexpr (EPV == 8)
    return (e & 1) ? __uint_as_float(w[e >> 1] & 0xFFFF0000u) : __uint_as_float(w[e >> 1] << 16);
  else
    return __uint_as_float(w[e]);
}

// Log-sum-exp update for one group of NV packed vectors per lane (slots
// outside the chunk hold -inf words, which add nothing). Returns the lane's
// group maximum.
template <int NV, int EPV>
__device__ __forceinline__ float group_lse(State& st, const u32x4_t (&w)[NV]) {
  float lm = elem<EPV>(w[0], 0);
#pragma unroll
  for (int u = 0; u < NV; ++u)
#pragma unroll
    for (int e = 0; e < EPV; ++e) lm = fmaxf(lm, elem<EPV>(w[u], e));
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
    for (int e = 0; e < EPV; ++e) t += __builtin_amdgcn_exp2f(fmaf(elem<EPV>(w[u], e), kL2E, -c));
    st.s += t;
  }
  return lm;
}

// Slow path over a group stashed in this wave's LDS area (vector slot u of
// lane l at stash[u * 64 + l]). Element (u, e) of a lane has row-local index
// base + (u * 64 + lane) * LS + e; -inf elements are outside the row.
template <int NV, int EPV, int LS>
__device__ __forceinline__ void group_slow(State& st, const u32x4_t* stash, int base, bool seed,
                                           int K, int lane) {
  int excl = -1;
  if (seed) {
    // the 64 lanes' best elements, bitonic-sorted (descending key); the first
    // K seed the list, so the threshold starts at the K-th best lane maximum
    float bv = -INFINITY;
    int bi = kInvalid;
    for (int u = 0; u < NV; ++u) {
      const u32x4_t w = stash[u * 64 + lane];
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const float x = elem<EPV>(w, e);
        const int id = base + (u * 64 + lane) * LS + e;
        if (x != -INFINITY && key_gt(x, id, bv, bi)) {
          bv = x;
          bi = id;
        }
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
    excl = bi;
  }
  for (int u = 0; u < NV; ++u) {
    const u32x4_t w = stash[u * 64 + lane];
    float vm = -INFINITY;
#pragma unroll
    for (int e = 0; e < EPV; ++e) vm = fmaxf(vm, elem<EPV>(w, e));
    if (!__any(vm >= st.th_v)) continue;
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      const float x = elem<EPV>(w, e);
      const int id = x == -INFINITY ? kInvalid : base + (u * 64 + lane) * LS + e;
      offer(st, x, id, id != excl, K, lane);
    }
  }
}

template <int EPV>
__device__ __forceinline__ void unpack(const u32x4_t& w, float (&x)[EPV]) {
#pragma unroll
  for (int e = 0; e < EPV; ++e) x[e] = elem<EPV>(w, e);
}

// One wave per (row, chunk). DT: 0 = fp32 logits, 1 = bf16 logits.
template <int DT, int NV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 8))) void topk_partial_kernel(const void* __restrict__ logits,
                                                           int rows, int V, int K, int P,
                                                           float* __restrict__ part_val,
                                                           int32_t* __restrict__ part_idx,
                                                           float* __restrict__ part_ms) {
  constexpr int EPV = DT == 1 ? 8 : 4;
  // a 32-bit word holding -inf in every element
  constexpr uint32_t kNegInfWord = DT == 1 ? 0xFF80FF80u : 0xFF800000u;
  __shared__ u32x4_t stash_all[4][NV * 64];
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  u32x4_t* stash = stash_all[wid];
  const int g = blockIdx.x * 4 + wid;
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

  // Head / tail elements (fewer than EPV, or a row shorter than two vectors):
  // one element per lane in slot (u = 0, e = 0), through the same slow path.
  auto do_edge = [&](int64_t start, int len) __attribute__((always_inline)) {
    const float x = lane < len ? load_scalar<DT>(logits, start + lane) : -INFINITY;
    u32x4_t w = {0, 0, 0, 0};
    if constexpr (EPV == 8)
      w[0] = (__float_as_uint(x) >> 16) | 0xFF800000u;  // element 0 (exact), element 1 = -inf
    else
      w[0] = __float_as_uint(x);
    w[1] = w[2] = w[3] = kNegInfWord;
    u32x4_t wg[NV];
    wg[0] = w;
#pragma unroll
    for (int u = 1; u < NV; ++u) wg[u] = u32x4_t{kNegInfWord, kNegInfWord, kNegInfWord, kNegInfWord};
    group_lse<NV, EPV>(st, wg);
#pragma unroll
    for (int u = 0; u < NV; ++u) stash[u * 64 + lane] = wg[u];
    __builtin_amdgcn_wave_barrier();
    group_slow<NV, EPV, 1>(st, stash, (int)(start - rs), !seeded, K, lane);
    __builtin_amdgcn_wave_barrier();
    seeded = true;
  };

  bool head_pending = unit == 0 && head_len > 0;
  // Interior vectors [vb, ve), 64 * NV per iteration. Loads are unconditional
  // (indices clamped into the chunk) so all NV of an iteration issue back to
  // back, and the next iteration's loads are in flight while the current one
  // is consumed. Only the final partial iteration has invalid slots.
  auto load_group = [&](int64_t v, u32x4_t (&w)[NV]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      int64_t vi = v + u * 64 + lane;
      vi = vi < ve ? vi : ve - 1;
      w[u] = __builtin_nontemporal_load(vbase + vi);
    }
  };
  auto consume = [&](u32x4_t (&w)[NV], int64_t v) __attribute__((always_inline)) {
    if (v + 64 * NV > ve) {
      // last, partial iteration: slots past the chunk end read as -inf
#pragma unroll
      for (int u = 0; u < NV; ++u)
        if (v + u * 64 + lane >= ve) w[u] = u32x4_t{kNegInfWord, kNegInfWord, kNegInfWord, kNegInfWord};
    }
    const float lm = group_lse<NV, EPV>(st, w);
    if (!seeded || __any(lm > st.th_v)) {
#pragma unroll
      for (int u = 0; u < NV; ++u) stash[u * 64 + lane] = w[u];
      __builtin_amdgcn_wave_barrier();
      group_slow<NV, EPV, EPV>(st, stash, (int)(a0 - rs + v * EPV), !seeded, K, lane);
      __builtin_amdgcn_wave_barrier();
      seeded = true;
    }
    if (head_pending) {
      do_edge(rs, head_len);
      head_pending = false;
    }
  };
  if (vb < ve) {
    u32x4_t wa[NV], wb[NV];
    int64_t v = vb;
    load_group(v, wa);
    while (true) {
      const int64_t v1 = v + 64 * NV;
      if (v1 < ve) load_group(v1, wb);
      consume(wa, v);
      if (v1 >= ve) break;
      const int64_t v2 = v1 + 64 * NV;
      if (v2 < ve) load_group(v2, wa);
      consume(wb, v1);
      if (v2 >= ve) break;
      v = v2;
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
    // wave argmax of the heads by (value desc, index asc); the winner is the
    // lowest lane holding that key (keys are unique except exhausted lists)
    float bv = hv;
    int bi = hi;
    wave_argmax(bv, bi);
    const int bl = __ffsll((long long)__ballot(hv == bv && hi == bi)) - 1;
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
