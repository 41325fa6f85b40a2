// Fused log-partition + exact top-K over vocabulary rows (one HBM pass).
//
// What it computes (LiLiCorr paper, Section 3.2 and Appendix A "Serving";
// SGLang PR "[Spec] Add LiLiCorr", section "Why the custom kernels"): for each
// row, lse = log sum_v exp(x_v) and the K entries ordered by (x desc, v asc),
// with logp = fl32(x - fl32(lse)).
//
// Design for gfx950 (the PR's Triton kernel pre-selects whole tiles; here the
// unit of work is one wave64 streaming a contiguous chunk of a row):
//  * each lane issues NV 16-byte non-temporal buffer loads per group (64 lanes
//    read 1 KiB contiguous per load); the next group is always in flight
//    while the current one is consumed;
//  * the log-partition is a per-lane sum of exp(x - ref) against a
//    wave-uniform reference max that is raised only when a term exceeds 2^23,
//    so the common path per element is unpack, fma, v_exp_f32 and add;
//  * the same exponential terms gate the top-K: the largest term of each
//    lane's vector is compared with exp(threshold - ref), so the streaming
//    pass adds only a max3 per three terms and one compare per vector;
//  * the running top-K is a sorted list held one entry per lane (lane k holds
//    the k-th best key); the threshold is entry K-1. Groups that pass the gate
//    are scanned element position by element position (one ballot each) and
//    candidates are inserted on the full (value, id) key; insertions number
//    about K ln(n/K) for n streamed elements in random order;
//  * the list is seeded from the first group by a 64-lane bitonic sort of the
//    lanes' best elements, so it starts at a tight threshold;
//  * a row split over several chunks is merged by a second kernel (one wave
//    per row: a K-step tournament over the chunks' sorted lists plus the
//    log-sum-exp combination of the chunks' (max, sum) pairs; few-row lattice
//    heads do this merge inside the node build instead); a row that is one
//    chunk is written directly.
// Exactness: the gate can only let extra elements through (its slack covers
// the rounding of the exponential); every element that reaches the scan is
// decided on the full (value, id) key, and the top-K of a set under a total
// order does not depend on the order the elements are offered in.
#include <cmath>

#include "common.hpp"
#include "kernels.hpp"
#include "layout.hpp"
#include "topk_merge.hpp"

namespace ll {
namespace {

// A term exp(x - ref) above 2^23 (x more than ~15.9 above the reference)
// triggers a rebase of the reference to the group maximum.
constexpr float kRebase = 8388608.0f;
// The top-K gate compares exp(x - ref) with exp(threshold - ref) scaled down
// by this factor, so that rounding of the exponential (a few ulp) can only
// let extra elements through, never drop one.
constexpr float kGateSlack = 0.99998474f;   // 1 - 2^-16
// Buffer descriptor word 3 for raw (untyped) loads on gfx9-family targets.
constexpr int kBufferWord3 = 0x00020000;
// Cache-policy operand of a buffer load: non-temporal (streamed once).
constexpr int kLoadNonTemporal = 2;

// Non-short-circuit form, so lane-varying uses compile to selects rather
// than exec-mask branches.
__device__ __forceinline__ bool key_gt(float av, int ai, float bv, int bi) {
  return (av > bv) | ((av == bv) & (ai < bi));
}

struct State {
  float ref;        // wave-uniform reference max (kMInit until a finite value is seen)
  float nc;         // -ref * log2(e)
  float s;          // per lane: sum of exp(x - ref)
  float lv;         // list entry of this lane (lanes >= K hold -inf)
  int li;
  float th_v;       // wave-uniform threshold = list entry K-1
  int th_i;
  float p_th;       // wave-uniform gate: exp(th_v - ref) * kGateSlack
  bool seeded;
};

__device__ __forceinline__ float exp_term(float x, float nc) {
  return __builtin_amdgcn_exp2f(fmaf(x, kL2E, nc));
}

__device__ __forceinline__ void update_gate(State& st) {
  st.p_th = exp_term(st.th_v, st.nc) * kGateSlack;
}

__device__ __forceinline__ void list_insert(State& st, float cv, int ci, int K, int lane) {
  const bool better = (lane < K) && key_gt(st.lv, st.li, cv, ci);
  const int pos = __popcll(__ballot(better));
  // wave_shr:1 (DPP): every lane receives the entry of the lane below it
  const float upv = dpp_f<0x138, 0xf>(st.lv, st.lv);
  const int upi = dpp_i<0x138, 0xf>(st.li, st.li);
  const bool here = lane == pos;
  const bool shift = (lane > pos) & (lane < K);
  st.lv = here ? cv : (shift ? upv : st.lv);
  st.li = here ? ci : (shift ? upi : st.li);
  st.th_v = readlane_f(st.lv, K - 1);
  st.th_i = readlane_i(st.li, K - 1);
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

// exp(x - ref) summed over a group of NV packed vectors per lane (-inf
// padding words add nothing); pm[u] receives the lane's largest term of
// vector slot u, t the lane's sum.
template <int NV, int EPV>
__device__ __forceinline__ void lse_pass(float nc, const u32x4_t (&w)[NV], float& t, float (&pm)[NV]) {
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    float a = exp_term(elem<EPV>(w[u], 0), nc);
    float m = a;
#pragma unroll
    for (int e = 1; e < EPV; ++e) {
      const float p = exp_term(elem<EPV>(w[u], e), nc);
      a += p;
      m = fmaxf(m, p);
    }
    t = u == 0 ? a : t + a;
    pm[u] = m;
  }
}

// A copy of a group that the compiler cannot relate to the original, so that
// the rarely taken paths unpack their own elements instead of keeping the
// streaming pass's unpacked values alive in registers.
template <int NV>
__device__ __forceinline__ void opaque_copy(const u32x4_t (&w)[NV], u32x4_t (&c)[NV]) {
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    c[u] = w[u];
    asm volatile("" : "+v"(c[u]));
  }
}

// Raise the reference to the group maximum and recompute the group's terms.
template <int NV, int EPV>
__device__ __forceinline__ void rebase(State& st, const u32x4_t (&w0)[NV], float& t, float (&pm)[NV]) {
  u32x4_t w[NV];
  opaque_copy<NV>(w0, w);
  float m = -INFINITY;
#pragma unroll
  for (int u = 0; u < NV; ++u)
#pragma unroll
    for (int e = 0; e < EPV; ++e) m = fmaxf(m, elem<EPV>(w[u], e));
  const float nm = fmaxf(st.ref, wave_max(m));
  if (nm > st.ref) {
    st.s *= __builtin_amdgcn_exp2f((st.ref - nm) * kL2E);
    st.ref = nm;
    st.nc = -nm * kL2E;
    update_gate(st);
  }
  lse_pass<NV, EPV>(st.nc, w, t, pm);
}

// Seed the list from a group: the 64 lanes' best elements, bitonic-sorted
// (descending key; lane exchanges by DPP and row-swap permutes, no LDS); the
// first K become the list. Returns this lane's best id
// (to be skipped by the candidate scan: inside the list it would be a
// duplicate, outside it fails the strict key test anyway).
template <int NV, int EPV, int LS>
__device__ __forceinline__ int seed_list(State& st, const u32x4_t (&w)[NV], int base, int K, int lane) {
  float bv = -INFINITY;
  int bi = kInvalid;
#pragma unroll
  for (int u = 0; u < NV; ++u)
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      // a lane's ids increase with (u, e): strict > keeps the lowest id of a tie
      const float x = elem<EPV>(w[u], e);
      const bool better = x > bv;
      bv = better ? x : bv;
      bi = better ? base + (u * 64 + lane) * LS + e : bi;
    }
  float sv = bv;
  int si = bi;
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const float ov = xor_lane(sv, j, lane);
      const int oi = xor_lane(si, j, lane);
      const bool keep_better = ((lane & j) == 0) == ((lane & k) == 0);
      const bool swap = keep_better != key_gt(sv, si, ov, oi);
      sv = swap ? ov : sv;
      si = swap ? oi : si;
    }
  }
  st.lv = lane < K ? sv : -INFINITY;
  st.li = lane < K ? si : kInvalid;
  st.th_v = readlane_f(st.lv, K - 1);
  st.th_i = readlane_i(st.li, K - 1);
  st.seeded = true;
  return bi;
}

// Top-K update from a group whose terms passed the gate somewhere. For each
// vector slot that may hold an element >= threshold, each element position e
// is tested in all lanes at once; the lanes that pass are visited one at a
// time and decided on the full (value, id) key.
// Element (u, e) of lane l has row-local id base + (u * 64 + l) * LS + e.
template <int NV, int EPV, int LS>
__device__ __forceinline__ void topk_pass(State& st, const u32x4_t (&w0)[NV], const float (&pm)[NV],
                                          int base, int K, int lane) {
  u32x4_t w[NV];
  opaque_copy<NV>(w0, w);
  int excl = -1;
  const bool seeding = !st.seeded;
  if (seeding) {
    excl = seed_list<NV, EPV, LS>(st, w, base, K, lane);
    update_gate(st);
  }
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    if (seeding) {
      // right after seeding every slot holding a seed passes the exp gate, so
      // count the elements that can still enter instead
      const float th = fmaxf(st.th_v, -3.402823466e38f);
      int c = 0;
#pragma unroll
      for (int e = 0; e < EPV; ++e)
        c += (elem<EPV>(w[u], e) >= th) & (base + (u * 64 + lane) * LS + e != excl);
      if (!__any(c > 0)) continue;
    } else if (!__any(pm[u] >= st.p_th)) {
      continue;
    }
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      const float x = elem<EPV>(w[u], e);
      const int id = base + (u * 64 + lane) * LS + e;
      // logits are finite: -inf elements are padding and never enter; an
      // element already placed by the seeding is dropped here
      uint64_t mask = __ballot((x >= fmaxf(st.th_v, -3.402823466e38f)) & (id != excl));
      while (mask) {
        const int l = __ffsll((long long)mask) - 1;
        mask &= mask - 1;
        const float cv = readlane_f(x, l);
        const int ci = base + (u * 64 + l) * LS + e;
        if (key_gt(cv, ci, st.th_v, st.th_i)) list_insert(st, cv, ci, K, lane);
      }
    }
  }
  update_gate(st);
}

// One group: log-partition terms, then the gated top-K update.
template <int NV, int EPV, int LS>
__device__ __forceinline__ void consume_group(State& st, const u32x4_t (&w)[NV], int base, int K,
                                              int lane) {
  float t, pm[NV];
  lse_pass<NV, EPV>(st.nc, w, t, pm);
  float pmax = pm[0];
#pragma unroll
  for (int u = 1; u < NV; ++u) pmax = fmaxf(pmax, pm[u]);
  if (__any(pmax > kRebase)) {
    rebase<NV, EPV>(st, w, t, pm);
    pmax = pm[0];
#pragma unroll
    for (int u = 1; u < NV; ++u) pmax = fmaxf(pmax, pm[u]);
  }
  st.s += t;
  if (!st.seeded || __any(pmax >= st.p_th)) topk_pass<NV, EPV, LS>(st, w, pm, base, K, lane);
}

// One wave streams chunk `unit` of P of a row: its sorted top-K list (one
// entry per lane) and its (reference max, per-lane sum) state.
// DT: 0 = fp32 logits, 1 = bf16 logits.
template <int DT, int NV>
__device__ __forceinline__ State stream_chunk(const void* __restrict__ logits, int row, int V, int K,
                                              int P, int unit, int lane) {
  constexpr int EPV = DT == 1 ? 8 : 4;
  // a 32-bit word holding -inf in every element
  constexpr uint32_t kNegInfWord = DT == 1 ? 0xFF80FF80u : 0xFF800000u;
  const int64_t rs = (int64_t)row * V, re = rs + V;
  int64_t a0 = (rs + EPV - 1) / EPV * EPV, a1 = re / EPV * EPV;
  if (a1 <= a0) {  // no whole aligned vector: the row is all head
    a0 = re;
    a1 = re;
  }
  // vector indices relative to the row's first aligned vector (< 2^31)
  const int nv = (int)((a1 - a0) / EPV);
  const int cv = (nv + P - 1) / P;
  const int vb = min(nv, unit * cv), ve = min(nv, vb + cv);
  const u32x4_t* vbase = (const u32x4_t*)logits + a0 / EPV;
  const int head_len = (int)(a0 - rs), tail_len = (int)(re - a1);

  State st;
  st.ref = kMInit;
  st.nc = -kMInit * kL2E;
  st.s = 0.f;
  st.lv = -INFINITY;
  st.li = kInvalid;
  st.th_v = -INFINITY;
  st.th_i = kInvalid;
  st.p_th = 0.f;
  st.seeded = false;

  // Interior vectors [vb, ve), 64 * NV per group, read with buffer loads
  // through a per-group descriptor whose range ends at the chunk end: a load
  // past it returns zero without touching memory, so every load is issued
  // unconditionally, the loop body is straight-line and the next group's
  // loads stay in flight while the current group is consumed. Only the final
  // partial group has padding slots (set to -inf below).
  auto load_group = [&](int v, u32x4_t (&w)[NV]) __attribute__((always_inline)) {
    const int bytes = max(0, ve - v) * 16;
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + v), 0, bytes, kBufferWord3);
#pragma unroll
    for (int u = 0; u < NV; ++u)
      w[u] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (u * 64 + lane) * 16, 0, kLoadNonTemporal);
  };
  auto consume = [&](u32x4_t (&w)[NV], int v) __attribute__((always_inline)) {
    if (v + 64 * NV > ve) {
#pragma unroll
      for (int u = 0; u < NV; ++u)
        if (v + u * 64 + lane >= ve) w[u] = u32x4_t{kNegInfWord, kNegInfWord, kNegInfWord, kNegInfWord};
    }
    consume_group<NV, EPV, EPV>(st, w, (int)(a0 - rs) + v * EPV, K, lane);
  };
  if (vb < ve) {
    u32x4_t wa[NV], wb[NV];
    int v = vb;
    load_group(v, wa);
    while (true) {
      load_group(v + 64 * NV, wb);
      consume(wa, v);
      if (v + 64 * NV >= ve) break;
      load_group(v + 128 * NV, wa);
      consume(wb, v + 64 * NV);
      if (v + 128 * NV >= ve) break;
      v += 128 * NV;
    }
  }

  // Head / tail elements (fewer than EPV each, or a row too short for an
  // aligned vector): one element per lane, as a one-vector group whose
  // element 0 is the lane's element.
  auto do_edge = [&](int64_t start, int len) __attribute__((always_inline)) {
    const float x = lane < len ? load_scalar<DT>(logits, start + lane) : -INFINITY;
    u32x4_t w1[1];
    w1[0] = u32x4_t{kNegInfWord, kNegInfWord, kNegInfWord, kNegInfWord};
    if constexpr (EPV == 8)
      w1[0][0] = (__float_as_uint(x) >> 16) | 0xFF800000u;  // element 0 exact, element 1 = -inf
    else
      w1[0][0] = __float_as_uint(x);
    consume_group<1, EPV, 1>(st, w1, (int)(start - rs), K, lane);
  };
  if (unit == 0 && head_len > 0) do_edge(rs, head_len);
  if (unit == P - 1 && tail_len > 0) do_edge(a1, tail_len);
  return st;
}

// One wave per (row, chunk).
template <int DT, int NV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 8))) void topk_partial_kernel(const void* __restrict__ logits,
                                                           int rows, int V, int K, int P,
                                                           int id_offset, int final_out,
                                                           float* __restrict__ part_val,
                                                           int32_t* __restrict__ part_idx,
                                                           float* __restrict__ part_ms,
                                                           int32_t* __restrict__ topk_idx,
                                                           float* __restrict__ topk_logp,
                                                           float* __restrict__ lse_out) {
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = blockIdx.x * 4 + wid;
  const int row = g / P, unit = g - (g / P) * P;
  if (row >= rows) return;
  const State st = stream_chunk<DT, NV>(logits, row, V, K, P, unit, lane);
  const float S = wave_sum(st.s);
  if (P == 1 && final_out) {
    // the row is one chunk: its sorted list is the answer
    const float lse = st.ref + logf(S);
    if (lane < K) {
      topk_idx[(int64_t)row * K + lane] = st.li;
      topk_logp[(int64_t)row * K + lane] = __fsub_rn(st.lv, lse);
    }
    if (lse_out != nullptr && lane == 0) lse_out[row] = lse;
    return;
  }
  // Chunk outputs: sorted list (ids shifted to the caller's numbering) and
  // (reference max, sum) of the wave.
  const int64_t o = (int64_t)row * P + unit;
  if (lane < K) {
    part_val[o * K + lane] = st.lv;
    part_idx[o * K + lane] = st.li == kInvalid ? kInvalid : st.li + id_offset;
  }
  if (lane == 0) {
    part_ms[2 * o] = st.ref;
    part_ms[2 * o + 1] = S;
  }
}

// One wave per row: combine the P chunk lists (tournament) and (max, sum)
// pairs. The row's P * K partial entries are staged in LDS first, so each of
// the K tournament steps reads the winner's next entry from LDS. Entry k of
// list p of a row sits at p * sp + row * sr + k (values and ids) and its
// (max, sum) pair at 2 * (p * mp + row * mr): the chunks of one row are
// [rows, P, K]; the shards of a split vocabulary are [P, rows, K]. Lists must
// be in ascending order of their id ranges. PARTIAL_OUT writes the merged
// list and the combined (max, sum) pair instead of (ids, logp, lse).
template <bool PARTIAL_OUT>
__global__ __launch_bounds__(64) void topk_merge_kernel(int rows, int K, int P, int64_t sp, int64_t sr,
                                                        int64_t mp, int64_t mr,
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
  float rv, M, S;
  int ri;
  const float lse = merge_row_lists(row, K, P, sp, sr, mp, mr, part_val, part_idx, part_ms, sv, si, lane,
                                    rv, ri, M, S);
  if (PARTIAL_OUT) {
    // topk_logp receives the merged values, lse_out the (max, sum) pair
    if (lane < K) {
      topk_idx[(int64_t)row * K + lane] = ri;
      topk_logp[(int64_t)row * K + lane] = rv;
    }
    if (lane == 0) {
      lse_out[2 * (int64_t)row] = M;
      lse_out[2 * (int64_t)row + 1] = S;
    }
    return;
  }
  if (lane < K) {
    topk_idx[(int64_t)row * K + lane] = ri;
    topk_logp[(int64_t)row * K + lane] = __fsub_rn(rv, lse);
  }
  if (lse_out != nullptr && lane == 0) lse_out[row] = lse;
}

}  // namespace

namespace {

hipError_t launch_partial(const void* logits, int rows, int V, int K, int dtype, int P, int id_offset,
                          int final_out, float* part_val, int32_t* part_idx, float* part_ms,
                          int32_t* topk_idx, float* topk_logp, float* lse, hipStream_t stream) {
  const int64_t waves = (int64_t)rows * P;
  const unsigned blocks = (unsigned)((waves + 3) / 4);
  if (dtype == 1)
    hipLaunchKernelGGL((topk_partial_kernel<1, 4>), dim3(blocks), dim3(256), 0, stream, logits,
                       rows, V, K, P, id_offset, final_out, part_val, part_idx, part_ms, topk_idx,
                       topk_logp, lse);
  else
    hipLaunchKernelGGL((topk_partial_kernel<0, 4>), dim3(blocks), dim3(256), 0, stream, logits,
                       rows, V, K, P, id_offset, final_out, part_val, part_idx, part_ms, topk_idx,
                       topk_logp, lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk_lse(const void* logits, int rows, int V, int K, int dtype, float* part_val,
                           int32_t* part_idx, float* part_ms, int32_t* topk_idx, float* topk_logp,
                           float* lse, hipStream_t stream, bool merge) {
  const int P = topk_chunks_per_row(rows, V);
  hipError_t e = launch_partial(logits, rows, V, K, dtype, P, 0, 1, part_val, part_idx, part_ms,
                                topk_idx, topk_logp, lse, stream);
  if (e != hipSuccess || P == 1 || !merge) return e;
  hipLaunchKernelGGL(topk_merge_kernel<false>, dim3((unsigned)rows), dim3(64), (size_t)P * K * 8,
                     stream, rows, K, P, (int64_t)K, (int64_t)P * K, (int64_t)1, (int64_t)P,
                     part_val, part_idx, part_ms, topk_idx, topk_logp, lse);
  return hipGetLastError();
}

hipError_t launch_topk_shard(const void* logits, int rows, int V, int K, int dtype, int id_offset,
                             float* part_val, int32_t* part_idx, float* part_ms, float* out_val,
                             int32_t* out_idx, float* out_ms, hipStream_t stream) {
  const int P = topk_chunks_per_row(rows, V);
  if (P == 1)   // one chunk per row: its list and (max, sum) are the shard's output
    return launch_partial(logits, rows, V, K, dtype, 1, id_offset, 0, out_val, out_idx, out_ms,
                          nullptr, nullptr, nullptr, stream);
  hipError_t e = launch_partial(logits, rows, V, K, dtype, P, id_offset, 0, part_val, part_idx,
                                part_ms, nullptr, nullptr, nullptr, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_merge_kernel<true>, dim3((unsigned)rows), dim3(64), (size_t)P * K * 8,
                     stream, rows, K, P, (int64_t)K, (int64_t)P * K, (int64_t)1, (int64_t)P,
                     part_val, part_idx, part_ms, out_idx, out_val, out_ms);
  return hipGetLastError();
}

hipError_t launch_topk_merge_shards(int G, int rows, int K, const float* val, const int32_t* idx,
                                    const float* ms, int32_t* topk_idx, float* topk_logp,
                                    float* lse, hipStream_t stream) {
  hipLaunchKernelGGL(topk_merge_kernel<false>, dim3((unsigned)rows), dim3(64), (size_t)G * K * 8,
                     stream, rows, K, G, (int64_t)rows * K, (int64_t)K, (int64_t)rows, (int64_t)1,
                     val, idx, ms, topk_idx, topk_logp, lse);
  return hipGetLastError();
}

}  // namespace ll
