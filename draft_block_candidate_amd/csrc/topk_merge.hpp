// Merge of a vocabulary row's chunk results (shared by the top-K merge kernel
// and the few-row node build, which merges its own row in place of that
// kernel): P lists of the K best (value, id) keys, each sorted by (value desc,
// id asc) with list p's ids all below list p + 1's, and P (reference max,
// sum of exp(x - max)) pairs. The result is the row's K best keys, lse =
// log sum exp, and logp = fl32(x - fl32(lse)) for each key.
#pragma once

#include "common.hpp"

namespace ll {

constexpr float kL2E = 1.4426950408889634f;
constexpr float kMInit = -1e30f;   // reference max before any finite value
constexpr int kInvalid = 0x7fffffff;

// K-step tournament over P sorted lists held in LDS (list p at sv/si + p K,
// ordered by (value desc, id asc), list p's ids all below list p + 1's):
// lane k < K receives the k-th best (value, id). Lane p < P walks list p; hp
// is its read position. Every step is straight-line (selects, a clamped LDS
// read in every lane).
__device__ __forceinline__ void tournament(const float* sv, const int* si, int P, int K, int lane,
                                           float& rv, int& ri) {
  const bool live = lane < P;
  const int lb = min(lane, P - 1) * K;
  float hv = live ? sv[lb] : -INFINITY;
  int hi = live ? si[lb] : kInvalid;
  int hp = 0;
  rv = -INFINITY;
  ri = kInvalid;
  const int width = P <= 16 ? 16 : (P <= 32 ? 32 : 64);   // lanes >= P hold -inf
  for (int k = 0; k < K; ++k) {
    // Winner by (value desc, id asc): among equal values the lowest lane
    // holds the lowest id, so a max plus the lowest lane of the ballot
    // decides it.
    const float bv = lanes_max(hv, width);
    const int bl = __ffsll((long long)__ballot(hv == bv)) - 1;
    const int bi = readlane_i(hi, bl);
    rv = lane == k ? bv : rv;
    ri = lane == k ? bi : ri;
    const bool adv = (lane == bl) & live;
    hp += adv ? 1 : 0;
    const float nv = sv[lb + min(hp, K - 1)];
    const int ni = si[lb + min(hp, K - 1)];
    const bool more = hp < K;
    hv = adv ? (more ? nv : -INFINITY) : hv;
    hi = adv ? (more ? ni : kInvalid) : hi;
  }
}

// One wave merges row `row`: entry k of list p at p * sp + row * sr + k
// (values and ids), its (max, sum) pair at 2 * (p * mp + row * mr). The P K
// entries are staged in the LDS scratch sv / si first (one memory round trip
// per 512 entries). Lane k < K receives the k-th best key in (rv, ri); M and S
// are the combined (max, sum) and the return value is lse = M + log S. Only
// this wave touches sv / si: the tournament's reads follow its own LDS
// writes, which one wave's LDS accesses see in issue order.
__device__ __forceinline__ float merge_row_lists(int row, int K, int P, int64_t sp, int64_t sr, int64_t mp,
                                                 int64_t mr, const float* __restrict__ part_val,
                                                 const int32_t* __restrict__ part_idx,
                                                 const float* __restrict__ part_ms, float* sv, int* si,
                                                 int lane, float& rv, int& ri, float& M, float& S) {
  const int64_t rbase = (int64_t)row * sr;
  const int n = P * K;
  // Eight entries per lane per batch, every load issued before the first
  // is used (indices clamped to the row, duplicates written twice with the
  // same value).
  for (int i0 = 0; i0 < n; i0 += 512) {
    float bv[8];
    int bi[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = min(i0 + j * 64 + lane, n - 1);
      int64_t a = rbase + i;         // lists of a row contiguous (sp == K)
      if (sp != K) {
        const int p = i / K;
        a = rbase + p * sp + (i - p * K);
      }
      bv[j] = part_val[a];
      bi[j] = part_idx[a];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = min(i0 + j * 64 + lane, n - 1);
      sv[i] = bv[j];
      si[i] = bi[j];
    }
  }
  const int pl = min(lane, P - 1);
  float m = part_ms[2 * (pl * mp + row * mr)];
  float s = part_ms[2 * (pl * mp + row * mr) + 1];
  if (lane >= P) {
    m = kMInit;
    s = 0.f;
  }
  M = wave_max(m);
  S = wave_sum(s * __builtin_amdgcn_exp2f((m - M) * kL2E));
  const float lse = M + logf(S);
  // the staged entries are complete before the tournament reads them
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  tournament(sv, si, P, K, lane, rv, ri);
  return lse;
}

}  // namespace ll
