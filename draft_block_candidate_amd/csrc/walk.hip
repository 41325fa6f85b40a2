// Pair scores and the commit rules.
//
// Pair scores (LiLiCorr paper, Eq. (1) and Section 3.5): for every adjacent
// slot pair, cos_s = out_{s-1} . in_s^T over unit vectors, one K x K product
// per pair. One wave per pair, 16 x 16 MFMA tiles over d_e.
//
// Greedy commit (Eq. (8); ties to the lower index as in the SGLang PR,
// "Why the custom kernels"): one wave per block, lane j scores candidate j.
// Only the walk is sequential, over slots.
//
// Exact best path (Appendix E, Eq. (12)) and sampled commit (SGLang PR,
// "Sampling the committed path (opt-in)"): further rules of the fused kernel,
// with the same per-step score z_s(i, j) = fl32(logp[s][j] + fl32(alpha *
// cos_s[i][j])).
#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace ll {
namespace {

// One K x K cosine matrix (rows of o against rows of in, d_e wide) by one
// wave, 16 x 16 MFMA tiles; emit(ra, b, value) receives every in-range entry.
// Rows past K are clamped to row K - 1 (their results are never emitted), so
// every load is unconditional and a 256-wide slice of d is loaded ahead of
// its MFMAs (conditional loads would be serialised).
// Only columns d0 .. d1 - 1 of the rows (row stride de) enter the sums.
// d0 and d1 must be wave-uniform values the compiler knows to be uniform
// (kernel arguments, readfirstlane results): an MFMA runs on every lane
// whatever the exec mask, so the guards below have to compile to branches,
// not to exec masks around unloaded fragments.
template <typename Emit>
__device__ __forceinline__ void pair_matrix(const uint16_t* __restrict__ o,
                                            const uint16_t* __restrict__ in, int K, int de,
                                            int d0, int d1, int lane, Emit emit) {
  const int g = lane >> 4, c = lane & 15;
  const int tiles = (K + 15) / 16;
  for (int at = 0; at < tiles; ++at)
    for (int bt = 0; bt < tiles; ++bt) {
      const int a = min(at * 16 + c, K - 1), b = min(bt * 16 + c, K - 1);
      const uint16_t* ar = o + (int64_t)a * de + 8 * g;
      const uint16_t* br = in + (int64_t)b * de + 8 * g;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      for (int k0 = d0; k0 < d1; k0 += 256) {
        u32x4_t af[8], bf[8];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
          if (k0 + ks * 32 < d1) {
            af[ks] = *(const u32x4_t*)(ar + k0 + ks * 32);
            bf[ks] = *(const u32x4_t*)(br + k0 + ks * 32);
          }
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
          if (k0 + ks * 32 < d1) acc = mfma16(af[ks], bf[ks], acc);
      }
      const int bc = bt * 16 + c;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ra = at * 16 + 4 * g + i;
        if (ra < K && bc < K) emit(ra, bc, acc[i]);
      }
    }
}

__global__ __launch_bounds__(256) void pair_scores_kernel(const uint16_t* __restrict__ outv,
                                                          const uint16_t* __restrict__ inv, int N,
                                                          int B, int K, int de,
                                                          float* __restrict__ cos) {
  const int lane = threadIdx.x & 63;
  const int64_t pair = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (pair >= (int64_t)N * (B - 1)) return;
  const int64_t n = pair / (B - 1);
  const int s = (int)(pair - n * (B - 1)) + 1;
  const uint16_t* o = outv + ((n * B + s - 1) * K) * (int64_t)de;
  const uint16_t* in = inv + ((n * B + s) * K) * (int64_t)de;
  float* dst = cos + pair * K * K;
  pair_matrix(o, in, K, de, 0, de, lane, [&](int ra, int b, float v) { dst[ra * K + b] = v; });
}

// Wide vectors (d_e of 512 and more), where one workgroup per block would
// stream every pair's rows through few waves: one wave per (pair, 256-wide
// slice of d_e), each writing its partial K x K matrix to
// part[(slice N (B-1) + pair) K K ..]; the walk kernel adds the slices in
// slice order.
__global__ __launch_bounds__(256) void pair_slices_kernel(const uint16_t* __restrict__ outv,
                                                          const uint16_t* __restrict__ inv, int N,
                                                          int B, int K, int de, int slices,
                                                          float* __restrict__ part) {
  const int lane = threadIdx.x & 63;
  const int64_t pairs = (int64_t)N * (B - 1);
  // wave-uniform, so the slice bounds below are scalar and their guards branch
  const int64_t item = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (item >= pairs * slices) return;
  const int sl = (int)(item / pairs);
  const int64_t pair = item - sl * pairs;
  const int64_t n = pair / (B - 1);
  const int s = (int)(pair - n * (B - 1)) + 1;
  const uint16_t* o = outv + ((n * B + s - 1) * K) * (int64_t)de;
  const uint16_t* in = inv + ((n * B + s) * K) * (int64_t)de;
  float* dst = part + item * K * K;
  pair_matrix(o, in, K, de, 256 * sl, min(de, 256 * sl + 256), lane,
              [&](int ra, int b, float v) { dst[ra * K + b] = v; });
}

__global__ __launch_bounds__(256) void greedy_walk_kernel(
    const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_logp,
    const float* __restrict__ cos, int N, int B, int K, float alpha, int use_logp,
    int32_t* __restrict__ out_tokens, float* __restrict__ score, float* __restrict__ gap) {
  const int lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const int64_t r0 = n * B;
  // as in the fused kernel: winner by max then lowest lane of the ballot;
  // step s's results are kept in lane s and written after the loop
  const int width = K <= 16 ? 16 : (K <= 32 ? 32 : 64);
  int choice = 0;
  float my_score = topk_logp[r0 * K], my_gap = 0.f;
  int cprev = 0;
  for (int s = 1; s < B; ++s) {
    float z = -INFINITY;
    if (lane < K) {
      const float cs = cos[((n * (B - 1) + s - 1) * K + cprev) * K + lane];
      const float term = mul_rn(alpha, cs);
      z = use_logp ? add_rn(topk_logp[(r0 + s) * K + lane], term) : term;
    }
    const float bz = lanes_max(z, width);
    int bl = __ffsll((long long)__ballot(z == bz)) - 1;
    if (bl < 0 || bl >= K) bl = 0;  // only reachable with non-finite scores; keeps every index in range
    const float second = gap ? wave_max(lane == bl ? -INFINITY : z) : 0.f;
    choice = lane == s ? bl : choice;
    my_score = lane == s ? bz : my_score;
    my_gap = lane == s ? (K > 1 ? sub_rn(bz, second) : 0.f) : my_gap;
    cprev = bl;
  }
  if (lane < B) {
    out_tokens[r0 + lane] = topk_idx[(r0 + lane) * K + choice];
    if (score) score[r0 + lane] = my_score;
    if (gap) gap[r0 + lane] = my_gap;
  }
}

// Pair scores + commit for the rerank path: one workgroup per block. The
// eight waves compute the block's B-1 K x K cosine matrices into LDS (and to
// global memory when requested), or copy them from cos_in when the scores are
// given. Then, by rule:
//   RULE_GREEDY  tabulate the walk's decision for every (slot, previous
//                candidate) pair; the sequential part is one LDS lookup per slot
//   RULE_EXACT   the highest-scoring path (LiLiCorr paper, Appendix E, Eq. (12))
//                by dynamic programming in wave 0, then the predecessor trace-back
//   RULE_SAMPLE  (SGLang PR, opt-in sampled commit) tabulate, for every (slot,
//                previous candidate) pair, the draw from softmax(z / T) with the
//                slot's input uniform, then walk the table; blocks with T <= 0
//                take the greedy table (the greedy path, bit for bit)
template <int RULE>
__global__ __launch_bounds__(512) void scores_walk_kernel(
    const uint16_t* __restrict__ outv, const uint16_t* __restrict__ inv,
    const float* __restrict__ cos_in, int cos_slices, int64_t slice_stride,
    const int32_t* __restrict__ topk_idx,
    const float* __restrict__ topk_logp, int B, int K, int de, float alpha, int use_logp,
    const float* __restrict__ temperature, const float* __restrict__ uniforms,
    float* __restrict__ proposal, float* __restrict__ cos_out, int32_t* __restrict__ out_tokens,
    float* __restrict__ score, float* __restrict__ gap) {
  extern __shared__ float sm[];
  const int KK = K * K;
  float* s_cos = sm;                                // [(B-1) K K]
  float* s_logp = sm + (B - 1) * KK;                // [B K]
  int* s_idx = (int*)(s_logp + B * K);              // [B K]
  int* s_tc = s_idx + B * K;                        // [(B-1) K] table: choice (EXACT: predecessor)
  float* s_tz = (float*)(s_tc + (B - 1) * K);       // [(B-1) K] its score (SAMPLE: the row max)
  float* s_tg = s_tz + (B - 1) * K;                 // [(B-1) K] its gap (SAMPLE: the row's exp sum)
  int* s_path = (int*)(s_tg + (B - 1) * K);         // [B] committed candidates
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t n = blockIdx.x;
  const int64_t base = n * B * K;
  for (int i = tid; i < B * K; i += blockDim.x) {
    s_logp[i] = topk_logp[base + i];
    s_idx[i] = topk_idx[base + i];
  }
  const int nw = blockDim.x >> 6;
  if (cos_in) {
    // one matrix per pair, or the partial sums of its d_e slices (added in
    // slice order)
    const float* src = cos_in + n * (int64_t)(B - 1) * KK;
    for (int i = tid; i < (B - 1) * KK; i += blockDim.x) {
      float v = src[i];
      for (int sl = 1; sl < cos_slices; ++sl) v += src[sl * slice_stride + i];
      s_cos[i] = v;
      if (cos_out) cos_out[n * (int64_t)(B - 1) * KK + i] = v;
    }
  } else {
    for (int p = wave; p < B - 1; p += nw) {
      const uint16_t* o = outv + (base + (int64_t)p * K) * de;
      const uint16_t* in = inv + (base + (int64_t)(p + 1) * K) * de;
      pair_matrix(o, in, K, de, 0, de, lane, [&](int ra, int b, float v) {
        s_cos[p * KK + ra * K + b] = v;
        if (cos_out) cos_out[(n * (B - 1) + p) * KK + ra * K + b] = v;
      });
    }
  }
  __syncthreads();
  // z_s(i, j): the walk's own arithmetic (fl32, each step rounded, never fused)
  auto zval = [&](int s, int i, int j) {
    const float term = mul_rn(alpha, s_cos[(s - 1) * KK + i * K + j]);
    return use_logp ? add_rn(s_logp[s * K + j], term) : term;
  };
  const float T = RULE == RULE_SAMPLE ? temperature[n] : 0.f;
  const bool draw = RULE == RULE_SAMPLE && T > 0.f;   // uniform over the workgroup
  const float inv_t = draw ? 1.0f / T : 0.f;
  const int NE = (B - 1) * K;
  if (RULE == RULE_GREEDY || (RULE == RULE_SAMPLE && !draw)) {
    // Walk table: for every slot s >= 1 and every candidate c of slot s - 1,
    // the choice the walk makes at s when it stands on c, with its score and
    // the gap to the runner-up. Entries are independent, so all threads build
    // them; the largest score wins and the lowest index breaks a tie.
    for (int e = tid; e < NE; e += blockDim.x) {
      const int s = e / K + 1, cp = e - (s - 1) * K;
      const float* crow = s_cos + (s - 1) * KK + cp * K;
      const float* lrow = s_logp + s * K;
      float best = -INFINITY, second = -INFINITY;
      int bj = K;
      // neighbouring entries start their scans at different j (their rows are
      // K floats apart, so equal j would hit a few LDS banks); the comparison
      // is on the full (score, lower index) key, so the order does not matter
      // (eight at a time, all eight pairs of reads issued before any is used)
      for (int jj0 = 0; jj0 < K; jj0 += 8) {
        float cv[8], lv[8];
        int jv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          int j = cp + min(jj0 + u, K - 1);
          j = j >= K ? j - K : j;
          jv[u] = j;
          cv[u] = crow[j];
          lv[u] = lrow[j];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float term = mul_rn(alpha, cv[u]);
          const float z = use_logp ? add_rn(lv[u], term) : term;
          const int j = jv[u];
          const bool better = (jj0 + u < K) & ((z > best) | ((z == best) & (j < bj)));
          second = (jj0 + u < K) ? (better ? best : fmaxf(second, z)) : second;
          best = better ? z : best;
          bj = better ? j : bj;
        }
      }
      s_tc[e] = bj < K ? bj : 0;   // bj == K only if every score is NaN; keeps the walk in range
      s_tz[e] = best;
      s_tg[e] = K > 1 ? sub_rn(best, second) : 0.f;
    }
  } else if (draw) {
    // Sample table: the row maximum m, the float32 sum S of e_j =
    // exp((z_j - m) / T) in ascending j, and the draw: the number of
    // cumulative sums C_j <= u_s * S (the smallest j whose cumulative
    // probability exceeds u_s), at most K - 1.
    for (int e = tid; e < NE; e += blockDim.x) {
      const int s = e / K + 1, cp = e - (s - 1) * K;
      float m = -INFINITY;
      for (int j = 0; j < K; ++j) m = fmaxf(m, zval(s, cp, j));
      float S = 0.f;
      for (int j = 0; j < K; ++j) S = add_rn(S, __expf(mul_rn(sub_rn(zval(s, cp, j), m), inv_t)));
      const float target = mul_rn(uniforms[n * B + s], S);
      float C = 0.f;
      int cnt = 0;
      for (int j = 0; j < K; ++j) {
        C = add_rn(C, __expf(mul_rn(sub_rn(zval(s, cp, j), m), inv_t)));
        cnt += C <= target ? 1 : 0;
      }
      s_tc[e] = min(cnt, K - 1);
      s_tz[e] = m;
      s_tg[e] = S;
    }
  }
  __syncthreads();
  if (wave == 0) {
    const int64_t r0 = n * B;
    int choice = 0;
    float my_score = s_logp[0], my_gap = 0.f;
    if (RULE == RULE_EXACT && K <= 8) {
      // K <= 8: every (predecessor i, candidate j) pair of a slot in its own
      // lane of an 8 x 8 grid. The lane layout alternates between slots so
      // that each slot's totals are already where the next slot reads them:
      //   layout A (odd s):  j = lane >> 3, i = lane & 7; the maximum over i
      //                      within each 8-lane group leaves G_s(lane >> 3);
      //   layout B (even s): i = lane >> 3, j = lane & 7; the maximum over i
      //                      across the eight groups leaves G_s(lane & 7),
      // and G_1(j) = z_1(0, j) starts as if made by layout A. Candidates are
      // fl32(G_{s-1}(i) + z_s(i, j)) (left-to-right sums); the lowest i among
      // equal maxima is the predecessor of j, as in the scan below.
      const int hi = lane >> 3, lo = lane & 7;
      float G = (B > 1 && hi < K) ? zval(1, 0, hi) : -INFINITY;
      int hlo = 0, hhi = 0;   // lane s: the ballot of slot s (B <= 64)
      // z operands of slot s in layout ODD (loaded one slot ahead)
      auto zload = [&](auto odd_tag, int s, float& c, float& lp) {
        constexpr bool ODD = decltype(odd_tag)::value;
        const int i = ODD ? lo : hi, j = ODD ? hi : lo;
        c = s_cos[(s - 1) * KK + min(i, K - 1) * K + min(j, K - 1)];
        lp = s_logp[s * K + min(j, K - 1)];
      };
      // one slot of the program in layout ODD, from its loaded operands
      auto step = [&](auto odd_tag, int s, float cc, float lc) {
        constexpr bool ODD = decltype(odd_tag)::value;
        const int i = ODD ? lo : hi, j = ODD ? hi : lo;
        const float term = mul_rn(alpha, cc);
        const float z = use_logp ? add_rn(lc, term) : term;
        const float cand = (i < K && j < K) ? add_rn(G, z) : -INFINITY;
        int key = fkey(cand);
        if (ODD) {
          // within each 8-lane group: the two quad permutes, then lane k
          // against lane 7 - k (row_half_mirror) joins the two quads
          key = max(key, xor_lane(key, 1, lane));
          key = max(key, xor_lane(key, 2, lane));
          key = max(key, __builtin_amdgcn_update_dpp(INT_MIN, key, 0x141, 0xf, 0xf, false));
        } else {
          // across the eight groups: lane k against k + 8 within its row
          // (row_ror:8), then the two row swaps
          key = max(key, __builtin_amdgcn_update_dpp(INT_MIN, key, 0x128, 0xf, 0xf, false));
          key = max(key, xor_lane(key, 16, lane));
          key = max(key, xor_lane(key, 32, lane));
        }
        G = fkey_inv(key);
        // lowest i reaching the maximum: from the ballot, in every lane of
        // the group; one lane per candidate stores it as slot s's byte j
        // the lanes that reach their candidate's maximum: slot s's ballot,
        // kept in lane s of (hlo, hhi); the trace-back reads the lowest
        // predecessor of its candidate from it
        const uint64_t hit = __ballot(cand == G && i < K);
        hlo = lane == s ? (int)(uint32_t)hit : hlo;
        hhi = lane == s ? (int)(uint32_t)(hit >> 32) : hhi;
      };
      using Even = std::integral_constant<bool, false>;
      using Odd = std::integral_constant<bool, true>;
      // slots in pairs (even s in layout B, odd s + 1 in layout A)
      float ce = 0.f, le = 0.f, co = 0.f, lo_ = 0.f;
      if (B > 2) zload(Even{}, 2, ce, le);
      for (int s = 2; s < B; s += 2) {
        if (s + 1 < B) zload(Odd{}, s + 1, co, lo_);
        step(Even{}, s, ce, le);
        if (s + 1 < B) {
          if (s + 2 < B) zload(Even{}, s + 2, ce, le);
          step(Odd{}, s + 1, co, lo_);
        }
      }
      if (B > 1) {
        // best final candidate (lowest index on a tie), then the trace-back,
        // scalar: slot s's ballot from lane s; in layout A (odd s) candidate
        // c's lanes are 8c .. 8c + 7 with i = lane - 8c, in layout B (even s)
        // lanes c, c + 8, .. with i = lane / 8; the lowest set lane is the
        // lowest predecessor
        float gv = G;
        int c = ((B - 1) & 1) || B == 2 ? hi : lo;    // the candidate this lane's total belongs to
        gv = c < K ? gv : -INFINITY;
        wave_argmax(gv, c);
        c = c < K ? c : 0;
        choice = lane == B - 1 ? c : choice;
        for (int s = B - 1; s >= 2; --s) {
          const uint64_t hit = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(hhi, s) << 32) |
                               (uint32_t)__builtin_amdgcn_readlane(hlo, s);
          const uint64_t bits = (s & 1) ? (hit >> (8 * c)) & 0xffull : (hit >> c) & 0x0101010101010101ull;
          int p = __ffsll((long long)bits) - 1;
          p = (s & 1) ? p : (p >> 3);
          c = p < 0 ? 0 : p;   // p < 0 only if no lane reached the maximum (non-finite scores)
          choice = lane == s - 1 ? c : choice;
        }
      }
    } else if (RULE == RULE_EXACT) {
      // G in lane j: the best float32 total of a path ending at candidate j of
      // slot s (left-to-right sums); s_tc[(s-2) K + j] its predecessor. The
      // predecessor scan runs i upward and keeps the first maximum.
      const int j = lane < K ? lane : K - 1;
      float G = (lane < K && B > 1) ? zval(1, 0, j) : -INFINITY;
      for (int s = 2; s < B; ++s) {
        float best = -INFINITY;
        int bi = 0;
        const float lj = s_logp[s * K + j];
        const float* ccol = s_cos + (s - 1) * KK + j;
        // eight predecessors at a time, their eight LDS reads issued together
        for (int i0 = 0; i0 < K; i0 += 8) {
          float cv[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) cv[u] = ccol[min(i0 + u, K - 1) * K];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int i = i0 + u;   // < 64: i0 <= 56 since K <= 64
            const float term = mul_rn(alpha, cv[u]);
            const float z = use_logp ? add_rn(lj, term) : term;
            const float cand = add_rn(readlane_f(G, i), z);
            const bool better = (i < K) & (cand > best);
            best = better ? cand : best;
            bi = better ? i : bi;
          }
        }
        if (lane < K) s_tc[(s - 2) * K + lane] = bi;
        G = lane < K ? best : -INFINITY;
      }
      if (B > 1) {
        // best final candidate, lowest index on a tie, then the trace-back
        float gv = G;
        int c = lane;
        lanes_argmax(gv, c, K <= 16 ? 16 : (K <= 32 ? 32 : 64));
        c = c < K ? c : 0;
        choice = lane == B - 1 ? c : choice;
        for (int s = B - 1; s >= 2; --s) {
          c = s_tc[(s - 2) * K + c];
          choice = lane == s - 1 ? c : choice;
        }
      }
    } else {
      // the walk proper: one table lookup per slot, starting from slot 0's top
      // candidate; step s's results are kept in lane s and written after the loop
      int c = 0;
      for (int s = 1; s < B; ++s) {
        const int e = (s - 1) * K + c;
        const int nc = s_tc[e];
        choice = lane == s ? nc : choice;
        if (RULE == RULE_GREEDY || !draw) {
          my_score = lane == s ? s_tz[e] : my_score;
          my_gap = lane == s ? s_tg[e] : my_gap;
        }
        c = nc;
      }
    }
    if (RULE == RULE_EXACT || draw) {
      // score of the committed candidate at each slot along the path
      const int prev = __shfl(choice, lane > 0 ? lane - 1 : 0);
      if (lane >= 1 && lane < B) my_score = zval(lane, prev, choice);
    }
    if (lane < B) {
      out_tokens[r0 + lane] = s_idx[lane * K + choice];
      if (score) score[r0 + lane] = my_score;
      if (gap) gap[r0 + lane] = my_gap;
      s_path[lane] = choice;
    }
  }
  if (RULE == RULE_SAMPLE && proposal) {
    // the distribution each slot was drawn from: softmax(z / T) of the row the
    // path stood on (one-hot for slot 0 and for greedy rows)
    __syncthreads();
    for (int t = tid; t < B * K; t += blockDim.x) {
      const int s = t / K, j = t - s * K;
      float q;
      if (s == 0 || !draw) {
        q = j == s_path[s] ? 1.f : 0.f;
      } else {
        const int cp = s_path[s - 1], e = (s - 1) * K + cp;
        q = __expf(mul_rn(sub_rn(zval(s, cp, j), s_tz[e]), inv_t)) / s_tg[e];
      }
      proposal[base + t] = q;
    }
  }
}

}  // namespace

size_t scores_walk_lds_bytes(int B, int K) {
  return ((size_t)(B - 1) * K * K + 2 * (size_t)B * K + 3 * (size_t)(B - 1) * K + B) * 4;
}

hipError_t launch_scores_walk(const uint16_t* outv, const uint16_t* inv, const float* cos_in,
                              int cos_slices, const int32_t* topk_idx, const float* topk_logp,
                              int N, int B, int K, int d_e, const CommitRule& rule, float* cos_out,
                              int32_t* out_tokens, float* score, float* gap, hipStream_t stream) {
  const int64_t slice_stride = (int64_t)N * (B - 1) * K * K;
  const size_t lds = scores_walk_lds_bytes(B, K);
  // The kernel's LDS may exceed the default 64 KiB limit: raise it once per
  // device (the attribute is set on the current device).
  static std::atomic<bool> attr_set[64];
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!attr_set[dev].load(std::memory_order_acquire)) {
    const void* fns[3] = {(const void*)scores_walk_kernel<RULE_GREEDY>,
                          (const void*)scores_walk_kernel<RULE_EXACT>,
                          (const void*)scores_walk_kernel<RULE_SAMPLE>};
    for (const void* f : fns) {
      err = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kScoresWalkMaxLds);
      if (err != hipSuccess) return err;
    }
    attr_set[dev].store(true, std::memory_order_release);
  }
#define LL_SW(R)                                                                                  \
  hipLaunchKernelGGL(scores_walk_kernel<R>, dim3((unsigned)N), dim3(512), lds, stream, outv, inv, \
                     cos_in, cos_slices, slice_stride, topk_idx, topk_logp, B, K, d_e,           \
                     rule.alpha, rule.use_logp,                                                   \
                     rule.temperature, rule.uniforms, rule.proposal, cos_out, out_tokens, score,  \
                     gap)
  if (rule.kind == RULE_EXACT)
    LL_SW(RULE_EXACT);
  else if (rule.kind == RULE_SAMPLE)
    LL_SW(RULE_SAMPLE);
  else
    LL_SW(RULE_GREEDY);
#undef LL_SW
  return hipGetLastError();
}

hipError_t launch_pair_scores(const uint16_t* outv, const uint16_t* inv, int N, int B, int K,
                              int d_e, float* cos, hipStream_t stream) {
  const int64_t pairs = (int64_t)N * (B - 1);
  if (pairs <= 0) return hipSuccess;
  hipLaunchKernelGGL(pair_scores_kernel, dim3((unsigned)((pairs + 3) / 4)), dim3(256), 0, stream,
                     outv, inv, N, B, K, d_e, cos);
  return hipGetLastError();
}

hipError_t launch_pair_slices(const uint16_t* outv, const uint16_t* inv, int N, int B, int K,
                              int d_e, float* part, hipStream_t stream) {
  const int64_t items = (int64_t)N * (B - 1) * pair_slice_count(d_e);
  if (items <= 0) return hipSuccess;
  hipLaunchKernelGGL(pair_slices_kernel, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, stream,
                     outv, inv, N, B, K, d_e, pair_slice_count(d_e), part);
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
