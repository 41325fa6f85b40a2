// Lattice attention (LiLiCorr paper, Section 3.2 and Appendix A: a
// bidirectional transformer over the whole candidate lattice of a block, with
// two per-head biases on the attention logits: one indexed by the signed slot
// distance between the two candidates, one for pairs in the same slot).
//
//   s_ij = q_i . k_j / sqrt(d_h) + Dist[slot_j - slot_i + 63] + Same [slot_i == slot_j]
//   p_ij = bf16(exp(s_ij - max_j s_ij)),  l_i = sum_j exp(s_ij - max_j s_ij)
//   o_i  = bf16(sum_j p_ij v_j / l_i)
//
// Scores are computed transposed (S^T = K Q^T), so each lane holds one
// query's column: that layout is directly the B operand of O^T = V^T P~^T,
// the second MFMA product. The row maximum is exact before any exponential
// (no online rescaling). Kernels: the resident one (K and V of a (head,
// block) in LDS, up to 256 tokens; at few rows it can also apply the output
// projection's per-head split-K slice) and the two-pass one (up to 512
// tokens, where K and V do not fit in LDS together).
#include "common.hpp"
#include "kernels.hpp"

namespace ll {
namespace {

// Resident variant for lattices of up to 256 tokens: one workgroup of eight
// waves per (head, block) loads the block's K and V (row-major, 16-byte
// chunks XOR-swizzled by key) into LDS once, with every global load in flight
// together, and the waves then loop over the block's 16-query tiles (wave w
// takes tiles w, w+8, ...). Per tile: S^T = K Q^T with the key tiles as
// independent MFMA chains, exact row max, P~ = bf16(exp(s - max)),
// O^T = V^T P~^T with V^T fragments read by ds_read_b64_tr_b16, O / l. K and V
// are read from HBM once per (block, head).
//
// With OPROJ (few rows: T of 65..128, d_h = 128) the kernel also applies the
// output projection's split-K slice of its head: workgroup z = half + 2 cq
// takes half `half` of the query tiles and columns 128 cq .. 128 cq + 127 of
// W_o, staged in LDS with K and V. Each wave multiplies its bf16 output tile
// (the attention output's rounding point) by that W_o slice over the head's
// d_h = 128 input columns and writes the fp32 partial
// part[head][row][column]; the linear's ordered split-K reduce (K slice =
// head) then adds bias, residual and RMSNorm. The attention output itself is
// not written.
template <int TMAX, int DH, int NW, int KM, bool OPROJ = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void attention_res_kernel(const uint16_t* __restrict__ qkv, int B,
                                                            int K, int H,
                                                            const float* __restrict__ dist,
                                                            const float* __restrict__ same,
                                                            uint16_t* __restrict__ out,
                                                            const uint16_t* __restrict__ wo = nullptr,
                                                            float* __restrict__ part = nullptr,
                                                            int M = 0) {
  constexpr int KT = TMAX / 16;   // 16-key tiles
  constexpr int KS = DH / 32;     // MFMA k-steps over d_h
  constexpr int DT = DH / 16;     // 16-wide d tiles of the output
  constexpr int CPR = DH / 8;     // 16-byte chunks per K or V row
  constexpr int SWM = DT - 1;     // V d-tile swizzle mask
  __shared__ __attribute__((aligned(16))) uint16_t Ks[TMAX * DH];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[TMAX * DH];
  __shared__ float bias_tab[128];
  static_assert(!OPROJ || (DH == 128 && TMAX == 128), "fused output projection tiling");
  constexpr int WCOLS = 128;   // W_o columns per workgroup (OPROJ)
  __shared__ __attribute__((aligned(16))) uint16_t Wos[OPROJ ? WCOLS * DH : 8];
  // K chunk (key, c) lives at chunk c ^ swz(key) of its row. A 16-byte LDS
  // read is served 16 lanes (256 bytes, all 64 banks) at a time, and a K
  // fragment read has those lanes on 16 consecutive keys at one chunk, so the
  // swizzle gives them 16 distinct 16-byte bank groups: 256 / (16 CPR) rows
  // share a 256-byte line, and the key's line index picks the chunk.
  auto kat = [](int key, int c) {
    constexpr int RPL = CPR >= 16 ? 1 : 16 / CPR;   // rows per 256-byte line
    const int sw = (key / RPL) & (CPR >= 16 ? 15 : CPR - 1);
    return key * DH + ((c ^ sw) << 3);
  };
  // V row-major; chunk c (8 columns) of row key sits in 32-byte d tile
  // ((c >> 1) ^ key) & SWM, so transposed fragment reads spread over the banks
  auto cat = [](int key, int c) { return key * DH + (((((c >> 1) ^ key) & SWM) << 1 | (c & 1)) << 3); };

  const int T = B * K;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int h = blockIdx.x;
  const int64_t n = blockIdx.y;
  const int64_t H3 = 3 * (int64_t)H;
  const uint16_t* blk = qkv + n * T * H3;

  // The block's query tiles are dealt to the gridDim.z workgroups of this
  // (head, block) and, within one, to its waves: tile qt0 + j * qstep.
  // OPROJ: z = half + 2 cq, the halves deal the tiles.
  const int zh = OPROJ ? (int)(blockIdx.z & 1) : (int)blockIdx.z;
  const int qt0 = zh * NW + wave, qstep = NW * (OPROJ ? 2 : (int)gridDim.z);
  const int64_t wn0 = OPROJ ? (int64_t)(blockIdx.z >> 1) * WCOLS : 0;   // first W_o column
  // Query fragments of this wave's first tile, issued before the staging
  // loads so that their latency overlaps them.
  u32x4_t qf0[KS];
  {
    const int qc = min(qt0 * 16 + c, T - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf0[ks] = *(const u32x4_t*)(blk + (int64_t)qc * H3 + h * DH + ks * 32 + 8 * g);
  }
  if (tid < 127) bias_tab[tid] = dist[h * 127 + tid];
  const float same_h = same[h];
  // K and V of this head (row-major, 16-byte chunks), all loads issued
  // before any store. Rows past the lattice are read from its last token
  // (a conditional load would serialise the loads): their keys are masked to
  // -inf and their values meet probability 0.
  constexpr int TOT = TMAX * CPR;                     // 16-byte chunks of each of K and V
  constexpr int NCH = (TOT + 64 * NW - 1) / (64 * NW);   // per thread
  constexpr bool EXACT = TOT % (64 * NW) == 0;
  u32x4_t kr[NCH], vr[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int ch = min(tid + 64 * NW * i, TOT - 1);
    const int kk = min(ch / CPR, T - 1), kc = ch % CPR;
    kr[i] = *(const u32x4_t*)(blk + (int64_t)kk * H3 + H + h * DH + kc * 8);
    vr[i] = *(const u32x4_t*)(blk + (int64_t)kk * H3 + 2 * H + h * DH + kc * 8);
  }
  // OPROJ: the W_o slice, rows wn0 .. wn0 + 127 (output columns), input
  // columns h DH .. h DH + DH - 1; 16-byte chunk c of row r at c ^ (r & 15)
  constexpr int WCH = OPROJ ? WCOLS * CPR / (64 * NW) : 1;   // chunks per thread
  u32x4_t wr[WCH];
  if constexpr (OPROJ) {
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int ch = tid + 64 * NW * i;
      wr[i] = *(const u32x4_t*)(wo + (wn0 + ch / CPR) * (int64_t)H + h * DH + (ch % CPR) * 8);
    }
  }
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int ch = tid + 64 * NW * i;
    if (!EXACT && ch >= TOT) break;
    *(u32x4_t*)(&Ks[kat(ch / CPR, ch % CPR)]) = kr[i];
    *(u32x4_t*)(&Vs[cat(ch / CPR, ch % CPR)]) = vr[i];
  }
  if constexpr (OPROJ) {
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int ch = tid + 64 * NW * i, r = ch / CPR, cc = ch % CPR;
      *(u32x4_t*)(&Wos[r * DH + ((cc ^ (r & 15)) << 3)]) = wr[i];
    }
  }
  __syncthreads();

  const float scale = 1.0f / __fsqrt_rn((float)DH);
  // slot of a token: (t * kmul) >> 16 equals t / K for t < 1024 and K <= 64
  const unsigned kmul = (65536u + K - 1) / K;
  const int ntile = (T + 15) / 16;
  for (int qt = qt0; qt < ntile; qt += qstep) {
    const int q = qt * 16 + c;   // this lane's query
    const bool q_ok = q < T;
    const int qc = min(q, T - 1);   // rows past the lattice compute a copy, never stored
    const int slot_q = (int)(((unsigned)qc * kmul) >> 16);
    u32x4_t qf[KS];
    if (qt == qt0) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = qf0[ks];
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qf[ks] = *(const u32x4_t*)(blk + (int64_t)qc * H3 + h * DH + ks * 32 + 8 * g);
    }
    // S^T tiles: key tiles are independent accumulation chains. Every tile of
    // TMAX is computed (rows past the lattice hold copies of its last token
    // and are masked below), so the loop has no branches and a k-step's LDS
    // reads are all issued before its MFMAs.
    f32x4_t acc[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) acc[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t kf[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) kf[kt] = *(const u32x4_t*)(&Ks[kat(kt * 16 + c, ks * 4 + g)]);
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) acc[kt] = mfma16(kf[kt], qf[ks], acc[kt]);
      __builtin_amdgcn_sched_group_barrier(0x100, KT, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, KT, 0);
      __builtin_amdgcn_sched_barrier(0);   // keep each k-step's reads with it
    }
    // Bias, same-slot term and mask (KM is 16 or 4 when K is a multiple of
    // it, else 0). With K a multiple of 4 a lane's four keys of a tile share one slot:
    // one slot computation, one bias-table read and one same-slot test per
    // tile and lane. Otherwise per element, with the bias-table reads
    // unconditional on a clamped slot (a read under a per-element branch is
    // waited for inside it) and issued together in a region of their own.
    // All compute fl32(fma(acc, scale, bias)), then + Same in its own
    // rounding on same-slot pairs (adding 0 elsewhere changes nothing).
    float s[KT][4];
    float mx = -INFINITY;
    if constexpr (KM == 16) {
      // K a multiple of 16: a 16-key tile and the 16-query tile each lie in
      // one slot and T is a multiple of 16, so the slots, the bias, the mask
      // and the same-slot test are wave-uniform per tile (scalar registers
      // and branches), leaving fma(acc, scale, bias) and the running max per
      // score, plus the Same add on the K / 16 same-slot tiles
      const int sq = __builtin_amdgcn_readfirstlane(slot_q);
      const float* __restrict__ dist_h = dist + h * 127;
      // the tiles' bias entries, read together (slot distances are within
      // +-63, so the clamped key's entry is always inside the table)
      float bt[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
        bt[kt] = dist_h[(int)(((unsigned)min(kt * 16, T - 1) * kmul) >> 16) - sq + 63];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const int key0 = kt * 16;
        const int sk = (int)(((unsigned)min(key0, T - 1) * kmul) >> 16);
        const float b = key0 < T ? bt[kt] : -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) s[kt][i] = acc[kt][i] * scale + b;
        if (sk == sq) {
#pragma unroll
          for (int i = 0; i < 4; ++i) s[kt][i] += same_h;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[kt][i]);
      }
    } else if constexpr (KM == 4) {
      // an opaque per-tile copy of the lane's key offset: the per-key masks
      // are recomputed per query tile instead of hoisted out of the tile
      // loop (a mask register pair per strip element, spilled)
      int g4 = 4 * g;
      asm volatile("" : "+v"(g4));
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        // T = B K is a multiple of 4 too, so the four keys are all inside the
        // lattice or all past it: the mask is a bias of -inf (fma(a, s, -inf)
        // is -inf for finite a)
        const int key0 = kt * 16 + g4;
        const int slot_k = (int)(((unsigned)min(key0, T - 1) * kmul) >> 16);
        const float b = key0 < T ? bias_tab[slot_k - slot_q + 63] : -INFINITY;
        const float sm = slot_k == slot_q ? same_h : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = (acc[kt][i] * scale + b) + sm;
          s[kt][i] = v;
          mx = fmaxf(mx, v);
        }
      }
    } else {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int slot_k = (int)(((unsigned)min(kt * 16 + 4 * g + i, T - 1) * kmul) >> 16);
          s[kt][i] = bias_tab[slot_k - slot_q + 63];
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kt * 16 + 4 * g + i;
          const int slot_k = (int)(((unsigned)min(key, T - 1) * kmul) >> 16);
          float v = acc[kt][i] * scale + s[kt][i];
          v = slot_k == slot_q ? v + same_h : v;
          v = key < T ? v : -INFINITY;
          s[kt][i] = v;
          mx = fmaxf(mx, v);
        }
    }
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
    // k-slot j of lane group g stands for key 32*ch + 4g + j (j < 4) or
    // 32*ch + 16 + 4g + (j - 4) (j >= 4), matching the score layout
    // chunks past the lattice carry probability 0 against finite values
#pragma unroll
    for (int ch = 0; ch < KT / 2; ++ch) {
      u32x4_t pb;
      pb[0] = pack_bf16x2(s[2 * ch][0], s[2 * ch][1]);
      pb[1] = pack_bf16x2(s[2 * ch][2], s[2 * ch][3]);
      pb[2] = pack_bf16x2(s[2 * ch + 1][0], s[2 * ch + 1][1]);
      pb[3] = pack_bf16x2(s[2 * ch + 1][2], s[2 * ch + 1][3]);
      // V^T fragments by ds_read_b64_tr_b16: within each 16-lane group,
      // source lane s addresses key k0 + s / 4, columns 4 (s % 4) .. + 3 of
      // the d tile, and output lane i receives keys k0 .. k0 + 3 of column i
      // (the MFMA A-operand layout); all of the chunk's reads are issued
      // before its MFMAs
      u32x4_t va[DT];
#pragma unroll
      for (int d = 0; d < DT; ++d) {
        const int k_lo = 32 * ch + 4 * g + c / 4, k_hi = k_lo + 16;
        const int c8 = 2 * d + (c & 3) / 2, off = 4 * (c & 1);
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16_t*)(&Vs[cat(k_lo, c8) + off]));
        const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16_t*)(&Vs[cat(k_hi, c8) + off]));
        const u32x2_t lo2 = __builtin_bit_cast(u32x2_t, lo), hi2 = __builtin_bit_cast(u32x2_t, hi);
        va[d] = u32x4_t{lo2[0], lo2[1], hi2[0], hi2[1]};
      }
#pragma unroll
      for (int d = 0; d < DT; ++d) oacc[d] = mfma16(va[d], pb, oacc[d]);
      // schedule: the chunk's LDS reads first, then its MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * DT, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, DT, 0);
      __builtin_amdgcn_sched_barrier(0);   // bound the V reads in flight
    }
    if constexpr (OPROJ) {
      // The tile's output, rounded to bf16 as stored otherwise, is the B
      // operand of P^T = W_o O^T: for k-step kk (d of 32 kk .. 32 kk + 31)
      // lane (g, c) holds query c at d = 32 kk + 4 g + 0..3 and
      // 32 kk + 16 + 4 g + 0..3 (its own accumulator elements), so the W_o
      // fragment takes the same d at the same k-slots. Output element
      // (row 4 g + i, column c) is column wn0 + 16 j + 4 g + i of query c.
      const float inv = 1.0f / lsum;
      u32x4_t ob[KS];
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        ob[kk] = u32x4_t{pack_bf16x2(oacc[2 * kk][0] * inv, oacc[2 * kk][1] * inv),
                         pack_bf16x2(oacc[2 * kk][2] * inv, oacc[2 * kk][3] * inv),
                         pack_bf16x2(oacc[2 * kk + 1][0] * inv, oacc[2 * kk + 1][1] * inv),
                         pack_bf16x2(oacc[2 * kk + 1][2] * inv, oacc[2 * kk + 1][3] * inv)};
      float* prow = part + ((int64_t)h * M + n * T + q) * (int64_t)H + wn0 + 4 * g;
#pragma unroll
      for (int j = 0; j < WCOLS / 16; ++j) {
        const int r = j * 16 + c;   // W_o row of this lane's A fragment
        u32x4_t wf[KS];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          const int c_lo = 4 * kk + (g >> 1), c_hi = c_lo + 2, hw = (g & 1) * 4;
          const u32x2_t lo = *(const u32x2_t*)(&Wos[r * DH + ((c_lo ^ (r & 15)) << 3) + hw]);
          const u32x2_t hi2 = *(const u32x2_t*)(&Wos[r * DH + ((c_hi ^ (r & 15)) << 3) + hw]);
          wf[kk] = u32x4_t{lo[0], lo[1], hi2[0], hi2[1]};
        }
        f32x4_t pacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) pacc = mfma16(wf[kk], ob[kk], pacc);
        if (q_ok) *(float4*)(prow + j * 16) = make_float4(pacc[0], pacc[1], pacc[2], pacc[3]);
      }
    } else if (q_ok) {
      const float inv = 1.0f / lsum;
      uint16_t* orow = out + (n * T + q) * (int64_t)H + h * DH;
#pragma unroll
      for (int d = 0; d < DT; ++d) {
        const uint32_t w0 = pack_bf16x2(oacc[d][0] * inv, oacc[d][1] * inv);
        const uint32_t w1 = pack_bf16x2(oacc[d][2] * inv, oacc[d][3] * inv);
        *(uint2*)(orow + d * 16 + 4 * g) = make_uint2(w0, w1);
      }
    }
  }
}

// Large lattices (T up to 512, where K and V do not fit in LDS together): one
// workgroup of eight waves per (head, block); each wave carries two 16-query
// tiles, so every K or V fragment it reads from LDS feeds two MFMAs (rounds of
// sixteen tiles). Pass 1 stages the head's K (row-major) and finds every
// query's exact row max. Pass 2 stages K and V of one half of the keys at a
// time (256 each) and, chunk of 32 keys by chunk, recomputes the identical
// scores, forms P~ = bf16(exp(s - max)) and accumulates O^T = V^T P~^T at once,
// so P~ lives for one chunk only. With K a multiple of 16 the first round's
// pass 1 also takes the second round's tiles, so K is staged whole once per
// block, and the first half of each pass 2 that follows a pass 1 reuses the K
// half still in LDS (staged bytes per block 768 -> 576 KiB at T = 512).
// V^T fragments are read by ds_read_b64_tr_b16:
// within each 16-lane group, source lane s addresses key k0 + s/4, columns
// 4 (s % 4) ..+3 of a 16-column d tile, and output lane i receives keys
// k0 .. k0 + 3 of column i, which is the MFMA A-operand layout. K and V rows
// keep their 32-byte d tiles XOR-swizzled by the LDS row, so fragment reads
// spread over the banks.
template <int DH>
__global__ __launch_bounds__(512) void attention_big_kernel(const uint16_t* __restrict__ qkv, int B,
                                                            int K, int H,
                                                            const float* __restrict__ dist,
                                                            const float* __restrict__ same,
                                                            uint16_t* __restrict__ out) {
  constexpr int TMAX = 512;
  constexpr int NW = 8;
  constexpr int KT = TMAX / 16, KS = DH / 32, DT = DH / 16, CPR = DH / 8;
  constexpr int SWM = DT - 1;         // d-tile swizzle mask
  constexpr int TOT = TMAX * CPR;     // 16-byte chunks of K (or V)
  constexpr int HCH = TOT / 2 / (64 * NW);   // per thread, one half of the keys
  static_assert(TOT % (2 * 64 * NW) == 0, "chunking");
  __shared__ __attribute__((aligned(16))) uint16_t buf[TMAX * DH];   // K, or K half | V half
  __shared__ float bias_tab[128];
  // element offset of 16-byte chunk c (8 columns) of LDS row r
  auto cat = [](int r, int c) { return r * DH + (((((c >> 1) ^ r) & SWM) << 1 | (c & 1)) << 3); };

  const int T = B * K;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int h = blockIdx.x;
  const int64_t n = blockIdx.y;
  const int64_t H3 = 3 * (int64_t)H;
  const uint16_t* blk = qkv + n * T * H3;
  if (tid < 127) bias_tab[tid] = dist[h * 127 + tid];
  const float same_h = same[h];

  // Stage keys [256 kh, 256 kh + 256) of K (which = 1) or V (which = 2) into
  // LDS rows [256 lh, 256 lh + 256); keys past the lattice are read from its
  // last token (masked to -inf / met with probability 0). Buffer loads with
  // 32-bit offsets from a descriptor of this block's rows, all issued before
  // any store.
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)blk, 0, (int)(T * H3 * 2), 0x00020000);
  auto stage_half = [&](int which, int kh, int lh) __attribute__((always_inline)) {
    // an opaque copy of the thread index: the offsets below are recomputed
    // per call instead of being kept live (and spilled) across rounds
    int t0 = tid;
    asm volatile("" : "+v"(t0));
    u32x4_t rr[HCH];
#pragma unroll
    for (int i = 0; i < HCH; ++i) {
      const int ch = t0 + 64 * NW * i;
      const int key = min(256 * kh + ch / CPR, T - 1), c8 = ch % CPR;
      const int off = (key * (int)H3 + which * H + h * DH + c8 * 8) * 2;
      rr[i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < HCH; ++i) {
      const int ch = t0 + 64 * NW * i;
      *(u32x4_t*)(&buf[cat(256 * lh + ch / CPR, ch % CPR)]) = rr[i];
    }
  };

  const float scale = 1.0f / __fsqrt_rn((float)DH);
  // slot of a token: (t * kmul) >> 16 equals t / K for t < 1024 and K <= 64
  const unsigned kmul = (65536u + K - 1) / K;
  const float* __restrict__ dist_h = dist + h * 127;
  const int ntile = (T + 15) / 16;
  // With K a multiple of 16 and a second round, round 0's pass 1 also takes
  // round 1's query tiles (K is then staged whole once per block), and their
  // maxima wait here.
  const bool ahead = K % 16 == 0 && ntile > 2 * NW;
  float mxc_s = -INFINITY, mxd_s = -INFINITY;
  for (int r0 = 0; r0 < ntile; r0 += 2 * NW) {
    const bool p1 = !(ahead && r0 > 0);   // this round runs pass 1
    const int qta = r0 + wave, qtb = r0 + NW + wave;
    const bool oka = qta < ntile, okb = qtb < ntile;
    const int qa = qta * 16 + c, qb = qtb * 16 + c;
    const int qca = min(qa, T - 1), qcb = min(qb, T - 1);
    const int slot_qa = qca / K, slot_qb = qcb / K;
    u32x4_t qfa[KS], qfb[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qfa[ks] = *(const u32x4_t*)(blk + (int64_t)qca * H3 + h * DH + ks * 32 + 8 * g);
      qfb[ks] = *(const u32x4_t*)(blk + (int64_t)qcb * H3 + h * DH + ks * 32 + 8 * g);
    }
    // LDS fragment addresses derive from an opaque per-round base, so they are
    // recomputed each round rather than hoisted out of the loop (and spilled)
    int zb = 0;
    asm volatile("" : "+v"(zb));
    const uint16_t* lb = buf + zb;
    if (p1) {
      __syncthreads();   // previous round done with buf
      stage_half(1, 0, 0);
      stage_half(1, 1, 1);
      __syncthreads();
    }
    // Scores of key tiles kt0, kt0 + 1 (LDS rows from lr0) for both query
    // tiles, masked and biased; each K fragment read feeds two MFMAs.
    auto scores2 = [&](int kt0, int lr0, float (&va)[2][4], float (&vb)[2][4]) __attribute__((always_inline)) {
      f32x4_t aa[2], ab[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        aa[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        ab[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const u32x4_t kf = *(const u32x4_t*)(&lb[cat(lr0 + j * 16 + c, ks * 4 + g)]);
          aa[j] = mfma16(kf, qfa[ks], aa[j]);
          ab[j] = mfma16(kf, qfb[ks], ab[j]);
        }
      if (K % 16 == 0) {
        // every 16-key tile lies in one slot, and T = B K is a multiple of 16,
        // so a tile is all inside the lattice or all past it: one table read
        // per tile and query tile, the mask a bias of -inf (fma(a, s, -inf) is
        // -inf for finite a) and the same-slot term one add
        // (slots, bias and the same-slot tests are wave-uniform: scalar)
        const int sqa = __builtin_amdgcn_readfirstlane(slot_qa), sqb = __builtin_amdgcn_readfirstlane(slot_qb);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int key0 = (kt0 + j) * 16;
          const int st = (int)(((unsigned)min(key0, T - 1) * kmul) >> 16);
          const bool in = key0 < T;
          const float ta = dist_h[st - sqa + 63], tb = dist_h[st - sqb + 63];   // clamped key: in the table
          const float ba = in ? ta : -INFINITY;
          const float bb = in ? tb : -INFINITY;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            va[j][i] = aa[j][i] * scale + ba;
            vb[j][i] = ab[j][i] * scale + bb;
          }
          if (st == sqa) {
#pragma unroll
            for (int i = 0; i < 4; ++i) va[j][i] += same_h;
          }
          if (st == sqb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) vb[j][i] += same_h;
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = (kt0 + j) * 16 + 4 * g + i + zb;   // zb == 0, opaque
            float x = -INFINITY, y = -INFINITY;
            if (key < T) {
              const int slot_k = (int)(((unsigned)key * kmul) >> 16);
              x = aa[j][i] * scale + bias_tab[slot_k - slot_qa + 63];
              y = ab[j][i] * scale + bias_tab[slot_k - slot_qb + 63];
              if (slot_k == slot_qa) x += same_h;
              if (slot_k == slot_qb) y += same_h;
            }
            va[j][i] = x;
            vb[j][i] = y;
          }
      }
    };
    // pass 1: the exact row maxima
    float mxa = -INFINITY, mxb = -INFINITY;
    if (!p1) {
      mxa = mxc_s;
      mxb = mxd_s;
    } else if (ahead) {
      // round 0 with round 1's tiles qta + 2 NW, qtb + 2 NW alongside: every
      // K fragment read feeds four MFMAs; raw-product maxima per tile as below
      const int qcc = min(qa + 32 * NW, T - 1), qcd = min(qb + 32 * NW, T - 1);
      const int sqa = __builtin_amdgcn_readfirstlane(slot_qa), sqb = __builtin_amdgcn_readfirstlane(slot_qb);
      const int sqc = __builtin_amdgcn_readfirstlane(qcc / K), sqd = __builtin_amdgcn_readfirstlane(qcd / K);
      u32x4_t qfc[KS], qfd[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        qfc[ks] = *(const u32x4_t*)(blk + (int64_t)qcc * H3 + h * DH + ks * 32 + 8 * g);
        qfd[ks] = *(const u32x4_t*)(blk + (int64_t)qcd * H3 + h * DH + ks * 32 + 8 * g);
      }
      float mxc = -INFINITY, mxd = -INFINITY;
#pragma unroll 2
      for (int kt0 = 0; kt0 < KT; kt0 += 2) {
        if (kt0 * 16 >= T) continue;
        f32x4_t a4[4][2];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int j = 0; j < 2; ++j) a4[t][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const u32x4_t kf = *(const u32x4_t*)(&lb[cat(kt0 * 16 + j * 16 + c, ks * 4 + g)]);
            a4[0][j] = mfma16(kf, qfa[ks], a4[0][j]);
            a4[1][j] = mfma16(kf, qfb[ks], a4[1][j]);
            a4[2][j] = mfma16(kf, qfc[ks], a4[2][j]);
            a4[3][j] = mfma16(kf, qfd[ks], a4[3][j]);
          }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int key0 = (kt0 + j) * 16;
          const int st = (int)(((unsigned)min(key0, T - 1) * kmul) >> 16);
          const bool in = key0 < T;
          const int sq[4] = {sqa, sqb, sqc, sqd};
          float* const mx[4] = {&mxa, &mxb, &mxc, &mxd};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float dv = dist_h[st - sq[t] + 63];   // clamped key: in the table
            const float b = in ? dv : -INFINITY;
            const float sm = st == sq[t] ? same_h : 0.f;
            const float tm = fmaxf(fmaxf(a4[t][j][0], a4[t][j][1]), fmaxf(a4[t][j][2], a4[t][j][3]));
            *mx[t] = fmaxf(*mx[t], (tm * scale + b) + sm);
          }
        }
      }
      mxa = fmaxf(mxa, __shfl_xor(mxa, 16, 64));
      mxa = fmaxf(mxa, __shfl_xor(mxa, 32, 64));
      mxb = fmaxf(mxb, __shfl_xor(mxb, 16, 64));
      mxb = fmaxf(mxb, __shfl_xor(mxb, 32, 64));
      mxc = fmaxf(mxc, __shfl_xor(mxc, 16, 64));
      mxc = fmaxf(mxc, __shfl_xor(mxc, 32, 64));
      mxd = fmaxf(mxd, __shfl_xor(mxd, 16, 64));
      mxd = fmaxf(mxd, __shfl_xor(mxd, 32, 64));
      mxc_s = mxc;
      mxd_s = mxd;
    } else if (oka) {
#pragma unroll 4
      for (int kt0 = 0; kt0 < KT; kt0 += 2) {
        if (kt0 * 16 >= T) continue;
        if (K % 16 == 0) {
          // fl(fl(a s + bias) + Same) does not decrease with a, and bias and
          // Same are one per 16-key tile here: the tile's largest score is
          // that of its largest product
          f32x4_t aa[2], ab[2];
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            aa[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            ab[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const u32x4_t kf = *(const u32x4_t*)(&lb[cat(kt0 * 16 + j * 16 + c, ks * 4 + g)]);
              aa[j] = mfma16(kf, qfa[ks], aa[j]);
              ab[j] = mfma16(kf, qfb[ks], ab[j]);
            }
          const int sqa = __builtin_amdgcn_readfirstlane(slot_qa), sqb = __builtin_amdgcn_readfirstlane(slot_qb);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int key0 = (kt0 + j) * 16;
            const int st = (int)(((unsigned)min(key0, T - 1) * kmul) >> 16);
            const bool in = key0 < T;
            const float da = dist_h[st - sqa + 63], db = dist_h[st - sqb + 63];   // clamped key: in the table
            const float ba = in ? da : -INFINITY;
            const float bb = in ? db : -INFINITY;
            const float sa = st == sqa ? same_h : 0.f, sb = st == sqb ? same_h : 0.f;
            const float ta = fmaxf(fmaxf(aa[j][0], aa[j][1]), fmaxf(aa[j][2], aa[j][3]));
            const float tb = fmaxf(fmaxf(ab[j][0], ab[j][1]), fmaxf(ab[j][2], ab[j][3]));
            mxa = fmaxf(mxa, (ta * scale + ba) + sa);
            mxb = fmaxf(mxb, (tb * scale + bb) + sb);
          }
        } else {
          float va[2][4], vb[2][4];
          scores2(kt0, kt0 * 16, va, vb);
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              mxa = fmaxf(mxa, va[j][i]);
              mxb = fmaxf(mxb, vb[j][i]);
            }
        }
      }
      mxa = fmaxf(mxa, __shfl_xor(mxa, 16, 64));
      mxa = fmaxf(mxa, __shfl_xor(mxa, 32, 64));
      mxb = fmaxf(mxb, __shfl_xor(mxb, 16, 64));
      mxb = fmaxf(mxb, __shfl_xor(mxb, 32, 64));
    }
    // pass 2: per half of the keys, K and V side by side in LDS
    f32x4_t oa[DT], ob[DT];
#pragma unroll
    for (int d = 0; d < DT; ++d) {
      oa[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      ob[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    float la = 0.f, lbs = 0.f;
    for (int kh = 0; kh < 2; ++kh) {
      if (256 * kh >= T) break;
      __syncthreads();   // every wave is done with the previous contents
      // after this round's pass 1 the first K half is still in rows 0..255
      if (kh > 0 || !p1) stage_half(1, kh, 0);
      stage_half(2, kh, 1);
      __syncthreads();
      if (!oka) continue;
      for (int ch = 0; ch < 8; ++ch) {
        const int gch = 8 * kh + ch;   // global 32-key chunk
        if (gch * 32 >= T) break;
        float va[2][4], vb[2][4];
        scores2(2 * gch, 32 * ch, va, vb);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            va[j][i] = __expf(va[j][i] - mxa);
            la += va[j][i];
            vb[j][i] = __expf(vb[j][i] - mxb);
            lbs += vb[j][i];
          }
        // k-slot j of lane group g stands for key 32 ch + 4g + j (j < 4) or
        // 32 ch + 16 + 4g + (j - 4) (j >= 4), matching the score layout
        const u32x4_t pa = {pack_bf16x2(va[0][0], va[0][1]), pack_bf16x2(va[0][2], va[0][3]),
                            pack_bf16x2(va[1][0], va[1][1]), pack_bf16x2(va[1][2], va[1][3])};
        const u32x4_t pb = {pack_bf16x2(vb[0][0], vb[0][1]), pack_bf16x2(vb[0][2], vb[0][3]),
                            pack_bf16x2(vb[1][0], vb[1][1]), pack_bf16x2(vb[1][2], vb[1][3])};
        const int s = c;   // source lane within the 16-lane group
#pragma unroll
        for (int d = 0; d < DT; ++d) {
          const int k_lo = 256 + 32 * ch + 4 * g + s / 4, k_hi = k_lo + 16;
          const int c8 = 2 * d + (s & 3) / 2, off = 4 * (s & 1);
          const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16_t*)(&lb[cat(k_lo, c8) + off]));
          const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16_t*)(&lb[cat(k_hi, c8) + off]));
          const u32x2_t lo2 = __builtin_bit_cast(u32x2_t, lo), hi2 = __builtin_bit_cast(u32x2_t, hi);
          const u32x4_t vf = {lo2[0], lo2[1], hi2[0], hi2[1]};
          oa[d] = mfma16(vf, pa, oa[d]);
          ob[d] = mfma16(vf, pb, ob[d]);
        }
      }
    }
    if (oka) {
      la += __shfl_xor(la, 16, 64);
      la += __shfl_xor(la, 32, 64);
      lbs += __shfl_xor(lbs, 16, 64);
      lbs += __shfl_xor(lbs, 32, 64);
      if (qa < T) {
        const float inv = 1.0f / la;
        uint16_t* orow = out + (n * T + qa) * (int64_t)H + h * DH;
#pragma unroll
        for (int d = 0; d < DT; ++d)
          *(uint2*)(orow + d * 16 + 4 * g) =
              make_uint2(pack_bf16x2(oa[d][0] * inv, oa[d][1] * inv), pack_bf16x2(oa[d][2] * inv, oa[d][3] * inv));
      }
      if (okb && qb < T) {
        const float inv = 1.0f / lbs;
        uint16_t* orow = out + (n * T + qb) * (int64_t)H + h * DH;
#pragma unroll
        for (int d = 0; d < DT; ++d)
          *(uint2*)(orow + d * 16 + 4 * g) =
              make_uint2(pack_bf16x2(ob[d][0] * inv, ob[d][1] * inv), pack_bf16x2(ob[d][2] * inv, ob[d][3] * inv));
      }
    }
  }
}

template <int TMAX>
hipError_t launch_res(int dh, const uint16_t* qkv, int N, int B, int K, int H, int heads,
                      const float* dist, const float* same, uint16_t* out, hipStream_t stream) {
  // Up to 128 tokens: two four-wave workgroups per (head, block), each with
  // half of the query tiles (every wave reads all of K and V from LDS, so
  // fewer waves per CU means less LDS traffic per CU); larger lattices: one
  // eight-wave workgroup.
  constexpr int NW = TMAX <= 128 ? 4 : 8;
  const int ntile = (B * K + 15) / 16;
  const dim3 grid((unsigned)heads, (unsigned)N, TMAX <= 128 && ntile > NW ? 2u : 1u);
#define LL_RES(DH)                                                                              \
  do {                                                                                        \
    if ((K & 15) == 0)                                                                        \
      hipLaunchKernelGGL((attention_res_kernel<TMAX, DH, NW, 16>), grid, dim3(64 * NW), 0,     \
                         stream, qkv, B, K, H, dist, same, out);                              \
    else if ((K & 3) == 0)                                                                    \
      hipLaunchKernelGGL((attention_res_kernel<TMAX, DH, NW, 4>), grid, dim3(64 * NW), 0,      \
                         stream, qkv, B, K, H, dist, same, out);                              \
    else                                                                                      \
      hipLaunchKernelGGL((attention_res_kernel<TMAX, DH, NW, 0>), grid, dim3(64 * NW), 0,      \
                         stream, qkv, B, K, H, dist, same, out);                              \
  } while (0)
  if (dh == 32) LL_RES(32);
  else if (dh == 64) LL_RES(64);
  else LL_RES(128);
#undef LL_RES
  return hipGetLastError();
}

}  // namespace

bool attention_o_fusable(int N, int B, int K, int H, int heads) {
  const int T = B * K;
  return heads >= 1 && H == heads * 128 && T > 64 && T <= 128 && (int64_t)N * T < 2048 &&
         (heads == 2 || heads == 3 || heads == 4 || heads == 6 || heads == 8 || heads == 12 || heads == 16);
}

hipError_t launch_attention_o(const uint16_t* qkv, int N, int B, int K, int H, int heads,
                              const float* dist, const float* same, const uint16_t* wo, float* part,
                              hipStream_t stream) {
  if (!attention_o_fusable(N, B, K, H, heads)) return hipErrorInvalidValue;
  const int M = N * B * K;
  const dim3 grid((unsigned)heads, (unsigned)N, (unsigned)(2 * (H / 128)));
  if ((K & 15) == 0)
    hipLaunchKernelGGL((attention_res_kernel<128, 128, 4, 16, true>), grid, dim3(256), 0, stream, qkv, B, K, H,
                       dist, same, nullptr, wo, part, M);
  else if ((K & 3) == 0)
    hipLaunchKernelGGL((attention_res_kernel<128, 128, 4, 4, true>), grid, dim3(256), 0, stream, qkv, B, K, H,
                       dist, same, nullptr, wo, part, M);
  else
    hipLaunchKernelGGL((attention_res_kernel<128, 128, 4, 0, true>), grid, dim3(256), 0, stream, qkv, B, K, H,
                       dist, same, nullptr, wo, part, M);
  return hipGetLastError();
}

hipError_t launch_attention(const uint16_t* qkv, int N, int B, int K, int H, int heads,
                            const float* dist, const float* same, uint16_t* out,
                            hipStream_t stream) {
  const int T = B * K, dh = H / heads;
  if (T <= 64) return launch_res<64>(dh, qkv, N, B, K, H, heads, dist, same, out, stream);
  if (T <= 128) return launch_res<128>(dh, qkv, N, B, K, H, heads, dist, same, out, stream);
  if (T <= 256) return launch_res<256>(dh, qkv, N, B, K, H, heads, dist, same, out, stream);
  const dim3 grid((unsigned)heads, (unsigned)N);
  if (dh == 32)
    hipLaunchKernelGGL(attention_big_kernel<32>, grid, dim3(512), 0, stream, qkv, B, K, H, dist, same, out);
  else if (dh == 64)
    hipLaunchKernelGGL(attention_big_kernel<64>, grid, dim3(512), 0, stream, qkv, B, K, H, dist, same, out);
  else
    hipLaunchKernelGGL(attention_big_kernel<128>, grid, dim3(512), 0, stream, qkv, B, K, H, dist, same, out);
  return hipGetLastError();
}

}  // namespace ll
