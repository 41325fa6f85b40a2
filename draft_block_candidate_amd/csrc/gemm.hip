// Linear layers of the candidate encoder on CDNA4 MFMA (bf16 in, fp32 acc).
//
// Y[M, N] = A[M, Kd] . W[N, Kd]^T + bias, both operands K-contiguous, so every
// MFMA operand fragment is one 16-byte LDS read. Epilogues fuse the bias, the
// bf16 rounding, SiLU and the fp32 residual add of the pre-norm transformer.
//
// Schedules:
//  * many rows (M >= 2048): the DMA-pipelined kernel (32 x 32 x 16 MFMA, four
//    LDS stages filled by direct global-to-LDS loads, LDS-staged coalesced
//    epilogue) with the largest of 256 x 256, 256 x 128 and 128 x 128 tiles
//    that still gives every CU a tile; eight waves (two per SIMD) for the
//    two large tiles, four for 128 x 128;
//  * many rows that the DMA kernel cannot take (K not a multiple of 32,
//    misaligned operands): 128 x 128 tiles over the whole K, double-buffered
//    in LDS, four waves in a 2 x 2 arrangement of 16 x 16 MFMA tiles;
//  * few rows (M <= 128) and at least 128 tiles of 16 columns: one DMA-
//    pipelined pass over K per 16-column tile (64 x 32 tiles from 65 rows)
//    with the epilogue fused;
//  * other few-row shapes (one or a few draft blocks, M = B*K*N of 64..2047):
//    the GEMM is weight-streaming and latency bound, so K is split S ways
//    (64 x 64 tiles from 65 rows, 64 x 32 below).
//    Each workgroup stages its whole A and W K-slice (64..256 wide) in LDS
//    with every load in flight at once, multiplies, and writes an fp32
//    partial tile. A second kernel sums the S partials in the fixed order
//    s = 0..S-1 (bit-reproducible) and applies the epilogue; it works on
//    whole rows, so the RMSNorm that follows a residual add and the unit
//    normalisation of the out/in heads fuse into it.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace ll {
namespace {

constexpr int BK = 64;
constexpr int LDS_STRIDE = BK + 8;  // bf16 elements per LDS row (16-byte pad)

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(const uint16_t* __restrict__ A,
                                                   const uint16_t* __restrict__ W, int M, int N,
                                                   int Kd, const float* __restrict__ bias,
                                                   const float* resid, void* out) {
  constexpr int MT = BM / 32;  // 16-row tiles per wave
  constexpr int NT = BN / 32;  // 16-col tiles per wave
  constexpr int A_CHUNKS = BM * BK / 8 / 256;  // 16-byte chunks per thread
  constexpr int W_CHUNKS = BN * BK / 8 / 256;
  static_assert(A_CHUNKS >= 1 && W_CHUNKS >= 1, "tile too small");
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t Ws[2][BN * LDS_STRIDE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 4, c = lane & 15;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int64_t n0 = (int64_t)blockIdx.x * BN;

  u32x4_t ra[A_CHUNKS], rw[W_CHUNKS];
  auto load_tiles = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
      const int ch = tid + 256 * i;
      const int r = ch >> 3, c8 = ch & 7;
      const int64_t gm = m0 + r;
      ra[i] = gm < M ? *(const u32x4_t*)(A + gm * Kd + k0 + c8 * 8) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < W_CHUNKS; ++i) {
      const int ch = tid + 256 * i;
      const int r = ch >> 3, c8 = ch & 7;
      const int64_t gn = n0 + r;
      rw[i] = gn < N ? *(const u32x4_t*)(W + gn * Kd + k0 + c8 * 8) : u32x4_t{0, 0, 0, 0};
    }
  };
  auto store_tiles = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
      const int ch = tid + 256 * i;
      *(u32x4_t*)(&As[buf][(ch >> 3) * LDS_STRIDE + (ch & 7) * 8]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < W_CHUNKS; ++i) {
      const int ch = tid + 256 * i;
      *(u32x4_t*)(&Ws[buf][(ch >> 3) * LDS_STRIDE + (ch & 7) * 8]) = rw[i];
    }
  };

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = Kd / BK;
  load_tiles(0);
  store_tiles(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_tiles((kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      u32x4_t af[MT], bfr[NT];
#pragma unroll
      for (int i = 0; i < MT; ++i)
        af[i] = *(const u32x4_t*)(&As[buf][(wm * (BM / 2) + i * 16 + c) * LDS_STRIDE + kk + 8 * g]);
#pragma unroll
      for (int j = 0; j < NT; ++j)
        bfr[j] = *(const u32x4_t*)(&Ws[buf][(wn * (BN / 2) + j * 16 + c) * LDS_STRIDE + kk + 8 * g]);
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = mfma16(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) store_tiles(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: lane holds rows 4g+q, column c of every 16 x 16 tile. Bias and
  // residual addresses are clamped so their loads are unconditional; only the
  // stores are predicated.
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int64_t n = n0 + wn * (BN / 2) + j * 16 + c;
    const int64_t nc = min(n, (int64_t)N - 1);
    const float bv = bias ? bias[nc] : 0.f;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t m = m0 + wm * (BM / 2) + i * 16 + 4 * g + q;
        const bool ok = m < M && n < N;
        const float y = acc[i][j][q] + bv;
        const int64_t o = m * N + n;
        if constexpr (EPI == EPI_F32) {
          if (ok) ((float*)out)[o] = y;
        } else if constexpr (EPI == EPI_BF16) {
          if (ok) ((uint16_t*)out)[o] = (uint16_t)f32_to_bf16(y);
        } else if constexpr (EPI == EPI_SILU_BF16) {
          if (ok) ((uint16_t*)out)[o] = (uint16_t)f32_to_bf16(silu(y));
        } else {
          const float r = resid[min(m, (int64_t)M - 1) * N + nc];
          if (ok) ((float*)out)[o] = r + y;
        }
      }
    }
  }
}

__device__ __forceinline__ f32x16_t mfma32(const u32x4_t& a, const u32x4_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Many-row GEMM on 32 x 32 x 16 MFMA, BM x BN tiles. NW waves in a
// 2 x (NW / 2) grid each hold a (BM / 2) x (2 BN / NW) fp32 accumulator block
// (with four waves and 256 x 256 tiles, 128 x 128: every 16-byte fragment
// read from LDS feeds four MFMAs). K advances 64 per stage
// through two or three LDS stages that global_load_lds fills directly (no
// register staging), NS - 1 stages ahead of the one being multiplied; each wave waits
// only for its own stage loads (vmcnt) and a bare s_barrier then makes the
// stage visible, so the loads behind it stay in flight. Within a stage the
// next k-step's fragment reads are interleaved with the current MFMAs. Stage
// rows are 128 bytes with the 16-byte chunk XOR-swizzled by (row >> 1) & 7:
// LDS serves a 16-byte-per-lane read 16 lanes (256 bytes, all 64 banks) at a
// time; the 16 rows those lanes read pair up on the two halves of the banks
// (row parity) and the swizzle gives the 8 rows of each half 8 distinct
// chunks, so every read touches each bank once. Workgroups are dealt to the XCDs
// round-robin; the tile order is remapped so that each XCD runs a contiguous
// run of tiles and shares their A row panels in its L2. The epilogue moves
// each wave's block out through LDS in 32-row slices as 16-byte stores.
// s_waitcnt immediate for "at most v vector-memory operations outstanding"
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt not waited).
constexpr int waitcnt_vm(int v) { return (v & 15) | ((v >> 4) << 14) | 0x70 | 0xF00; }

// Residual epilogue whose residual is the node build's table sum (NodeSource)
constexpr int EPI_NODE = 4;

// Token id of row m, clamped into E (the ids come from the top-K stage; a
// row never reads outside the table).
__device__ __forceinline__ int node_token(const NodeSource& nd, uint32_t m) {
  const int64_t tok = nd.tok[m];
  return tok < 0 || tok >= nd.V ? 0 : (int)tok;
}

// ((E[tok] + S[s]) + R[j]) of row m, columns n .. n + 3 (float32, the order
// the node is written in); N is the row length of the tables.
__device__ __forceinline__ float4 node_sum4(const NodeSource& nd, uint32_t m, int tok, int64_t n, int N) {
  const uint32_t q = div_by(m, nd.magic_k);
  const int j = (int)(m - q * (uint32_t)nd.K);
  const int s = (int)(q - div_by(q, nd.magic_b) * (uint32_t)nd.B);
  const uint2 e = *(const uint2*)(nd.E + (int64_t)tok * N + n);
  const uint2 sv = *(const uint2*)(nd.S + (int64_t)s * N + n);
  const uint2 rv = *(const uint2*)(nd.R + (int64_t)j * N + n);
  auto lo = [](uint32_t w) { return __uint_as_float(w << 16); };
  auto hi = [](uint32_t w) { return __uint_as_float(w & 0xffff0000u); };
  return make_float4((lo(e.x) + lo(sv.x)) + lo(rv.x), (hi(e.x) + hi(sv.x)) + hi(rv.x),
                     (lo(e.y) + lo(sv.y)) + lo(rv.y), (hi(e.y) + hi(sv.y)) + hi(rv.y));
}

__device__ __forceinline__ float4 node_resid4(const NodeSource& nd, uint32_t m, int64_t n, int N) {
  return node_sum4(nd, m, node_token(nd, m), n, N);
}

template <int BM, int BN, int EPI, int NW = 4>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(BM * BN * 4 / NW >= 32768 ? 1 : 2, BM * BN * 4 / NW >= 32768 ? 1 : 2))) void gemm_dma_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W, int M, int N, int Kd,
    const float* __restrict__ bias, const float* resid, void* out, int tiles_n, int ntiles,
    NodeSource node) {
  constexpr bool RES = EPI == EPI_RESID_F32 || EPI == EPI_NODE;   // a residual is added
  // K advances 64 per stage, so a stage row is one whole 128-byte line of A or
  // W (10-17 % faster than 32 per stage, whose load instructions each touched
  // half of 16 lines). Stages in LDS: three for 256 x 128 tiles (144 KiB), two
  // otherwise (128 KiB for 256 x 256; 64 KiB for 128 x 128, two workgroups per CU).
  constexpr int BK = 64, NS = BM == 256 && BN == 128 ? 3 : 2;
  constexpr int CPR = BK / 8, RPI = 64 / CPR;   // 16-byte chunks per stage row; rows per load instruction
  constexpr int WGN = NW / 2;                  // waves: 2 x WGN grid
  constexpr int WM = BM / 2, WN = BN / WGN, MT = WM / 32, NT = WN / 32;
  constexpr int UA = BM / RPI / NW, UW = BN / RPI / NW;   // 1 KiB stage-load instructions per wave
  static_assert(UA >= 1 && UW >= 1 && BM % (RPI * NW) == 0 && BN % (RPI * NW) == 0, "stage loads");
  constexpr int PER = UA + UW;                 // per wave per stage
  constexpr int STAGE = (BM + BN) * BK;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[NS * STAGE];

  const int wg = blockIdx.x;
  const int q = ntiles / 8, r = ntiles % 8, x = wg % 8;
  const int t = x * q + min(x, r) + wg / 8;
  if (t >= ntiles) return;
  // Within an XCD's run, tiles go column-major over groups of 8 row panels
  // when the output is at least 8 tiles wide: the 32 tiles an XCD runs at once
  // then share 8 A panels and 4 W panels instead of 2 and 16, which cuts the
  // L2 misses of wide outputs by about a third. Narrower outputs go row-major
  // (already 8 row panels per 32 tiles).
  int tm, tn;
  if (tiles_n >= 8) {
    const int tiles_m = ntiles / tiles_n;
    const int grp = t / (8 * tiles_n), first_m = grp * 8;
    const int gm = min(8, tiles_m - first_m), tin = t - grp * 8 * tiles_n;
    tm = first_m + tin % gm;
    tn = tin / gm;
  } else {
    tm = t / tiles_n;
    tn = t % tiles_n;
  }
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int l32 = lane & 31, hi = lane >> 5;

  // Stage loads: instruction j of A (0 .. BM/8 - 1 over the workgroup) covers
  // tile rows 8 j .. 8 j + 7, and its lane i fills LDS slot i (row 8 j + i / 8,
  // chunk' = i % 8), which holds chunk chunk' ^ ((row >> 1) & 7) of that row;
  // likewise for W. Rows past the matrix are clamped.
  const uint16_t* srcA[UA];
  const uint16_t* srcW[UW];
#pragma unroll
  for (int u = 0; u < UA; ++u) {
    const int row = RPI * (wave * UA + u) + lane / CPR;
    const int chunk = (lane % CPR) ^ ((row >> 1) & 7);
    srcA[u] = A + min(m0 + row, (int64_t)M - 1) * Kd + chunk * 8;
  }
#pragma unroll
  for (int u = 0; u < UW; ++u) {
    const int row = RPI * (wave * UW + u) + lane / CPR;
    const int chunk = (lane % CPR) ^ ((row >> 1) & 7);
    srcW[u] = W + min(n0 + row, (int64_t)N - 1) * Kd + chunk * 8;
  }
  auto issue = [&](int kt) __attribute__((always_inline)) {
    uint16_t* st = smem + (kt % NS) * STAGE;
    const int k0 = kt * BK;
#pragma unroll
    for (int u = 0; u < UA; ++u)
      __builtin_amdgcn_global_load_lds((const void*)(srcA[u] + k0),
                                       (__attribute__((address_space(3))) void*)(st + (wave * UA + u) * 512),
                                       16, 0, 0);
#pragma unroll
    for (int u = 0; u < UW; ++u)
      __builtin_amdgcn_global_load_lds((const void*)(srcW[u] + k0),
                                       (__attribute__((address_space(3))) void*)(st + BM * BK + (wave * UW + u) * 512),
                                       16, 0, 0);
  };
  auto fat = [](int row, int chunk) { return row * BK + ((chunk ^ ((row >> 1) & 7)) << 3); };

  f32x16_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nk = Kd / BK;
#pragma unroll
  for (int st = 0; st < NS - 1; ++st)
    if (st < nk) issue(st);
  for (int kt = 0; kt < nk; ++kt) {
    // this wave's loads of stage kt are done once at most those of the stages
    // issued after it (up to NS - 2, PER instructions each) are outstanding
    const int after = min(NS - 2, nk - 1 - kt);
    if (NS >= 5 && after >= 3) __builtin_amdgcn_s_waitcnt(waitcnt_vm(3 * PER));
    else if (after >= 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * PER));
    else if (after == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(PER));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_barrier();
    // every wave has finished stage kt - 1, so its buffer takes stage kt + NS - 1
    if (kt + NS - 1 < nk) issue(kt + NS - 1);
    const uint16_t* as = smem + (kt % NS) * STAGE;
    const uint16_t* ws = as + BM * BK;
    u32x4_t fa[2][MT], fb[2][NT];
    auto rd = [&](int ks, int slot) __attribute__((always_inline)) {
      const int ch = ks * 2 + hi;
#pragma unroll
      for (int i = 0; i < MT; ++i) fa[slot][i] = *(const u32x4_t*)(&as[fat(wm * WM + i * 32 + l32, ch)]);
#pragma unroll
      for (int j = 0; j < NT; ++j) fb[slot][j] = *(const u32x4_t*)(&ws[fat(wn * WN + j * 32 + l32, ch)]);
    };
    rd(0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      if (ks + 1 < BK / 16) rd(ks + 1, (ks + 1) & 1);   // next k-step's fragments in flight
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = mfma32(fa[ks & 1][i], fb[ks & 1][j], acc[i][j]);
      if (ks + 1 < BK / 16) {
        // MFMAs and the next k-step's fragment reads, interleaved
        constexpr int RD = MT + NT, G = MT * NT, PERRD = G / RD > 0 ? G / RD : 1;
#pragma unroll
        for (int r2 = 0; r2 < RD; ++r2) {
          __builtin_amdgcn_sched_group_barrier(0x008, PERRD, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Epilogue through LDS: each wave owns a slice and moves its WM x WN block
  // out 32 rows at a time as full rows of 16-byte stores (N % 4 == 0, so a
  // 4-column chunk is entirely inside or outside the matrix).
  __syncthreads();   // every wave is done reading the pipeline stages
  constexpr int ES = WN + 4;          // floats per staged row (16-byte pad)
  constexpr int CPRW = WN / 4;        // 4-column chunks per row
  static_assert(NW * (32 * ES + 64) * 4 <= NS * STAGE * 2, "epilogue staging fits");
  static_assert(64 % CPRW == 0, "a lane keeps one column chunk");
  float* stg = (float*)smem + wave * (32 * ES + 64);
  // A lane stores the same 4-column chunk in every row it handles, so its
  // bias is loaded once. Loads never sit behind the row/column predicate
  // (the residual address is clamped instead): a load under a branch is
  // waited for before the branch closes, serialising the whole epilogue.
  const int c4 = (lane % CPRW) * 4;
  const int64_t n = n0 + wn * WN + c4;
  const bool col_ok = n < N;
  const int64_t nc = min(n, (int64_t)N - 4);
  float4 bv = make_float4(0.f, 0.f, 0.f, 0.f);
  if (bias) bv = *(const float4*)(bias + nc);
  // Residual epilogue: the residual rows of slice i + 1 are loaded while
  // slice i is staged and stored (double-buffered), so the reads overlap.
  // The node-table residual (three row gathers and the index arithmetic per
  // row) does not fit twice in the register budget: it is loaded per slice,
  // before the slice is staged, so the staging overlaps its reads, and only
  // its token ids are read ahead.
  constexpr int U = 32 * CPRW / 64;
  constexpr int RB = EPI == EPI_NODE ? 1 : 2;
  float4 rbuf[RB][RES ? U : 1];
  auto load_resid = [&](int i, float4 (&r)[RES ? U : 1]) __attribute__((always_inline)) {
    if constexpr (EPI == EPI_RESID_F32) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t m = m0 + wm * WM + i * 32 + (lane + 64 * u) / CPRW;
        r[u] = *(const float4*)(resid + min(m, (int64_t)M - 1) * N + nc);
      }
    }
  };
  // The node-table residual's token ids (the first of its two dependent
  // gathers) are read one slice ahead; the E, S and R rows at use.
  int tbuf[EPI == EPI_NODE ? U : 1];
  auto load_tok = [&](int i) __attribute__((always_inline)) {
    if constexpr (EPI == EPI_NODE) {
#pragma unroll
      for (int u = 0; u < U; ++u)
        tbuf[u] = node_token(node, (uint32_t)min(m0 + wm * WM + i * 32 + (lane + 64 * u) / CPRW, (int64_t)M - 1));
    }
  };
  auto load_node = [&](int i, float4 (&r)[RES ? U : 1]) __attribute__((always_inline)) {
    if constexpr (EPI == EPI_NODE) {
#pragma unroll
      for (int u = 0; u < U; ++u)
        r[u] = node_sum4(node, (uint32_t)min(m0 + wm * WM + i * 32 + (lane + 64 * u) / CPRW, (int64_t)M - 1),
                         tbuf[u], nc, N);
    }
  };
  // Whole tiles (the wave-uniform common case) store with no predicate at
  // all: a predicated store sits in its own exec branch, and the wait the
  // compiler puts at its head (for a bias or residual load that may still be
  // outstanding on the skipped path) also waits for every earlier store.
  const bool full = m0 + BM <= M && n0 + BN <= N;
  auto slices = [&](auto full_tag) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_tag)::value;
    if constexpr (RB == 2) load_resid(0, rbuf[0]);
    if constexpr (EPI == EPI_NODE) load_tok(0);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      if constexpr (RB == 2) {
        if (i + 1 < MT) load_resid(i + 1, rbuf[(i + 1) & 1]);
      } else {
        load_node(i, rbuf[0]);
        if (i + 1 < MT) load_tok(i + 1);
      }
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          stg[(8 * (e >> 2) + 4 * hi + (e & 3)) * ES + j * 32 + l32] = acc[i][j][e];
      __builtin_amdgcn_wave_barrier();
      // the slice's staged values are read together, except in the residual
      // epilogue, whose double-buffered residual rows leave no registers
      constexpr int UY = RES ? 1 : U;
      float4 ys[UY];
      if constexpr (UY > 1) {
#pragma unroll
        for (int u = 0; u < U; ++u) ys[u] = *(const float4*)(&stg[((lane + 64 * u) / CPRW) * ES + c4]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int rr = (lane + 64 * u) / CPRW;
        const int64_t m = m0 + wm * WM + i * 32 + rr;
        const bool ok = FULL || (col_ok && m < M);
        float4 y = UY > 1 ? ys[u % UY] : *(const float4*)(&stg[rr * ES + c4]);
        y.x += bv.x; y.y += bv.y; y.z += bv.z; y.w += bv.w;
        const int64_t o = m * N + n;
        if constexpr (EPI == EPI_F32) {
          if (ok) *(float4*)((float*)out + o) = y;
        } else if constexpr (EPI == EPI_BF16) {
          if (ok) *(uint2*)((uint16_t*)out + o) = make_uint2(pack_bf16x2(y.x, y.y), pack_bf16x2(y.z, y.w));
        } else if constexpr (EPI == EPI_SILU_BF16) {
          if (ok)
            *(uint2*)((uint16_t*)out + o) =
                make_uint2(pack_bf16x2(silu(y.x), silu(y.y)), pack_bf16x2(silu(y.z), silu(y.w)));
        } else {
          const float4 rv = rbuf[RB == 2 ? (i & 1) : 0][u];
          if (ok) *(float4*)((float*)out + o) = make_float4(rv.x + y.x, rv.y + y.y, rv.z + y.z, rv.w + y.w);
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  };
  if (full) slices(std::true_type{});
  else slices(std::false_type{});
}

template <int BM, int BN, int NW = 4>
hipError_t launch_dma(const uint16_t* A, int M, int Kd, const uint16_t* W, int N, const float* bias,
                      int epi, const float* resid, void* out, hipStream_t stream,
                      const NodeSource* node = nullptr) {
  const NodeSource nd = node ? *node : NodeSource{};
  const int tiles_n = (N + BN - 1) / BN;
  const int ntiles = ((M + BM - 1) / BM) * tiles_n;
  const dim3 grid((unsigned)ntiles), block(64 * NW);
  switch (epi) {
    case EPI_F32:
      hipLaunchKernelGGL((gemm_dma_kernel<BM, BN, EPI_F32, NW>), grid, block, 0, stream, A, W, M, N,
                         Kd, bias, resid, out, tiles_n, ntiles, nd);
      break;
    case EPI_BF16:
      hipLaunchKernelGGL((gemm_dma_kernel<BM, BN, EPI_BF16, NW>), grid, block, 0, stream, A, W, M, N,
                         Kd, bias, resid, out, tiles_n, ntiles, nd);
      break;
    case EPI_SILU_BF16:
      hipLaunchKernelGGL((gemm_dma_kernel<BM, BN, EPI_SILU_BF16, NW>), grid, block, 0, stream, A, W,
                         M, N, Kd, bias, resid, out, tiles_n, ntiles, nd);
      break;
    default:
      if (node)
        hipLaunchKernelGGL((gemm_dma_kernel<BM, BN, EPI_NODE, NW>), grid, block, 0, stream, A, W,
                           M, N, Kd, bias, resid, out, tiles_n, ntiles, nd);
      else
        hipLaunchKernelGGL((gemm_dma_kernel<BM, BN, EPI_RESID_F32, NW>), grid, block, 0, stream, A, W,
                           M, N, Kd, bias, resid, out, tiles_n, ntiles, nd);
      break;
  }
  return hipGetLastError();
}

template <int EPI>
__device__ __forceinline__ void epilogue_store(void* out, const float* resid, int64_t o, float y) {
  if constexpr (EPI == EPI_F32) {
    ((float*)out)[o] = y;
  } else if constexpr (EPI == EPI_BF16) {
    ((uint16_t*)out)[o] = (uint16_t)f32_to_bf16(y);
  } else if constexpr (EPI == EPI_SILU_BF16) {
    ((uint16_t*)out)[o] = (uint16_t)f32_to_bf16(silu(y));
  } else {
    ((float*)out)[o] = resid[o] + y;
  }
}

// Split-K partial products for few rows: block (tile, s) writes
// part[s][m][n] for its BM x BN tile over k in [s*KS, (s+1)*KS). The A and W
// slices sit unpadded in LDS with the 16-byte chunk index XOR-swizzled by the
// row, so the 16 rows an MFMA fragment read touches hit distinct banks and
// two 80 KiB workgroups fit on one CU.
template <int BM, int BN, int KS>
__global__ __launch_bounds__(256) void gemm_part_kernel(const uint16_t* __restrict__ A,
                                                        const uint16_t* __restrict__ W, int M, int N,
                                                        int Kd, float* __restrict__ part,
                                                        int tiles_n) {
  constexpr int CPR = KS / 8;                  // 16-byte chunks per row
  constexpr int SWM = CPR >= 16 ? 15 : CPR - 1;
  constexpr int MT = BM / 32, NT = BN / 32;
  constexpr int CH_A = BM * CPR, CH_W = BN * CPR;
  constexpr int NCH = (CH_A + CH_W) / 256;
  static_assert((CH_A + CH_W) % 256 == 0, "chunking");
  // the A and W slices, later the fp32 tile (row-major, 4-float pad) staged for the stores
  constexpr int ES = BN + 4;
  constexpr int SMEM = (BM + BN) * KS > BM * ES * 2 ? (BM + BN) * KS : BM * ES * 2;
  __shared__ __attribute__((aligned(16))) uint16_t smem[SMEM];
  uint16_t* As = smem;
  uint16_t* Ws = smem + BM * KS;
  auto at = [](int row, int chunk) { return row * KS + ((chunk ^ (row & SWM)) << 3); };

  const int tile = blockIdx.x, s = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 4, c = lane & 15;
  const int64_t m0 = (int64_t)(tile / tiles_n) * BM, n0 = (int64_t)(tile % tiles_n) * BN;
  const int64_t k0 = (int64_t)s * KS;

  // Every load is issued unconditionally (rows past the matrix are clamped to
  // its last row; their products land in rows that are never stored), so all
  // of them are in flight together: one memory round trip per workgroup.
  u32x4_t r[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int ch = tid + 256 * i;
    const uint16_t* src;
    if (ch < CH_A) {   // uniform per i: CH_A is a multiple of 256
      const int64_t gm = min(m0 + ch / CPR, (int64_t)M - 1);
      src = A + gm * Kd + k0 + (ch % CPR) * 8;
    } else {
      const int cw = ch - CH_A;
      const int64_t gn = min(n0 + cw / CPR, (int64_t)N - 1);
      src = W + gn * Kd + k0 + (cw % CPR) * 8;
    }
    r[i] = *(const u32x4_t*)src;
  }
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int ch = tid + 256 * i;
    if (ch < CH_A)
      *(u32x4_t*)(&As[at(ch / CPR, ch % CPR)]) = r[i];
    else
      *(u32x4_t*)(&Ws[at((ch - CH_A) / CPR, (ch - CH_A) % CPR)]) = r[i];
  }
  __syncthreads();

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < KS; kk += 32) {
    u32x4_t af[MT], bfr[NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
      af[i] = *(const u32x4_t*)(&As[at(wm * (BM / 2) + i * 16 + c, kk / 8 + g)]);
#pragma unroll
    for (int j = 0; j < NT; ++j)
      bfr[j] = *(const u32x4_t*)(&Ws[at(wn * (BN / 2) + j * 16 + c, kk / 8 + g)]);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[i][j] = mfma16(af[i], bfr[j], acc[i][j]);
  }

  // The tile goes out through LDS (row-major, 4-float pad) as 16-byte row
  // stores; N % 4 == 0, so a 4-column chunk is entirely inside or outside.
  __syncthreads();   // every wave is done with the A and W slices
  float* stg = (float*)smem;
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
        stg[(wm * (BM / 2) + i * 16 + 4 * g + qq) * ES + wn * (BN / 2) + j * 16 + c] = acc[i][j][qq];
  __syncthreads();
  float* ps = part + (int64_t)s * M * N;
  constexpr int C4 = BN / 4;
#pragma unroll
  for (int u = 0; u < BM * C4 / 256; ++u) {
    const int idx = tid + 256 * u, row = idx / C4, c4 = (idx % C4) * 4;
    const int64_t m = m0 + row, n = n0 + c4;
    if (m < M && n < N) *(float4*)(ps + m * N + n) = *(const float4*)(&stg[row * ES + c4]);
  }
}

// Few-row linear (M <= 128): one workgroup of four waves per 16 output
// columns over the whole of K, so there are no split-K partials and the
// epilogue is fused. Every workgroup streams all of A, so the kernel is bound
// by how fast A reaches each CU: A and the 16 W rows go through LDS in
// 128-wide K stages by global_load_lds, three stages ahead of the one being
// multiplied; each DMA instruction moves four whole 256-byte row segments
// (full cache lines), with the 16-byte chunk index XOR-swizzled by the row so
// that fragment reads touch every bank once. Wave w multiplies rows
// 32 w .. 32 w + 31 (two 16-row MFMA tiles) against the 16 columns. Rows and
// columns past the matrix are clamped on load and never stored.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(const uint16_t* __restrict__ A,
                                                          const uint16_t* __restrict__ W, int M,
                                                          int N, int Kd,
                                                          const float* __restrict__ bias,
                                                          const float* resid, void* out) {
  constexpr int BM = 128, BN = 16, BK = 128, NS = 4;
  constexpr int STAGE = (BM + BN) * BK;        // bf16 elements per stage
  constexpr int NI = STAGE / 512;              // 1 KiB DMA instructions per stage (36)
  constexpr int PER = NI / 4;                  // per wave (9)
  static_assert(NI % 4 == 0, "stage split");
  __shared__ __attribute__((aligned(1024))) uint16_t smem[NS * STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int64_t n0 = (int64_t)blockIdx.x * BN;

  // Instruction j of a stage fills elements [512 j, 512 j + 512): rows
  // 4 j .. 4 j + 3 of the stage (A rows first, then the W rows); lane i
  // fills row 4 j + i / 16, slot i % 16, which holds chunk (i % 16) ^ (row & 15).
  const uint16_t* src[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int j = wave * PER + u, row = 4 * j + lane / 16;
    const int chunk = (lane % 16) ^ (row & 15);
    src[u] = row < BM ? A + (int64_t)min(row, M - 1) * Kd + chunk * 8
                      : W + min(n0 + (row - BM), (int64_t)N - 1) * Kd + chunk * 8;
  }
  auto issue = [&](int kt) __attribute__((always_inline)) {
    uint16_t* st = smem + (kt % NS) * STAGE;
#pragma unroll
    for (int u = 0; u < PER; ++u)
      __builtin_amdgcn_global_load_lds((const void*)(src[u] + kt * BK),
                                       (__attribute__((address_space(3))) void*)(st + (wave * PER + u) * 512),
                                       16, 0, 0);
  };
  auto at = [](int row, int chunk) { return row * BK + ((chunk ^ (row & 15)) << 3); };

  f32x4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  const int nk = Kd / BK;
  issue(0);
  if (nk > 1) issue(1);
  if (nk > 2) issue(2);
  for (int kt = 0; kt < nk; ++kt) {
    // this wave's loads of stage kt are done once at most those of the
    // stages issued after it are outstanding; the barrier makes them visible
    if (kt + 2 < nk) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * PER));
    else if (kt + 1 < nk) __builtin_amdgcn_s_waitcnt(waitcnt_vm(PER));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_barrier();
    // every wave is done with stage kt - 1, whose buffer takes stage kt + 3
    if (kt + 3 < nk) issue(kt + 3);
    const uint16_t* st = smem + (kt % NS) * STAGE;
    u32x4_t fa[BK / 32][2], fw[BK / 32];
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
#pragma unroll
      for (int i = 0; i < 2; ++i) fa[ks][i] = *(const u32x4_t*)(&st[at(wave * 32 + i * 16 + c, ks * 4 + g)]);
      fw[ks] = *(const u32x4_t*)(&st[at(BM + c, ks * 4 + g)]);
    }
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks)
#pragma unroll
      for (int i = 0; i < 2; ++i) acc[i] = mfma16(fa[ks][i], fw[ks], acc[i]);
  }
  // acc[i][q]: row 32 w + 16 i + 4 g + q, column n0 + c
  const int64_t n = n0 + c, nc = min(n, (int64_t)N - 1);
  const float bv = bias ? bias[nc] : 0.f;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t m = wave * 32 + i * 16 + 4 * g + q;
      const bool ok = m < M && n < N;
      const float y = acc[i][q] + bv;
      const int64_t o = m * N + n;
      if constexpr (EPI == EPI_F32) {
        if (ok) ((float*)out)[o] = y;
      } else if constexpr (EPI == EPI_BF16) {
        if (ok) ((uint16_t*)out)[o] = (uint16_t)f32_to_bf16(y);
      } else if constexpr (EPI == EPI_SILU_BF16) {
        if (ok) ((uint16_t*)out)[o] = (uint16_t)f32_to_bf16(silu(y));
      } else {
        const float r = resid[min(m, (int64_t)M - 1) * N + nc];
        if (ok) ((float*)out)[o] = r + y;
      }
    }
}

// The same pass for 65..128 rows on 64 x 32 tiles: workgroup (x, y) takes
// columns 32 x .. 32 x + 31 of rows 64 y .. 64 y + 63. Each workgroup then
// streams 64 rows of A and 32 of W (192 KiB at K = 1,024) instead of all 128
// rows of A and 16 of W (288 KiB), with as many workgroups; the per-CU rate
// of these streams, not the L2 total, bounds the pass. Wave w multiplies rows
// 16 w .. 16 w + 15 against both 16-column halves. The two row halves of a
// column tile are tiles_n apart in launch order, which is a multiple of 8 for
// the encoder's widths, so they run on one XCD and W is read from HBM once.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_skinny2_kernel(const uint16_t* __restrict__ A,
                                                           const uint16_t* __restrict__ W, int M,
                                                           int N, int Kd,
                                                           const float* __restrict__ bias,
                                                           const float* resid, void* out) {
  constexpr int BM = 64, BN = 32, BK = 128, NS = 4;
  constexpr int STAGE = (BM + BN) * BK;        // bf16 elements per stage
  constexpr int NI = STAGE / 512;              // 1 KiB DMA instructions per stage (24)
  constexpr int PER = NI / 4;                  // per wave (6)
  static_assert(NI % 4 == 0, "stage split");
  __shared__ __attribute__((aligned(1024))) uint16_t smem[NS * STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int64_t n0 = (int64_t)blockIdx.x * BN, m0 = (int64_t)blockIdx.y * BM;

  // Instruction j of a stage fills elements [512 j, 512 j + 512): rows
  // 4 j .. 4 j + 3 of the stage (A rows first, then the W rows); lane i
  // fills row 4 j + i / 16, slot i % 16, which holds chunk (i % 16) ^ (row & 15).
  const uint16_t* src[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int j = wave * PER + u, row = 4 * j + lane / 16;
    const int chunk = (lane % 16) ^ (row & 15);
    src[u] = row < BM ? A + min(m0 + row, (int64_t)M - 1) * Kd + chunk * 8
                      : W + min(n0 + (row - BM), (int64_t)N - 1) * Kd + chunk * 8;
  }
  auto issue = [&](int kt) __attribute__((always_inline)) {
    uint16_t* st = smem + (kt % NS) * STAGE;
#pragma unroll
    for (int u = 0; u < PER; ++u)
      __builtin_amdgcn_global_load_lds((const void*)(src[u] + kt * BK),
                                       (__attribute__((address_space(3))) void*)(st + (wave * PER + u) * 512),
                                       16, 0, 0);
  };
  auto at = [](int row, int chunk) { return row * BK + ((chunk ^ (row & 15)) << 3); };

  f32x4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  const int nk = Kd / BK;
  issue(0);
  if (nk > 1) issue(1);
  if (nk > 2) issue(2);
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 2 < nk) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * PER));
    else if (kt + 1 < nk) __builtin_amdgcn_s_waitcnt(waitcnt_vm(PER));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_barrier();
    if (kt + 3 < nk) issue(kt + 3);
    const uint16_t* st = smem + (kt % NS) * STAGE;
    u32x4_t fa[BK / 32], fw[BK / 32][2];
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      fa[ks] = *(const u32x4_t*)(&st[at(wave * 16 + c, ks * 4 + g)]);
#pragma unroll
      for (int j = 0; j < 2; ++j) fw[ks][j] = *(const u32x4_t*)(&st[at(BM + j * 16 + c, ks * 4 + g)]);
    }
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[j] = mfma16(fa[ks], fw[ks][j], acc[j]);
  }
  // acc[j][q]: row m0 + 16 w + 4 g + q, column n0 + 16 j + c
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t n = n0 + 16 * j + c, nc = min(n, (int64_t)N - 1);
    const float bv = bias ? bias[nc] : 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t m = m0 + wave * 16 + 4 * g + q;
      const bool ok = m < M && n < N;
      const float y = acc[j][q] + bv;
      const int64_t o = m * N + n;
      if constexpr (EPI == EPI_F32) {
        if (ok) ((float*)out)[o] = y;
      } else if constexpr (EPI == EPI_BF16) {
        if (ok) ((uint16_t*)out)[o] = (uint16_t)f32_to_bf16(y);
      } else if constexpr (EPI == EPI_SILU_BF16) {
        if (ok) ((uint16_t*)out)[o] = (uint16_t)f32_to_bf16(silu(y));
      } else {
        const float r = resid[min(m, (int64_t)M - 1) * N + nc];
        if (ok) ((float*)out)[o] = r + y;
      }
    }
  }
}

// Partial sums are added in the fixed order s = 0..S-1; S is a compile-time
// constant so the S loads of a group are issued together.
template <int S>
__device__ __forceinline__ float4 splitk_sum4(const float4* __restrict__ part4, int64_t MN4,
                                              int64_t q) {
  float4 v = part4[q];
#pragma unroll
  for (int s = 1; s < S; ++s) {
    const float4 p = part4[(int64_t)s * MN4 + q];
    v.x += p.x;
    v.y += p.y;
    v.z += p.z;
    v.w += p.w;
  }
  return v;
}

template <int EPI>
__device__ __forceinline__ void store4(void* out, const float* resid, int64_t o, float4 y) {
  if constexpr (EPI == EPI_F32) {
    *(float4*)((float*)out + o) = y;
  } else if constexpr (EPI == EPI_RESID_F32) {
    const float4 r = *(const float4*)(resid + o);
    *(float4*)((float*)out + o) = make_float4(r.x + y.x, r.y + y.y, r.z + y.z, r.w + y.w);
  } else if constexpr (EPI == EPI_BF16) {
    *(uint2*)((uint16_t*)out + o) = make_uint2(pack_bf16x2(y.x, y.y), pack_bf16x2(y.z, y.w));
  } else {
    *(uint2*)((uint16_t*)out + o) =
        make_uint2(pack_bf16x2(silu(y.x), silu(y.y)), pack_bf16x2(silu(y.z), silu(y.w)));
  }
}

// Plain epilogues, 4 consecutive outputs per thread (N % 4 == 0).
template <int EPI, int S>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int M,
                                                            int N, const float* __restrict__ bias,
                                                            const float* resid, void* out) {
  const int64_t MN4 = (int64_t)M * N / 4;
  const float4* part4 = (const float4*)part;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < MN4; q += (int64_t)gridDim.x * blockDim.x) {
    float4 v = splitk_sum4<S>(part4, MN4, q);
    const int n = (int)((q * 4) % N);
    if (bias) {
      const float4 b = *(const float4*)(bias + n);
      v.x += b.x;
      v.y += b.y;
      v.z += b.z;
      v.w += b.w;
    }
    store4<EPI>(out, resid, q * 4, v);
  }
}

// Residual add fused with the RMSNorm that follows it: one 256-thread
// workgroup per row (few rows here, so the row is spread over four waves),
// x = resid + (y + bias) written back, then u = bf16(x * rstd * gamma).
// Thread t holds the 4-column groups t, t + 256, ...; the sum of squares is
// reduced per wave, then over the four waves in a fixed order.
template <int S, int NV, bool NODE = false>
__global__ __launch_bounds__(256) void splitk_resid_rmsnorm_kernel(
    const float* __restrict__ part, int M, int N, const float* __restrict__ bias,
    const float* resid, float* x_out, const float* __restrict__ gamma, float eps,
    uint16_t* __restrict__ u_out, NodeSource node) {
  __shared__ float red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t m = blockIdx.x;
  const int64_t MN4 = (int64_t)M * N / 4;
  const int n4 = N / 4;
  const float4* part4 = (const float4*)part;
  // Loads use clamped indices and are unconditional, so every column group's
  // partials, bias, residual and gamma are in flight at once; only the
  // stores and the sum are predicated.
  float4 v[NV], gv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int gi = tid + 256 * i;
    const int gc = min(gi, n4 - 1);
    const int64_t q = m * n4 + gc;
    const float4 y = splitk_sum4<S>(part4, MN4, q);
    const float4 b = bias ? ((const float4*)bias)[gc] : make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 r = NODE ? node_resid4(node, (uint32_t)m, (int64_t)gc * 4, N) : ((const float4*)resid)[q];
    gv[i] = ((const float4*)gamma)[gc];
    v[i] = make_float4(r.x + (y.x + b.x), r.y + (y.y + b.y), r.z + (y.z + b.z), r.w + (y.w + b.w));
    if (gi >= n4) v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int gi = tid + 256 * i;
    if (gi < n4) ((float4*)x_out)[m * n4 + gi] = v[i];
    ss = fmaf(v[i].x, v[i].x, ss);
    ss = fmaf(v[i].y, v[i].y, ss);
    ss = fmaf(v[i].z, v[i].z, ss);
    ss = fmaf(v[i].w, v[i].w, ss);
  }
  ss = wave_sum(ss);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  ss = ((red[0] + red[1]) + red[2]) + red[3];
  const float rstd = 1.0f / __fsqrt_rn(ss / (float)N + eps);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int gi = tid + 256 * i;
    if (gi < n4)
      ((uint2*)(u_out + m * N))[gi] =
          make_uint2(pack_bf16x2(v[i].x * rstd * gv[i].x, v[i].y * rstd * gv[i].y),
                     pack_bf16x2(v[i].z * rstd * gv[i].z, v[i].w * rstd * gv[i].w));
  }
}

// Out/in heads: y = A W^T + b over N = 2 d_e, each half normalised to unit
// length and rounded to bf16, stored in row heads_row(m, group, skip). One
// wave per row; d_e % 4 == 0. With S = 1 and no bias it normalises rows the
// many-row GEMM has already finished (16-byte loads, a whole row per wave).
template <int S, int NV>
__global__ __launch_bounds__(256) void splitk_heads_l2norm_kernel(
    const float* __restrict__ part, int M, int de, const float* __restrict__ bias,
    uint16_t* __restrict__ outv, uint16_t* __restrict__ inv, int group, int skip) {
  const int lane = threadIdx.x & 63;
  const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  const int N = 2 * de, n4 = N / 4, h4 = de / 4;
  const int64_t MN4 = (int64_t)M * n4;
  const float4* part4 = (const float4*)part;
  float4 v[NV];
  float ss0 = 0.f, ss1 = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int gi = lane + 64 * i;
    const int gc = min(gi, n4 - 1);   // clamped: loads stay unconditional
    const float4 y = splitk_sum4<S>(part4, MN4, m * n4 + gc);
    const float4 b = bias ? ((const float4*)bias)[gc] : make_float4(0.f, 0.f, 0.f, 0.f);
    v[i] = make_float4(y.x + b.x, y.y + b.y, y.z + b.z, y.w + b.w);
    if (gi >= n4) v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int gi = lane + 64 * i;
    const float sq = v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
    if (gi < h4) ss0 += sq; else ss1 += sq;
  }
  const float n0 = fmaxf(__fsqrt_rn(wave_sum(ss0)), 1e-12f);
  const float n1 = fmaxf(__fsqrt_rn(wave_sum(ss1)), 1e-12f);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int gi = lane + 64 * i;
    if (gi < n4) {
      const bool hi = gi >= h4;
      const float nr = hi ? n1 : n0;
      uint16_t* dst = (hi ? inv : outv) + heads_row(m, group, skip) * de + (hi ? gi - h4 : gi) * 4;
      *(uint2*)dst = make_uint2(pack_bf16x2(__fdiv_rn(v[i].x, nr), __fdiv_rn(v[i].y, nr)),
                                pack_bf16x2(__fdiv_rn(v[i].z, nr), __fdiv_rn(v[i].w, nr)));
    }
  }
}

// The same for wide heads over few rows (N = 2 d_e > 256): one 256-thread
// workgroup per row, thread t holding the 4-column groups t, t + 256, ...;
// each half's sum of squares is reduced per wave, then over the four waves in
// a fixed order (a wave per row left most CUs idle at one block).
template <int S, int NV>
__global__ __launch_bounds__(256) void splitk_heads_l2norm_row_kernel(
    const float* __restrict__ part, int M, int de, const float* __restrict__ bias,
    uint16_t* __restrict__ outv, uint16_t* __restrict__ inv, int group, int skip) {
  __shared__ float red[4][2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t m = blockIdx.x;
  const int N = 2 * de, n4 = N / 4, h4 = de / 4;
  const int64_t MN4 = (int64_t)M * n4;
  const float4* part4 = (const float4*)part;
  float4 v[NV];
  float ss0 = 0.f, ss1 = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int gi = tid + 256 * i;
    const int gc = min(gi, n4 - 1);   // clamped: loads stay unconditional
    const float4 y = splitk_sum4<S>(part4, MN4, m * n4 + gc);
    const float4 b = bias ? ((const float4*)bias)[gc] : make_float4(0.f, 0.f, 0.f, 0.f);
    v[i] = make_float4(y.x + b.x, y.y + b.y, y.z + b.z, y.w + b.w);
    if (gi >= n4) v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int gi = tid + 256 * i;
    const float sq = v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
    if (gi < h4) ss0 += sq; else ss1 += sq;
  }
  ss0 = wave_sum(ss0);
  ss1 = wave_sum(ss1);
  if (lane == 0) {
    red[wave][0] = ss0;
    red[wave][1] = ss1;
  }
  __syncthreads();
  const float t0 = ((red[0][0] + red[1][0]) + red[2][0]) + red[3][0];
  const float t1 = ((red[0][1] + red[1][1]) + red[2][1]) + red[3][1];
  const float n0 = fmaxf(__fsqrt_rn(t0), 1e-12f);
  const float n1 = fmaxf(__fsqrt_rn(t1), 1e-12f);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int gi = tid + 256 * i;
    if (gi < n4) {
      const bool hi = gi >= h4;
      const float nr = hi ? n1 : n0;
      uint16_t* dst = (hi ? inv : outv) + heads_row(m, group, skip) * de + (hi ? gi - h4 : gi) * 4;
      *(uint2*)dst = make_uint2(pack_bf16x2(__fdiv_rn(v[i].x, nr), __fdiv_rn(v[i].y, nr)),
                                pack_bf16x2(__fdiv_rn(v[i].z, nr), __fdiv_rn(v[i].w, nr)));
    }
  }
}

template <int BM, int BN>
hipError_t launch_tile(const uint16_t* A, int M, int Kd, const uint16_t* W, int N,
                       const float* bias, int epi, const float* resid, void* out,
                       hipStream_t stream) {
  dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
  switch (epi) {
    case EPI_F32:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, EPI_F32>), grid, dim3(256), 0, stream, A, W, M, N,
                         Kd, bias, resid, out);
      break;
    case EPI_BF16:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, EPI_BF16>), grid, dim3(256), 0, stream, A, W, M, N,
                         Kd, bias, resid, out);
      break;
    case EPI_SILU_BF16:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, EPI_SILU_BF16>), grid, dim3(256), 0, stream, A, W,
                         M, N, Kd, bias, resid, out);
      break;
    default:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, EPI_RESID_F32>), grid, dim3(256), 0, stream, A, W,
                         M, N, Kd, bias, resid, out);
      break;
  }
  return hipGetLastError();
}

template <int KS>
hipError_t launch_part(const uint16_t* A, int M, int Kd, const uint16_t* W, int N, float* part,
                       int S, int bm, int bn, hipStream_t stream) {
  if (bm == 128) {
    const int tiles_n = (N + 31) / 32;
    const dim3 grid((unsigned)(((M + 127) / 128) * tiles_n), (unsigned)S);
    hipLaunchKernelGGL((gemm_part_kernel<128, 32, KS>), grid, dim3(256), 0, stream, A, W, M, N, Kd,
                       part, tiles_n);
  } else if (bn == 64) {
    const int tiles_n = (N + 63) / 64;
    const dim3 grid((unsigned)(((M + 63) / 64) * tiles_n), (unsigned)S);
    hipLaunchKernelGGL((gemm_part_kernel<64, 64, KS>), grid, dim3(256), 0, stream, A, W, M, N, Kd,
                       part, tiles_n);
  } else {
    const int tiles_n = (N + 31) / 32;
    const dim3 grid((unsigned)(((M + 63) / 64) * tiles_n), (unsigned)S);
    hipLaunchKernelGGL((gemm_part_kernel<64, 32, KS>), grid, dim3(256), 0, stream, A, W, M, N, Kd,
                       part, tiles_n);
  }
  return hipGetLastError();
}

template <int S>
hipError_t launch_reduce(int M, int N, const float* bias, const LinearEpilogue& ep, void* out,
                         const float* part, hipStream_t stream) {
  const unsigned row_blocks = (unsigned)((M + 3) / 4);
  if (ep.kind == EPI_RESID_F32 && ep.norm_out) {
    const NodeSource nd = ep.node ? *ep.node : NodeSource{};
#define LL_RRN(NV)                                                                                 \
  do {                                                                                             \
    if (ep.node)                                                                                   \
      hipLaunchKernelGGL((splitk_resid_rmsnorm_kernel<S, NV, true>), dim3((unsigned)M), dim3(256), 0, \
                         stream, part, M, N, bias, ep.resid, (float*)out, ep.norm_gamma, ep.eps,    \
                         ep.norm_out, nd);                                                         \
    else                                                                                           \
      hipLaunchKernelGGL((splitk_resid_rmsnorm_kernel<S, NV, false>), dim3((unsigned)M), dim3(256), 0, \
                         stream, part, M, N, bias, ep.resid, (float*)out, ep.norm_gamma, ep.eps,    \
                         ep.norm_out, nd);                                                         \
  } while (0)
    if (N <= 1024) LL_RRN(1);
    else if (N <= 2048) LL_RRN(2);
    else LL_RRN(4);
#undef LL_RRN
    return hipGetLastError();
  }
  if (ep.kind == EPI_F32 && ep.heads_out) {
    if (N > 256 && N <= 2048 && M < 1024) {
      // wide vectors, few rows: a workgroup per row
      if (N <= 1024)
        hipLaunchKernelGGL((splitk_heads_l2norm_row_kernel<S, 1>), dim3((unsigned)M), dim3(256), 0, stream,
                           part, M, N / 2, bias, ep.heads_out, ep.heads_in, ep.heads_group, ep.heads_skip);
      else
        hipLaunchKernelGGL((splitk_heads_l2norm_row_kernel<S, 2>), dim3((unsigned)M), dim3(256), 0, stream,
                           part, M, N / 2, bias, ep.heads_out, ep.heads_in, ep.heads_group, ep.heads_skip);
      return hipGetLastError();
    }
    if (N <= 256)
      hipLaunchKernelGGL((splitk_heads_l2norm_kernel<S, 1>), dim3(row_blocks), dim3(256), 0, stream,
                         part, M, N / 2, bias, ep.heads_out, ep.heads_in, ep.heads_group,
                         ep.heads_skip);
    else if (N <= 1024)
      hipLaunchKernelGGL((splitk_heads_l2norm_kernel<S, 4>), dim3(row_blocks), dim3(256), 0, stream,
                         part, M, N / 2, bias, ep.heads_out, ep.heads_in, ep.heads_group,
                         ep.heads_skip);
    else
      hipLaunchKernelGGL((splitk_heads_l2norm_kernel<S, 8>), dim3(row_blocks), dim3(256), 0, stream,
                         part, M, N / 2, bias, ep.heads_out, ep.heads_in, ep.heads_group,
                         ep.heads_skip);
    return hipGetLastError();
  }
  const int64_t MN4 = (int64_t)M * N / 4;
  // 64-thread workgroups when 256-thread ones would leave most CUs idle (one
  // output group per thread either way; few rows: the S loads of a group are
  // the whole per-thread work)
  const int tpb = (MN4 + 255) / 256 < 256 ? 64 : 256;
  const unsigned blocks = (unsigned)std::min<int64_t>((MN4 + tpb - 1) / tpb, 4096);
  switch (ep.kind) {
    case EPI_F32:
      hipLaunchKernelGGL((splitk_reduce_kernel<EPI_F32, S>), dim3(blocks), dim3(tpb), 0, stream,
                         part, M, N, bias, ep.resid, out);
      break;
    case EPI_BF16:
      hipLaunchKernelGGL((splitk_reduce_kernel<EPI_BF16, S>), dim3(blocks), dim3(tpb), 0, stream,
                         part, M, N, bias, ep.resid, out);
      break;
    case EPI_SILU_BF16:
      hipLaunchKernelGGL((splitk_reduce_kernel<EPI_SILU_BF16, S>), dim3(blocks), dim3(tpb), 0,
                         stream, part, M, N, bias, ep.resid, out);
      break;
    default:
      hipLaunchKernelGGL((splitk_reduce_kernel<EPI_RESID_F32, S>), dim3(blocks), dim3(tpb), 0,
                         stream, part, M, N, bias, ep.resid, out);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_skinny(const uint16_t* A, int M, int Kd, const uint16_t* W, int N,
                         const float* bias, int epi, const float* resid, void* out,
                         hipStream_t stream) {
  if (M > 64) {
    const dim3 grid2((unsigned)((N + 31) / 32), (unsigned)((M + 63) / 64));
    switch (epi) {
      case EPI_F32:
        hipLaunchKernelGGL((gemm_skinny2_kernel<EPI_F32>), grid2, dim3(256), 0, stream, A, W, M, N, Kd,
                           bias, resid, out);
        break;
      case EPI_BF16:
        hipLaunchKernelGGL((gemm_skinny2_kernel<EPI_BF16>), grid2, dim3(256), 0, stream, A, W, M, N, Kd,
                           bias, resid, out);
        break;
      case EPI_SILU_BF16:
        hipLaunchKernelGGL((gemm_skinny2_kernel<EPI_SILU_BF16>), grid2, dim3(256), 0, stream, A, W, M,
                           N, Kd, bias, resid, out);
        break;
      default:
        hipLaunchKernelGGL((gemm_skinny2_kernel<EPI_RESID_F32>), grid2, dim3(256), 0, stream, A, W, M,
                           N, Kd, bias, resid, out);
        break;
    }
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((N + 15) / 16));
  switch (epi) {
    case EPI_F32:
      hipLaunchKernelGGL((gemm_skinny_kernel<EPI_F32>), grid, dim3(256), 0, stream, A, W, M, N, Kd,
                         bias, resid, out);
      break;
    case EPI_BF16:
      hipLaunchKernelGGL((gemm_skinny_kernel<EPI_BF16>), grid, dim3(256), 0, stream, A, W, M, N, Kd,
                         bias, resid, out);
      break;
    case EPI_SILU_BF16:
      hipLaunchKernelGGL((gemm_skinny_kernel<EPI_SILU_BF16>), grid, dim3(256), 0, stream, A, W, M,
                         N, Kd, bias, resid, out);
      break;
    default:
      hipLaunchKernelGGL((gemm_skinny_kernel<EPI_RESID_F32>), grid, dim3(256), 0, stream, A, W, M,
                         N, Kd, bias, resid, out);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_splitk_reduce(int S, int M, int N, const float* bias, const LinearEpilogue& ep,
                                void* out, const float* part, hipStream_t stream) {
  switch (S) {
    case 2: return launch_reduce<2>(M, N, bias, ep, out, part, stream);
    case 3: return launch_reduce<3>(M, N, bias, ep, out, part, stream);
    case 4: return launch_reduce<4>(M, N, bias, ep, out, part, stream);
    case 6: return launch_reduce<6>(M, N, bias, ep, out, part, stream);
    case 8: return launch_reduce<8>(M, N, bias, ep, out, part, stream);
    case 12: return launch_reduce<12>(M, N, bias, ep, out, part, stream);
    case 16: return launch_reduce<16>(M, N, bias, ep, out, part, stream);
    default: return hipErrorInvalidValue;
  }
}

bool uses_skinny(int M, int Kd, int N) {
  return M <= 128 && Kd % 128 == 0 && (N + 15) / 16 >= 128;
}

GemmPlan plan_linear(int M, int Kd, int N) {
  GemmPlan p{};
  p.split = 1;
  if (M >= 2048 || Kd < 128 || Kd % 64) return p;
  // 64 x 64 tiles above 64 rows: as many workgroups as 128 x 32 ones, each
  // staging 128 rows of A and W per K slice instead of 160
  p.bm = 64;
  p.bn = M > 64 ? 64 : 32;
  p.tiles = ((M + p.bm - 1) / p.bm) * ((N + p.bn - 1) / p.bn);
  // Widest K slice (<= 256, so the slice sits in LDS) that still gives about
  // 256 workgroups; at least two slices.
  int ks = 256;
  while (ks > 64 && (Kd % ks || (int64_t)p.tiles * (Kd / ks) < 256)) ks >>= 1;
  const int S = Kd / ks;
  // slice counts the reduce kernels are built for (3, 6 and 12 serve K = 3 x 2^k,
  // the fusion layer of the paper's head)
  const bool s_ok = S == 2 || S == 3 || S == 4 || S == 6 || S == 8 || S == 12 || S == 16;
  if (Kd % ks || !s_ok || N % 4) return p;
  p.ks = ks;
  p.split = Kd / ks;
  p.part_floats = (size_t)p.split * M * N;
  return p;
}

bool linear_takes_node_source(int M, int Kd, int N) {
  // the many-row DMA kernel (M >= 2048, K a multiple of 64, N of 4, aligned
  // operands) or the split-K row reduce (plan_linear splits K)
  if (M >= 2048) return Kd % 64 == 0 && N % 4 == 0;
  return plan_linear(M, Kd, N).split > 1;
}

hipError_t launch_linear(const uint16_t* A, int M, int Kd, const uint16_t* W, int N,
                         const float* bias, const LinearEpilogue& ep, void* out, float* part,
                         hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (ep.node && (ep.kind != EPI_RESID_F32 || !ep.norm_out || !linear_takes_node_source(M, Kd, N)))
    return hipErrorInvalidValue;
  // Few rows and enough 16-column tiles to occupy the GPU: one pass over K
  // with the epilogue fused (row-wide epilogues need whole rows: not here).
  if (uses_skinny(M, Kd, N) && ep.norm_out == nullptr && ep.heads_out == nullptr)
    return launch_skinny(A, M, Kd, W, N, bias, ep.kind, ep.resid, out, stream);
  const GemmPlan p = plan_linear(M, Kd, N);
  if (p.split == 1) {
    hipError_t e;
    const auto al16 = [](const void* ptr) { return ((uintptr_t)ptr & 15) == 0; };
    const auto tiles = [&](int bm, int bn) { return (int64_t)((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
    if (M >= 2048 && Kd % 64 == 0 && N % 4 == 0 && al16(out) && (bias == nullptr || al16(bias)) &&
        (ep.resid == nullptr || al16(ep.resid))) {
      const NodeSource* nd = ep.node;
      // the largest tile that still gives (nearly) every CU work
      // (eight waves, two per SIMD, for the large tiles: each wave then owns a
      // 128 x 64 or 128 x 32 block, and one wave's barrier wait overlaps the
      // other's MFMAs). Three quarters of the CUs busy with 256 x 256 tiles
      // beat all of them with 256 x 128 ones (QKV at 4,096 rows: 36 against
      // 43 us).
      if (tiles(256, 256) >= 192)
        e = launch_dma<256, 256, 8>(A, M, Kd, W, N, bias, ep.kind, ep.resid, out, stream, nd);
      else if (tiles(256, 128) >= 256)
        e = launch_dma<256, 128, 8>(A, M, Kd, W, N, bias, ep.kind, ep.resid, out, stream, nd);
      else if (tiles(128, 128) >= 384)
        e = launch_dma<128, 128, 4>(A, M, Kd, W, N, bias, ep.kind, ep.resid, out, stream, nd);
      else   // a few thousand rows of a narrow output: 128 x 64 tiles, three workgroups per CU
        e = launch_dma<128, 64, 4>(A, M, Kd, W, N, bias, ep.kind, ep.resid, out, stream, nd);
    } else if (ep.node) {
      return hipErrorInvalidValue;   // misaligned operands: no node-source kernel here
    } else if (M >= 2048)
      e = launch_tile<128, 128>(A, M, Kd, W, N, bias, ep.kind, ep.resid, out, stream);
    else if (M > 64)
      e = launch_tile<128, 32>(A, M, Kd, W, N, bias, ep.kind, ep.resid, out, stream);
    else
      e = launch_tile<64, 32>(A, M, Kd, W, N, bias, ep.kind, ep.resid, out, stream);
    if (e != hipSuccess) return e;
    if (ep.norm_out) return launch_rmsnorm((const float*)out, M, N, ep.norm_gamma, ep.eps, ep.norm_out, stream);
    if (ep.heads_out) {
      const dim3 grid((unsigned)((M + 3) / 4));
      const float* y = (const float*)out;
      if (N <= 256)
        hipLaunchKernelGGL((splitk_heads_l2norm_kernel<1, 1>), grid, dim3(256), 0, stream, y, M, N / 2,
                           nullptr, ep.heads_out, ep.heads_in, ep.heads_group, ep.heads_skip);
      else if (N <= 1024)
        hipLaunchKernelGGL((splitk_heads_l2norm_kernel<1, 4>), grid, dim3(256), 0, stream, y, M, N / 2,
                           nullptr, ep.heads_out, ep.heads_in, ep.heads_group, ep.heads_skip);
      else
        hipLaunchKernelGGL((splitk_heads_l2norm_kernel<1, 8>), grid, dim3(256), 0, stream, y, M, N / 2,
                           nullptr, ep.heads_out, ep.heads_in, ep.heads_group, ep.heads_skip);
      return hipGetLastError();
    }
    return hipSuccess;
  }
  hipError_t e;
  if (p.ks == 64) e = launch_part<64>(A, M, Kd, W, N, part, p.split, p.bm, p.bn, stream);
  else if (p.ks == 128) e = launch_part<128>(A, M, Kd, W, N, part, p.split, p.bm, p.bn, stream);
  else e = launch_part<256>(A, M, Kd, W, N, part, p.split, p.bm, p.bn, stream);
  if (e != hipSuccess) return e;
  switch (p.split) {
    case 2: return launch_reduce<2>(M, N, bias, ep, out, part, stream);
    case 3: return launch_reduce<3>(M, N, bias, ep, out, part, stream);
    case 4: return launch_reduce<4>(M, N, bias, ep, out, part, stream);
    case 6: return launch_reduce<6>(M, N, bias, ep, out, part, stream);
    case 8: return launch_reduce<8>(M, N, bias, ep, out, part, stream);
    case 12: return launch_reduce<12>(M, N, bias, ep, out, part, stream);
    default: return launch_reduce<16>(M, N, bias, ep, out, part, stream);
  }
}

}  // namespace ll
