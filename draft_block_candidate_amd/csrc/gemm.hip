// Linear layers of the candidate encoder on CDNA4 MFMA (bf16 in, fp32 acc).
//
// Y[M, N] = A[M, Kd] . W[N, Kd]^T + bias, both operands K-contiguous, so every
// MFMA operand fragment is one 16-byte LDS read. Four waves per workgroup in a
// 2 x 2 arrangement; each wave owns a (BM/2) x (BN/2) patch of 16 x 16
// v_mfma_f32_16x16x32_bf16 tiles. Epilogues fuse the bias, the bf16 rounding,
// SiLU and the fp32 residual add of the pre-norm transformer.
//
// Two schedules:
//  * many rows (M >= 2048): BM x BN = 128 x 128 tiles over the whole K,
//    double-buffered in LDS with one barrier per 64-wide k-step;
//  * few rows (one or a few draft blocks, M = B*K*N of 64..1024): the GEMM is
//    weight-streaming and latency bound, so K is split S ways. Each workgroup
//    stages its whole A and W K-slice in LDS with every load in flight at
//    once, multiplies, and writes an fp32 partial tile; the last workgroup of
//    a tile to finish (an atomic arrival counter) sums the S partials in the
//    fixed order s = 0..S-1 (bit-reproducible) and applies the epilogue.
//    Workgroups of one tile are mapped to the same XCD (consecutive block ids
//    go round-robin over the 8 XCDs), so its partials stay in one L2.
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

  // Epilogue: lane holds rows 4g+q, column c of every 16 x 16 tile.
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int64_t n = n0 + wn * (BN / 2) + j * 16 + c;
    if (n >= N) continue;
    const float bv = bias ? bias[n] : 0.f;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t m = m0 + wm * (BM / 2) + i * 16 + 4 * g + q;
        if (m >= M) continue;
        const float y = acc[i][j][q] + bv;
        const int64_t o = m * N + n;
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
    }
  }
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

// Split-K schedule for few rows. Block b -> XCD x = b % 8, q = b / 8,
// tile = (q / S) * 8 + x, split s = q % S.
template <int BM, int BN, int KS, int EPI>
__global__ __launch_bounds__(256) void gemm_splitk_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W, int M, int N, int Kd,
    const float* __restrict__ bias, const float* resid, void* out, float* __restrict__ part,
    int* __restrict__ cnt, int S, int tiles_n, int tiles) {
  constexpr int STR = KS + 8;
  constexpr int MT = BM / 32, NT = BN / 32;
  constexpr int CH_A = BM * KS / 8, CH_W = BN * KS / 8;
  constexpr int NCH = (CH_A + CH_W) / 256;
  static_assert((CH_A + CH_W) % 256 == 0, "chunking");
  __shared__ __attribute__((aligned(16))) uint16_t smem[(BM + BN) * STR];
  uint16_t* As = smem;
  uint16_t* Ws = smem + BM * STR;
  __shared__ int is_last;

  const int b = blockIdx.x;
  const int x = b & 7, q = b >> 3;
  const int tile = (q / S) * 8 + x, s = q % S;
  if (tile >= tiles) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 4, c = lane & 15;
  const int64_t m0 = (int64_t)(tile / tiles_n) * BM, n0 = (int64_t)(tile % tiles_n) * BN;
  const int64_t k0 = (int64_t)s * KS;

  u32x4_t r[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int ch = tid + 256 * i;
    if (ch < CH_A) {
      const int row = ch / (KS / 8), c8 = ch % (KS / 8);
      const int64_t gm = m0 + row;
      r[i] = gm < M ? *(const u32x4_t*)(A + gm * Kd + k0 + c8 * 8) : u32x4_t{0, 0, 0, 0};
    } else {
      const int cw = ch - CH_A;
      const int row = cw / (KS / 8), c8 = cw % (KS / 8);
      const int64_t gn = n0 + row;
      r[i] = gn < N ? *(const u32x4_t*)(W + gn * Kd + k0 + c8 * 8) : u32x4_t{0, 0, 0, 0};
    }
  }
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int ch = tid + 256 * i;
    if (ch < CH_A)
      *(u32x4_t*)(&As[(ch / (KS / 8)) * STR + (ch % (KS / 8)) * 8]) = r[i];
    else
      *(u32x4_t*)(&Ws[((ch - CH_A) / (KS / 8)) * STR + ((ch - CH_A) % (KS / 8)) * 8]) = r[i];
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
      af[i] = *(const u32x4_t*)(&As[(wm * (BM / 2) + i * 16 + c) * STR + kk + 8 * g]);
#pragma unroll
    for (int j = 0; j < NT; ++j)
      bfr[j] = *(const u32x4_t*)(&Ws[(wn * (BN / 2) + j * 16 + c) * STR + kk + 8 * g]);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[i][j] = mfma16(af[i], bfr[j], acc[i][j]);
  }

  float* mypart = part + ((int64_t)tile * S + s) * (BM * BN);
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int row = wm * (BM / 2) + i * 16 + 4 * g + qq;
        const int col = wn * (BN / 2) + j * 16 + c;
        mypart[row * BN + col] = acc[i][j][qq];
      }
  __threadfence();
  __syncthreads();
  if (tid == 0) is_last = atomicAdd(&cnt[tile], 1) == S - 1;
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  const float* tp = part + (int64_t)tile * S * (BM * BN);
  for (int e = tid; e < BM * BN; e += 256) {
    const int row = e / BN, col = e % BN;
    const int64_t m = m0 + row, n = n0 + col;
    if (m >= M || n >= N) continue;
    float v = tp[e];
    for (int t = 1; t < S; ++t) v += tp[(int64_t)t * (BM * BN) + e];
    epilogue_store<EPI>(out, resid, m * N + n, v + (bias ? bias[n] : 0.f));
  }
  if (tid == 0) cnt[tile] = 0;
}

__global__ void clear_counters_kernel(int* cnt, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) cnt[i] = 0;
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

template <int BM, int BN, int KS>
hipError_t launch_splitk(const uint16_t* A, int M, int Kd, const uint16_t* W, int N,
                         const float* bias, int epi, const float* resid, void* out, float* part,
                         int* cnt, int S, hipStream_t stream) {
  const int tiles_n = (N + BN - 1) / BN;
  const int tiles = ((M + BM - 1) / BM) * tiles_n;
  const int blocks = ((tiles + 7) / 8) * 8 * S;
#define LL_SPLITK(E)                                                                            \
  hipLaunchKernelGGL((gemm_splitk_kernel<BM, BN, KS, E>), dim3(blocks), dim3(256), 0, stream, A, \
                     W, M, N, Kd, bias, resid, out, part, cnt, S, tiles_n, tiles)
  switch (epi) {
    case EPI_F32: LL_SPLITK(EPI_F32); break;
    case EPI_BF16: LL_SPLITK(EPI_BF16); break;
    case EPI_SILU_BF16: LL_SPLITK(EPI_SILU_BF16); break;
    default: LL_SPLITK(EPI_RESID_F32); break;
  }
#undef LL_SPLITK
  return hipGetLastError();
}

}  // namespace

GemmPlan plan_linear(int M, int Kd, int N) {
  GemmPlan p{};
  if (M >= 2048 || Kd < 128) {
    p.split = 1;
    return p;
  }
  p.bm = M > 64 ? 128 : 64;
  p.bn = 32;
  p.tiles = ((M + p.bm - 1) / p.bm) * ((N + p.bn - 1) / p.bn);
  // about 512 workgroups; K slices of 64..256 (the whole slice sits in LDS)
  int S = 1;
  while (S * 2 * p.tiles <= 512 && Kd / (S * 2) >= 64 && (Kd % (S * 2)) == 0) S *= 2;
  while (Kd / S > 256) S *= 2;
  if (Kd % S || (Kd / S) % 64) {
    p.split = 1;
    return p;
  }
  p.split = S;
  p.ks = Kd / S;
  if (S == 1) return p;
  p.part_floats = (size_t)p.tiles * S * p.bm * p.bn;
  p.counters = p.tiles;
  return p;
}

hipError_t launch_clear_counters(int* cnt, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(clear_counters_kernel, dim3((unsigned)((n + 255) / 256 < 64 ? (n + 255) / 256 : 64)),
                     dim3(256), 0, stream, cnt, n);
  return hipGetLastError();
}

hipError_t launch_linear(const uint16_t* A, int M, int Kd, const uint16_t* W, int N,
                         const float* bias, int epi, const float* resid, void* out, float* part,
                         int* cnt, hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const GemmPlan p = plan_linear(M, Kd, N);
  if (p.split > 1) {
    if (p.bm == 128) {
      if (p.ks == 64) return launch_splitk<128, 32, 64>(A, M, Kd, W, N, bias, epi, resid, out, part, cnt, p.split, stream);
      if (p.ks == 128) return launch_splitk<128, 32, 128>(A, M, Kd, W, N, bias, epi, resid, out, part, cnt, p.split, stream);
      return launch_splitk<128, 32, 256>(A, M, Kd, W, N, bias, epi, resid, out, part, cnt, p.split, stream);
    }
    if (p.ks == 64) return launch_splitk<64, 32, 64>(A, M, Kd, W, N, bias, epi, resid, out, part, cnt, p.split, stream);
    if (p.ks == 128) return launch_splitk<64, 32, 128>(A, M, Kd, W, N, bias, epi, resid, out, part, cnt, p.split, stream);
    return launch_splitk<64, 32, 256>(A, M, Kd, W, N, bias, epi, resid, out, part, cnt, p.split, stream);
  }
  if (M >= 2048) return launch_tile<128, 128>(A, M, Kd, W, N, bias, epi, resid, out, stream);
  if (M > 64) return launch_tile<128, 32>(A, M, Kd, W, N, bias, epi, resid, out, stream);
  return launch_tile<64, 32>(A, M, Kd, W, N, bias, epi, resid, out, stream);
}

}  // namespace ll
