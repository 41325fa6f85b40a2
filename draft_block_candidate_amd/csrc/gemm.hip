// Linear layers of the candidate encoder on CDNA4 MFMA (bf16 in, fp32 acc).
//
// Y[M, N] = A[M, Kd] . W[N, Kd]^T + bias, both operands K-contiguous, so every
// MFMA operand fragment is one 16-byte LDS read. Block tile BM x BN x 64 with
// four waves in a 2 x 2 arrangement; each wave owns a (BM/2) x (BN/2) patch of
// 16 x 16 v_mfma_f32_16x16x32_bf16 tiles. Tiles are double-buffered in LDS
// with one barrier per k-step; the next tile's global loads are in flight
// while the current one is multiplied. Epilogues fuse the bias, the bf16
// rounding, SiLU and the fp32 residual add of the pre-norm transformer.
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

}  // namespace

hipError_t launch_linear(const uint16_t* A, int M, int Kd, const uint16_t* W, int N,
                         const float* bias, int epi, const float* resid, void* out,
                         hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (M >= 2048) return launch_tile<128, 128>(A, M, Kd, W, N, bias, epi, resid, out, stream);
  if (M > 64) return launch_tile<128, 32>(A, M, Kd, W, N, bias, epi, resid, out, stream);
  return launch_tile<64, 32>(A, M, Kd, W, N, bias, epi, resid, out, stream);
}

}  // namespace ll
