// Shared device helpers for the gfx950 kernels: bf16 conversion, wave64
// reductions and MFMA operand types.
#pragma once

#include <hip/hip_runtime.h>
#include <climits>
#include <stdint.h>

#define LL_WAVE 64

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));

namespace ll {

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round a finite float to bfloat16, to nearest with ties to even.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two floats to packed bfloat16 (lo in bits 15:0), round to nearest even:
// one v_cvt_pk_bf16_f32, the same rounding as f32_to_bf16 for finite values.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// 16x16x32 bf16 MFMA on gfx950: acc += A(16x32) * B(32x16).
// Operand layout (lane l, g = l / 16): A row l%16, k = 8g..8g+7;
// B column l%16, k = 8g..8g+7; acc row 4g+i, column l%16 (i = 0..3).
__device__ __forceinline__ f32x4_t mfma16(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Wave64 reductions on DPP (GFX9 data-parallel primitives): row_shr:1/2/4/8
// combine within each 16-lane row, row_bcast:15 and row_bcast:31 fold the
// rows, leaving the result in lane 63, which readlane broadcasts. Lanes with no
// DPP source contribute the identity passed as `old`. Must be called by all 64
// lanes (wave-uniform control flow). The order of the combination is fixed.
enum : int {
  kDppShr1 = 0x111,
  kDppShr2 = 0x112,
  kDppShr4 = 0x114,
  kDppShr8 = 0x118,
  kDppBcast15 = 0x142,
  kDppBcast31 = 0x143
};

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_i(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xf, false);
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float old, float v) {
  return __int_as_float(dpp_i<CTRL, ROW_MASK>(__float_as_int(old), __float_as_int(v)));
}
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ int readlane_i(int v, int l) { return __builtin_amdgcn_readlane(v, l); }

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<kDppShr1, 0xf>(0.f, v);
  v += dpp_f<kDppShr2, 0xf>(0.f, v);
  v += dpp_f<kDppShr4, 0xf>(0.f, v);
  v += dpp_f<kDppShr8, 0xf>(0.f, v);
  v += dpp_f<kDppBcast15, 0xa>(0.f, v);
  v += dpp_f<kDppBcast31, 0xc>(0.f, v);
  return readlane_f(v, 63);
}

// Order-preserving map of a float to a signed int (and back): for non-NaN
// values, a < b exactly when key(a) < key(b) (with -0 below +0). Maxima are
// taken on the keys so that each DPP step is one integer max, which the
// compiler folds into a v_max_i32 with a DPP operand.
__device__ __forceinline__ int fkey(float x) {
  const int i = __float_as_int(x);
  return i ^ ((i >> 31) & 0x7fffffff);
}
__device__ __forceinline__ float fkey_inv(int k) { return __int_as_float(k ^ ((k >> 31) & 0x7fffffff)); }

__device__ __forceinline__ float wave_max(float x) {
  int v = fkey(x);
  v = max(v, dpp_i<kDppShr1, 0xf>(INT_MIN, v));
  v = max(v, dpp_i<kDppShr2, 0xf>(INT_MIN, v));
  v = max(v, dpp_i<kDppShr4, 0xf>(INT_MIN, v));
  v = max(v, dpp_i<kDppShr8, 0xf>(INT_MIN, v));
  v = max(v, dpp_i<kDppBcast15, 0xa>(INT_MIN, v));
  v = max(v, dpp_i<kDppBcast31, 0xc>(INT_MIN, v));
  return fkey_inv(readlane_i(v, 63));
}

// Largest (v, i) by v descending, then i ascending; result in every lane.
// Written with non-short-circuit operators and selects: a branchy form
// compiles to exec-mask updates whose hazards stall every step.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void argmax_step(float& v, int& i) {
  const float ov = dpp_f<CTRL, ROW_MASK>(-INFINITY, v);
  const int oi = dpp_i<CTRL, ROW_MASK>(0x7fffffff, i);
  const bool take = (ov > v) | ((ov == v) & (oi < i));
  v = take ? ov : v;
  i = take ? oi : i;
}
// Maximum over lanes 0 .. n - 1 only (n = 16, 32 or 64); result in every lane.
__device__ __forceinline__ float lanes_max(float x, int n) {
  int v = fkey(x);
  v = max(v, dpp_i<kDppShr1, 0xf>(INT_MIN, v));
  v = max(v, dpp_i<kDppShr2, 0xf>(INT_MIN, v));
  v = max(v, dpp_i<kDppShr4, 0xf>(INT_MIN, v));
  v = max(v, dpp_i<kDppShr8, 0xf>(INT_MIN, v));
  if (n > 16) v = max(v, dpp_i<kDppBcast15, 0xa>(INT_MIN, v));
  if (n > 32) v = max(v, dpp_i<kDppBcast31, 0xc>(INT_MIN, v));
  return fkey_inv(readlane_i(v, n > 32 ? 63 : (n > 16 ? 31 : 15)));
}

// Argmax over lanes 0 .. n - 1 only (n = 16, 32 or 64); fewer DPP steps for
// small n. Result in every lane.
__device__ __forceinline__ void lanes_argmax(float& v, int& i, int n) {
  argmax_step<kDppShr1, 0xf>(v, i);
  argmax_step<kDppShr2, 0xf>(v, i);
  argmax_step<kDppShr4, 0xf>(v, i);
  argmax_step<kDppShr8, 0xf>(v, i);
  if (n > 16) argmax_step<kDppBcast15, 0xa>(v, i);
  if (n > 32) argmax_step<kDppBcast31, 0xc>(v, i);
  const int last = n > 32 ? 63 : (n > 16 ? 31 : 15);
  v = readlane_f(v, last);
  i = readlane_i(i, last);
}
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  argmax_step<kDppShr1, 0xf>(v, i);
  argmax_step<kDppShr2, 0xf>(v, i);
  argmax_step<kDppShr4, 0xf>(v, i);
  argmax_step<kDppShr8, 0xf>(v, i);
  argmax_step<kDppBcast15, 0xa>(v, i);
  argmax_step<kDppBcast31, 0xc>(v, i);
  v = readlane_f(v, 63);
  i = readlane_i(i, 63);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Float32 product, sum and difference, each rounded once, that the compiler
// may not fuse into an FMA with a neighbouring operation (HIP compiles with
// floating-point contraction on, and __fmul_rn / __fadd_rn are plain operators
// there). The commit rules' score fl32(logp + fl32(alpha * cos)) is two
// roundings; an FMA would round once.
__device__ __forceinline__ float mul_rn(float a, float b) {
#pragma clang fp contract(off)
  return a * b;
}
__device__ __forceinline__ float add_rn(float a, float b) {
#pragma clang fp contract(off)
  return a + b;
}
__device__ __forceinline__ float sub_rn(float a, float b) {
#pragma clang fp contract(off)
  return a - b;
}

// The value held by lane (lane ^ j), j in {1, 2, 4, 8, 16, 32}, without the
// LDS crossbar: quad permutes for 1 and 2, a row shift each way for 4 and 8
// (each lane keeps the one that stays in its 16-lane row), and the gfx950
// row-swap permutes for 16 and 32. Lane layout of the swaps (measured): with
// both operands v, permlane16_swap returns {v of lane l - 16 on odd rows,
// own on even rows} and {v of lane l + 16 on even rows, own on odd rows};
// permlane32_swap likewise for the halves. j must fold to a constant (call
// from fully unrolled loops); every lane must take part.
__device__ __forceinline__ int xor_lane(int v, int j, int lane) {
  switch (j) {
    case 1: return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xf, 0xf, false);   // quad_perm [1,0,3,2]
    case 2: return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xf, 0xf, false);   // quad_perm [2,3,0,1]
    case 4: {
      const int dn = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
      const int up = __builtin_amdgcn_update_dpp(0, v, 0x104, 0xf, 0xf, false);  // row_shl:4
      return (lane & 4) ? dn : up;
    }
    case 8: {
      const int dn = __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
      const int up = __builtin_amdgcn_update_dpp(0, v, 0x108, 0xf, 0xf, false);  // row_shl:8
      return (lane & 8) ? dn : up;
    }
    case 16: {
      const auto r = __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false);
      return (int)((lane & 16) ? r[0] : r[1]);
    }
    default: {
      const auto r = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
      return (int)((lane & 32) ? r[0] : r[1]);
    }
  }
}
__device__ __forceinline__ float xor_lane(float v, int j, int lane) {
  return __int_as_float(xor_lane(__float_as_int(v), j, lane));
}

// SiLU with the hardware exponential and reciprocal (v_exp_f32, v_rcp_f32;
// about 1 ulp each): the result is rounded to bfloat16 by every caller.
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

}  // namespace ll
