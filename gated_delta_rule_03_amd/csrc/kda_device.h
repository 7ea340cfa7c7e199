// Device-side helpers shared by the KDA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Element i of an io tensor stored as bf16 (BF16 = true) or fp32.
template <bool BF16>
__device__ __forceinline__ float ld(const void* p, size_t i) {
  if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  else return static_cast<const float*>(p)[i];
}

template <bool BF16>
__device__ __forceinline__ void st(void* p, size_t i, float x) {
  if constexpr (BF16) static_cast<uint16_t*>(p)[i] = f32_to_bf16(x);
  else static_cast<float*>(p)[i] = x;
}

// Two consecutive io elements (i even).
template <bool BF16>
__device__ __forceinline__ float2 ld2(const void* p, size_t i) {
  if constexpr (BF16) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p) + i);
    return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
  } else {
    return *reinterpret_cast<const float2*>(static_cast<const float*>(p) + i);
  }
}

template <bool BF16>
__device__ __forceinline__ void st2(void* p, size_t i, float2 x) {
  if constexpr (BF16) {
    const uint32_t w = static_cast<uint32_t>(f32_to_bf16(x.x)) | (static_cast<uint32_t>(f32_to_bf16(x.y)) << 16);
    *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p) + i) = w;
  } else {
    *reinterpret_cast<float2*>(static_cast<float*>(p) + i) = x;
  }
}

// e^x through the hardware base-2 exponential (v_exp_f32): a few ulp, no
// range-reduction sequence.  Underflows to 0 below about -87.
__device__ __forceinline__ float exp_fast(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// e^x to about 2 ulp over the whole fp32 range: the rounding residual of
// x * log2(e) is carried to first order instead of being lost (it reaches
// ~5e-6 relative for |x| ~ 80, the span of a 16-token decay sub-block).
__device__ __forceinline__ float exp_precise(float x) {
  constexpr float kLog2e = 1.4426950408889634f;           // fp32 rounding of log2(e)
  constexpr float kLog2eLo = 1.925963033500011e-08f;      // log2(e) - kLog2e
  const float t = x * kLog2e;
  const float r = fmaf(x, kLog2e, -t) + x * kLog2eLo;
  return __builtin_amdgcn_exp2f(t) * fmaf(r, 0.6931471805599453f, 1.0f);
}

// 1/x through the hardware reciprocal (v_rcp_f32, 1 ulp).
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ __forceinline__ float sigmoidf_(float x) { return rcp_fast(1.0f + exp_fast(-x)); }

// log(1 + e^x) without overflow: max(x, 0) + log(1 + e^-|x|), the second
// term through the hardware base-2 logarithm (v_log_f32).  Its absolute
// error is ~1e-7, which is all that matters here: the result enters the gate
// additively.
__device__ __forceinline__ float softplusf_(float x) {
  return fmaxf(x, 0.0f) + __builtin_amdgcn_logf(1.0f + exp_fast(-fabsf(x))) * 0.6931471805599453f;
}

// y * sigmoid(y); for y below about -87 the exponential overflows and the
// reciprocal gives 0, the correct limit.
__device__ __forceinline__ float siluf_(float y) { return y * rcp_fast(1.0f + exp_fast(-y)); }

// Sum over groups of `width` consecutive lanes (width a power of two <= 64).
template <int width>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int m = width / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, width);
  return x;
}

// One DPP move within rows of 16 lanes (gfx9 encodings): quad_perm
// [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E, row_half_mirror = 0x141,
// row_mirror = 0x140.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of W = 8 or 16 lanes, in every lane of the group:
// pairs, quads, then the mirrored half row (lane i with 7 - i joins the two
// quads of a half) and, for 16, the mirrored row (lane i with 15 - i joins
// the halves).
template <int W>
__device__ __forceinline__ float lane_group_sum(float x) {
  static_assert(W == 8 || W == 16, "DPP row groups of 8 or 16 lanes");
  x += dpp_mov<0xB1>(x);
  x += dpp_mov<0x4E>(x);
  x += dpp_mov<0x141>(x);
  if constexpr (W == 16) x += dpp_mov<0x140>(x);
  return x;
}

// Gate of one channel: max(-exp(A_log) * softplus(alpha + dt_bias), lower bound).
__device__ __forceinline__ float gate_value(float alpha, float dt_bias, float a_exp, float lower_bound) {
  return fmaxf(-a_exp * softplusf_(alpha + dt_bias), lower_bound);
}

}  // namespace kda
