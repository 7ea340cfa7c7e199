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

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + expf(-x)); }

// log(1 + e^x) without overflow: max(x, 0) + log1p(e^-|x|).
__device__ __forceinline__ float softplusf_(float x) { return fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x))); }

__device__ __forceinline__ float siluf_(float y) { return y / (1.0f + expf(-y)); }

// Sum over groups of `width` consecutive lanes (width a power of two <= 64).
template <int width>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int m = width / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, width);
  return x;
}

// Gate of one channel: max(-exp(A_log) * softplus(alpha + dt_bias), lower bound).
__device__ __forceinline__ float gate_value(float alpha, float dt_bias, float a_exp, float lower_bound) {
  return fmaxf(-a_exp * softplusf_(alpha + dt_bias), lower_bound);
}

}  // namespace kda
