// bf16 matrix-core helpers for gfx950 (wave64, v_mfma_f32_16x16x32_bf16).
//
// Operand layouts of one 16x16x32 step (verified on MI355X):
//   A (16 x 32, M x K): lane l holds A[l % 16][8 * (l / 16) + i], i < 8
//   B (32 x 16, K x N): lane l holds B[8 * (l / 16) + i][l % 16], i < 8
//   C (16 x 16):        lane l holds C[4 * (l / 16) + i][l % 16], i < 4
//
// Compensated products.  Plain bf16 operands (8 significant bits) are far too
// coarse for the chunked form of the delta rule, so every fp32 operand x is
// split into NP bf16 pieces, x ~ p0 + p1 (+ p2), each piece the bf16 rounding
// of what the earlier pieces left, and a product accumulates in fp32 all
// piece pairs (i, j) with i + j < NP, smallest terms first.  NP = 2 gives 16
// significant bits with 3 matrix-core passes (dropping only p1*p1, ~2^-16
// relative): the path for bf16 inputs.  NP = 3 gives fp32's 24 bits with 6
// passes: the all-fp32 path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int NP>
struct SplitN {
  bf16x8 v[NP];
};

// c += a * b over all piece pairs i + j < NP, smallest terms first.
template <int NP>
__device__ __forceinline__ f32x4 mfmaN(const SplitN<NP>& a, const SplitN<NP>& b, f32x4 c) {
#pragma unroll
  for (int sum = NP - 1; sum >= 0; --sum)
#pragma unroll
    for (int i = 0; i <= sum; ++i) c = mfma(a.v[i], b.v[sum - i], c);
  return c;
}

// Two products sharing the B operand, c1 += a1 b and c2 += a2 b, their passes
// interleaved so that consecutive matrix-core steps are independent.
template <int NP>
__device__ __forceinline__ void mfmaN2(const SplitN<NP>& a1, const SplitN<NP>& a2, const SplitN<NP>& b, f32x4& c1,
                                       f32x4& c2) {
#pragma unroll
  for (int sum = NP - 1; sum >= 0; --sum)
#pragma unroll
    for (int i = 0; i <= sum; ++i) {
      c1 = mfma(a1.v[i], b.v[sum - i], c1);
      c2 = mfma(a2.v[i], b.v[sum - i], c2);
    }
}

// Two independent products, c1 += a1 b1 and c2 += a2 b2, their passes
// interleaved.
template <int NP>
__device__ __forceinline__ void mfmaNx2(const SplitN<NP>& a1, const SplitN<NP>& b1, f32x4& c1, const SplitN<NP>& a2,
                                        const SplitN<NP>& b2, f32x4& c2) {
#pragma unroll
  for (int sum = NP - 1; sum >= 0; --sum)
#pragma unroll
    for (int i = 0; i <= sum; ++i) {
      c1 = mfma(a1.v[i], b1.v[sum - i], c1);
      c2 = mfma(a2.v[i], b2.v[sum - i], c2);
    }
}

// The NP bf16 pieces of one fp32 value.
template <int NP>
__device__ __forceinline__ void split_pieces(float x, __bf16 (&pc)[NP]) {
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    pc[k] = static_cast<__bf16>(x);
    x -= static_cast<float>(pc[k]);
  }
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to bf16 (nearest even) in one packed word
// (v_cvt_pk_bf16_f32): a in the low half, b in the high half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// x - (the low or the high bf16 half of the packed word w), in one packed
// bf16 dot product with (-1, 0) or (0, -1): both products are exact and the
// difference of x and its own bf16 rounding is exact in fp32, so no rounding
// takes place.  (A shift or a mask and a subtraction would take two
// instructions.)
// The constant words are passed through a scalar register the compiler cannot
// see into.  Written as constants, (-1, 0) is encoded as the inline constant
// -1.0, which the hardware applies to both halves of a packed bf16 operand
// (measured: the result was x minus both halves), not to the low one alone.
__device__ __forceinline__ uint32_t sreg(uint32_t c) {
  asm("" : "+s"(c));   // not volatile: equal uses share one register
  return c;
}
__device__ __forceinline__ float minus_lo(uint32_t w, float x) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, sreg(0x0000bf80u)),
                                         x, false);
}
__device__ __forceinline__ float minus_hi(uint32_t w, float x) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, sreg(0xbf800000u)),
                                         x, false);
}

// The NP pieces of the pair (a, b), each a packed bf16 word: piece k + 1
// splits what is left after piece k.
template <int NP>
__device__ __forceinline__ void split_pair(float a, float b, uint32_t (&w)[NP]) {
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    w[k] = pack_bf16x2(a, b);
    if (k + 1 < NP) {
      a = minus_lo(w[k], a);
      b = minus_hi(w[k], b);
    }
  }
}

template <int NP>
__device__ __forceinline__ SplitN<NP> splitN(const float (&x)[8]) {
  uint32_t w[4][NP];
#pragma unroll
  for (int j = 0; j < 4; ++j) split_pair<NP>(x[2 * j], x[2 * j + 1], w[j]);
  SplitN<NP> s;
#pragma unroll
  for (int k = 0; k < NP; ++k) s.v[k] = __builtin_bit_cast(bf16x8, make_uint4(w[0][k], w[1][k], w[2][k], w[3][k]));
  return s;
}

// Eight consecutive fp32 values (16-byte aligned) split into pieces.
template <int NP>
__device__ __forceinline__ SplitN<NP> load_split(const float* p) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  return splitN<NP>(x);
}

template <int NP>
__device__ __forceinline__ SplitN<NP> zero_split() {
  SplitN<NP> s;
#pragma unroll
  for (int k = 0; k < NP; ++k) s.v[k] = __builtin_bit_cast(bf16x8, make_uint4(0u, 0u, 0u, 0u));
  return s;
}

__device__ __forceinline__ bf16x8 load_bf16x8(const void* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

}  // namespace kda
