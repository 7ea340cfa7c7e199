// The KDA layer's output epilogue: o_norm, an RMS norm over each (token,
// head) row of dv outputs with one weight per channel, times the sigmoid of
// the output gate (AliceAI page, section 三: KDA's o_norm and sigmoid gate;
// section 二: output_gate among the per-token control inputs):
//   y[j] = o[j] / sqrt(mean_j' o[j']^2 + eps) * w[j] * sigmoid(gate[j])
//
// HBM-bound (read o and gate, write y).  A row belongs to 16 consecutive
// lanes (one DPP row), dv / 16 elements each, so a bf16 row of 128 is one
// 16-byte load per lane and operand, and the row's sum of squares is four
// DPP steps with no LDS.  A wave covers four rows; workgroups stride over
// the rows.
#include "kda_device.h"
#include "kda_internal.h"
#include "mfma.h"

namespace kda {

namespace {

constexpr int kEpiThreads = 256;

// EPL consecutive io elements (EPL in {1, 2, 4, 8}) at index i of a bf16 or
// fp32 tensor, as floats, with the widest aligned loads.
template <bool BF16, int EPL>
__device__ __forceinline__ void load_n(const void* p, size_t i, float (&x)[EPL]) {
  if constexpr (BF16) {
    const uint16_t* q = static_cast<const uint16_t*>(p) + i;
    uint32_t w[(EPL + 1) / 2];
    if constexpr (EPL == 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(q);
      w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else if constexpr (EPL == 4) {
      const uint2 v = *reinterpret_cast<const uint2*>(q);
      w[0] = v.x; w[1] = v.y;
    } else if constexpr (EPL == 2) {
      w[0] = *reinterpret_cast<const uint32_t*>(q);
    } else {
      w[0] = *q;
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) x[e] = __uint_as_float((e & 1) ? (w[e / 2] & 0xffff0000u) : (w[e / 2] << 16));
  } else {
    const float* q = static_cast<const float*>(p) + i;
#pragma unroll
    for (int e = 0; e < EPL; e += (EPL >= 4 ? 4 : EPL)) {
      if constexpr (EPL >= 4) {
        const float4 v = *reinterpret_cast<const float4*>(q + e);
        x[e] = v.x; x[e + 1] = v.y; x[e + 2] = v.z; x[e + 3] = v.w;
      } else if constexpr (EPL == 2) {
        const float2 v = *reinterpret_cast<const float2*>(q);
        x[0] = v.x; x[1] = v.y;
      } else {
        x[0] = *q;
      }
    }
  }
}

template <bool BF16, int EPL>
__device__ __forceinline__ void store_n(void* p, size_t i, const float (&x)[EPL]) {
  if constexpr (BF16) {
    uint16_t* q = static_cast<uint16_t*>(p) + i;
    if constexpr (EPL == 1) {
      *q = static_cast<uint16_t>(pack_bf16x2(x[0], 0.f));
    } else {
      uint32_t w[EPL / 2];
#pragma unroll
      for (int e = 0; e < EPL / 2; ++e) w[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
      if constexpr (EPL == 8) *reinterpret_cast<uint4*>(q) = make_uint4(w[0], w[1], w[2], w[3]);
      else if constexpr (EPL == 4) *reinterpret_cast<uint2*>(q) = make_uint2(w[0], w[1]);
      else *reinterpret_cast<uint32_t*>(q) = w[0];
    }
  } else {
    float* q = static_cast<float*>(p) + i;
    if constexpr (EPL >= 4) {
#pragma unroll
      for (int e = 0; e < EPL; e += 4) *reinterpret_cast<float4*>(q + e) = make_float4(x[e], x[e + 1], x[e + 2], x[e + 3]);
    } else if constexpr (EPL == 2) {
      *reinterpret_cast<float2*>(q) = make_float2(x[0], x[1]);
    } else {
      *q = x[0];
    }
  }
}

}  // namespace

template <int DV, bool O_BF16, bool G_BF16>
__global__ __launch_bounds__(kEpiThreads) void output_gate_kernel(int64_t rows, const void* o, const void* gate,
                                                                  const float* __restrict__ w, float eps, void* y) {
  constexpr int EPL = DV / 16;
  const int l16 = threadIdx.x & 15;
  const int64_t first = (static_cast<int64_t>(blockIdx.x) * kEpiThreads + threadIdx.x) >> 4;
  const int64_t step = (static_cast<int64_t>(gridDim.x) * kEpiThreads) >> 4;
  float wv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) wv[e] = w[l16 * EPL + e];
  // every lane of a 16-lane group takes the same rows, so a group is either
  // wholly active or wholly idle and its DPP sums stay inside it
  for (int64_t r = first; r < rows; r += step) {
    const size_t base = static_cast<size_t>(r) * DV + static_cast<size_t>(l16) * EPL;
    float ov[EPL], gv[EPL];
    load_n<O_BF16, EPL>(o, base, ov);
    load_n<G_BF16, EPL>(gate, base, gv);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) ss = fmaf(ov[e], ov[e], ss);
    ss = lane_group_sum<16>(ss);
    const float inv = 1.0f / sqrtf(ss * (1.0f / DV) + eps);
    float yv[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) yv[e] = ov[e] * inv * wv[e] * sigmoidf_(gv[e]);
    store_n<O_BF16, EPL>(y, base, yv);
  }
}

template <int DV>
static hipError_t launch_output_gate_d(int64_t rows, const void* o, const void* gate, const float* w, float eps,
                                       void* y, bool o_bf16, bool g_bf16, hipStream_t st) {
  const int64_t groups_per_block = kEpiThreads / 16;
  const int64_t blocks = (rows + groups_per_block - 1) / groups_per_block;
  const dim3 grid(static_cast<unsigned>(blocks < (1 << 20) ? blocks : (1 << 20)));
  if (o_bf16 && g_bf16) output_gate_kernel<DV, true, true><<<grid, kEpiThreads, 0, st>>>(rows, o, gate, w, eps, y);
  else if (o_bf16) output_gate_kernel<DV, true, false><<<grid, kEpiThreads, 0, st>>>(rows, o, gate, w, eps, y);
  else if (g_bf16) output_gate_kernel<DV, false, true><<<grid, kEpiThreads, 0, st>>>(rows, o, gate, w, eps, y);
  else output_gate_kernel<DV, false, false><<<grid, kEpiThreads, 0, st>>>(rows, o, gate, w, eps, y);
  return hipGetLastError();
}

hipError_t launch_output_gate(int D, int64_t rows, const void* o, const void* gate, const float* w, float eps,
                              void* y, bool o_bf16, bool g_bf16, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  switch (D) {
    case 16: return launch_output_gate_d<16>(rows, o, gate, w, eps, y, o_bf16, g_bf16, st);
    case 32: return launch_output_gate_d<32>(rows, o, gate, w, eps, y, o_bf16, g_bf16, st);
    case 64: return launch_output_gate_d<64>(rows, o, gate, w, eps, y, o_bf16, g_bf16, st);
    case 128: return launch_output_gate_d<128>(rows, o, gate, w, eps, y, o_bf16, g_bf16, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kda
