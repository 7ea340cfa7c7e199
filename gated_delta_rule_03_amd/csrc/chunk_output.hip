// Chunk output of the chunked KDA prefill: one workgroup per (chunk, head)
//   O = Q+ S_start + Aqk Delta
// the cross-chunk read q^T S of the chunk-start state (with the in-chunk decay
// folded into Q+ = Q * e^G) plus the masked intra-chunk attention applied to
// the corrected values.  The pages' loop reads o from the state updated by the
// current token (AliceAI page, section 二), which is why Aqk includes its
// diagonal.  Rows past the end of a partial chunk are not written.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(256) void chunk_output_kernel(Params p, ChunkTable t, PrefillIO io, ChunkBuffers b) {
  constexpr int NT = 256;
  constexpr int RG = NT / D;               // row groups
  constexpr int RPT = kChunk / RG;         // rows per lane
  constexpr int LD = D + 1;
  __shared__ float Qs[kChunk * LD];
  __shared__ float Ss[D * D];
  __shared__ float As[kChunk * (kChunk + 1)];
  __shared__ float Ds[kChunk * D];

  const int c = blockIdx.x, h = blockIdx.y;
  if (c >= t.chunk0[t.N]) return;
  const int H = p.H;
  const int s = t.chunk_seq[c];
  const int64_t tok0 = static_cast<int64_t>(t.cu[s]) + (c - t.chunk0[s]) * kChunk;
  const int len = min(kChunk, t.cu[s + 1] - static_cast<int>(tok0));
  const int tid = threadIdx.x;
  const size_t tile = (static_cast<size_t>(c) * H + h) * kChunk;
  const float* sst = b.Sst + (static_cast<size_t>(c) * H + h) * D * D;

  for (int e = tid; e < kChunk * D; e += NT) {
    const int r = e / D, i = e % D;
    Qs[r * LD + i] = b.Qp[(tile + r) * D + i];
    Ds[e] = b.U[(tile + r) * D + i];
  }
  for (int e = tid; e < D * D; e += NT) Ss[e] = sst[e];
  for (int e = tid; e < kChunk * kChunk; e += NT) {
    const int r = e / kChunk, i = e % kChunk;
    As[r * (kChunk + 1) + i] = b.Aqk[tile * kChunk + e];
  }
  __syncthreads();

  const int j = tid % D, rg = tid / D;
  float acc[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m) acc[m] = 0.f;
  for (int i = 0; i < D; ++i) {
    const float sv = Ss[i * D + j];
#pragma unroll
    for (int m = 0; m < RPT; ++m) acc[m] += Qs[(rg * RPT + m) * LD + i] * sv;
  }
  for (int i = 0; i < kChunk; ++i) {
    const float dv = Ds[i * D + j];
#pragma unroll
    for (int m = 0; m < RPT; ++m) acc[m] += As[(rg * RPT + m) * (kChunk + 1) + i] * dv;
  }
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int r = rg * RPT + m;
    if (r < len) st<OUT_BF16>(io.o, (static_cast<size_t>(tok0 + r) * H + h) * D + j, acc[m]);
  }
}

template <int D>
static hipError_t launch_out_d(const Params& p, const ChunkTable& t, const PrefillIO& io, const ChunkBuffers& b,
                               int max_chunks, bool out_bf16, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(max_chunks), static_cast<unsigned>(p.H));
  if (out_bf16) chunk_output_kernel<D, true><<<grid, 256, 0, st>>>(p, t, io, b);
  else chunk_output_kernel<D, false><<<grid, 256, 0, st>>>(p, t, io, b);
  return hipGetLastError();
}

hipError_t launch_chunk_output(const Params& p, const ChunkTable& t, const PrefillIO& io, const ChunkBuffers& b,
                               int max_chunks, bool out_bf16, hipStream_t st) {
  switch (p.D) {
    case 16: return launch_out_d<16>(p, t, io, b, max_chunks, out_bf16, st);
    case 32: return launch_out_d<32>(p, t, io, b, max_chunks, out_bf16, st);
    case 64: return launch_out_d<64>(p, t, io, b, max_chunks, out_bf16, st);
    case 128: return launch_out_d<128>(p, t, io, b, max_chunks, out_bf16, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kda
