// Inter-chunk state propagation of the chunked KDA prefill.
//
// One workgroup per (sequence, head, dv tile of DVT columns): the columns of
// the dk x dv state evolve independently, so a workgroup owns a dk x DVT slice
// and walks the sequence's chunks in order:
//   record S as the chunk-start state (for the output step)
//   Delta = U - W S                     [64 x DVT]
//   S     = Diag(e^{G_C}) S + K~^T Delta
// with W, U, K~, e^{G_C} from the intra-chunk step.  Delta overwrites U.  The
// state starts from initial_state (or zeros) and the last S is the final
// state: the same state interface as the decode step (AliceAI page, section 五).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <int D, int DVT>
__global__ __launch_bounds__(256) void chunk_state_kernel(Params p, ChunkTable t, PrefillIO io, ChunkBuffers b) {
  constexpr int NT = 256;
  constexpr int NTILE = D / DVT;
  constexpr int LD = D + 1;
  __shared__ float Ws[kChunk * LD];
  __shared__ float Ks[kChunk * LD];
  __shared__ float Ss[D * DVT];
  __shared__ float Dl[kChunk * DVT];
  __shared__ float eg[D];

  const int H = p.H;
  const int tile_id = blockIdx.x % NTILE;
  const int h = (blockIdx.x / NTILE) % H;
  const int s = blockIdx.x / (NTILE * H);
  const int j0 = tile_id * DVT;
  const int tid = threadIdx.x;
  const size_t sbase = (static_cast<size_t>(s) * H + h) * D * D;

  for (int e = tid; e < D * DVT; e += NT) {
    const int i = e / DVT, jj = e % DVT;
    Ss[e] = io.S0 ? io.S0[sbase + static_cast<size_t>(i) * D + j0 + jj] : 0.f;
  }
  const int c_first = t.chunk0[s], c_end = t.chunk0[s + 1];
  for (int c = c_first; c < c_end; ++c) {
    const size_t tile = (static_cast<size_t>(c) * H + h) * kChunk;
    __syncthreads();
    for (int e = tid; e < kChunk * D; e += NT) {
      const int r = e / D, i = e % D;
      Ws[r * LD + i] = b.W[(tile + r) * D + i];
      Ks[r * LD + i] = b.Kt[(tile + r) * D + i];
    }
    for (int e = tid; e < kChunk * DVT; e += NT) {
      const int r = e / DVT, jj = e % DVT;
      Dl[e] = b.U[(tile + r) * D + j0 + jj];
    }
    for (int i = tid; i < D; i += NT) eg[i] = b.eGC[(static_cast<size_t>(c) * H + h) * D + i];
    // chunk-start state for the output step
    float* sst = b.Sst + (static_cast<size_t>(c) * H + h) * D * D;
    for (int e = tid; e < D * DVT; e += NT) {
      const int i = e / DVT, jj = e % DVT;
      sst[static_cast<size_t>(i) * D + j0 + jj] = Ss[e];
    }
    __syncthreads();
    // Delta = U - W S
    for (int e = tid; e < kChunk * DVT; e += NT) {
      const int r = e / DVT, jj = e % DVT;
      float acc = Dl[e];
      for (int i = 0; i < D; ++i) acc -= Ws[r * LD + i] * Ss[i * DVT + jj];
      Dl[e] = acc;
    }
    __syncthreads();
    // S = e^{G_C} S + K~^T Delta; Delta back to global
    for (int e = tid; e < D * DVT; e += NT) {
      const int i = e / DVT, jj = e % DVT;
      float acc = eg[i] * Ss[e];
      for (int r = 0; r < kChunk; ++r) acc += Ks[r * LD + i] * Dl[r * DVT + jj];
      Ss[e] = acc;
    }
    for (int e = tid; e < kChunk * DVT; e += NT) {
      const int r = e / DVT, jj = e % DVT;
      b.U[(tile + r) * D + j0 + jj] = Dl[e];
    }
  }
  __syncthreads();
  if (io.S_out) {
    for (int e = tid; e < D * DVT; e += NT) {
      const int i = e / DVT, jj = e % DVT;
      io.S_out[sbase + static_cast<size_t>(i) * D + j0 + jj] = Ss[e];
    }
  }
}

template <int D, int DVT>
static hipError_t launch_state_d(const Params& p, const ChunkTable& t, const PrefillIO& io, const ChunkBuffers& b,
                                 hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(t.N) * p.H * (D / DVT));
  chunk_state_kernel<D, DVT><<<grid, 256, 0, st>>>(p, t, io, b);
  return hipGetLastError();
}

hipError_t launch_chunk_state(const Params& p, const ChunkTable& t, const PrefillIO& io, const ChunkBuffers& b,
                              hipStream_t st) {
  switch (p.D) {
    case 16: return launch_state_d<16, 16>(p, t, io, b, st);
    case 32: return launch_state_d<32, 32>(p, t, io, b, st);
    case 64: return launch_state_d<64, 32>(p, t, io, b, st);
    case 128: return launch_state_d<128, 32>(p, t, io, b, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kda
