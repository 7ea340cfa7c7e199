// Kernel argument blocks and launchers of the KDA library (host + device).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/kda.h"

namespace kda {

constexpr int kChunk = 64;   // tokens per chunk of the chunked form
constexpr int kSub = 16;     // tokens per decay sub-block inside a chunk

// Parameters every kernel that touches raw inputs needs.
struct Params {
  int H;
  int D;                 // dk == dv
  float scale;
  float lower_bound;
  float eps;
  uint32_t flags;
  const float* A_log;    // [H]
  const float* dt_bias;  // [H*D]
  const void* wq;        // [H*D][4]
  const void* wk;
  const void* wv;
};

// Device-side description of a packed batch, built by the chunk-table kernel.
struct ChunkTable {
  const int32_t* cu;         // [N+1] token offsets
  const int32_t* chunk0;     // [N+1] first chunk of each sequence; chunk0[N] = total chunks
  const int32_t* chunk_seq;  // [max_chunks] sequence of each chunk
  int32_t N;
};

// Per-chunk fp32 intermediates, chunk-major: [chunk][H][64][D] unless noted.
struct ChunkBuffers {
  float* qh;     // normalised, scaled q
  float* kh;     // normalised k
  float* vh;     // v after conv + SiLU
  float* g;      // per-channel log decay
  float* beta;   // [chunk][H][64]
  float* W;      // T (beta * k * e^G)
  float* U;      // T (beta * v); overwritten by Delta = U - W S
  float* Qp;     // q * e^G
  float* Kt;     // k * e^{G_C - G}
  float* eGC;    // [chunk][H][D] e^{G_C}
  float* Aqk;    // [chunk][H][64][64] masked intra-chunk attention
  float* Sst;    // [chunk][H][D][D] state at chunk start
};

struct PrefillIO {
  const void* q;
  const void* k;
  const void* v;
  const void* alpha;
  const void* b;
  const float* S0;        // [N][H][D][D] or null
  const void* conv_in;    // [N][3][Ctot] or null
  void* o;
  float* S_out;           // or null
  void* conv_out;         // or null
};

hipError_t launch_build_chunks(const int32_t* cu_in, int32_t N, int32_t T_uniform, int32_t* cu_ws,
                               int32_t* chunk0, int32_t* chunk_seq, int32_t max_chunks, hipStream_t st);
hipError_t launch_preprocess(const Params& p, const ChunkTable& t, const PrefillIO& io, const ChunkBuffers& b,
                             int max_chunks, bool io_bf16, hipStream_t st);
hipError_t launch_chunk_intra(const Params& p, const ChunkTable& t, const ChunkBuffers& b, int max_chunks,
                              hipStream_t st);
hipError_t launch_chunk_state(const Params& p, const ChunkTable& t, const PrefillIO& io, const ChunkBuffers& b,
                              hipStream_t st);
hipError_t launch_chunk_output(const Params& p, const ChunkTable& t, const PrefillIO& io, const ChunkBuffers& b,
                               int max_chunks, bool out_bf16, hipStream_t st);
hipError_t launch_conv_state_out(const Params& p, const ChunkTable& t, const PrefillIO& io, bool io_bf16,
                                 hipStream_t st);

struct DecodeIO {
  const void* q;
  const void* k;
  const void* v;
  const void* alpha;
  const void* b;
  float* state;
  void* conv_state;
  void* o;
};

hipError_t launch_decode(const Params& p, const DecodeIO& io, int N, bool io_bf16, bool out_bf16, hipStream_t st);

}  // namespace kda
