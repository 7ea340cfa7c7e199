// Kernel argument blocks and launchers of the KDA library (host + device).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/kda.h"

namespace kda {

constexpr int kChunk = 64;   // tokens per chunk of the chunked form
constexpr int kSub = 16;     // tokens per decay sub-block inside a chunk

// Per (chunk, head) record written by the chunk-prep kernels and read by the
// chunk-scan kernel: the operands of the state recurrence.  The four matrix
// operands are stored as NP bf16 piece planes (x ~ p0 + p1 (+ p2), see mfma.h),
// so the sequential scan loads them ready for the matrix cores; U and e^{G_C}
// stay fp32.
//   W   [NP][64][KPD]  W = (I + A)^-1 Diag(beta) (K * e^G), token rows
//   Qp  [NP][64][KPD]  Q+ = Q * e^G, token rows
//   KT  [NP][D][64]    K~^T = (K * e^{G_C - G})^T, channel rows
//   Aqk [NP][64][64]   the masked intra-chunk attention, token rows
//   UT  [D][64]        U^T = ((I + A)^-1 Diag(beta) V)^T, fp32
//   eGC [D]            e^{G_C}, the whole-chunk decay, fp32
// (KPD = max(D, 32): channel columns in whole 32-wide matrix-core steps.)
//
// Every tile is stored in matrix-core fragment order (frag_index, ut_index):
// the 16 bytes that lane l of a wave loads for one 16x16x32 step sit at
// ((row block * steps + step) * 64 + l) * 16, so each wave-wide load reads
// 1 KB of contiguous memory, eight whole cache lines.
struct Record {
  size_t W, Qp, KT, Aqk, UT, eGC, bytes;
  size_t tile_plane, aqk_plane;   // bytes of one piece plane of a [64][KPD] tile / of Aqk
};

__host__ __device__ constexpr Record record_layout(int D, int NP) {
  const int KPD = D < 32 ? 32 : D;
  const size_t tp = static_cast<size_t>(64) * KPD * 2;
  const size_t ap = static_cast<size_t>(64) * 64 * 2;
  Record r{};
  r.tile_plane = tp;
  r.aqk_plane = ap;
  r.W = 0;
  r.Qp = r.W + NP * tp;
  r.KT = r.Qp + NP * tp;
  r.Aqk = r.KT + NP * tp;
  r.UT = r.Aqk + NP * ap;
  r.eGC = r.UT + static_cast<size_t>(64) * D * 4;
  r.bytes = (r.eGC + static_cast<size_t>(D) * 4 + 255) / 256 * 256;
  return r;
}

// Element index of X[row][col] in a fragment-ordered bf16 tile with `cols`
// columns (a multiple of 32): lane = row % 16 + 16 * (col % 32 / 8) of step
// (row / 16, col / 32) holds columns col - col % 8 .. +7.
__host__ __device__ constexpr size_t frag_index(int row, int col, int cols) {
  return ((static_cast<size_t>(row >> 4) * (cols >> 5) + (col >> 5)) * 64 + (row & 15) + 16 * ((col & 31) >> 3)) * 8 +
         (col & 7);
}

// Element index of U^T[v][t] (64 token columns, fp32): lane = v % 16 +
// 16 * (t % 16 / 4) of block (v / 16, t / 16) holds tokens t - t % 4 .. +3.
__host__ __device__ constexpr size_t ut_index(int v, int t) {
  return ((static_cast<size_t>(v >> 4) * 4 + (t >> 4)) * 64 + (v & 15) + 16 * ((t & 15) >> 2)) * 4 + (t & 3);
}

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
  const int32_t* chunk0;     // [2N+2] first chunk of each sequence; chunk0[N] = total chunks;
                             // chunk0[N+1] = 1 when the scan takes its narrow value tile;
                             // chunk0[N+2+i] = the i-th sequence in the scan's dispatch order
  const int32_t* chunk_seq;  // [max_chunks] sequence of each chunk
  const int4* desc;          // [max_chunks] (sequence, first token in it, tokens, first packed token)
  int32_t N;
  int32_t s0;                // the table covers positions [s0, s0 + span) of every sequence (0 and
                             // the whole sequence unless the prefill runs in slabs); a multiple of 64
  // The sequence the scan's i-th (sequence, head) group of workgroups runs:
  // the long sequences first, so that their serial chains start at once.
  __device__ int32_t scan_seq(int32_t i) const { return chunk0[N + 2 + i]; }
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
                               int32_t* chunk0, int32_t* chunk_seq, int4* desc, int32_t max_chunks, int32_t H,
                               int32_t D, hipStream_t st, int32_t s0 = 0, int32_t span = INT32_MAX);
// Compute units of the current device (queried on every call).
hipError_t device_cus(int* ncu);
hipError_t launch_chunk_prep(const Params& p, const ChunkTable& t, const PrefillIO& io, uint8_t* records,
                             int max_chunks, bool io_bf16, hipStream_t st);
// The row-block prep kernel (bf16 inputs, dk = dv in {64, 128}, 16-byte
// aligned q/k/v/alpha/conv history); launch_chunk_prep uses it when it applies.
bool chunk_prep_rows_supported(const Params& p, const PrefillIO& io, bool io_bf16);
hipError_t launch_chunk_prep_rows(const Params& p, const ChunkTable& t, const PrefillIO& io, uint8_t* records,
                                  int max_chunks, hipStream_t st);
// device_choice: the value-tile width between the wide and the narrow one
// is taken on the device from chunk0[N+1] (sequence lengths the host does
// not see); otherwise from the batch shape alone.
hipError_t launch_chunk_scan(const Params& p, const ChunkTable& t, const PrefillIO& io, const uint8_t* records,
                             bool io_bf16, bool out_bf16, bool device_choice, hipStream_t st);
hipError_t launch_conv_state_out(const Params& p, const ChunkTable& t, const PrefillIO& io, bool io_bf16,
                                 hipStream_t st);

// The recurrent-form prefill (gates below the chunked form's floor): a token
// preprocess writing one fp32 record of recurrent_record_bytes(D) per (head,
// packed token) into `recs` ([H][total_T] records), and the sequential scan
// over those records, one workgroup per (sequence, head, value tile).
size_t recurrent_record_bytes(int D);
hipError_t launch_token_prep(const Params& p, const ChunkTable& t, const PrefillIO& io, float* recs,
                             int64_t total_T, int max_chunks, bool io_bf16, hipStream_t st);
hipError_t launch_recurrent_scan(const Params& p, const ChunkTable& t, const PrefillIO& io, const float* recs,
                                 int64_t total_T, bool out_bf16, hipStream_t st);

// The output epilogue over `rows` (token, head) rows of D outputs:
// y = o / sqrt(mean(o^2) + eps) * w * sigmoid(gate); y may alias o.
hipError_t launch_output_gate(int D, int64_t rows, const void* o, const void* gate, const float* w, float eps,
                              void* y, bool o_bf16, bool g_bf16, hipStream_t st);

struct DecodeIO {
  const void* q;
  const void* k;
  const void* v;
  const void* alpha;
  const void* b;
  float* state;
  void* conv_state;
  void* o;                   // o, or y when gate is set
  const void* gate;          // [N][H][dv] io dtype: the output epilogue's gate, or null for plain o
  const float* onw;          // [dv] o_norm weight (with gate)
  float oeps;                // o_norm epsilon (with gate)
};

hipError_t launch_decode(const Params& p, const DecodeIO& io, int N, bool io_bf16, bool out_bf16, hipStream_t st);

// K tokens per sequence through state / conv-history pools.
struct DecodeMultiIO {
  const int32_t* slots;      // [N] pool index per sequence (negative: skipped), or null for n
  const int32_t* n_commit;   // [N] tokens whose updates are kept (0..K), or null for K
  const void* q;             // [N][K][H*dk]
  const void* k;
  const void* v;
  const void* alpha;         // [N][K][H][dk]
  const void* b;             // [N][K][H]
  float* state_pool;         // [P][H][dk][dv]
  void* conv_pool;           // [P][3][Ctot]
  void* o;                   // [N][K][H][dv]: o, or y when gate is set
  const void* gate;          // [N][K][H][dv] io dtype, or null for plain o
  const float* onw;          // [dv] o_norm weight (with gate)
  float oeps;                // o_norm epsilon (with gate)
};

hipError_t launch_decode_multi(const Params& p, const DecodeMultiIO& io, int N, int K, bool io_bf16, bool out_bf16,
                               hipStream_t st);

// The backward pass (gradient of o and of the final state).
struct BackwardIO {
  const void* dO;            // [total_T][H][dv] out dtype: gradient of o
  const float* dS_final;     // [N][H][dk][dv] gradient of the final state, or null
  float* dq;                 // [total_T][H*dk] gradient of raw q (fp32)
  float* dk;
  float* dv;                 // [total_T][H*dv]
  float* dalpha;             // [total_T][H][dk]
  float* db;                 // [total_T][H]
  float* dS_init;            // [N][H][dk][dv] or null
  float* dconv;              // [N][3][Ctot] or null
  float* dw_q;               // [H*dk][4]
  float* dw_k;
  float* dw_v;               // [H*dv][4]
  float* ddt_bias;           // [H*dk]
  float* dA_log;             // [H]
};

// Workspace of the backward (besides the chunk table).
struct BackwardWS {
  uint8_t* recs;             // per (16-token block, head) records
  float* Sblk;               // state at every block's start   [blocks][H][D][D]
  float* dSblk;              // adjoint of every block's end state
  float* Dblk;               // Delta of every block            [blocks][H][16][D]
  float* dDblk;              // its gradient
  float* dy;                 // gradient of the conv outputs    [total_T][3][H*D]
  float* pdw;                // per-chunk conv-weight partials  [chunks][3][H*D][4]
  float* pdtb;               // per-block dt_bias partials      [blocks][H][D]
  float* pAlog;              // per-block A_log partials        [blocks][H]
  float* pstage;             // first-pass sums of the partials [bwd_reduce_parts()][3*H*D*4 + H*D + H]
};

int bwd_reduce_parts();

size_t bwd_record_bytes(int D);
hipError_t launch_backward(const Params& p, const ChunkTable& t, const PrefillIO& io, const BackwardIO& g,
                           const BackwardWS& ws, int N, int max_chunks, bool io_bf16, bool do_bf16, hipStream_t st);

}  // namespace kda
