// Host side of the KDA C ABI: validation, workspace layout and launch
// sequencing on the caller's stream.  No allocation, no synchronisation, no
// host reads of device memory.
#include <cmath>
#include <cstddef>
#include <cstdint>

#include "kda_internal.h"

namespace {

using kda::ChunkTable;
using kda::Params;
using kda::PrefillIO;

constexpr size_t kAlign = 256;
constexpr uint32_t kKnownFlags = KDA_FLAG_SKIP_CONV | KDA_FLAG_SKIP_L2NORM | KDA_FLAG_RAW_GATE |
                                 KDA_FLAG_RAW_BETA | KDA_FLAG_BETA_X2;
// Sub-block decay factors e^{-P} of 16 tokens stay finite in fp32 when every
// log decay is >= -5.4 (16 * 5.4 = 86.4 < ln FLT_MAX).  A lower bound below
// it (down to -inf, no clamp) routes a prefill to the recurrent form, whose
// state is only ever multiplied by e^g <= 1.
constexpr float kChunkedGateFloor = -5.4f;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

kda_status_t check_config(const kda_config_t* cfg, bool chunked) {
  if (!cfg) return KDA_ERR_INVALID_ARGUMENT;
  if (cfg->num_heads < 1 || cfg->head_k_dim < 1 || cfg->head_v_dim < 1) return KDA_ERR_INVALID_ARGUMENT;
  if (cfg->num_heads > 65535) return KDA_ERR_UNSUPPORTED;
  if (cfg->head_k_dim != cfg->head_v_dim) return KDA_ERR_UNSUPPORTED;
  const int d = cfg->head_k_dim;
  if (d != 16 && d != 32 && d != 64 && d != 128) return KDA_ERR_UNSUPPORTED;
  if ((cfg->io_dtype != KDA_BF16 && cfg->io_dtype != KDA_FP32) ||
      (cfg->out_dtype != KDA_BF16 && cfg->out_dtype != KDA_FP32))
    return KDA_ERR_UNSUPPORTED;
  if (cfg->flags & ~kKnownFlags) return KDA_ERR_UNSUPPORTED;
  if (chunked && cfg->chunk_size != kda::kChunk) return KDA_ERR_UNSUPPORTED;
  if (std::isnan(cfg->gate_lower_bound) || std::isnan(cfg->l2norm_eps) || std::isnan(cfg->scale))
    return KDA_ERR_INVALID_ARGUMENT;
  if (!cfg->A_log || !cfg->dt_bias) return KDA_ERR_INVALID_ARGUMENT;
  if (!(cfg->flags & KDA_FLAG_SKIP_CONV) && (!cfg->conv_w_q || !cfg->conv_w_k || !cfg->conv_w_v))
    return KDA_ERR_INVALID_ARGUMENT;
  return KDA_OK;
}

// The prefill form a configuration takes: chunked unless the gate's lower
// bound is below the floor.  With KDA_FLAG_RAW_GATE the bound is not applied
// to g, but it still selects the form.
bool recurrent_form(const kda_config_t* cfg) { return !(cfg->gate_lower_bound >= kChunkedGateFloor); }

Params make_params(const kda_config_t* cfg) {
  Params p;
  p.H = cfg->num_heads;
  p.D = cfg->head_k_dim;
  p.scale = cfg->scale;
  p.lower_bound = cfg->gate_lower_bound;
  p.eps = cfg->l2norm_eps;
  p.flags = cfg->flags;
  p.A_log = cfg->A_log;
  p.dt_bias = cfg->dt_bias;
  p.wq = cfg->conv_w_q;
  p.wk = cfg->conv_w_k;
  p.wv = cfg->conv_w_v;
  return p;
}

// bf16 pieces per matrix operand: 2 for bf16 inputs, 3 for the all-fp32 path.
int pieces(const kda_config_t* cfg) { return cfg->io_dtype == KDA_BF16 ? 2 : 3; }

struct Layout {
  size_t cu, chunk0, chunk_seq, desc, records, total;
};

// records: the chunked form's per-(chunk, head) records, or the recurrent
// form's per-(head, token) records.
Layout make_layout(const kda_config_t* cfg, int64_t N, int64_t max_chunks, int64_t total_T) {
  const int64_t H = cfg->num_heads, D = cfg->head_k_dim;
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
  L.cu = take((N + 1) * sizeof(int32_t));
  L.chunk0 = take((2 * N + 2) * sizeof(int32_t));   // and the scan's sequence order
  L.chunk_seq = take(static_cast<size_t>(max_chunks > 0 ? max_chunks : 1) * sizeof(int32_t));
  L.desc = take(static_cast<size_t>(max_chunks > 0 ? max_chunks : 1) * sizeof(int4));
  if (recurrent_form(cfg))
    L.records = take(static_cast<size_t>(H) * total_T * kda::recurrent_record_bytes(static_cast<int>(D)));
  else
    L.records = take(static_cast<size_t>(max_chunks) * H * kda::record_layout(static_cast<int>(D), pieces(cfg)).bytes);
  L.total = off;
  return L;
}

int64_t chunks_uniform(int64_t B, int64_t T) { return B * ((T + kda::kChunk - 1) / kda::kChunk); }
int64_t chunks_varlen(int64_t N, int64_t total_T) { return (total_T + kda::kChunk - 1) / kda::kChunk + N; }

kda_status_t hip_status(hipError_t e) { return e == hipSuccess ? KDA_OK : KDA_ERR_HIP; }

// Records the caller's timing event `which` (0 = before, 1 = after) of a stage.
void mark(const kda_config_t* cfg, int stage, int which, hipStream_t st) {
  if (!cfg->stage_events) return;
  void* ev = cfg->stage_events[2 * stage + which];
  if (ev) (void)hipEventRecord(static_cast<hipEvent_t>(ev), st);
}

// Runs one stage's launcher between its two timing marks.
template <class F>
kda_status_t stage(const kda_config_t* cfg, int s, hipStream_t st, F&& launch) {
  mark(cfg, s, 0, st);
  const hipError_t e = launch();
  mark(cfg, s, 1, st);
  return hip_status(e);
}

// The shared prefill pipeline over a packed batch.
kda_status_t run_prefill(const kda_config_t* cfg, int32_t N, int64_t total_T, int64_t max_chunks,
                         const int32_t* cu_in, int32_t T_uniform, const PrefillIO& io, void* workspace,
                         hipStream_t st) {
  const Params p = make_params(cfg);
  const Layout L = make_layout(cfg, N, max_chunks, total_T);
  char* ws = static_cast<char*>(workspace);
  int32_t* cu_ws = reinterpret_cast<int32_t*>(ws + L.cu);
  int32_t* chunk0 = reinterpret_cast<int32_t*>(ws + L.chunk0);
  int32_t* chunk_seq = reinterpret_cast<int32_t*>(ws + L.chunk_seq);
  int4* desc = reinterpret_cast<int4*>(ws + L.desc);
  ChunkTable t{cu_ws, chunk0, chunk_seq, desc, N, 0};
  uint8_t* records = reinterpret_cast<uint8_t*>(ws + L.records);
  const bool io_bf16 = cfg->io_dtype == KDA_BF16;
  const bool out_bf16 = cfg->out_dtype == KDA_BF16;
  const int mc = static_cast<int>(max_chunks);

  kda_status_t s = stage(cfg, KDA_STAGE_CHUNK_TABLE, st, [&] {
    return kda::launch_build_chunks(cu_in, N, T_uniform, cu_ws, chunk0, chunk_seq, desc, mc, p.H, p.D, st);
  });
  if (s != KDA_OK) return s;
  if (recurrent_form(cfg)) {
    float* recs = reinterpret_cast<float*>(records);
    s = stage(cfg, KDA_STAGE_CHUNK_PREP, st,
              [&] { return kda::launch_token_prep(p, t, io, recs, total_T, mc, io_bf16, st); });
    if (s != KDA_OK) return s;
    s = stage(cfg, KDA_STAGE_CHUNK_SCAN, st,
              [&] { return kda::launch_recurrent_scan(p, t, io, recs, total_T, out_bf16, st); });
    if (s != KDA_OK) return s;
  } else {
    if (total_T > 0 && mc > 0) {
      s = stage(cfg, KDA_STAGE_CHUNK_PREP, st,
                [&] { return kda::launch_chunk_prep(p, t, io, records, mc, io_bf16, st); });
      if (s != KDA_OK) return s;
    }
    // equal lengths: the host knows the batch shape; packed sequences of any
    // lengths: the value-tile width is chosen on the device
    const bool device_choice = cu_in != nullptr;
    s = stage(cfg, KDA_STAGE_CHUNK_SCAN, st, [&] {
      return kda::launch_chunk_scan(p, t, io, records, io_bf16, out_bf16, device_choice, st);
    });
    if (s != KDA_OK) return s;
  }
  if (io.conv_out) {
    s = stage(cfg, KDA_STAGE_CONV_STATE, st, [&] { return kda::launch_conv_state_out(p, t, io, io_bf16, st); });
    if (s != KDA_OK) return s;
  }
  return KDA_OK;
}

// The chunked prefill in slabs, for a workspace smaller than a whole pass
// needs: windows of `slab` positions (a multiple of 64) of every sequence,
// one after the other, each a chunk table, a prep and a scan over the
// window's chunks, with the state carried from window to window in place
// (in the caller's final state, or in a buffer of the workspace).  The
// result is bit-identical to one pass: the scan's state at a chunk boundary
// is the same fp32 value whether it stays in registers or goes to memory.
struct SlabLayout {
  Layout L;
  size_t state, total;
};

SlabLayout make_slab_layout(const kda_config_t* cfg, int64_t N, int64_t slab) {
  SlabLayout S{};
  S.L = make_layout(cfg, N, N * (slab / kda::kChunk), 0);
  S.state = S.L.total;
  S.total = align_up(S.state + static_cast<size_t>(N) * cfg->num_heads * cfg->head_k_dim * cfg->head_v_dim * 4);
  return S;
}

// The longest slab (a multiple of 64 tokens, at most `cap`) whose workspace
// fits in `bytes`, or 0.
int64_t slab_for(const kda_config_t* cfg, int64_t N, size_t bytes, int64_t cap) {
  if (N <= 0 || make_slab_layout(cfg, N, kda::kChunk).total > bytes) return 0;
  int64_t lo = 1, hi = (cap + kda::kChunk - 1) / kda::kChunk;   // in chunks
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) / 2;
    if (make_slab_layout(cfg, N, mid * kda::kChunk).total <= bytes) lo = mid; else hi = mid - 1;
  }
  return lo * kda::kChunk;
}

kda_status_t run_prefill_slabs(const kda_config_t* cfg, int32_t N, int64_t total_T, const int32_t* cu_in,
                               int32_t T_uniform, const PrefillIO& io, void* workspace, int64_t slab,
                               hipStream_t st) {
  const Params p = make_params(cfg);
  const SlabLayout S = make_slab_layout(cfg, N, slab);
  char* ws = static_cast<char*>(workspace);
  int32_t* cu_ws = reinterpret_cast<int32_t*>(ws + S.L.cu);
  int32_t* chunk0 = reinterpret_cast<int32_t*>(ws + S.L.chunk0);
  int32_t* chunk_seq = reinterpret_cast<int32_t*>(ws + S.L.chunk_seq);
  int4* desc = reinterpret_cast<int4*>(ws + S.L.desc);
  uint8_t* records = reinterpret_cast<uint8_t*>(ws + S.L.records);
  float* state = io.S_out ? io.S_out : reinterpret_cast<float*>(ws + S.state);
  const bool io_bf16 = cfg->io_dtype == KDA_BF16;
  const bool out_bf16 = cfg->out_dtype == KDA_BF16;
  const int mc = static_cast<int>(static_cast<int64_t>(N) * (slab / kda::kChunk));
  // the longest a sequence can be: the batch's length, or all its tokens
  const int64_t longest = cu_in ? total_T : T_uniform;
  const int64_t nslabs = longest > 0 ? (longest + slab - 1) / slab : 1;   // (one pass writes the states of an empty batch)
  for (int64_t k = 0; k < nslabs; ++k) {
    const int32_t s0 = static_cast<int32_t>(k * slab);
    PrefillIO sio = io;
    sio.S0 = k == 0 ? io.S0 : state;
    sio.S_out = state;
    sio.conv_out = nullptr;
    ChunkTable t{cu_ws, chunk0, chunk_seq, desc, N, s0};
    hipError_t e = kda::launch_build_chunks(cu_in, N, T_uniform, cu_ws, chunk0, chunk_seq, desc, mc, p.H, p.D, st,
                                            s0, static_cast<int32_t>(slab));
    if (e == hipSuccess) e = kda::launch_chunk_prep(p, t, sio, records, mc, io_bf16, st);
    if (e == hipSuccess) e = kda::launch_chunk_scan(p, t, sio, records, io_bf16, out_bf16, cu_in != nullptr, st);
    if (e != hipSuccess) return KDA_ERR_HIP;
  }
  if (io.conv_out) {   // (the table's sequence offsets are the whole batch's)
    const ChunkTable t{cu_ws, chunk0, chunk_seq, desc, N, 0};
    return stage(cfg, KDA_STAGE_CONV_STATE, st, [&] { return kda::launch_conv_state_out(p, t, io, io_bf16, st); });
  }
  return KDA_OK;
}

// The backward's workspace: the chunk table, then per 16-token block and
// head its record, the block-start state and the block-end adjoint, Delta and
// its gradient; the conv outputs' gradient per token; the partial parameter
// gradients per chunk / block and their first-pass sums.
struct BwdLayout {
  size_t cu, chunk0, chunk_seq, desc, recs, Sblk, dSblk, Dblk, dDblk, dy, pdw, pdtb, pAlog, pstage, total;
};

BwdLayout make_bwd_layout(const kda_config_t* cfg, int64_t N, int64_t max_chunks, int64_t total_T) {
  const int64_t H = cfg->num_heads, D = cfg->head_k_dim;
  const int64_t mc = max_chunks > 0 ? max_chunks : 1;
  const int64_t blocks = mc * (kda::kChunk / 16);
  BwdLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
  L.cu = take((N + 1) * sizeof(int32_t));
  L.chunk0 = take((2 * N + 2) * sizeof(int32_t));   // and the scan's sequence order
  L.chunk_seq = take(static_cast<size_t>(mc) * sizeof(int32_t));
  L.desc = take(static_cast<size_t>(mc) * sizeof(int4));
  L.recs = take(static_cast<size_t>(blocks) * H * kda::bwd_record_bytes(static_cast<int>(D)));
  L.Sblk = take(static_cast<size_t>(blocks) * H * D * D * 4);
  L.dSblk = take(static_cast<size_t>(blocks) * H * D * D * 4);
  L.Dblk = take(static_cast<size_t>(blocks) * H * 16 * D * 4);
  L.dDblk = take(static_cast<size_t>(blocks) * H * 16 * D * 4);
  L.dy = take(static_cast<size_t>(total_T > 0 ? total_T : 1) * 3 * H * D * 4);
  L.pdw = take(static_cast<size_t>(mc) * 3 * H * D * 4 * 4);
  L.pdtb = take(static_cast<size_t>(blocks) * H * D * 4);
  L.pAlog = take(static_cast<size_t>(blocks) * H * 4);
  L.pstage = take(static_cast<size_t>(kda::bwd_reduce_parts()) * (H * D * (3 * 4 + 1) + H) * 4);
  L.total = off;
  return L;
}

// The backward handles the method as described plus beta x2; the other test
// hooks and the recurrent form's gates (below -5.4) are not built.
kda_status_t check_backward(const kda_config_t* cfg) {
  kda_status_t s = check_config(cfg, true);
  if (s != KDA_OK) return s;
  if (cfg->flags & ~static_cast<uint32_t>(KDA_FLAG_BETA_X2)) return KDA_ERR_UNSUPPORTED;
  if (recurrent_form(cfg)) return KDA_ERR_UNSUPPORTED;
  return KDA_OK;
}

}  // namespace

extern "C" {

int32_t kda_version(void) { return 105; }

size_t kda_varlen_backward_workspace_bytes(const kda_config_t* cfg, int32_t N, int32_t total_T) {
  if (check_backward(cfg) != KDA_OK || N < 0 || total_T < 0) return 0;
  return make_bwd_layout(cfg, N, chunks_varlen(N, total_T), total_T).total;
}

kda_status_t kda_varlen_backward(const kda_config_t* cfg, int32_t N, int32_t total_T, const int32_t* cu_seqlens,
                                 const void* q, const void* k, const void* v, const void* alpha, const void* b,
                                 const float* initial_state, const void* conv_state_in, const void* d_o,
                                 const float* d_final_state, float* dq, float* dk, float* dv, float* dalpha, float* db,
                                 float* d_initial_state, float* d_conv_state_in, float* dw_q, float* dw_k,
                                 float* dw_v, float* ddt_bias, float* dA_log, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  kda_status_t s = check_backward(cfg);
  if (s != KDA_OK) return s;
  if (N < 0 || total_T < 0) return KDA_ERR_INVALID_ARGUMENT;
  if (N == 0) return KDA_OK;
  if (!cu_seqlens || !dw_q || !dw_k || !dw_v || !ddt_bias || !dA_log) return KDA_ERR_INVALID_ARGUMENT;
  if (total_T > 0 && (!q || !k || !v || !alpha || !b || !d_o || !dq || !dk || !dv || !dalpha || !db))
    return KDA_ERR_INVALID_ARGUMENT;
  const int64_t mc = chunks_varlen(N, total_T);
  if (mc * (kda::kChunk / 16) * cfg->num_heads > INT32_MAX) return KDA_ERR_UNSUPPORTED;
  const BwdLayout L = make_bwd_layout(cfg, N, mc, total_T);
  if (!workspace) return KDA_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < L.total) return KDA_ERR_WORKSPACE_TOO_SMALL;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const Params p = make_params(cfg);
  char* ws = static_cast<char*>(workspace);
  int32_t* cu_ws = reinterpret_cast<int32_t*>(ws + L.cu);
  int32_t* chunk0 = reinterpret_cast<int32_t*>(ws + L.chunk0);
  int32_t* chunk_seq = reinterpret_cast<int32_t*>(ws + L.chunk_seq);
  int4* desc = reinterpret_cast<int4*>(ws + L.desc);
  ChunkTable t{cu_ws, chunk0, chunk_seq, desc, N, 0};
  PrefillIO io{q, k, v, alpha, b, initial_state, conv_state_in, nullptr, nullptr, nullptr};
  kda::BackwardIO g{d_o, d_final_state, dq, dk, dv, dalpha, db, d_initial_state, d_conv_state_in,
                    dw_q, dw_k, dw_v, ddt_bias, dA_log};
  kda::BackwardWS w{reinterpret_cast<uint8_t*>(ws + L.recs), reinterpret_cast<float*>(ws + L.Sblk),
                    reinterpret_cast<float*>(ws + L.dSblk), reinterpret_cast<float*>(ws + L.Dblk),
                    reinterpret_cast<float*>(ws + L.dDblk), reinterpret_cast<float*>(ws + L.dy),
                    reinterpret_cast<float*>(ws + L.pdw), reinterpret_cast<float*>(ws + L.pdtb),
                    reinterpret_cast<float*>(ws + L.pAlog), reinterpret_cast<float*>(ws + L.pstage)};
  const int imc = static_cast<int>(mc);
  s = stage(cfg, KDA_STAGE_CHUNK_TABLE, st, [&] {
    return kda::launch_build_chunks(cu_seqlens, N, 0, cu_ws, chunk0, chunk_seq, desc, imc, p.H, p.D, st);
  });
  if (s != KDA_OK) return s;
  return stage(cfg, KDA_STAGE_BACKWARD, st, [&] {
    return kda::launch_backward(p, t, io, g, w, N, imc, cfg->io_dtype == KDA_BF16, cfg->out_dtype == KDA_BF16, st);
  });
}

const char* kda_status_string(kda_status_t status) {
  switch (status) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARGUMENT: return "KDA_ERR_INVALID_ARGUMENT";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_WORKSPACE_TOO_SMALL: return "KDA_ERR_WORKSPACE_TOO_SMALL";
    case KDA_ERR_HIP: return "KDA_ERR_HIP";
    default: return "KDA_ERR_UNKNOWN";
  }
}

size_t kda_prefill_workspace_bytes(const kda_config_t* cfg, int32_t B, int32_t T) {
  if (check_config(cfg, true) != KDA_OK || B < 0 || T < 0) return 0;
  const int64_t mc = chunks_uniform(B, T);
  if (static_cast<int64_t>(B) * T > INT32_MAX || mc > INT32_MAX) return 0;
  return make_layout(cfg, B, mc, static_cast<int64_t>(B) * T).total;
}

size_t kda_varlen_workspace_bytes(const kda_config_t* cfg, int32_t N, int32_t total_T) {
  if (check_config(cfg, true) != KDA_OK || N < 0 || total_T < 0) return 0;
  return make_layout(cfg, N, chunks_varlen(N, total_T), total_T).total;
}

size_t kda_prefill_slab_workspace_bytes(const kda_config_t* cfg, int32_t N, int32_t slab_tokens) {
  if (check_config(cfg, true) != KDA_OK || N < 1 || slab_tokens < 1 || recurrent_form(cfg)) return 0;
  const int64_t slab = (static_cast<int64_t>(slab_tokens) + kda::kChunk - 1) / kda::kChunk * kda::kChunk;
  if (static_cast<int64_t>(N) * (slab / kda::kChunk) > INT32_MAX) return 0;
  return make_slab_layout(cfg, N, slab).total;
}

kda_status_t kda_prefill(const kda_config_t* cfg, int32_t B, int32_t T, const void* q, const void* k, const void* v,
                         const void* alpha, const void* b, const float* initial_state, const void* conv_state_in,
                         void* o, float* final_state, void* conv_state_out, void* workspace, size_t workspace_bytes,
                         void* stream) {
  kda_status_t s = check_config(cfg, true);
  if (s != KDA_OK) return s;
  if (B < 0 || T < 0) return KDA_ERR_INVALID_ARGUMENT;
  if (static_cast<int64_t>(B) * T > INT32_MAX) return KDA_ERR_UNSUPPORTED;
  if (B == 0) return KDA_OK;
  if (T > 0 && (!q || !k || !v || !alpha || !b || !o)) return KDA_ERR_INVALID_ARGUMENT;
  const int64_t mc = chunks_uniform(B, T);
  const size_t need = make_layout(cfg, B, mc, static_cast<int64_t>(B) * T).total;
  if (!workspace) return KDA_ERR_INVALID_ARGUMENT;
  PrefillIO io{q, k, v, alpha, b, initial_state, conv_state_in, o, final_state, conv_state_out};
  if (workspace_bytes < need) {   // the chunked form runs in slabs of T, if one of 64 tokens fits
    const int64_t slab = recurrent_form(cfg) ? 0 : slab_for(cfg, B, workspace_bytes, T);
    if (slab <= 0) return KDA_ERR_WORKSPACE_TOO_SMALL;
    return run_prefill_slabs(cfg, B, static_cast<int64_t>(B) * T, nullptr, T, io, workspace, slab,
                             static_cast<hipStream_t>(stream));
  }
  return run_prefill(cfg, B, static_cast<int64_t>(B) * T, mc, nullptr, T, io, workspace,
                     static_cast<hipStream_t>(stream));
}

kda_status_t kda_varlen_prefill(const kda_config_t* cfg, int32_t N, int32_t total_T, const int32_t* cu_seqlens,
                                const void* q, const void* k, const void* v, const void* alpha, const void* b,
                                const float* initial_state, const void* conv_state_in, void* o, float* final_state,
                                void* conv_state_out, void* workspace, size_t workspace_bytes, void* stream) {
  kda_status_t s = check_config(cfg, true);
  if (s != KDA_OK) return s;
  if (N < 0 || total_T < 0) return KDA_ERR_INVALID_ARGUMENT;
  if (N == 0) return KDA_OK;
  if (!cu_seqlens) return KDA_ERR_INVALID_ARGUMENT;
  if (total_T > 0 && (!q || !k || !v || !alpha || !b || !o)) return KDA_ERR_INVALID_ARGUMENT;
  const int64_t mc = chunks_varlen(N, total_T);
  if (mc > INT32_MAX) return KDA_ERR_UNSUPPORTED;
  const size_t need = make_layout(cfg, N, mc, total_T).total;
  if (!workspace) return KDA_ERR_INVALID_ARGUMENT;
  PrefillIO io{q, k, v, alpha, b, initial_state, conv_state_in, o, final_state, conv_state_out};
  if (workspace_bytes < need) {   // the chunked form runs in slabs, if one of 64 tokens per sequence fits
    const int64_t slab = recurrent_form(cfg) ? 0 : slab_for(cfg, N, workspace_bytes, total_T);
    if (slab <= 0) return KDA_ERR_WORKSPACE_TOO_SMALL;
    return run_prefill_slabs(cfg, N, total_T, cu_seqlens, 0, io, workspace, slab, static_cast<hipStream_t>(stream));
  }
  return run_prefill(cfg, N, total_T, mc, cu_seqlens, 0, io, workspace, static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// Shared by the plain and the gated decode entry points; gate == nullptr for
// the plain one.
kda_status_t decode_step(const kda_config_t* cfg, int32_t N, const void* q, const void* k, const void* v,
                         const void* alpha, const void* b, float* state, void* conv_state, const void* gate,
                         const float* onw, float oeps, void* o, void* stream) {
  kda_status_t s = check_config(cfg, false);
  if (s != KDA_OK) return s;
  if (N < 0) return KDA_ERR_INVALID_ARGUMENT;
  if (static_cast<int64_t>(N) * cfg->num_heads > INT32_MAX) return KDA_ERR_UNSUPPORTED;
  if (N == 0) return KDA_OK;
  if (!q || !k || !v || !alpha || !b || !state || !conv_state || !o) return KDA_ERR_INVALID_ARGUMENT;
  const Params p = make_params(cfg);
  kda::DecodeIO io{q, k, v, alpha, b, state, conv_state, o, gate, onw, oeps};
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return stage(cfg, KDA_STAGE_DECODE, st, [&] {
    return kda::launch_decode(p, io, N, cfg->io_dtype == KDA_BF16, cfg->out_dtype == KDA_BF16, st);
  });
}

kda_status_t decode_multi(const kda_config_t* cfg, int32_t N, int32_t K, const int32_t* slots, const void* q,
                          const void* k, const void* v, const void* alpha, const void* b, float* state_pool,
                          void* conv_pool, const void* gate, const float* onw, float oeps, void* o,
                          const int32_t* n_commit, void* stream) {
  kda_status_t s = check_config(cfg, false);
  if (s != KDA_OK) return s;
  if (N < 0 || K < 1) return KDA_ERR_INVALID_ARGUMENT;
  if (K > 64) return KDA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(N) * cfg->num_heads > INT32_MAX) return KDA_ERR_UNSUPPORTED;
  if (N == 0) return KDA_OK;
  if (!q || !k || !v || !alpha || !b || !state_pool || !conv_pool || !o) return KDA_ERR_INVALID_ARGUMENT;
  const Params p = make_params(cfg);
  kda::DecodeMultiIO io{slots, n_commit, q, k, v, alpha, b, state_pool, conv_pool, o, gate, onw, oeps};
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return stage(cfg, KDA_STAGE_DECODE, st, [&] {
    return kda::launch_decode_multi(p, io, N, K, cfg->io_dtype == KDA_BF16, cfg->out_dtype == KDA_BF16, st);
  });
}

bool bad_epilogue_args(const void* gate, const float* onw, float eps) {
  return !gate || !onw || std::isnan(eps) || eps < 0.f;
}

}  // namespace

extern "C" {

kda_status_t kda_decode_step(const kda_config_t* cfg, int32_t N, const void* q, const void* k, const void* v,
                             const void* alpha, const void* b, float* state, void* conv_state, void* o,
                             void* stream) {
  return decode_step(cfg, N, q, k, v, alpha, b, state, conv_state, nullptr, nullptr, 0.f, o, stream);
}

kda_status_t kda_decode_step_gated(const kda_config_t* cfg, int32_t N, const void* q, const void* k, const void* v,
                                   const void* alpha, const void* b, float* state, void* conv_state,
                                   const void* gate, const float* o_norm_weight, float eps, void* y, void* stream) {
  if (cfg && N > 0 && bad_epilogue_args(gate, o_norm_weight, eps)) return KDA_ERR_INVALID_ARGUMENT;
  return decode_step(cfg, N, q, k, v, alpha, b, state, conv_state, gate, o_norm_weight, eps, y, stream);
}

kda_status_t kda_decode_multi(const kda_config_t* cfg, int32_t N, int32_t K, const int32_t* slots, const void* q,
                              const void* k, const void* v, const void* alpha, const void* b, float* state_pool,
                              void* conv_pool, void* o, const int32_t* n_commit, void* stream) {
  return decode_multi(cfg, N, K, slots, q, k, v, alpha, b, state_pool, conv_pool, nullptr, nullptr, 0.f, o,
                      n_commit, stream);
}

kda_status_t kda_decode_multi_gated(const kda_config_t* cfg, int32_t N, int32_t K, const int32_t* slots,
                                    const void* q, const void* k, const void* v, const void* alpha, const void* b,
                                    float* state_pool, void* conv_pool, const void* gate,
                                    const float* o_norm_weight, float eps, void* y, const int32_t* n_commit,
                                    void* stream) {
  if (cfg && N > 0 && bad_epilogue_args(gate, o_norm_weight, eps)) return KDA_ERR_INVALID_ARGUMENT;
  return decode_multi(cfg, N, K, slots, q, k, v, alpha, b, state_pool, conv_pool, gate, o_norm_weight, eps, y,
                      n_commit, stream);
}

kda_status_t kda_output_gate(const kda_config_t* cfg, int64_t n_tokens, const void* o, const void* gate,
                             const float* o_norm_weight, float eps, void* y, void* stream) {
  if (!cfg) return KDA_ERR_INVALID_ARGUMENT;
  if (cfg->num_heads < 1 || cfg->head_v_dim < 1) return KDA_ERR_INVALID_ARGUMENT;
  if (cfg->num_heads > 65535) return KDA_ERR_UNSUPPORTED;
  const int dv = cfg->head_v_dim;
  if (dv != 16 && dv != 32 && dv != 64 && dv != 128) return KDA_ERR_UNSUPPORTED;
  if ((cfg->io_dtype != KDA_BF16 && cfg->io_dtype != KDA_FP32) ||
      (cfg->out_dtype != KDA_BF16 && cfg->out_dtype != KDA_FP32))
    return KDA_ERR_UNSUPPORTED;
  if (n_tokens < 0 || std::isnan(eps) || eps < 0.f) return KDA_ERR_INVALID_ARGUMENT;
  if (n_tokens > INT64_MAX / cfg->num_heads / dv) return KDA_ERR_UNSUPPORTED;
  if (n_tokens == 0) return KDA_OK;
  if (!o || !gate || !o_norm_weight || !y) return KDA_ERR_INVALID_ARGUMENT;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t rows = n_tokens * cfg->num_heads;
  return stage(cfg, KDA_STAGE_OUTPUT_GATE, st, [&] {
    return kda::launch_output_gate(dv, rows, o, gate, o_norm_weight, eps, y, cfg->out_dtype == KDA_BF16,
                                   cfg->io_dtype == KDA_BF16, st);
  });
}

}  // extern "C"
