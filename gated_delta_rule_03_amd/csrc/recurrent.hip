// Prefill in the token-by-token recurrent form, for gates without the safe
// lower bound (gate_lower_bound below the chunked form's floor, down to
// -inf).
//
// The chunked form factors the decay of a 16-token sub-block into e^{+P} and
// e^{-P}; with unbounded log decays e^{-P} overflows fp32.  The recurrence of
// the AliceAI page (section 二, the delta-rule loop) only ever multiplies the
// state by e^g <= 1, so it holds for any gate:
//   S~ = Diag(e^g) S;  delta = beta (v - k^T S~);  S = S~ + k delta^T;
//   o = q^T S = q^T S~ + (q . k) delta
// Two kernels:
//  1. token_prep_kernel, parallel over (64-token chunk, head) through the same
//     chunk table as the chunked form: conv + SiLU, L2 norms, gate and beta
//     per token, written as one fp32 token record per (head, token):
//       [0, D) q^ (scale applied)  [D, 2D) k^  [2D, 3D) e^g  [3D, 4D) v^
//       [4D] beta  [4D+1] q^ . k^  [4D+2, 4D+4) zero
//     Records of one head are consecutive in token order, so the scan of one
//     (sequence, head) streams a contiguous range.
//  2. recurrent_scan_kernel, one workgroup per (sequence, head, value tile):
//     the fp32 state slice lives in registers for the whole sequence.  Lane
//     (rg, cg) of a wave holds D/16 key rows x CPL value columns; the column
//     sums k^T S~ and q^T S~ are reduced over the 16 lanes of a row group with
//     four DPP steps, so a token needs no barrier.  The waves of a workgroup
//     share the token records, staged 16 tokens at a time in LDS
//     (double-buffered, one barrier per 16 tokens; the next block's loads are
//     in flight while the current one is computed).
#include "kda_device.h"
#include "kda_internal.h"
#include "mfma.h"

namespace kda {

namespace {

constexpr int kTokBlock = 16;       // tokens staged per LDS block

__host__ __device__ constexpr int rec_floats(int D) { return 4 * D + 4; }

}  // namespace

size_t recurrent_record_bytes(int D) { return static_cast<size_t>(rec_floats(D)) * 4; }

// ---- 1. token preprocess ---------------------------------------------------
// 4D lanes: lane t has role t / D (q, k, v, alpha) and channel t % D and
// slides the conv window down the chunk, as in the chunked form's prep.
template <int D, bool IO_BF16>
__global__ __launch_bounds__(4 * D) void token_prep_kernel(Params p, ChunkTable t, float* __restrict__ recs,
                                                           int64_t total_T, const void* conv_in, const void* qin,
                                                           const void* kin, const void* vin, const void* ain,
                                                           const void* bin) {
  constexpr int RF = rec_floats(D);
  constexpr int LQ = D + 4;        // LDS row stride of the q and k tiles (16-byte rows)
  constexpr int TPT = D / 16;      // threads per token in the norm step (16 channels each)
  __shared__ __align__(16) float sQ[kChunk * LQ];
  __shared__ __align__(16) float sK[kChunk * LQ];

  // one-dimensional grid, head fastest (grid dimension y holds at most 65536)
  const int h = static_cast<int>(blockIdx.x % static_cast<unsigned>(p.H));
  const int c = static_cast<int>(blockIdx.x / static_cast<unsigned>(p.H));
  if (c >= t.chunk0[t.N]) return;
  const int H = p.H;
  const int4 dsc = t.desc[c];      // (sequence, first token in it, tokens, first packed token)
  const int s = dsc.x, tau0 = dsc.y;
  const int64_t tok0 = dsc.w;
  const int len = static_cast<int>(min(static_cast<int64_t>(dsc.z), total_T - tok0));
  if (len <= 0) return;
  const int tid = threadIdx.x;
  const int role = tid / D, ch = tid % D;
  const size_t HD = static_cast<size_t>(H) * D;
  const size_t Ctot = 3 * HD;
  const size_t col = static_cast<size_t>(h) * D + ch;
  const uint32_t flags = p.flags;
  float* rbase = recs + (static_cast<size_t>(h) * total_T + tok0) * RF;

  if (role < 3) {
    const void* xin = role == 0 ? qin : (role == 1 ? kin : vin);
    const void* w = role == 0 ? p.wq : (role == 1 ? p.wk : p.wv);
    const bool raw = flags & KDA_FLAG_SKIP_CONV;
    // every load goes out unconditionally (a load under a condition compiles
    // to a branch that waits for it), the unused values replaced afterwards
    float w0 = ld<IO_BF16>(w, col * 4), w1 = ld<IO_BF16>(w, col * 4 + 1);
    float w2 = ld<IO_BF16>(w, col * 4 + 2), w3 = ld<IO_BF16>(w, col * 4 + 3);
    float hm[3];
#pragma unroll
    for (int m = 0; m < 3; ++m) {
      const int tau = tau0 - 3 + m;
      const bool hist = tau < 0 && conv_in != nullptr;
      const void* src = hist ? conv_in : xin;
      const size_t idx = hist ? (static_cast<size_t>(s) * 3 + (3 + tau)) * Ctot + role * HD + col
                              : static_cast<size_t>(tok0 - tau0 + max(tau, 0)) * HD + col;
      hm[m] = ld<IO_BF16>(src, idx);
    }
#pragma unroll
    for (int m = 0; m < 3; ++m)
      if (tau0 - 3 + m < 0 && conv_in == nullptr) hm[m] = 0.f;
    if (raw) { w0 = 0.f; w1 = 0.f; w2 = 0.f; w3 = 1.f; }
    float x[kChunk];
#pragma unroll
    for (int r = 0; r < kChunk; ++r)   // rows past the chunk's end re-read its last row
      x[r] = ld<IO_BF16>(xin, static_cast<size_t>(tok0 + min(r, len - 1)) * HD + col);
#pragma unroll
    for (int r = 0; r < kChunk; ++r) {
      const float xm3 = r >= 3 ? x[r - 3] : hm[r], xm2 = r >= 2 ? x[r - 2] : hm[r + 1];
      const float xm1 = r >= 1 ? x[r - 1] : hm[2], xt = x[r];
      const float u = raw ? xt : siluf_(w0 * xm3 + w1 * xm2 + w2 * xm1 + w3 * xt);
      if (role == 0) sQ[r * LQ + ch] = u;
      else if (role == 1) sK[r * LQ + ch] = u;
      else if (r < len) rbase[static_cast<size_t>(r) * RF + 3 * D + ch] = u;
    }
  } else {
    const float a_exp = expf(p.A_log[h]);
    const float dtb = p.dt_bias[col];
    float ar[kChunk];
#pragma unroll
    for (int r = 0; r < kChunk; ++r) ar[r] = ld<IO_BF16>(ain, static_cast<size_t>(tok0 + min(r, len - 1)) * HD + col);
#pragma unroll
    for (int r = 0; r < kChunk; ++r) {
      const float g = (flags & KDA_FLAG_RAW_GATE) ? ar[r] : gate_value(ar[r], dtb, a_exp, p.lower_bound);
      if (r < len) rbase[static_cast<size_t>(r) * RF + 2 * D + ch] = expf(g);
    }
  }
  const float bb = ld<IO_BF16>(bin, static_cast<size_t>(tok0 + min(tid, len - 1)) * H + h);
  if (tid < len) {
    float be = (flags & KDA_FLAG_RAW_BETA) ? bb : sigmoidf_(bb);
    if (flags & KDA_FLAG_BETA_X2) be *= 2.0f;
    float* rr = rbase + static_cast<size_t>(tid) * RF + 4 * D;
    rr[0] = be;
    rr[2] = 0.f;
    rr[3] = 0.f;
  }
  __syncthreads();

  // L2 norms and q.k: TPT lanes per token, 16 channels each
  const bool norm = !(flags & KDA_FLAG_SKIP_L2NORM);
  for (int r0 = 0; r0 < kChunk; r0 += 4 * D / TPT) {
    const int r = r0 + tid / TPT, part = tid % TPT;
    const float4* qp = reinterpret_cast<const float4*>(sQ + r * LQ + part * 16);
    const float4* kp = reinterpret_cast<const float4*>(sK + r * LQ + part * 16);
    float4 qv[4], kv[4];
    float sq = 0.f, sk = 0.f, sqk = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qv[i] = qp[i];
      kv[i] = kp[i];
      sq += qv[i].x * qv[i].x + qv[i].y * qv[i].y + qv[i].z * qv[i].z + qv[i].w * qv[i].w;
      sk += kv[i].x * kv[i].x + kv[i].y * kv[i].y + kv[i].z * kv[i].z + kv[i].w * kv[i].w;
      sqk += qv[i].x * kv[i].x + qv[i].y * kv[i].y + qv[i].z * kv[i].z + qv[i].w * kv[i].w;
    }
    sq = group_sum<TPT>(sq);
    sk = group_sum<TPT>(sk);
    sqk = group_sum<TPT>(sqk);
    if (r < len) {
      const float iq = (norm ? 1.0f / sqrtf(sq + p.eps) : 1.0f) * p.scale;
      const float ik = norm ? 1.0f / sqrtf(sk + p.eps) : 1.0f;
      float* rr = rbase + static_cast<size_t>(r) * RF;
      float4* qo = reinterpret_cast<float4*>(rr + part * 16);
      float4* ko = reinterpret_cast<float4*>(rr + D + part * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qo[i] = make_float4(qv[i].x * iq, qv[i].y * iq, qv[i].z * iq, qv[i].w * iq);
        ko[i] = make_float4(kv[i].x * ik, kv[i].y * ik, kv[i].z * ik, kv[i].w * ik);
      }
      if (part == 0) rr[4 * D + 1] = sqk * iq * ik;
    }
  }
}

// ---- 2. the recurrence -----------------------------------------------------
// NW waves; lane l of wave w: rg = l % RGW (a group of RGW = 8 or 16 lanes
// that splits the D key rows), cg = l / RGW.  Its RPL = D / RGW key rows are
// row(i) = 4 RGW (i / 4) + 4 rg + i % 4 when RPL >= 4 (float4 groups spread
// over the row groups, so a wave's LDS read of one group touches 4 RGW
// consecutive floats), else RPL rg + i; its value columns are
// col0 = tile * DVT + (CG w + cg) CPL .. + CPL - 1, with CG = 64 / RGW and
// DVT = NW CG CPL.
template <int D, int RGW, int NW, int CPL, bool OUT_BF16>
__global__ __launch_bounds__(kWave * NW) void recurrent_scan_kernel(Params p, const int32_t* __restrict__ cu,
                                                                 const int32_t* __restrict__ order,
                                                                 int32_t N, const float* __restrict__ recs,
                                                                 int64_t total_T, const float* S0, float* S_out,
                                                                 void* o) {
  constexpr int NT = kWave * NW;
  constexpr int RF = rec_floats(D);
  constexpr int RPL = D / RGW;                // key rows per lane
  constexpr int CG = kWave / RGW;             // column groups per wave
  constexpr int DVT = NW * CG * CPL;          // value columns per workgroup
  constexpr int NTILE = D / DVT;
  constexpr int BLK4 = kTokBlock * RF / 4;    // float4s of one staged block
  constexpr int PER = (BLK4 + NT - 1) / NT;
  static_assert(D % DVT == 0, "value tiles must cover dv");
  // each buffer holds PER * NT float4s, every lane's share of a block
  // (BLK4 of them are records), so that the deposit is unconditional too
  __shared__ float4 sRec4[2][PER * NT];

  const int H = p.H;
  // the tiles of one (sequence, head) run on one XCD (workgroup i goes to XCD
  // i % 8), so its token records are fetched into one L2
  const int G = N * H * NTILE;
  int L = blockIdx.x;
  if (G % 8 == 0) L = (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8;
  const int tile = L % NTILE, nh = L / NTILE;
  const int n = order[nh / H], h = nh % H;   // the chunk table's order: long sequences first
  const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave;
  const int rg = lane % RGW, cg = lane / RGW;
  const int col0 = tile * DVT + (CG * w + cg) * CPL;

  int row[RPL];
#pragma unroll
  for (int i = 0; i < RPL; ++i) row[i] = RPL >= 4 ? 4 * RGW * (i / 4) + 4 * rg + i % 4 : RPL * rg + i;

  const int64_t tok0 = cu[n];
  const int len = static_cast<int>(max<int64_t>(0, min<int64_t>(cu[n + 1], total_T) - tok0));
  const size_t sbase = (static_cast<size_t>(n) * H + h) * D * D;

  float S[RPL][CPL];
#pragma unroll
  for (int i = 0; i < RPL; ++i)
#pragma unroll
    for (int c = 0; c < CPL; ++c) S[i][c] = S0 ? S0[sbase + static_cast<size_t>(row[i]) * D + col0 + c] : 0.f;
  // The state loads are conditional; without this wait the compiler keeps
  // them pending into the token loop and waits there for every memory
  // access in flight, the next block's prefetch included, at every token.
  __builtin_amdgcn_s_waitcnt(0);

  const float4* src = reinterpret_cast<const float4*>(recs + (static_cast<size_t>(h) * total_T + tok0) * RF);
  const int nb = (len + kTokBlock - 1) / kTokBlock;
  float4 pre[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) pre[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  // Every lane loads unconditionally (exec-masked loads would make the
  // compiler wait for them early); past the block's last token the index is
  // clamped to its last float4, and those copies are never read.
  auto fetch = [&](int b) {
    const int lim = min(kTokBlock, len - b * kTokBlock) * (RF / 4);
    const float4* bs = src + static_cast<size_t>(b) * BLK4;
#pragma unroll
    for (int j = 0; j < PER; ++j) pre[j] = bs[min(tid + j * NT, lim - 1)];
  };
  auto deposit = [&](int buf) {
#pragma unroll
    for (int j = 0; j < PER; ++j) sRec4[buf][tid + j * NT] = pre[j];
  };
  if (nb > 0) {
    fetch(0);
    deposit(0);
  }
  __syncthreads();

  // Outputs: after a token's column sums every lane of a row group holds
  // them, so lane rg keeps the output of token rg of the block (kTokBlock
  // == 16 >= RGW covers every token) and the block's outputs leave in one
  // store per lane after the token loop, which then holds no memory access
  // (a store inside it would make the wait for the next block's loads
  // come before the loop instead of at the LDS deposit).
  static_assert(kTokBlock == 16 && RGW <= kTokBlock, "token t of a block is kept by lane t % 16 of a group");
  const size_t ostride = static_cast<size_t>(H) * D;
  for (int b = 0; b < nb; ++b) {
    // unconditional: the last block fetches itself again into the idle
    // buffer (straight-line code, so the only wait for the loads is at the
    // deposit)
    fetch(min(b + 1, nb - 1));
    const float* blk = reinterpret_cast<const float*>(sRec4[b & 1]);
    const int nt = min(kTokBlock, len - b * kTokBlock);
    float mo[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) mo[c] = 0.f;
#pragma unroll
    for (int tt = 0; tt < kTokBlock; ++tt) {
      if (tt < nt) {
        const float* rec = blk + tt * RF;
        float kk[RPL], qq[RPL], ee[RPL];
        if constexpr (RPL >= 4) {
#pragma unroll
          for (int g4 = 0; g4 < RPL / 4; ++g4) {
            const int r0 = 4 * RGW * g4 + 4 * rg;
            const float4 q4 = *reinterpret_cast<const float4*>(rec + r0);
            const float4 k4 = *reinterpret_cast<const float4*>(rec + D + r0);
            const float4 e4 = *reinterpret_cast<const float4*>(rec + 2 * D + r0);
            qq[4 * g4] = q4.x; qq[4 * g4 + 1] = q4.y; qq[4 * g4 + 2] = q4.z; qq[4 * g4 + 3] = q4.w;
            kk[4 * g4] = k4.x; kk[4 * g4 + 1] = k4.y; kk[4 * g4 + 2] = k4.z; kk[4 * g4 + 3] = k4.w;
            ee[4 * g4] = e4.x; ee[4 * g4 + 1] = e4.y; ee[4 * g4 + 2] = e4.z; ee[4 * g4 + 3] = e4.w;
          }
        } else {
#pragma unroll
          for (int i = 0; i < RPL; ++i) {
            qq[i] = rec[row[i]];
            kk[i] = rec[D + row[i]];
            ee[i] = rec[2 * D + row[i]];
          }
        }
        float pk[CPL], pq[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          pk[c] = 0.f;
          pq[c] = 0.f;
        }
#pragma unroll
        for (int i = 0; i < RPL; ++i)
#pragma unroll
          for (int c = 0; c < CPL; ++c) {
            const float sv = S[i][c] * ee[i];
            S[i][c] = sv;
            pk[c] = fmaf(kk[i], sv, pk[c]);
            pq[c] = fmaf(qq[i], sv, pq[c]);
          }
        const float beta = rec[4 * D], qk = rec[4 * D + 1];
        float dl[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const float kS = lane_group_sum<RGW>(pk[c]);
          const float qS = lane_group_sum<RGW>(pq[c]);
          dl[c] = beta * (rec[3 * D + col0 + c] - kS);
          const float ov = fmaf(qk, dl[c], qS);
          mo[c] = (tt % RGW) == rg ? ov : mo[c];
        }
#pragma unroll
        for (int i = 0; i < RPL; ++i)
#pragma unroll
          for (int c = 0; c < CPL; ++c) S[i][c] = fmaf(kk[i], dl[c], S[i][c]);
      }
      if ((tt + 1) % RGW == 0 || tt + 1 == kTokBlock) {
        // tokens tt + 1 - RGW .. tt are complete: lane rg stores token tt + 1 - RGW + rg
        const int tok = tt + 1 - RGW + rg;
        if (tok < nt) {
          const size_t oi =
              static_cast<size_t>(tok0 + b * kTokBlock + tok) * ostride + static_cast<size_t>(h) * D + col0;
          if constexpr (!OUT_BF16) {
#pragma unroll
            for (int c = 0; c < CPL; ++c) static_cast<float*>(o)[oi + c] = mo[c];
          } else if constexpr (CPL == 1) {
            static_cast<uint16_t*>(o)[oi] = static_cast<uint16_t>(pack_bf16x2(mo[0], 0.f));
          } else {
#pragma unroll
            for (int c = 0; c < CPL; c += 2)
              *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(o) + oi + c) = pack_bf16x2(mo[c], mo[c + 1]);
          }
        }
      }
    }
    deposit((b + 1) & 1);
    __syncthreads();
  }

  if (S_out) {
#pragma unroll
    for (int i = 0; i < RPL; ++i)
#pragma unroll
      for (int c = 0; c < CPL; ++c) S_out[sbase + static_cast<size_t>(row[i]) * D + col0 + c] = S[i][c];
  }
}

template <int D>
static hipError_t launch_token_prep_d(const Params& p, const ChunkTable& t, const PrefillIO& io, float* recs,
                                      int64_t total_T, int max_chunks, bool io_bf16, hipStream_t st) {
  const int64_t blocks = static_cast<int64_t>(p.H) * max_chunks;
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(blocks));
  if (io_bf16)
    token_prep_kernel<D, true><<<grid, 4 * D, 0, st>>>(p, t, recs, total_T, io.conv_in, io.q, io.k, io.v, io.alpha, io.b);
  else
    token_prep_kernel<D, false><<<grid, 4 * D, 0, st>>>(p, t, recs, total_T, io.conv_in, io.q, io.k, io.v, io.alpha, io.b);
  return hipGetLastError();
}

hipError_t launch_token_prep(const Params& p, const ChunkTable& t, const PrefillIO& io, float* recs,
                             int64_t total_T, int max_chunks, bool io_bf16, hipStream_t st) {
  if (max_chunks <= 0 || total_T <= 0) return hipSuccess;
  switch (p.D) {
    case 16: return launch_token_prep_d<16>(p, t, io, recs, total_T, max_chunks, io_bf16, st);
    case 32: return launch_token_prep_d<32>(p, t, io, recs, total_T, max_chunks, io_bf16, st);
    case 64: return launch_token_prep_d<64>(p, t, io, recs, total_T, max_chunks, io_bf16, st);
    case 128: return launch_token_prep_d<128>(p, t, io, recs, total_T, max_chunks, io_bf16, st);
    default: return hipErrorInvalidValue;
  }
}

template <int D, int RGW, int NW, int CPL>
static hipError_t launch_recurrent_scan_dc(const Params& p, const ChunkTable& t, const PrefillIO& io,
                                           const float* recs, int64_t total_T, bool out_bf16, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(t.N) * p.H * (D / (NW * (kWave / RGW) * CPL)));
  if (out_bf16)
    recurrent_scan_kernel<D, RGW, NW, CPL, true>
        <<<grid, kWave * NW, 0, st>>>(p, t.cu, t.chunk0 + t.N + 2, t.N, recs, total_T, io.S0, io.S_out, io.o);
  else
    recurrent_scan_kernel<D, RGW, NW, CPL, false>
        <<<grid, kWave * NW, 0, st>>>(p, t.cu, t.chunk0 + t.N + 2, t.N, recs, total_T, io.S0, io.S_out, io.o);
  return hipGetLastError();
}

hipError_t launch_recurrent_scan(const Params& p, const ChunkTable& t, const PrefillIO& io, const float* recs,
                                 int64_t total_T, bool out_bf16, hipStream_t st) {
  if (t.N <= 0) return hipSuccess;
  switch (p.D) {
    // one value column per lane and as many waves as fit: measured on four
    // 32K-token sequences, 16 waves of 1 column took the scan to 10.5 ms at
    // dk = dv = 128 (32 heads) against 12.6 ms for 4 waves of 4 columns, and
    // to 6.9 against 8.8 ms at 64 (64 heads)
    case 16: return launch_recurrent_scan_dc<16, 16, 4, 1>(p, t, io, recs, total_T, out_bf16, st);
    case 32: return launch_recurrent_scan_dc<32, 16, 8, 1>(p, t, io, recs, total_T, out_bf16, st);
    case 64: return launch_recurrent_scan_dc<64, 16, 16, 1>(p, t, io, recs, total_T, out_bf16, st);
    case 128: return launch_recurrent_scan_dc<128, 16, 16, 1>(p, t, io, recs, total_T, out_bf16, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kda
