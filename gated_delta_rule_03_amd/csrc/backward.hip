// Backward pass of the KDA core: the gradient of o and of the final state
// with respect to every input and parameter (the models on the pages are
// trained natively with KDA layers: Ling page, section on the 5:1 hybrid
// stacking; the pages give only the forward token loop, AliceAI page,
// section 二, and its derivative is worked out here).
//
// The backward runs in the chunked form with blocks of 16 tokens.  With
// every log-decay >= -5.4, the in-block factors e^{+-G} (G the in-block
// prefix sum) stay inside fp32 (16 * 5.4 < 88), so no sub-block references
// are needed.  Per (block, head), with S0 the state at the block start and
// G_C the block's total:
//   K+ = K e^G, K- = K e^-G, Q+ = Q e^G, K~ = K e^{G_C - G}
//   A = strict_lower(Diag(beta) K+ K-^T),  T = (I + A)^-1
//   W = T Diag(beta) K+,  U = T Diag(beta) V,  Aqk = lower(Q+ K-^T)
//   Delta = U - W S0,  O = Q+ S0 + Aqk Delta,  S_C = e^{G_C} S0 + K~^T Delta
// and, reversing the last three lines with dO and dS_C (adjoint of S_C):
//   dDelta = Aqk^T dO + K~ dS_C
//   dS0 = Q+^T dO + e^{G_C} dS_C - W^T dDelta          (the adjoint scan)
//   dQ+ = dO S0^T + dAqk K-,  dAqk = lower(dO Delta^T)
//   dK~ = Delta dS_C^T,       dG_C += e^{G_C} rowsum(dS_C * S0)
//   dW = -dDelta S0^T,  dU = dDelta;  [dXw | dXu] = T^T [dW | dU]
//   dA = -strict_lower(dXw W^T + dXu U^T)
//   dbeta = rowsum(dXw K+ + dXu V) + rowsum(dA * K+ K-^T)
//   dK+ = Diag(beta) dXw + (Diag(beta) dA) K-,  dK- = (Diag(beta) dA)^T K+ + dAqk^T Q+
//   dV = Diag(beta) dXu
//   dQ = dQ+ e^G,  dK = dK+ e^G + dK- e^-G + dK~ e^{G_C - G}
//   dG = dQ+ Q+ + dK+ K+ - dK- K-   (through the prefix sums)
//   dGs = dK~ K~                    (through the suffix sums G_C - G)
//   dg_t = sum_{r >= t} dG_r + sum_{r < t} dGs_r + dG_C
// where the terms of dG that come from A and Aqk are summed pair by pair over
// i < t <= r instead (they cancel elsewhere; see bwd_block_grad_kernel).
// then the preprocess in reverse (L2 norm, SiLU, conv, gate, beta).
//
// Kernels, in launch order (all fp32 arithmetic):
//   bwd_block_prep    per (block, head): preprocess, A, T, W, U, Q+, K~, Aqk
//   bwd_state_scan    per (sequence, head, value tile): S0 of every block, Delta
//   bwd_adjoint_scan  per (sequence, head, value tile), blocks in reverse:
//                     dS_C of every block, dDelta, d initial state
//   bwd_block_grad    per (block, head): everything above the scans, then the
//                     preprocess's reverse down to the conv outputs' gradient,
//                     d alpha, d b and per-block partial parameter gradients
//   bwd_conv          per (64-token chunk, head): the conv's reverse: d raw
//                     q, k, v, the conv history's gradient, per-chunk d conv w
//   bwd_param_partial, bwd_param_final
//                     partial parameter gradients summed in two fixed-order passes
#include "kda_device.h"
#include "kda_internal.h"
#include "mfma.h"

namespace kda {

namespace {

constexpr int kBlk = 16;             // tokens per block
constexpr int kBT = 256;             // threads of the per-block and scan kernels
constexpr int kBlocksPerChunk = kChunk / kBlk;
constexpr int kReduceParts = 64;     // row ranges of the parameter sums' first pass

// A block of the packed batch: block index = chunk * 4 + sub.
struct BlockInfo {
  int seq, ntok;       // ntok <= 0: empty (past a partial chunk's end)
  int tau0;            // position of its first token in the sequence
  int64_t tok0;        // its first packed token
};

__device__ __forceinline__ BlockInfo block_info(const ChunkTable& t, int blk) {
  const int c = blk / kBlocksPerChunk, sub = blk % kBlocksPerChunk;
  const int4 d = t.desc[c];
  BlockInfo b;
  b.seq = d.x;
  b.tau0 = d.y + sub * kBlk;
  b.ntok = min(kBlk, d.z - sub * kBlk);
  b.tok0 = static_cast<int64_t>(d.w) + sub * kBlk;
  return b;
}

// Shared-memory image of one block's preprocessed inputs (one head).
// Rows are padded by one float: matrix-core operand reads take a column
// across 16 rows, which then fall in 16 different banks.
template <int D>
struct BlockSmem {
  static constexpr int LD = D + 1;
  float q[kBlk][LD];     // q^ (normalised, scaled)
  float k[kBlk][LD];     // k^ (normalised)
  float v[kBlk][LD];     // v^
  float eP[kBlk][LD];    // e^{G}, G the inclusive in-block prefix sum of g
  float eM[kBlk][LD];    // e^{-G}
  float eS[kBlk][LD];    // e^{G_C - G}, from the exclusive in-block suffix sum of g
  float beta[kBlk];
  // per row, with n = sqrt(|u|^2 + eps) the L2 norm: scale / n for q, 1 / n
  // for k (one division per row; the elementwise steps multiply)
  float rq[kBlk], rk[kBlk];
};

// The raw inputs of one thread's preprocess tasks, loaded together before any
// of them is used.  Task m of thread tid is tid + m NT: tasks 0 .. 3D - 1 are
// (q | k | v, channel), holding the three inputs before the block (the conv
// history, or zeros at a sequence start without one) and the block's 16
// (zeros past its end); tasks 3D .. 4D - 1 are the gate's channels, holding
// the block's alphas.
template <int D, int NT>
struct BlockRaw {
  static constexpr int kTasks = (4 * D + NT - 1) / NT;
  float x[kTasks][3 + kBlk];
  float w[kTasks][4];    // conv taps (q | k | v tasks); dt_bias in w[m][0] (gate tasks)
  float bb;              // b of token tid (tid < kBlk)
};

// Every load goes out unconditionally and outside any branch, from an
// address clamped into the sequence (the block's last token stands in for
// rows past its end; a valid row for a missing history row, or for the
// window of a gate task), and the zeros are selected after the loads: a load
// under a condition is compiled as a branch that waits for it.
template <int D, bool IO_BF16, int NT>
__device__ __forceinline__ void block_load_raw(const Params& p, const PrefillIO& io, const BlockInfo& b, int h,
                                               BlockRaw<D, NT>& raw) {
  const int tid = threadIdx.x;
  const size_t HD = static_cast<size_t>(p.H) * D;
  const size_t Ctot = 3 * HD;
  const int64_t seq0 = b.tok0 - b.tau0;   // packed index of the sequence's first token
  const int last = b.ntok - 1;
  const bool have_hist = io.conv_in != nullptr;
#pragma unroll
  for (int m = 0; m < BlockRaw<D, NT>::kTasks; ++m) {
    const int task = tid + m * NT;
    const int role = task / D, ch = task % D;
    const int rq = min(role, 2);                 // the q | k | v tensor the window reads
    const size_t col = static_cast<size_t>(h) * D + ch;
    const void* xin = rq == 0 ? io.q : (rq == 1 ? io.k : io.v);
    const void* tok_src = role == 3 ? io.alpha : xin;     // the block's 16 rows: inputs or alpha
    const void* w = rq == 0 ? p.wq : (rq == 1 ? p.wk : p.wv);
#pragma unroll
    for (int j = 0; j < 4; ++j) raw.w[m][j] = ld<IO_BF16>(w, col * 4 + j);
    const float dtb = p.dt_bias[col];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int tau = b.tau0 - 3 + i;
      const bool hist = tau < 0 && have_hist;
      const void* src = hist ? io.conv_in : xin;
      const size_t idx = hist ? (static_cast<size_t>(b.seq) * 3 + (3 + tau)) * Ctot + rq * HD + col
                              : static_cast<size_t>(seq0 + max(tau, 0)) * HD + col;
      raw.x[m][i] = ld<IO_BF16>(src, idx);
    }
#pragma unroll
    for (int r = 0; r < kBlk; ++r)
      raw.x[m][3 + r] = ld<IO_BF16>(tok_src, static_cast<size_t>(b.tok0 + min(r, last)) * HD + col);
#pragma unroll
    for (int i = 0; i < 3; ++i)
      if (b.tau0 - 3 + i < 0 && !have_hist) raw.x[m][i] = 0.f;
#pragma unroll
    for (int r = 0; r < kBlk; ++r)
      if (r > last) raw.x[m][3 + r] = 0.f;
    if (role == 3) raw.w[m][0] = dtb;
  }
  raw.bb = ld<IO_BF16>(io.b, static_cast<size_t>(b.tok0 + min(tid % kBlk, last)) * p.H + h);
  if (tid >= b.ntok) raw.bb = 0.f;
}

// Conv + SiLU, L2 norm, gate and beta of one block's tokens for head h, from
// the loaded raw inputs into shared memory.  Rows past the block's end are
// zero, with g = beta = 0.
template <int D, int NT>
__device__ __forceinline__ void block_preprocess(const Params& p, const BlockInfo& b, int h, const BlockRaw<D, NT>& raw,
                                 BlockSmem<D>& s) {
  static_assert(NT >= 2 * kBlk * 8, "the L2 norms take 8 lanes for each of 32 rows");
  const int tid = threadIdx.x;
#pragma unroll
  for (int m = 0; m < BlockRaw<D, NT>::kTasks; ++m) {
    const int task = tid + m * NT;
    const int role = task / D, ch = task % D;
    if (role < 3) {
      const float w0 = raw.w[m][0], w1 = raw.w[m][1], w2 = raw.w[m][2], w3 = raw.w[m][3];
      float* dst = role == 0 ? &s.q[0][0] : (role == 1 ? &s.k[0][0] : &s.v[0][0]);
#pragma unroll
      for (int r = 0; r < kBlk; ++r) {
        const float y = w0 * raw.x[m][r] + w1 * raw.x[m][r + 1] + w2 * raw.x[m][r + 2] + w3 * raw.x[m][r + 3];
        dst[r * BlockSmem<D>::LD + ch] = r < b.ntok ? siluf_(y) : 0.f;
      }
    } else if (role == 3) {
      const float a_exp = expf(p.A_log[h]);
      const float dtb = raw.w[m][0];
      float run = 0.f;
      float g[kBlk];
#pragma unroll
      for (int r = 0; r < kBlk; ++r) {
        const float al = raw.x[m][3 + r];
        g[r] = r < b.ntok ? ((p.flags & KDA_FLAG_RAW_GATE) ? al : gate_value(al, dtb, a_exp, p.lower_bound)) : 0.f;
        run += g[r];
        s.eP[r][ch] = run;   // exponentiated below, by every thread
      }
      float suf = 0.f;
#pragma unroll
      for (int r = kBlk - 1; r >= 0; --r) {
        s.eS[r][ch] = suf;
        suf += g[r];
      }
    }
  }
  if (tid < kBlk) {
    float be = 0.f;
    if (tid < b.ntok) {
      be = sigmoidf_(raw.bb);
      if (p.flags & KDA_FLAG_BETA_X2) be *= 2.0f;
    }
    s.beta[tid] = be;
  }
  __syncthreads();
  // L2 norms of q and k: 32 rows, 8 lanes each (whole waves: 256 threads)
  if (tid < 2 * kBlk * 8) {
    const int row = tid / 8, l8 = tid % 8;     // rows 0..15 q, 16..31 k
    const float* src = row < kBlk ? s.q[row] : s.k[row - kBlk];
    float ss = 0.f;
    for (int c = l8; c < D; c += 8) ss += src[c] * src[c];
    ss += __shfl_xor(ss, 1, 8);
    ss += __shfl_xor(ss, 2, 8);
    ss += __shfl_xor(ss, 4, 8);
    if (l8 == 0) {
      const float n = sqrtf(ss + p.eps);
      if (row < kBlk) s.rq[row] = p.scale / n; else s.rk[row - kBlk] = 1.f / n;
    }
  }
  __syncthreads();
  // the normalisation, and the decays' exponentials spread over every thread
  // (the gate's threads formed their exponents: G_r, and G_C - G_r); the
  // hardware base-2 exponential with the rounding residual carried, ~2 ulp
  for (int e = tid; e < kBlk * D; e += NT) {
    const int r = e / D, c = e % D;
    s.q[r][c] *= s.rq[r];
    s.k[r][c] *= s.rk[r];
    const float G = s.eP[r][c];
    s.eP[r][c] = exp_precise(G);
    s.eM[r][c] = exp_precise(-G);
    s.eS[r][c] = exp_precise(s.eS[r][c]);
  }
  __syncthreads();
}

}  // namespace

// Per (block, head) record of the backward's forward quantities (fp32).
struct BwdRecord {
  size_t W, U, Qp, Kt, T, Aqk, eGC, bytes;
};

__host__ __device__ constexpr BwdRecord bwd_record(int D) {
  BwdRecord r{};
  const size_t tile = static_cast<size_t>(kBlk) * D * 4;
  r.W = 0;
  r.U = r.W + tile;
  r.Qp = r.U + tile;
  r.Kt = r.Qp + tile;
  r.T = r.Kt + tile;
  r.Aqk = r.T + kBlk * kBlk * 4;
  r.eGC = r.Aqk + kBlk * kBlk * 4;
  r.bytes = (r.eGC + static_cast<size_t>(D) * 4 + 255) / 256 * 256;
  return r;
}

size_t bwd_record_bytes(int D) { return bwd_record(D).bytes; }
int bwd_reduce_parts() { return kReduceParts; }

namespace {

// The block states (S0 of every block, the adjoint dS_C at every block end)
// are stored in the order the block-gradient kernel's lanes read them.  Its
// wave w owns state rows 16w .. 16w + 15 and lane l reads KS = D / 4
// consecutive columns KS (l / 16) .. of row 16w + l % 16 as KS / 4 float4s;
// element (c, j) therefore sits at
//   ((c / 16 * (KS / 4) + (j % KS) / 4) * 64 + (j / KS) * 16 + c % 16) * 4 + j % 4,
// so that each of the reader's 16-byte wave loads covers 1 KB of contiguous
// memory (in row order a load touches 64 cache lines for 16 bytes each).
template <int D>
__device__ __forceinline__ size_t state_index(int c, int j) {
  constexpr int KS = D / 4;
  return static_cast<size_t>(((c / 16 * (KS / 4) + (j % KS) / 4) * 64 + (j / KS) * 16 + c % 16) * 4 + j % 4);
}


// A scan wave's state slice (columns j0 .. j0 + 15, accumulator layout) to
// memory in state_index order.  At d >= 64 the slice is 32 runs of 256
// contiguous bytes there (one per row tile and 4-column group); it is laid
// out in that order in the wave's shared-memory area first, then leaves in
// 16-byte stores covering 1 KB each.  Smaller d store element by element.
constexpr int kRun = 68;

template <int D>
__device__ __forceinline__ void store_state(float* dst, const f32x4 (&acc)[D / 16], float* stg, int j0, int lane) {
  constexpr int KS = D / 4;
  const int l16 = lane % 16, g = lane / 16;
  if constexpr (D >= 64) {
    // stg[(t16 * 4 + m) * kRun + r16 * 4 + e]: row 16 t16 + r16, column
    // j0 + 4 m + e (runs padded to 68 floats against bank conflicts)
#pragma unroll
    for (int t16 = 0; t16 < D / 16; ++t16)
#pragma unroll
      for (int i = 0; i < 4; ++i) stg[(t16 * 4 + l16 / 4) * kRun + (4 * g + i) * 4 + l16 % 4] = acc[t16][i];
    const int m0 = (j0 % KS) / 4, g4 = j0 / KS;
#pragma unroll
    for (int k = 0; k < D / 16; ++k) {      // 4 runs of 256 B per 16-byte wave store
      const int run = k * 4 + lane / 16, t16 = run / 4, m = run % 4;
      const float4 v = *reinterpret_cast<const float4*>(&stg[run * kRun + (lane % 16) * 4]);
      *reinterpret_cast<float4*>(&dst[((t16 * (KS / 4) + m0 + m) * 64 + g4 * 16 + lane % 16) * 4]) = v;
    }
  } else {
#pragma unroll
    for (int t16 = 0; t16 < D / 16; ++t16)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[state_index<D>(16 * t16 + 4 * g + i, j0 + l16)] = acc[t16][i];
  }
}
}  // namespace

// ---------------------------------------------------------------- block prep
template <int D, bool IO_BF16>
__global__ __launch_bounds__(kBT, 3) void bwd_block_prep_kernel(Params p, ChunkTable t, PrefillIO io, uint8_t* recs) {
  constexpr BwdRecord R = bwd_record(D);
  __shared__ BlockSmem<D> s;
  // The half-channel partial products of A and Aqk, then T.  Where they fit
  // (d = 128) they go into the area of e^{G_C - G}, which is no longer needed
  // after the first pass below: shared memory is then the preprocessed block
  // alone, ~49 KB, and three workgroups fit on a compute unit instead of two
  // (the launch bound holds the registers to three waves per SIMD's share).
  constexpr int kPT = 5 * kBlk * kBlk;
  constexpr bool kAlias = kBlk * (D + 1) >= kPT;
  __shared__ float sPT_own[kAlias ? 1 : kPT];
  float* const pt = kAlias ? &s.eS[0][0] : sPT_own;
  float (*sPart)[kBlk][kBlk] = reinterpret_cast<float (*)[kBlk][kBlk]>(pt);
  float (*sT)[kBlk] = reinterpret_cast<float (*)[kBlk]>(pt + 4 * kBlk * kBlk);
  const int h = static_cast<int>(blockIdx.x % static_cast<unsigned>(p.H));
  const int blk = static_cast<int>(blockIdx.x / static_cast<unsigned>(p.H));
  if (blk / kBlocksPerChunk >= t.chunk0[t.N]) return;
  const BlockInfo b = block_info(t, blk);
  if (b.ntok <= 0) return;
  const int tid = threadIdx.x;
  {
    BlockRaw<D, kBT> raw;
    block_load_raw<D, IO_BF16, kBT>(p, io, b, h, raw);
    block_preprocess<D, kBT>(p, b, h, raw, s);
  }
  uint8_t* rec = recs + (static_cast<size_t>(blk) * p.H + h) * R.bytes;
  float* gW = reinterpret_cast<float*>(rec + R.W);
  float* gU = reinterpret_cast<float*>(rec + R.U);
  float* gQp = reinterpret_cast<float*>(rec + R.Qp);
  float* gKt = reinterpret_cast<float*>(rec + R.Kt);
  float* gT = reinterpret_cast<float*>(rec + R.T);
  float* gAqk = reinterpret_cast<float*>(rec + R.Aqk);
  float* geGC = reinterpret_cast<float*>(rec + R.eGC);
  // Q+, K~ and e^{G_C}
  for (int e = tid; e < kBlk * D; e += kBT) {
    const int r = e / D, c = e % D;
    gQp[e] = s.q[r][c] * s.eP[r][c];
    gKt[e] = s.k[r][c] * s.eS[r][c];
    if (r == 0) geGC[c] = s.eP[kBlk - 1][c];
  }
  __syncthreads();
  // A (strictly lower) and Aqk (lower with the diagonal) on the fp32 matrix
  // cores: K+ K-^T and Q+ K-^T over K = D, each product on two waves that take
  // half the channels each, 8 of every 16 (lane layout as in
  // bwd_block_grad_kernel); the halves meet in shared memory
  const int wave = tid / kWave, lane = tid % kWave, l16 = lane % 16, g4 = lane / 16;
  static_assert(kBT / kWave == 4, "A and Aqk take two waves each");
  {
    const int prod = wave >> 1, half = wave & 1;   // prod 0: A, 1: Aqk
    f32x4 acc[4] = {zero4(), zero4(), zero4(), zero4()};   // four independent chains
#pragma unroll
    for (int k0 = 0; k0 < D; k0 += 16) {
#pragma unroll
      for (int j2 = 0; j2 < 2; ++j2) {
        const int k = k0 + 4 * (2 * half + j2) + g4;
        const float a = (prod == 0 ? s.k[l16][k] : s.q[l16][k]) * s.eP[l16][k];
        const int ch = 2 * ((k0 / 16) & 1) + j2;
        acc[ch] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, s.k[l16][k] * s.eM[l16][k], acc[ch], 0, 0, 0);   // K-
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) sPart[wave][4 * g4 + i][l16] = (acc[0][i] + acc[1][i]) + (acc[2][i] + acc[3][i]);
  }
  __syncthreads();
  if (wave == 0) {
    // T = (I + A)^-1 by forward substitution, lane i < 16 owns column i.  The
    // strictly lower A is read into registers first (120 values, the halves
    // added), so the substitution chain does no shared-memory reads; each
    // row's sum runs in four partial sums.
    const int i = lane;
    float a[kBlk * (kBlk - 1) / 2];
#pragma unroll
    for (int r = 1, q = 0; r < kBlk; ++r)
#pragma unroll
      for (int m = 0; m < r; ++m, ++q) a[q] = s.beta[r] * (sPart[0][r][m] + sPart[1][r][m]);
    float col[kBlk];
#pragma unroll
    for (int r = 0, q = 0; r < kBlk; ++r) {
      float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < r; ++m, ++q) ps[m & 3] += a[q] * col[m];
      const float v = ((r == i) ? 1.f : 0.f) - ((ps[0] + ps[1]) + (ps[2] + ps[3]));
      col[r] = r < i ? 0.f : v;
    }
    if (i < kBlk) {
#pragma unroll
      for (int r = 0; r < kBlk; ++r) sT[r][i] = col[r];
    }
  } else if (wave == 1) {
    // Aqk out (the two halves added; lower with the diagonal)
#pragma unroll
    for (int e4 = 0; e4 < kBlk * kBlk / kWave; ++e4) {
      const int e = lane + e4 * kWave, r = e / kBlk, c = e % kBlk;
      gAqk[e] = c <= r ? sPart[2][r][c] + sPart[3][r][c] : 0.f;
    }
  }
  __syncthreads();
  for (int e = tid; e < kBlk * kBlk; e += kBT) gT[e] = sT[e / kBlk][e % kBlk];
  // W = T Diag(beta) K+,  U = T Diag(beta) V (K = 16), 16 channels per wave pass
  for (int c0 = wave * 16; c0 < D; c0 += (kBT / kWave) * 16) {
    const int c = c0 + l16;
    f32x4 w = zero4(), u = zero4();
#pragma unroll
    for (int st = 0; st < kBlk / 4; ++st) {
      const int k = 4 * st + g4;
      const float a = sT[l16][k] * s.beta[k];
      w = __builtin_amdgcn_mfma_f32_16x16x4f32(a, s.k[k][c] * s.eP[k][c], w, 0, 0, 0);
      u = __builtin_amdgcn_mfma_f32_16x16x4f32(a, s.v[k][c], u, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * g4 + i;
      gW[r * D + c] = w[i];
      gU[r * D + c] = u[i];
    }
  }
}

// ---------------------------------------------------------------- the two scans
// A workgroup per (sequence, head, TW consecutive 16-column value tiles), a
// wave per tile.  The state slice (or its adjoint) S[0..D) x [j0, j0 + 16) of
// a wave lives in fp32 matrix-core accumulators: row tile t (rows 16t ..
// 16t + 15) in acc[t], lane l holding rows 16t + 4 (l / 16) + i (i < 4) of
// column j0 + l % 16.  A product that contracts over the state's rows then
// takes its B operand straight from the accumulators: step (t, i) of
// v_mfma_f32_16x16x4_f32 covers rows 16t + 4g + i for the four lane groups g.
// A sequence's blocks are consecutive (block index = 4 x its first chunk +
// its position).  The block operands the waves share (W, K~, Q+, Aqk,
// e^{G_C}) are loaded once per workgroup, into registers two blocks ahead
// (two alternating sets), and moved to shared memory at the step that uses
// them.  Workgroups are numbered so that those of one (sequence, head) share
// an XCD (workgroups are dealt to the 8 XCDs round robin) and read its
// records through one L2.
constexpr int kScanTile = 16;

template <int D>
constexpr int scan_waves() { return D / kScanTile >= 4 ? 4 : D / kScanTile; }

__device__ __forceinline__ bool scan_coords(int nh_total, int ngroups, int& nh, int& grp) {
  const int bid = static_cast<int>(blockIdx.x);
  const int lo = bid % 8, rest = bid / 8;
  grp = rest % ngroups;
  nh = (rest / ngroups) * 8 + lo;
  return nh < nh_total;
}

template <int D>
__global__ __launch_bounds__(kWave * scan_waves<D>()) void bwd_state_scan_kernel(Params p, ChunkTable t,
                                                                                const float* S_init,
                                                                                const uint8_t* recs, float* Sblk,
                                                                                float* Dblk) {
  constexpr BwdRecord R = bwd_record(D);
  constexpr int TW = scan_waves<D>();
  constexpr int NTH = kWave * TW;
  constexpr int NT16 = D / 16;               // row tiles of the state
  constexpr int CW = kScanTile * TW;         // value columns of the workgroup
  constexpr int PF = kBlk * D / NTH;         // W / K~ elements per thread
  constexpr int PU = kBlk * CW / NTH;        // U elements per thread
  constexpr int PE = (D + NTH - 1) / NTH;    // e^{G_C} elements per thread
  struct Ops { float w[PF], k[PF], u[PU], e[PE]; };
  __shared__ float sW[kBlk][D + 1], sKt[kBlk][D + 1], seG[D], sU[kBlk][CW + 1];
  __shared__ float sDel[TW][kBlk][kScanTile + 1];
  __shared__ __align__(16) float sStg[TW][D >= 64 ? D / 4 * kRun : 4];   // staged state stores
  int nh, grp;
  if (!scan_coords(t.N * p.H, D / CW, nh, grp)) return;
  const int h = nh % p.H, n = t.scan_seq(nh / p.H);   // long sequences first
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave, l16 = lane % 16, g = lane / 16;
  const int c0 = grp * CW, jw = wave * kScanTile, j0 = c0 + jw;
  const size_t SZ = static_cast<size_t>(D) * D;
  f32x4 acc[NT16];
#pragma unroll
  for (int t16 = 0; t16 < NT16; ++t16)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * t16 + 4 * g + i;
      acc[t16][i] = S_init ? S_init[(static_cast<size_t>(n) * p.H + h) * SZ + static_cast<size_t>(r) * D + j0 + l16]
                           : 0.f;
    }
  const int L = t.cu[n + 1] - t.cu[n];
  const int nb = (L + kBlk - 1) / kBlk;
  const int blk0 = t.chunk0[n] * kBlocksPerChunk;
  auto fetch = [&](Ops& o, int jb) {
    const uint8_t* rec = recs + (static_cast<size_t>(blk0 + jb) * p.H + h) * R.bytes;
    const float* gW = reinterpret_cast<const float*>(rec + R.W);
    const float* gU = reinterpret_cast<const float*>(rec + R.U);
    const float* gKt = reinterpret_cast<const float*>(rec + R.Kt);
    const float* geG = reinterpret_cast<const float*>(rec + R.eGC);
#pragma unroll
    for (int m = 0; m < PF; ++m) { o.w[m] = gW[tid + m * NTH]; o.k[m] = gKt[tid + m * NTH]; }
#pragma unroll
    for (int m = 0; m < PU; ++m) {
      const int e = tid + m * NTH;
      o.u[m] = gU[(e / CW) * D + c0 + e % CW];
    }
#pragma unroll
    for (int m = 0; m < PE; ++m)
      if (tid + m * NTH < D) o.e[m] = geG[tid + m * NTH];
  };
  auto to_shared = [&](const Ops& o) {
#pragma unroll
    for (int m = 0; m < PF; ++m) {
      const int e = tid + m * NTH;
      sW[e / D][e % D] = o.w[m];
      sKt[e / D][e % D] = o.k[m];
    }
#pragma unroll
    for (int m = 0; m < PU; ++m) {
      const int e = tid + m * NTH;
      sU[e / CW][e % CW] = o.u[m];
    }
#pragma unroll
    for (int m = 0; m < PE; ++m)
      if (tid + m * NTH < D) seG[tid + m * NTH] = o.e[m];
  };
  // one block: its operands are in shared memory; Sblk <- S, Delta, S update
  auto step = [&](int jb) {
    const size_t bh = static_cast<size_t>(blk0 + jb) * p.H + h;
    store_state<D>(Sblk + bh * SZ, acc, &sStg[wave][0], j0, lane);
    // Delta = U - W S  (contracting the state's rows; four accumulators by i)
    f32x4 d4[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
    for (int t16 = 0; t16 < NT16; ++t16)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        d4[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(sW[l16][16 * t16 + 4 * g + i], acc[t16][i], d4[i], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float del = sU[4 * g + i][jw + l16] - ((d4[0][i] + d4[1][i]) + (d4[2][i] + d4[3][i]));
      sDel[wave][4 * g + i][l16] = del;
      Dblk[bh * kBlk * D + static_cast<size_t>(4 * g + i) * D + j0 + l16] = del;
    }
    // S <- e^{G_C} S + K~^T Delta  (K = the block's 16 rows; sDel is this
    // wave's own: the wave's LDS operations complete in order)
#pragma unroll
    for (int t16 = 0; t16 < NT16; ++t16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[t16][i] *= seG[16 * t16 + 4 * g + i];
#pragma unroll
      for (int st = 0; st < kBlk / 4; ++st) {
        const int k = 4 * st + g;
        acc[t16] = __builtin_amdgcn_mfma_f32_16x16x4f32(sKt[k][16 * t16 + l16], sDel[wave][k][l16], acc[t16], 0, 0,
                                                        0);
      }
    }
  };
  Ops A, B;
  if (nb > 0) fetch(A, 0);
  if (nb > 1) fetch(B, 1);
  for (int jb = 0; jb < nb; jb += 2) {
    to_shared(A);
    __syncthreads();
    if (jb + 2 < nb) fetch(A, jb + 2);
    step(jb);
    __syncthreads();
    if (jb + 1 < nb) {
      to_shared(B);
      __syncthreads();
      if (jb + 3 < nb) fetch(B, jb + 3);
      step(jb + 1);
      __syncthreads();
    }
  }
}

// The state scan's layout, blocks in reverse:
//   dDelta = Aqk^T dO + K~ dS_C,   dS0 = Q+^T dO + e^{G_C} dS_C - W^T dDelta
template <int D, bool DO_BF16>
__global__ __launch_bounds__(kWave * scan_waves<D>()) void bwd_adjoint_scan_kernel(Params p, ChunkTable t,
                                                                                  const uint8_t* recs,
                                                                                  const void* dO,
                                                                                  const float* dS_final,
                                                                                  float* dSblk, float* dDblk,
                                                                                  float* dS_init, float* dconv) {
  constexpr BwdRecord R = bwd_record(D);
  constexpr int TW = scan_waves<D>();
  constexpr int NTH = kWave * TW;
  constexpr int NT16 = D / 16;
  constexpr int CW = kScanTile * TW;
  constexpr int PF = kBlk * D / NTH;
  constexpr int PA = (kBlk * kBlk + NTH - 1) / NTH;   // Aqk elements per thread
  constexpr int PE = (D + NTH - 1) / NTH;
  struct Ops { float w[PF], k[PF], q[PF], a[PA], o[4], e[PE]; };
  __shared__ float sW[kBlk][D + 1], sKt[kBlk][D + 1], sQp[kBlk][D + 1], seG[D];
  __shared__ float sAqk[kBlk][kBlk + 1];
  __shared__ float sdO[TW][kBlk][kScanTile + 1], sdDel[TW][kBlk][kScanTile + 1];
  __shared__ __align__(16) float sStg[TW][D >= 64 ? D / 4 * kRun : 4];   // staged state stores
  int nh, grp;
  if (!scan_coords(t.N * p.H, D / CW, nh, grp)) return;
  const int h = nh % p.H, n = t.scan_seq(nh / p.H);   // long sequences first
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave, l16 = lane % 16, g = lane / 16;
  const int c0 = grp * CW, j0 = c0 + wave * kScanTile;
  const size_t SZ = static_cast<size_t>(D) * D;
  const size_t HD = static_cast<size_t>(p.H) * D;
  f32x4 acc[NT16];
#pragma unroll
  for (int t16 = 0; t16 < NT16; ++t16)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * t16 + 4 * g + i;
      acc[t16][i] = dS_final ? dS_final[(static_cast<size_t>(n) * p.H + h) * SZ + static_cast<size_t>(r) * D + j0 + l16]
                             : 0.f;
    }
  const int L = t.cu[n + 1] - t.cu[n];
  const int nb = (L + kBlk - 1) / kBlk;
  const int blk0 = t.chunk0[n] * kBlocksPerChunk;
  const int64_t seq0 = t.cu[n];
  auto fetch = [&](Ops& o, int jb) {
    const int ntok = min(kBlk, L - jb * kBlk);
    const uint8_t* rec = recs + (static_cast<size_t>(blk0 + jb) * p.H + h) * R.bytes;
    const float* gW = reinterpret_cast<const float*>(rec + R.W);
    const float* gKt = reinterpret_cast<const float*>(rec + R.Kt);
    const float* gQp = reinterpret_cast<const float*>(rec + R.Qp);
    const float* gAqk = reinterpret_cast<const float*>(rec + R.Aqk);
    const float* geG = reinterpret_cast<const float*>(rec + R.eGC);
#pragma unroll
    for (int m = 0; m < PF; ++m) {
      o.w[m] = gW[tid + m * NTH];
      o.k[m] = gKt[tid + m * NTH];
      o.q[m] = gQp[tid + m * NTH];
    }
#pragma unroll
    for (int m = 0; m < PA; ++m)
      if (tid + m * NTH < kBlk * kBlk) o.a[m] = gAqk[tid + m * NTH];
#pragma unroll
    for (int m = 0; m < 4; ++m) {      // this wave's 16 x 16 tile of dO (rows past the end: zeros)
      const int q = (lane + m * kWave) / kScanTile, jj = (lane + m * kWave) % kScanTile;
      o.o[m] = ld<DO_BF16>(dO, (static_cast<size_t>(seq0 + jb * kBlk + min(q, ntok - 1)) * p.H + h) * D + j0 + jj);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
      if ((lane + m * kWave) / kScanTile >= ntok) o.o[m] = 0.f;
#pragma unroll
    for (int m = 0; m < PE; ++m)
      if (tid + m * NTH < D) o.e[m] = geG[tid + m * NTH];
  };
  auto to_shared = [&](const Ops& o) {
#pragma unroll
    for (int m = 0; m < PF; ++m) {
      const int e = tid + m * NTH;
      sW[e / D][e % D] = o.w[m];
      sKt[e / D][e % D] = o.k[m];
      sQp[e / D][e % D] = o.q[m];
    }
#pragma unroll
    for (int m = 0; m < PA; ++m) {
      const int e = tid + m * NTH;
      if (e < kBlk * kBlk) sAqk[e / kBlk][e % kBlk] = o.a[m];
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int e = lane + m * kWave;
      sdO[wave][e / kScanTile][e % kScanTile] = o.o[m];
    }
#pragma unroll
    for (int m = 0; m < PE; ++m)
      if (tid + m * NTH < D) seG[tid + m * NTH] = o.e[m];
  };
  auto step = [&](int jb) {
    const size_t bh = static_cast<size_t>(blk0 + jb) * p.H + h;
    // the adjoint of the block's end state
    store_state<D>(dSblk + bh * SZ, acc, &sStg[wave][0], j0, lane);
    // dDelta = K~ dS_C (contracting the state's rows) + Aqk^T dO
    f32x4 d4[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
    for (int t16 = 0; t16 < NT16; ++t16)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        d4[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(sKt[l16][16 * t16 + 4 * g + i], acc[t16][i], d4[i], 0, 0, 0);
#pragma unroll
    for (int st = 0; st < kBlk / 4; ++st) {
      const int k = 4 * st + g;
      d4[st] = __builtin_amdgcn_mfma_f32_16x16x4f32(sAqk[k][l16], sdO[wave][k][l16], d4[st], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float dd = (d4[0][i] + d4[1][i]) + (d4[2][i] + d4[3][i]);
      sdDel[wave][4 * g + i][l16] = dd;
      dDblk[bh * kBlk * D + static_cast<size_t>(4 * g + i) * D + j0 + l16] = dd;
    }
    // dS0 = e^{G_C} dS_C + Q+^T dO - W^T dDelta  (sdDel is this wave's own)
#pragma unroll
    for (int t16 = 0; t16 < NT16; ++t16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[t16][i] *= seG[16 * t16 + 4 * g + i];
#pragma unroll
      for (int st = 0; st < kBlk / 4; ++st) {
        const int k = 4 * st + g;
        acc[t16] = __builtin_amdgcn_mfma_f32_16x16x4f32(sQp[k][16 * t16 + l16], sdO[wave][k][l16], acc[t16], 0, 0, 0);
        acc[t16] = __builtin_amdgcn_mfma_f32_16x16x4f32(-sW[k][16 * t16 + l16], sdDel[wave][k][l16], acc[t16], 0, 0,
                                                        0);
      }
    }
  };
  Ops A, B;
  if (nb > 0) fetch(A, nb - 1);
  if (nb > 1) fetch(B, nb - 2);
  for (int i = 0; i < nb; i += 2) {
    const int jb = nb - 1 - i;
    to_shared(A);
    __syncthreads();
    if (jb - 2 >= 0) fetch(A, jb - 2);
    step(jb);
    __syncthreads();
    if (jb - 1 >= 0) {
      to_shared(B);
      __syncthreads();
      if (jb - 3 >= 0) fetch(B, jb - 3);
      step(jb - 1);
      __syncthreads();
    }
  }
  if (dS_init) {
#pragma unroll
    for (int t16 = 0; t16 < NT16; ++t16)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * t16 + 4 * g + i;
        dS_init[(static_cast<size_t>(n) * p.H + h) * SZ + static_cast<size_t>(r) * D + j0 + l16] = acc[t16][i];
      }
  }
  // an empty sequence passes its conv history through: no gradient reaches it
  if (dconv && grp == 0 && nb == 0) {
    for (int e = tid; e < 3 * D; e += NTH) {
      const int role = e / D, ch = e % D;
      for (int m = 0; m < 3; ++m)
        dconv[(static_cast<size_t>(n) * 3 + m) * 3 * HD + role * HD + static_cast<size_t>(h) * D + ch] = 0.f;
    }
  }
}

// ---------------------------------------------------------------- block gradients
// Threads of the block-gradient kernel: its shared memory (~134 KB at d = 128)
// allows one workgroup per compute unit, so it takes two waves per SIMD.
template <int D>
constexpr int grad_threads() { return D >= 32 ? 512 : 256; }

template <int D, bool IO_BF16, bool DO_BF16>
__global__ __launch_bounds__(grad_threads<D>()) void bwd_block_grad_kernel(Params p, ChunkTable t, PrefillIO io, const uint8_t* recs,
                                                              const float* Sblk, const float* dSblk, const float* Dblk,
                                                              const float* dDblk, const void* dO, float* dy,
                                                              float* dalpha, float* db, float* pdtb, float* pAlog) {
  constexpr BwdRecord R = bwd_record(D);
  constexpr int NT = grad_threads<D>();
  constexpr int EL = (kBlk * D + NT - 1) / NT;   // block-tile elements per thread
  constexpr int KS = D / 4;                      // S0 / dS_C columns per lane of the matrix-core waves
  using Raw = BlockRaw<D, NT>;
  __shared__ BlockSmem<D> s;
  __shared__ float sDel[kBlk][D + 1], sdDel[kBlk][D + 1], sdO[kBlk][D + 1];   // padded: matrix-core A reads
  __shared__ float sdQp[kBlk][D + 1], sdKp[kBlk][D + 1], sdKm[kBlk][D + 1], sdKt[kBlk][D + 1];
  __shared__ float sX[kBlk][D + 1];       // dW, then dXw, then dV
  __shared__ __align__(16) float sT[kBlk][kBlk], sAun[kBlk][kBlk], sdA[kBlk][kBlk], sdAqk[kBlk][kBlk];
  __shared__ float sdbeta[kBlk], sdGC[D];
  __shared__ float sWt[kBlk][D + 1], sUt[kBlk][D + 1];  // W and U
  __shared__ float sPart[NT / kWave][kBlk][kBlk];        // the waves' partial 16 x 16 products
  const int h = static_cast<int>(blockIdx.x % static_cast<unsigned>(p.H));
  const int blk = static_cast<int>(blockIdx.x / static_cast<unsigned>(p.H));
  const bool live_chunk = blk / kBlocksPerChunk < t.chunk0[t.N];
  const BlockInfo b = live_chunk ? block_info(t, blk) : BlockInfo{0, 0, 0, 0};
  const int tid = threadIdx.x;
  const size_t HD = static_cast<size_t>(p.H) * D;
  float* pd = pdtb + (static_cast<size_t>(blk) * p.H + h) * D;
  if (b.ntok <= 0) {          // an empty block adds nothing to the parameter sums
    for (int e = tid; e < D; e += NT) pd[e] = 0.f;
    if (tid == 0) pAlog[static_cast<size_t>(blk) * p.H + h] = 0.f;
    return;
  }
  const size_t bh = static_cast<size_t>(blk) * p.H + h;
  const uint8_t* rec = recs + bh * R.bytes;
  const float* gW = reinterpret_cast<const float*>(rec + R.W);
  const float* gU = reinterpret_cast<const float*>(rec + R.U);
  const float* gT = reinterpret_cast<const float*>(rec + R.T);
  const float* geG = reinterpret_cast<const float*>(rec + R.eGC);
  const int wave = tid / kWave, lane = tid % kWave, l16 = lane % 16, g4 = lane / 16;

  // ---- every load of the block goes out here, before any arithmetic: the
  // raw inputs (kept for the reverse of the conv and the gate at the end),
  // then the scans' outputs and the record, whose latency the preprocess hides
  Raw raw;
  block_load_raw<D, IO_BF16, NT>(p, io, b, h, raw);
  float lDel[EL], ldDel[EL], ldO[EL], lW[EL], lU[EL];
#pragma unroll
  for (int m = 0; m < EL; ++m) {
    const int e = tid + m * NT;
    if (e < kBlk * D) {
      const int r = e / D, c = e % D;
      lDel[m] = Dblk[bh * kBlk * D + e];
      ldDel[m] = dDblk[bh * kBlk * D + e];
      ldO[m] = ld<DO_BF16>(dO, (static_cast<size_t>(b.tok0 + min(r, b.ntok - 1)) * p.H + h) * D + c);
      lW[m] = gW[e];
      lU[m] = gU[e];
    }
  }
#pragma unroll
  for (int m = 0; m < EL; ++m)
    if ((tid + m * NT) / D >= b.ntok) ldO[m] = 0.f;
  const float lT = gT[tid % (kBlk * kBlk)];
  // rows of S0 and dS_C for the matrix-core products: wave w owns output
  // channels 16w .. 16w + 15, lane l the contiguous state columns
  // KS (l / 16) .. KS (l / 16) + KS - 1 of row 16w + l % 16 (stored in that
  // order: state_index)
  float sv[KS], dsv[KS], lgeG = 0.f;
  if (D / 16 >= NT / kWave || wave < D / 16) {   // (every wave at d = 128: no branch)
    const int c = wave * 16 + l16;
    const size_t base = bh * D * D + (static_cast<size_t>(wave) * (KS / 4) * 64 + lane) * 4;
    const float* s0row = Sblk + base;
    const float* dsrow = dSblk + base;
#pragma unroll
    for (int q = 0; q < KS; q += 4) {
      const float4 a = *reinterpret_cast<const float4*>(s0row + q * 64);
      const float4 d4 = *reinterpret_cast<const float4*>(dsrow + q * 64);
      sv[q] = a.x; sv[q + 1] = a.y; sv[q + 2] = a.z; sv[q + 3] = a.w;
      dsv[q] = d4.x; dsv[q + 1] = d4.y; dsv[q + 2] = d4.z; dsv[q + 3] = d4.w;
    }
    lgeG = geG[c];
  }
  block_preprocess<D, NT>(p, b, h, raw, s);
#pragma unroll
  for (int m = 0; m < EL; ++m) {
    const int e = tid + m * NT;
    if (e < kBlk * D) {
      const int r = e / D, c = e % D;
      sDel[r][c] = lDel[m];
      sdDel[r][c] = ldDel[m];
      sdO[r][c] = ldO[m];
    }
  }
  if (tid < kBlk * kBlk) sT[tid / kBlk][tid % kBlk] = lT;
  __syncthreads();

  // ---- products with S0 and dS_C on the fp32 matrix cores (v_mfma_f32_16x16x4_f32):
  //   dQ+ = dO S0^T, dW = -dDelta S0^T, dK~ = Delta dS_C^T  (16 x D each) and
  //   dG_C = e^{G_C} rowsum(dS_C * S0).
  // Step s of lane l covers state column KS (l / 16) + s, the lane's own row
  // pieces loaded above.
  if (wave < D / 16) {
    const int c = wave * 16 + l16;
    float gc = 0.f;
#pragma unroll
    for (int q = 0; q < KS; ++q) gc += sv[q] * dsv[q];
    gc += __shfl_xor(gc, 16);
    gc += __shfl_xor(gc, 32);
    f32x4 aQ = zero4(), aW = zero4(), aK = zero4();
#pragma unroll
    for (int q = 0; q < KS; ++q) {
      const int j = g4 * KS + q;
      aQ = __builtin_amdgcn_mfma_f32_16x16x4f32(sdO[l16][j], sv[q], aQ, 0, 0, 0);
      aW = __builtin_amdgcn_mfma_f32_16x16x4f32(sdDel[l16][j], sv[q], aW, 0, 0, 0);
      aK = __builtin_amdgcn_mfma_f32_16x16x4f32(sDel[l16][j], dsv[q], aK, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * g4 + i;
      sdQp[r][c] = aQ[i];
      sX[r][c] = -aW[i];
      sdKt[r][c] = aK[i];
    }
    if (g4 == 0) sdGC[c] = lgeG * gc;
  }
  __syncthreads();
  // ---- the 16 x 16 and 16 x D products of the block on the fp32 matrix cores
  // (v_mfma_f32_16x16x4_f32: lane l gives A[l % 16][k] and B[k][l % 16] with k
  // the step's K index 4 s + l / 16, and holds C[4 (l / 16) + i][l % 16]).
  // dXw = T^T dW, dXu = T^T dDelta (K = 16); wave w: channels 16w .. 16w + 15
  {
    f32x4 xw = zero4(), xu = zero4();
    const int c = wave * 16 + l16;
    if (wave < D / 16) {
#pragma unroll
      for (int st = 0; st < kBlk / 4; ++st) {
        const int k = 4 * st + g4;
        const float a = sT[k][l16];            // T^T[m][k] = T[k][m]
        xw = __builtin_amdgcn_mfma_f32_16x16x4f32(a, sX[k][c], xw, 0, 0, 0);
        xu = __builtin_amdgcn_mfma_f32_16x16x4f32(a, sdDel[k][c], xu, 0, 0, 0);
      }
    }
    __syncthreads();
    if (wave < D / 16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sX[4 * g4 + i][c] = xw[i];
        sdKm[4 * g4 + i][c] = xu[i];          // dXu parked in sdKm until dV is formed
      }
    }
  }
#pragma unroll
  for (int m = 0; m < EL; ++m) {
    const int e = tid + m * NT;
    if (e < kBlk * D) {
      sWt[e / D][e % D] = lW[m];
      sUt[e / D][e % D] = lU[m];
    }
  }
  __syncthreads();
  // dA = -strict_lower(dXw W^T + dXu U^T), A_un = strict_lower(K+ K-^T) and
  // dAqk = lower(dO Delta^T): 16 x 16 each over K = D, the channel range split
  // over the waves (dA, two products a step, on half of them; A_un and dAqk on
  // a quarter each), four independent accumulators per wave, then the waves'
  // partial sums added in a fixed order
  {
    constexpr int NW = NT / kWave;
    constexpr int nA = NW / 2, nU = NW / 4;              // waves per product (nQ = nU)
    const int prod = wave < nA ? 0 : (wave < nA + nU ? 1 : 2);
    const int part = prod == 0 ? wave : (prod == 1 ? wave - nA : wave - nA - nU);
    const int KW = prod == 0 ? D / nA : D / nU;          // channels of this wave
    const int kbeg = part * KW;
    f32x4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
    for (int st0 = 0; st0 < KW / 4; st0 += 4) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (st0 + j >= KW / 4) break;
        const int k = kbeg + 4 * (st0 + j) + g4;
        if (prod == 0) {
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(sX[l16][k], sWt[l16][k], acc[j], 0, 0, 0);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(sdKm[l16][k], sUt[l16][k], acc[j], 0, 0, 0);
        } else if (prod == 1) {
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(s.k[l16][k] * s.eP[l16][k], s.k[l16][k] * s.eM[l16][k],
                                                        acc[j], 0, 0, 0);
        } else {
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(sdO[l16][k], sDel[l16][k], acc[j], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sPart[wave][4 * g4 + i][l16] = (acc[0][i] + acc[1][i]) + (acc[2][i] + acc[3][i]);
    __syncthreads();
    for (int e = tid; e < 3 * kBlk * kBlk; e += NT) {
      const int pr = e / (kBlk * kBlk), r = (e / kBlk) % kBlk, i = e % kBlk;
      const int w0 = pr == 0 ? 0 : (pr == 1 ? nA : nA + nU), nw = pr == 0 ? nA : nU;
      float v = 0.f;
      for (int w = 0; w < nw; ++w) v += sPart[w0 + w][r][i];
      if (pr == 0) sdA[r][i] = i < r ? -v : 0.f;
      else if (pr == 1) sAun[r][i] = i < r ? v : 0.f;
      else sdAqk[r][i] = i <= r ? v : 0.f;
    }
  }
  __syncthreads();
  // ---- dbeta (all threads: NT / 16 lanes per row, a shuffle sum); dV; dK+
  // and dK- from X and A; dQ+ and dK- from Aqk
  {
    constexpr int TPR = NT / kBlk;      // lanes per row (a power of two, at most 64)
    const int r = tid / TPR, lr = tid % TPR;
    float d = 0.f;
    for (int c = lr; c < D; c += TPR) d += sX[r][c] * s.k[r][c] * s.eP[r][c] + sdKm[r][c] * s.v[r][c];
    for (int i = lr; i < r; i += TPR) d += sdA[r][i] * sAun[r][i];
#pragma unroll
    for (int o = TPR / 2; o >= 1; o /= 2) d += __shfl_xor(d, o, TPR);
    if (lr == 0) sdbeta[r] = d;
  }
  {
    // (beta dA) K-,  (beta dA)^T K+ + dAqk^T Q+,  dAqk K-  (K = 16)
    f32x4 kpM = zero4(), kmM = zero4(), qpM = zero4();
    const int c = wave * 16 + l16;
    if (wave < D / 16) {
#pragma unroll
      for (int st = 0; st < kBlk / 4; ++st) {
        const int k = 4 * st + g4;
        const float kmi = s.k[k][c] * s.eM[k][c], kpi = s.k[k][c] * s.eP[k][c], qpi = s.q[k][c] * s.eP[k][c];
        kpM = __builtin_amdgcn_mfma_f32_16x16x4f32(s.beta[l16] * sdA[l16][k], kmi, kpM, 0, 0, 0);
        kmM = __builtin_amdgcn_mfma_f32_16x16x4f32(s.beta[k] * sdA[k][l16], kpi, kmM, 0, 0, 0);
        kmM = __builtin_amdgcn_mfma_f32_16x16x4f32(sdAqk[k][l16], qpi, kmM, 0, 0, 0);
        qpM = __builtin_amdgcn_mfma_f32_16x16x4f32(sdAqk[l16][k], kmi, qpM, 0, 0, 0);
      }
    }
    float dKp[4], dKm[4], dQp[4], dV[4], gnp[4];
    if (wave < D / 16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g4 + i;
        const float be = s.beta[r];
        const float xw = be * sX[r][c];         // Diag(beta) dXw
        const float q0 = sdQp[r][c];            // dO S0^T
        // the decay's gradient through the single-token terms (dO S0^T on Q+,
        // beta dXw on K+); the pair terms of A and Aqk are summed separately
        gnp[i] = (q0 * s.q[r][c] + xw * s.k[r][c]) * s.eP[r][c];
        dKp[i] = xw + kpM[i];
        dKm[i] = kmM[i];
        dQp[i] = q0 + qpM[i];
        dV[i] = be * sdKm[r][c];
      }
    }
    __syncthreads();
    if (wave < D / 16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g4 + i;
        sdKp[r][c] = dKp[i];
        sdKm[r][c] = dKm[i];
        sdQp[r][c] = dQp[i];
        sX[r][c] = dV[i];                       // sX now holds dV
        sDel[r][c] = gnp[i];                    // Delta is no longer needed
      }
    }
  }
  __syncthreads();
  // ---- chain to q^, k^ (into sdQp, sdKp) and the gate (dg into sdKm), per channel.
  // A pair (r, i < r) of A or Aqk enters the decays through e^{G_r - G_i}:
  // +T_ri on G_r and -T_ri on G_i, with T_ri = (beta_r dA[r][i] k_r
  // + dAqk[r][i] q_r) k_i e^{G_r - G_i}.  Summed into dg_t = sum_{r >= t} dG_r
  // the two cancel unless i < t <= r, so the pairs are added directly over
  // that rectangle (row by row, prefix sums over i): nothing is subtracted,
  // and no rounding residue of two large canceling sums is left over.
  // Four parts per channel (waves at d = 128), part p taking rows p, p + 4, ...:
  // the elementwise terms, then the pair terms of its rows into a partial P,
  // which meet in shared memory (buffers no longer needed: W, U, dDelta, dO)
  // and are added in part order by the channel's first thread.
  {
    constexpr int PT = NT / D >= 4 ? 4 : NT / D;
    static_assert(kBlk % PT == 0, "rows split evenly over the parts");
    const int c = tid % D, part = tid / D;
    float (*pp)[D + 1] = part == 0 ? sWt : (part == 1 ? sUt : (part == 2 ? sdDel : sdO));
    if (part < PT) {
      float P[kBlk];
#pragma unroll
      for (int t2 = 0; t2 < kBlk; ++t2) P[t2] = 0.f;
#pragma unroll
      for (int j = 0; j < kBlk / PT; ++j) {
        const int r = part + PT * j;
        const float eP = s.eP[r][c], eM = s.eM[r][c], eS = s.eS[r][c];
        const float k = s.k[r][c];
        const float dqp = sdQp[r][c], dkp = sdKp[r][c], dkm = sdKm[r][c], dkt = sdKt[r][c];
        sdQp[r][c] = dqp * eP;                          // d q^
        sdKp[r][c] = dkp * eP + dkm * eM + dkt * eS;    // d k^
        sdKt[r][c] = dkt * k * eS;                      // dGs, in place of dK~
      }
      // K-[i][c] for every column i of the pairs, and each row's dA, dAqk as
      // 16-byte reads: the loop below then reads nothing from shared memory
      float km[kBlk - 1];
#pragma unroll
      for (int i = 0; i < kBlk - 1; ++i) km[i] = s.k[i][c] * s.eM[i][c];
#pragma unroll
      for (int j = 0; j < kBlk / PT; ++j) {
        const int r = part + PT * j;
        const float ar = s.beta[r] * s.k[r][c] * s.eP[r][c], br = s.q[r][c] * s.eP[r][c];
        float da[kBlk], dq[kBlk];
#pragma unroll
        for (int q = 0; q < kBlk / 4; ++q) {
          const float4 a4 = *reinterpret_cast<const float4*>(&sdA[r][4 * q]);
          const float4 b4 = *reinterpret_cast<const float4*>(&sdAqk[r][4 * q]);
          da[4 * q] = a4.x; da[4 * q + 1] = a4.y; da[4 * q + 2] = a4.z; da[4 * q + 3] = a4.w;
          dq[4 * q] = b4.x; dq[4 * q + 1] = b4.y; dq[4 * q + 2] = b4.z; dq[4 * q + 3] = b4.w;
        }
        float rp = 0.f;
#pragma unroll
        for (int t2 = 1; t2 < kBlk; ++t2) {
          if (t2 <= r) {
            const int i = t2 - 1;
            rp += (da[i] * ar + dq[i] * br) * km[i];
            P[t2] += rp;
          }
        }
      }
#pragma unroll
      for (int t2 = 0; t2 < kBlk; ++t2) pp[t2][c] = P[t2];
    }
    __syncthreads();
    // dg_t = sum_{r >= t} dG_r + sum_{r < t} dGs_r + dG_C + P_t, for the block's
    // tokens: every part's thread forms the channel's suffix and prefix sums
    // (all reads first) and writes its own kBlk / PT rows
    if (part < PT) {
      float dG[kBlk], pre[kBlk];
#pragma unroll
      for (int r = 0; r < kBlk; ++r) {
        dG[r] = sDel[r][c];
        pre[r] = sdKt[r][c];
      }
      const float gc = sdGC[c];
      float suffix = 0.f, prefix = 0.f;
#pragma unroll
      for (int r = kBlk - 1; r >= 0; --r) {
        suffix += dG[r];
        dG[r] = suffix;
      }
#pragma unroll
      for (int r = 0; r < kBlk; ++r) {
        const float g = pre[r];
        pre[r] = prefix;
        prefix += g;
      }
#pragma unroll
      for (int r = 0; r < kBlk; ++r) {
        if (r / (kBlk / PT) != part) continue;   // (uniform over the wave)
        float Pr = sWt[r][c];
        if (PT > 1) Pr += sUt[r][c];
        if (PT > 2) Pr += sdDel[r][c];
        if (PT > 3) Pr += sdO[r][c];
        sdKm[r][c] = r < b.ntok ? dG[r] + pre[r] + gc + Pr : 0.f;   // dg
      }
    }
  }
  __syncthreads();
  // ---- the preprocess in reverse, on the threads whose registers hold the
  // raw inputs of the same (tensor, channel) task.  The gate's tasks, v's
  // SiLU and the L2 norms' dot products need nothing from one another and go
  // in one phase (different threads); the SiLU of q and k follows, after the
  // dot products are in shared memory.
  __shared__ float sAl[NT / kWave];
  __shared__ float sDot[2][kBlk];
  // SiLU: dy = du sigmoid(y) (1 + y (1 - sigmoid(y))), with y recomputed from
  // the raw inputs; roles 0 and 1 (q, k) through the L2 norm's reverse
  auto silu_reverse = [&](bool qk) {
#pragma unroll
    for (int m = 0; m < Raw::kTasks; ++m) {
      const int task = tid + m * NT;
      if (task >= 3 * D || (task < 2 * D) != qk) continue;
      const int role = task / D, ch = task % D;
      const size_t col = static_cast<size_t>(h) * D + ch;
      const float w0 = raw.w[m][0], w1 = raw.w[m][1], w2 = raw.w[m][2], w3 = raw.w[m][3];
#pragma unroll
      for (int r = 0; r < kBlk; ++r) {
        if (r >= b.ntok) continue;
        const float y = w0 * raw.x[m][r] + w1 * raw.x[m][r + 1] + w2 * raw.x[m][r + 2] + w3 * raw.x[m][r + 3];
        float du;
        if (role == 0) {
          du = s.rq[r] * (sdQp[r][ch] - s.q[r][ch] * sDot[0][r]);
        } else if (role == 1) {
          du = s.rk[r] * (sdKp[r][ch] - s.k[r][ch] * sDot[1][r]);
        } else {
          du = sX[r][ch];            // dV
        }
        const float sg = sigmoidf_(y);
        dy[static_cast<size_t>(b.tok0 + r) * 3 * HD + role * HD + col] = du * sg * (1.f + y * (1.f - sg));
      }
    }
  };
  // gate: d alpha, and the block's partial sums for d dt_bias and d A_log
  {
    const float a_exp = expf(p.A_log[h]);
    float alog_part = 0.f;
#pragma unroll
    for (int m = 0; m < Raw::kTasks; ++m) {
      const int task = tid + m * NT;
      if (task < 3 * D || task >= 4 * D) continue;
      const int c = task - 3 * D;
      const size_t col = static_cast<size_t>(h) * D + c;
      const float dtb = raw.w[m][0];
      float dtb_part = 0.f;
#pragma unroll
      for (int r = 0; r < kBlk; ++r) {
        if (r >= b.ntok) continue;
        const float al = raw.x[m][3 + r];
        const float dg = sdKm[r][c];
        float da;
        if (p.flags & KDA_FLAG_RAW_GATE) {
          da = dg;
        } else {
          const float z = al + dtb;
          const float graw = -a_exp * softplusf_(z);
          if (graw >= p.lower_bound) {
            da = -dg * a_exp * sigmoidf_(z);
            dtb_part += da;
            alog_part += dg * graw;
          } else {
            da = 0.f;
          }
        }
        dalpha[static_cast<size_t>(b.tok0 + r) * HD + col] = da;
      }
      pd[c] = dtb_part;
    }
    // d A_log: the waves' sums, added after the barrier below
    const float wsum = group_sum<kWave>(alog_part);
    if (tid % kWave == 0) sAl[tid / kWave] = wsum;
  }
  // beta
  if (tid < b.ntok) {
    const float sg = sigmoidf_(raw.bb);
    float dbv = sdbeta[tid] * sg * (1.f - sg);
    if (p.flags & KDA_FLAG_BETA_X2) dbv *= 2.f;
    db[static_cast<size_t>(b.tok0 + tid) * p.H + h] = dbv;
  }
  // L2 norm (q with its scale, k): du = (s / n) (dq^ - q^ (q^ . dq^) / s^2);
  // sDot holds (q^ . dq^) / s^2 and k^ . dk^
  if (tid < 2 * kBlk * 8) {
    const int row = tid / 8, l8 = tid % 8;
    const bool isq = row < kBlk;
    const int r = isq ? row : row - kBlk;
    float dot = 0.f;
    for (int c = l8; c < D; c += 8) dot += isq ? s.q[r][c] * sdQp[r][c] : s.k[r][c] * sdKp[r][c];
    dot += __shfl_xor(dot, 1, 8);
    dot += __shfl_xor(dot, 2, 8);
    dot += __shfl_xor(dot, 4, 8);
    if (l8 == 0) sDot[isq ? 0 : 1][r] = isq ? dot / (p.scale * p.scale) : dot;
  }
  silu_reverse(false);   // v
  __syncthreads();
  if (tid == 0) {
    float tot = 0.f;
    for (int w = 0; w < NT / kWave; ++w) tot += sAl[w];
    pAlog[bh] = tot;
  }
  silu_reverse(true);    // q, k
}

// ---------------------------------------------------------------- conv reverse
// One workgroup per (64-token chunk, head); a thread per (q/k/v, channel)
// walks the chunk's tokens: dx_t = sum_j w[j] dy_{t+3-j} over tokens of the
// same sequence, the history's gradient for the sequence's first chunk, and
// the chunk's partial d w[j] = sum_t dy_t x_{t-3+j}.  The tokens go in four
// steps of 16, each step's loads issued before the previous step's
// arithmetic; addresses are clamped into the sequence and the zeros outside
// it selected afterwards, so a step's loads go out back to back.
template <int D, bool IO_BF16>
__global__ __launch_bounds__(3 * D) void bwd_conv_kernel(Params p, ChunkTable t, PrefillIO io, const float* dy,
                                                          float* dq, float* dk, float* dv, float* dconv,
                                                          float* pdw) {
  constexpr int SB = 16;                   // tokens per step
  const int h = static_cast<int>(blockIdx.x % static_cast<unsigned>(p.H));
  const int c = static_cast<int>(blockIdx.x / static_cast<unsigned>(p.H));
  const int tid = threadIdx.x, role = tid / D, ch = tid % D;
  const size_t HD = static_cast<size_t>(p.H) * D;
  const size_t col = static_cast<size_t>(h) * D + ch;
  float* pw = pdw + ((static_cast<size_t>(c) * 3 + role) * HD + col) * 4;
  if (c >= t.chunk0[t.N]) return;
  const int4 d = t.desc[c];
  const int seq = d.x, tau0 = d.y, cnt = d.z;
  const int64_t tok0 = d.w, seq0 = tok0 - tau0;
  const int L = t.cu[seq + 1] - t.cu[seq];
  const void* xin = role == 0 ? io.q : (role == 1 ? io.k : io.v);
  const void* w = role == 0 ? p.wq : (role == 1 ? p.wk : p.wv);
  float* dx = role == 0 ? dq : (role == 1 ? dk : dv);
  const float* dyc = dy + static_cast<size_t>(seq0) * 3 * HD + role * HD + col;   // dy at sequence position 0
  const size_t xcol = static_cast<size_t>(seq0) * HD + col;                       // x at sequence position 0
  float wj[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) wj[j] = ld<IO_BF16>(w, col * 4 + j);
  // the window before the first step: x at positions tau0 - 3 .. tau0 - 1 (the
  // sequence's inputs, or at its start the conv history, zeros without one),
  // dy at tau0 .. tau0 + 2
  const bool hist = tau0 == 0;
  const bool from_hist = hist && io.conv_in != nullptr;
  const void* xsrc = from_hist ? io.conv_in : xin;   // one load from whichever holds the row
  float xw[3], dyw[3];
#pragma unroll
  for (int m = 0; m < 3; ++m) {
    const size_t xi = xcol + static_cast<size_t>(hist ? 0 : tau0 - 3 + m) * HD;
    const size_t hi = (static_cast<size_t>(seq) * 3 + m) * 3 * HD + role * HD + col;
    xw[m] = ld<IO_BF16>(xsrc, from_hist ? hi : xi);
    dyw[m] = dyc[static_cast<size_t>(min(tau0 + m, L - 1)) * 3 * HD];
  }
  // step k's operands: x at tau0 + 16k .. + 15, dy at tau0 + 16k + 3 .. + 18
  float xn[SB], dyn[SB];
  auto fetch = [&](int k) {
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      xn[i] = ld<IO_BF16>(xin, xcol + static_cast<size_t>(tau0 + min(SB * k + i, cnt - 1)) * HD);
      dyn[i] = dyc[static_cast<size_t>(min(tau0 + SB * k + 3 + i, L - 1)) * 3 * HD];
    }
  };
  fetch(0);
#pragma unroll
  for (int m = 0; m < 3; ++m) {
    if (hist && !from_hist) xw[m] = 0.f;
    if (tau0 + m >= L) dyw[m] = 0.f;
  }
  // history slot m holds position m - 3: dx_{m-3} = sum_j w[j] dy_{m-j}
  if (hist && dconv) {
#pragma unroll
    for (int m = 0; m < 3; ++m) {
      float g = 0.f;
#pragma unroll
      for (int j = 0; j <= m; ++j) g += wj[j] * dyw[m - j];
      dconv[(static_cast<size_t>(seq) * 3 + m) * 3 * HD + role * HD + col] = g;
    }
  }
  float aw[4] = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < kChunk / SB; ++k) {
    if (SB * k >= cnt) break;   // uniform over the workgroup
    float xx[SB + 3], dd[SB + 3];
#pragma unroll
    for (int m = 0; m < 3; ++m) { xx[m] = xw[m]; dd[m] = dyw[m]; }
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      xx[3 + i] = SB * k + i < cnt ? xn[i] : 0.f;
      dd[3 + i] = tau0 + SB * k + 3 + i < L ? dyn[i] : 0.f;
    }
    if (k + 1 < kChunk / SB) fetch(k + 1);
#pragma unroll
    for (int r = 0; r < SB; ++r) {
      if (SB * k + r < cnt) {
        float g = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) g += wj[j] * dd[r + 3 - j];
        dx[xcol + static_cast<size_t>(tau0 + SB * k + r) * HD] = g;
#pragma unroll
        for (int j = 0; j < 4; ++j) aw[j] += dd[r] * xx[r + j];
      }
    }
#pragma unroll
    for (int m = 0; m < 3; ++m) { xw[m] = xx[SB + m]; dyw[m] = dd[SB + m]; }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) pw[j] = aw[j];
}

// ---------------------------------------------------------------- parameter sums
// The partial parameter gradients (per chunk for the conv weights, per block
// for dt_bias and A_log) are summed in two deterministic passes: the rows are
// cut into kReduceParts contiguous ranges, each range summed by four threads
// per element (rows interleaved) and their sums added in a fixed order; then
// the ranges' sums are added in range order.  Element e runs over the conv
// weights' partials [0, n_w), dt_bias's [n_w, n_w + HD) and A_log's after.
struct ParamSums {
  const float* pdw;
  const float* pdtb;
  const float* pAlog;
  int64_t n_w, n_dtb, n_al;
  const int* nchunks;        // the chunk table's count of chunks (on the device)
  __device__ int64_t total() const { return n_w + n_dtb + n_al; }
  // the partial of element e in row r, and the element's number of rows
  // (chunks for the conv weights, 16-token blocks for the others)
  __device__ int rows(int64_t e) const { return *nchunks * (e < n_w ? 1 : kBlocksPerChunk); }
  __device__ float at(int64_t e, int r) const {
    if (e < n_w) return pdw[static_cast<size_t>(r) * n_w + e];
    if (e < n_w + n_dtb) return pdtb[static_cast<size_t>(r) * n_dtb + (e - n_w)];
    return pAlog[static_cast<size_t>(r) * n_al + (e - n_w - n_dtb)];
  }
};

__global__ __launch_bounds__(256) void bwd_param_partial_kernel(ParamSums ps, float* stage) {
  __shared__ float red[4][64];
  const int tid = threadIdx.x, el = tid % 64, sub = tid / 64;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 64 + el;
  const int part = static_cast<int>(blockIdx.y);
  float acc = 0.f;
  if (e < ps.total()) {
    const int rows = ps.rows(e);
    const int lo = static_cast<int>(static_cast<int64_t>(rows) * part / kReduceParts);
    const int hi = static_cast<int>(static_cast<int64_t>(rows) * (part + 1) / kReduceParts);
    for (int r = lo + sub; r < hi; r += 4) acc += ps.at(e, r);
  }
  red[sub][el] = acc;
  __syncthreads();
  if (sub == 0 && e < ps.total())
    stage[static_cast<size_t>(part) * ps.total() + e] = (red[0][el] + red[1][el]) + (red[2][el] + red[3][el]);
}

__global__ void bwd_param_final_kernel(ParamSums ps, const float* stage, float* dw_q, float* dw_k, float* dw_v,
                                       float* ddt_bias, float* dA_log) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= ps.total()) return;
  float acc = 0.f;
  for (int part = 0; part < kReduceParts; ++part) acc += stage[static_cast<size_t>(part) * ps.total() + e];
  if (e < ps.n_w) {
    const int64_t per = ps.n_w / 3, role = e / per, rest = e % per;
    (role == 0 ? dw_q : (role == 1 ? dw_k : dw_v))[rest] = acc;
  } else if (e < ps.n_w + ps.n_dtb) {
    ddt_bias[e - ps.n_w] = acc;
  } else {
    dA_log[e - ps.n_w - ps.n_dtb] = acc;
  }
}

// ---------------------------------------------------------------- launchers
namespace {

template <int D, bool IO_BF16, bool DO_BF16>
hipError_t launch_backward_d(const Params& p, const ChunkTable& t, const PrefillIO& io, const BackwardIO& g,
                             const BackwardWS& ws, int N, int max_chunks, hipStream_t st) {
  const unsigned nblk = static_cast<unsigned>(max_chunks) * kBlocksPerChunk * static_cast<unsigned>(p.H);
  bwd_block_prep_kernel<D, IO_BF16><<<nblk, kBT, 0, st>>>(p, t, io, ws.recs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned nh8 = (static_cast<unsigned>(N) * p.H + 7) / 8 * 8;   // (sequence, head) pairs, padded to 8 XCDs
  constexpr int TW = scan_waves<D>();
  const unsigned nscan = nh8 * (D / (kScanTile * TW));
  bwd_state_scan_kernel<D><<<nscan, kWave * TW, 0, st>>>(p, t, io.S0, ws.recs, ws.Sblk, ws.Dblk);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  bwd_adjoint_scan_kernel<D, DO_BF16><<<nscan, kWave * TW, 0, st>>>(p, t, ws.recs, g.dO, g.dS_final, ws.dSblk,
                                                                    ws.dDblk, g.dS_init, g.dconv);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  bwd_block_grad_kernel<D, IO_BF16, DO_BF16><<<nblk, grad_threads<D>(), 0, st>>>(p, t, io, ws.recs, ws.Sblk, ws.dSblk, ws.Dblk,
                                                                   ws.dDblk, g.dO, ws.dy, g.dalpha, g.db, ws.pdtb,
                                                                   ws.pAlog);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  bwd_conv_kernel<D, IO_BF16><<<static_cast<unsigned>(max_chunks) * p.H, 3 * D, 0, st>>>(p, t, io, ws.dy, g.dq, g.dk,
                                                                                       g.dv, g.dconv, ws.pdw);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  ParamSums ps{ws.pdw, ws.pdtb, ws.pAlog, 3 * static_cast<int64_t>(p.H) * D * 4, static_cast<int64_t>(p.H) * D,
               p.H, t.chunk0 + t.N};
  const int64_t n_out = ps.n_w + ps.n_dtb + ps.n_al;
  bwd_param_partial_kernel<<<dim3(static_cast<unsigned>((n_out + 63) / 64), kReduceParts), 256, 0, st>>>(ps, ws.pstage);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  bwd_param_final_kernel<<<static_cast<unsigned>((n_out + 255) / 256), 256, 0, st>>>(ps, ws.pstage, g.dw_q, g.dw_k,
                                                                                     g.dw_v, g.ddt_bias, g.dA_log);
  return hipGetLastError();
}

template <int D>
hipError_t launch_backward_io(const Params& p, const ChunkTable& t, const PrefillIO& io, const BackwardIO& g,
                              const BackwardWS& ws, int N, int max_chunks, bool io_bf16, bool do_bf16,
                              hipStream_t st) {
  if (io_bf16 && do_bf16) return launch_backward_d<D, true, true>(p, t, io, g, ws, N, max_chunks, st);
  if (io_bf16) return launch_backward_d<D, true, false>(p, t, io, g, ws, N, max_chunks, st);
  if (do_bf16) return launch_backward_d<D, false, true>(p, t, io, g, ws, N, max_chunks, st);
  return launch_backward_d<D, false, false>(p, t, io, g, ws, N, max_chunks, st);
}

}  // namespace

hipError_t launch_backward(const Params& p, const ChunkTable& t, const PrefillIO& io, const BackwardIO& g,
                           const BackwardWS& ws, int N, int max_chunks, bool io_bf16, bool do_bf16, hipStream_t st) {
  switch (p.D) {
    case 16: return launch_backward_io<16>(p, t, io, g, ws, N, max_chunks, io_bf16, do_bf16, st);
    case 32: return launch_backward_io<32>(p, t, io, g, ws, N, max_chunks, io_bf16, do_bf16, st);
    case 64: return launch_backward_io<64>(p, t, io, g, ws, N, max_chunks, io_bf16, do_bf16, st);
    case 128: return launch_backward_io<128>(p, t, io, g, ws, N, max_chunks, io_bf16, do_bf16, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kda
