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
//   bwd_param_reduce  partial parameter gradients summed in block order
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kBlk = 16;             // tokens per block
constexpr int kBT = 256;             // threads of the per-block and scan kernels
constexpr int kBlocksPerChunk = kChunk / kBlk;

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
template <int D>
struct BlockSmem {
  float q[kBlk][D];      // q^ (normalised, scaled)
  float k[kBlk][D];      // k^ (normalised)
  float v[kBlk][D];      // v^
  float eP[kBlk][D];     // e^{G}, G the inclusive in-block prefix sum of g
  float eM[kBlk][D];     // e^{-G}
  float eS[kBlk][D];     // e^{G_C - G}, from the exclusive in-block suffix sum of g
  float beta[kBlk];
  float nq[kBlk], nk[kBlk];   // the L2 norms sqrt(|u|^2 + eps) of q and k
};

// Conv + SiLU, L2 norm, gate and beta of one block's tokens for head h, into
// shared memory.  Rows past the block's end are zero, with g = beta = 0.
template <int D, bool IO_BF16, int NT>
__device__ void block_preprocess(const Params& p, const PrefillIO& io, const BlockInfo& b, int h, BlockSmem<D>& s) {
  static_assert(NT >= 2 * kBlk * 8, "the L2 norms take 8 lanes for each of 32 rows");
  const int tid = threadIdx.x;
  const size_t HD = static_cast<size_t>(p.H) * D;
  const size_t Ctot = 3 * HD;
  const int seq = b.seq;
  const int64_t seq0 = b.tok0 - b.tau0;   // packed index of the sequence's first token
  for (int task = tid; task < 4 * D; task += NT) {
    const int role = task / D, ch = task % D;
    const size_t col = static_cast<size_t>(h) * D + ch;
    if (role < 3) {
      const void* xin = role == 0 ? io.q : (role == 1 ? io.k : io.v);
      const void* w = role == 0 ? p.wq : (role == 1 ? p.wk : p.wv);
      const float w0 = ld<IO_BF16>(w, col * 4), w1 = ld<IO_BF16>(w, col * 4 + 1);
      const float w2 = ld<IO_BF16>(w, col * 4 + 2), w3 = ld<IO_BF16>(w, col * 4 + 3);
      float win[3];
#pragma unroll
      for (int m = 0; m < 3; ++m) {
        const int tau = b.tau0 - 3 + m;
        if (tau >= 0) win[m] = ld<IO_BF16>(xin, static_cast<size_t>(seq0 + tau) * HD + col);
        else if (io.conv_in) win[m] = ld<IO_BF16>(io.conv_in, (static_cast<size_t>(seq) * 3 + (3 + tau)) * Ctot + role * HD + col);
        else win[m] = 0.f;
      }
      float* dst = role == 0 ? &s.q[0][0] : (role == 1 ? &s.k[0][0] : &s.v[0][0]);
      for (int r = 0; r < kBlk; ++r) {
        float u = 0.f;
        if (r < b.ntok) {
          const float xt = ld<IO_BF16>(xin, static_cast<size_t>(b.tok0 + r) * HD + col);
          u = siluf_(w0 * win[0] + w1 * win[1] + w2 * win[2] + w3 * xt);
          win[0] = win[1]; win[1] = win[2]; win[2] = xt;
        }
        dst[r * D + ch] = u;
      }
    } else {
      const float a_exp = expf(p.A_log[h]);
      const float dtb = p.dt_bias[col];
      float run = 0.f;
      float g[kBlk];
      for (int r = 0; r < kBlk; ++r) {
        g[r] = 0.f;
        if (r < b.ntok) {
          const float al = ld<IO_BF16>(io.alpha, static_cast<size_t>(b.tok0 + r) * HD + col);
          g[r] = (p.flags & KDA_FLAG_RAW_GATE) ? al : gate_value(al, dtb, a_exp, p.lower_bound);
        }
        run += g[r];
        s.eP[r][ch] = expf(run);
        s.eM[r][ch] = expf(-run);
      }
      float suf = 0.f;
      for (int r = kBlk - 1; r >= 0; --r) {
        s.eS[r][ch] = expf(suf);
        suf += g[r];
      }
    }
  }
  if (tid < kBlk) {
    float be = 0.f;
    if (tid < b.ntok) {
      const float bb = ld<IO_BF16>(io.b, static_cast<size_t>(b.tok0 + tid) * p.H + h);
      be = sigmoidf_(bb);
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
      if (row < kBlk) s.nq[row] = n; else s.nk[row - kBlk] = n;
    }
  }
  __syncthreads();
  for (int e = tid; e < kBlk * D; e += NT) {
    const int r = e / D, c = e % D;
    s.q[r][c] = s.q[r][c] / s.nq[r] * p.scale;
    s.k[r][c] = s.k[r][c] / s.nk[r];
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

// ---------------------------------------------------------------- block prep
template <int D, bool IO_BF16>
__global__ __launch_bounds__(kBT) void bwd_block_prep_kernel(Params p, ChunkTable t, PrefillIO io, uint8_t* recs) {
  constexpr BwdRecord R = bwd_record(D);
  __shared__ BlockSmem<D> s;
  __shared__ float sKm[kBlk][D];       // K e^{-G}
  __shared__ float sA[kBlk][kBlk];     // A, then T
  __shared__ float sT[kBlk][kBlk];
  const int h = static_cast<int>(blockIdx.x % static_cast<unsigned>(p.H));
  const int blk = static_cast<int>(blockIdx.x / static_cast<unsigned>(p.H));
  if (blk / kBlocksPerChunk >= t.chunk0[t.N]) return;
  const BlockInfo b = block_info(t, blk);
  if (b.ntok <= 0) return;
  const int tid = threadIdx.x;
  block_preprocess<D, IO_BF16, kBT>(p, io, b, h, s);
  uint8_t* rec = recs + (static_cast<size_t>(blk) * p.H + h) * R.bytes;
  float* gW = reinterpret_cast<float*>(rec + R.W);
  float* gU = reinterpret_cast<float*>(rec + R.U);
  float* gQp = reinterpret_cast<float*>(rec + R.Qp);
  float* gKt = reinterpret_cast<float*>(rec + R.Kt);
  float* gT = reinterpret_cast<float*>(rec + R.T);
  float* gAqk = reinterpret_cast<float*>(rec + R.Aqk);
  float* geGC = reinterpret_cast<float*>(rec + R.eGC);
  // K-, Q+, K~ and e^{G_C}
  for (int e = tid; e < kBlk * D; e += kBT) {
    const int r = e / D, c = e % D;
    sKm[r][c] = s.k[r][c] * s.eM[r][c];
    gQp[e] = s.q[r][c] * s.eP[r][c];
    gKt[e] = s.k[r][c] * s.eS[r][c];
    if (r == 0) geGC[c] = s.eP[kBlk - 1][c];
  }
  __syncthreads();
  // A (strictly lower) and Aqk (lower with the diagonal): one entry each per thread
  {
    const int r = tid / kBlk, i = tid % kBlk;
    float a = 0.f, aq = 0.f;
    if (i <= r) {
      for (int c = 0; c < D; ++c) {
        const float eg = s.eP[r][c];
        const float km = sKm[i][c];
        aq += s.q[r][c] * eg * km;
        if (i < r) a += s.k[r][c] * eg * km;
      }
    }
    sA[r][i] = s.beta[r] * a;
    gAqk[tid] = aq;
  }
  __syncthreads();
  // T = (I + A)^-1 by forward substitution, lane i owns column i
  if (tid < kBlk) {
    const int i = tid;
    float col[kBlk];
    for (int r = 0; r < kBlk; ++r) {
      float v = (r == i) ? 1.f : 0.f;
      for (int m = 0; m < r; ++m) v -= sA[r][m] * col[m];
      col[r] = r < i ? 0.f : v;
    }
    for (int r = 0; r < kBlk; ++r) sT[r][i] = col[r];
  }
  __syncthreads();
  for (int e = tid; e < kBlk * kBlk; e += kBT) gT[e] = sT[e / kBlk][e % kBlk];
  // W = T Diag(beta) K+,  U = T Diag(beta) V
  for (int e = tid; e < kBlk * D; e += kBT) {
    const int r = e / D, c = e % D;
    float w = 0.f, u = 0.f;
    for (int m = 0; m <= r; ++m) {
      const float tb = sT[r][m] * s.beta[m];
      w += tb * s.k[m][c] * s.eP[m][c];
      u += tb * s.v[m][c];
    }
    gW[e] = w;
    gU[e] = u;
  }
}

// ---------------------------------------------------------------- state scan
// One workgroup per (sequence, head, value tile of VT columns): the state
// slice in registers, a thread holding column j = tid % VT of rows
// tid / VT + m * (256 / VT).  A sequence's blocks are consecutive (block
// index = 4 x its first chunk + its position); each block's operands are
// loaded into registers one block ahead and moved to shared memory at the
// top of the next step, so their latency hides behind a step's arithmetic.
template <int D, int VT>
__global__ __launch_bounds__(kBT) void bwd_state_scan_kernel(Params p, ChunkTable t, const float* S_init,
                                                              const uint8_t* recs, float* Sblk, float* Dblk) {
  constexpr BwdRecord R = bwd_record(D);
  constexpr int RG = kBT / VT;          // row groups
  constexpr int RPT = D / RG;           // rows per thread
  constexpr int TE = (kBlk * D + kBT - 1) / kBT;    // tile elements per thread
  constexpr int UE = (kBlk * VT + kBT - 1) / kBT;   // U elements per thread
  static_assert(D % RG == 0, "rows split evenly");
  __shared__ float sW[kBlk][D], sKt[kBlk][D], seG[D], sU[kBlk][VT];
  __shared__ float red[RG][kBlk][VT];
  __shared__ float sDel[kBlk][VT];
  const int ntile = D / VT;
  const int tile = static_cast<int>(blockIdx.x % static_cast<unsigned>(ntile));
  const int nh = static_cast<int>(blockIdx.x / static_cast<unsigned>(ntile));
  const int h = nh % p.H, n = nh / p.H;
  const int tid = threadIdx.x, j = tid % VT, rg = tid / VT, j0 = tile * VT;
  const size_t SZ = static_cast<size_t>(D) * D;
  float S[RPT];
  for (int m = 0; m < RPT; ++m) {
    const int r = rg + m * RG;
    S[m] = S_init ? S_init[(static_cast<size_t>(n) * p.H + h) * SZ + static_cast<size_t>(r) * D + j0 + j] : 0.f;
  }
  const int L = t.cu[n + 1] - t.cu[n];
  const int nb = (L + kBlk - 1) / kBlk;
  const int blk0 = t.chunk0[n] * kBlocksPerChunk;
  float pW[TE], pK[TE], pU[UE], pE = 0.f;
  auto fetch = [&](int blk) {
    const uint8_t* rec = recs + (static_cast<size_t>(blk) * p.H + h) * R.bytes;
    const float* gW = reinterpret_cast<const float*>(rec + R.W);
    const float* gU = reinterpret_cast<const float*>(rec + R.U);
    const float* gKt = reinterpret_cast<const float*>(rec + R.Kt);
    const float* geG = reinterpret_cast<const float*>(rec + R.eGC);
    for (int m = 0; m < TE; ++m) {
      const int e = tid + m * kBT;
      if (e < kBlk * D) { pW[m] = gW[e]; pK[m] = gKt[e]; }
    }
    for (int m = 0; m < UE; ++m) {
      const int e = tid + m * kBT;
      if (e < kBlk * VT) pU[m] = gU[(e / VT) * D + j0 + e % VT];
    }
    if (tid < D) pE = geG[tid];
  };
  if (nb > 0) fetch(blk0);
  for (int jb = 0; jb < nb; ++jb) {
    const int blk = blk0 + jb;
    const size_t bh = static_cast<size_t>(blk) * p.H + h;
    for (int m = 0; m < TE; ++m) {
      const int e = tid + m * kBT;
      if (e < kBlk * D) { sW[e / D][e % D] = pW[m]; sKt[e / D][e % D] = pK[m]; }
    }
    for (int m = 0; m < UE; ++m) {
      const int e = tid + m * kBT;
      if (e < kBlk * VT) sU[e / VT][e % VT] = pU[m];
    }
    if (tid < D) seG[tid] = pE;
    // the state at the block's start
    for (int m = 0; m < RPT; ++m) {
      const int r = rg + m * RG;
      Sblk[bh * SZ + static_cast<size_t>(r) * D + j0 + j] = S[m];
    }
    __syncthreads();
    if (jb + 1 < nb) fetch(blk + 1);
    // Delta = U - W S
    float acc[kBlk];
    for (int q = 0; q < kBlk; ++q) acc[q] = 0.f;
    for (int m = 0; m < RPT; ++m) {
      const int r = rg + m * RG;
      for (int q = 0; q < kBlk; ++q) acc[q] += sW[q][r] * S[m];
    }
    for (int q = 0; q < kBlk; ++q) red[rg][q][j] = acc[q];
    __syncthreads();
    for (int e = tid; e < kBlk * VT; e += kBT) {
      const int q = e / VT, jj = e % VT;
      float sum = 0.f;
      for (int g2 = 0; g2 < RG; ++g2) sum += red[g2][q][jj];
      const float del = sU[q][jj] - sum;
      sDel[q][jj] = del;
      Dblk[bh * kBlk * D + static_cast<size_t>(q) * D + j0 + jj] = del;
    }
    __syncthreads();
    // S <- e^{G_C} S + K~^T Delta
    for (int m = 0; m < RPT; ++m) {
      const int r = rg + m * RG;
      float v = seG[r] * S[m];
      for (int q = 0; q < kBlk; ++q) v += sKt[q][r] * sDel[q][j];
      S[m] = v;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- adjoint scan
// The state scan's layout, blocks in reverse, operands one block ahead.
template <int D, int VT, bool DO_BF16>
__global__ __launch_bounds__(kBT) void bwd_adjoint_scan_kernel(Params p, ChunkTable t, const uint8_t* recs,
                                                                const void* dO, const float* dS_final, float* dSblk,
                                                                float* dDblk, float* dS_init, float* dconv) {
  constexpr BwdRecord R = bwd_record(D);
  constexpr int RG = kBT / VT;
  constexpr int RPT = D / RG;
  constexpr int TE = (kBlk * D + kBT - 1) / kBT;
  constexpr int OE = (kBlk * VT + kBT - 1) / kBT;
  constexpr int AE = (kBlk * kBlk + kBT - 1) / kBT;
  __shared__ float sW[kBlk][D], sKt[kBlk][D], sQp[kBlk][D], seG[D];
  __shared__ float sAqk[kBlk][kBlk];
  __shared__ float sdO[kBlk][VT];
  __shared__ float red[RG][kBlk][VT];
  __shared__ float sdDel[kBlk][VT];
  const int ntile = D / VT;
  const int tile = static_cast<int>(blockIdx.x % static_cast<unsigned>(ntile));
  const int nh = static_cast<int>(blockIdx.x / static_cast<unsigned>(ntile));
  const int h = nh % p.H, n = nh / p.H;
  const int tid = threadIdx.x, j = tid % VT, rg = tid / VT, j0 = tile * VT;
  const size_t SZ = static_cast<size_t>(D) * D;
  const size_t HD = static_cast<size_t>(p.H) * D;
  float dS[RPT];
  for (int m = 0; m < RPT; ++m) {
    const int r = rg + m * RG;
    dS[m] = dS_final ? dS_final[(static_cast<size_t>(n) * p.H + h) * SZ + static_cast<size_t>(r) * D + j0 + j] : 0.f;
  }
  const int L = t.cu[n + 1] - t.cu[n];
  const int nb = (L + kBlk - 1) / kBlk;
  const int blk0 = t.chunk0[n] * kBlocksPerChunk;
  const int64_t seq0 = t.cu[n];
  float pW[TE], pK[TE], pQ[TE], pO[OE], pA[AE], pE = 0.f;
  auto fetch = [&](int jb) {
    const int blk = blk0 + jb;
    const int ntok = min(kBlk, L - jb * kBlk);
    const uint8_t* rec = recs + (static_cast<size_t>(blk) * p.H + h) * R.bytes;
    const float* gW = reinterpret_cast<const float*>(rec + R.W);
    const float* gKt = reinterpret_cast<const float*>(rec + R.Kt);
    const float* gQp = reinterpret_cast<const float*>(rec + R.Qp);
    const float* gAqk = reinterpret_cast<const float*>(rec + R.Aqk);
    const float* geG = reinterpret_cast<const float*>(rec + R.eGC);
    for (int m = 0; m < TE; ++m) {
      const int e = tid + m * kBT;
      if (e < kBlk * D) { pW[m] = gW[e]; pK[m] = gKt[e]; pQ[m] = gQp[e]; }
    }
    for (int m = 0; m < AE; ++m) {
      const int e = tid + m * kBT;
      if (e < kBlk * kBlk) pA[m] = gAqk[e];
    }
    for (int m = 0; m < OE; ++m) {
      const int e = tid + m * kBT;
      const int q = e / VT, jj = e % VT;
      if (e < kBlk * VT)
        pO[m] = q < ntok ? ld<DO_BF16>(dO, (static_cast<size_t>(seq0 + jb * kBlk + q) * p.H + h) * D + j0 + jj) : 0.f;
    }
    if (tid < D) pE = geG[tid];
  };
  if (nb > 0) fetch(nb - 1);
  for (int jb = nb - 1; jb >= 0; --jb) {
    const size_t bh = static_cast<size_t>(blk0 + jb) * p.H + h;
    for (int m = 0; m < TE; ++m) {
      const int e = tid + m * kBT;
      if (e < kBlk * D) { sW[e / D][e % D] = pW[m]; sKt[e / D][e % D] = pK[m]; sQp[e / D][e % D] = pQ[m]; }
    }
    for (int m = 0; m < AE; ++m) {
      const int e = tid + m * kBT;
      if (e < kBlk * kBlk) sAqk[e / kBlk][e % kBlk] = pA[m];
    }
    for (int m = 0; m < OE; ++m) {
      const int e = tid + m * kBT;
      if (e < kBlk * VT) sdO[e / VT][e % VT] = pO[m];
    }
    if (tid < D) seG[tid] = pE;
    // the adjoint of the block's end state
    for (int m = 0; m < RPT; ++m) {
      const int r = rg + m * RG;
      dSblk[bh * SZ + static_cast<size_t>(r) * D + j0 + j] = dS[m];
    }
    __syncthreads();
    if (jb > 0) fetch(jb - 1);
    // dDelta = Aqk^T dO + K~ dS_C
    float acc[kBlk];
    for (int q = 0; q < kBlk; ++q) acc[q] = 0.f;
    for (int m = 0; m < RPT; ++m) {
      const int r = rg + m * RG;
      for (int q = 0; q < kBlk; ++q) acc[q] += sKt[q][r] * dS[m];
    }
    for (int q = 0; q < kBlk; ++q) red[rg][q][j] = acc[q];
    __syncthreads();
    for (int e = tid; e < kBlk * VT; e += kBT) {
      const int q = e / VT, jj = e % VT;
      float sum = 0.f;
      for (int g2 = 0; g2 < RG; ++g2) sum += red[g2][q][jj];
      for (int r2 = q; r2 < kBlk; ++r2) sum += sAqk[r2][q] * sdO[r2][jj];
      sdDel[q][jj] = sum;
      dDblk[bh * kBlk * D + static_cast<size_t>(q) * D + j0 + jj] = sum;
    }
    __syncthreads();
    // dS0 = Q+^T dO + e^{G_C} dS_C - W^T dDelta
    for (int m = 0; m < RPT; ++m) {
      const int r = rg + m * RG;
      float v = seG[r] * dS[m];
      for (int q = 0; q < kBlk; ++q) v += sQp[q][r] * sdO[q][j] - sW[q][r] * sdDel[q][j];
      dS[m] = v;
    }
    __syncthreads();
  }
  if (dS_init) {
    for (int m = 0; m < RPT; ++m) {
      const int r = rg + m * RG;
      dS_init[(static_cast<size_t>(n) * p.H + h) * SZ + static_cast<size_t>(r) * D + j0 + j] = dS[m];
    }
  }
  // an empty sequence passes its conv history through: no gradient reaches it
  if (dconv && tile == 0 && nb == 0) {
    for (int e = tid; e < 3 * D; e += kBT) {
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
  constexpr int SC = 16;                  // state columns staged at a time
  __shared__ BlockSmem<D> s;
  __shared__ float sDel[kBlk][D], sdDel[kBlk][D], sdO[kBlk][D];
  __shared__ float sdQp[kBlk][D], sdKp[kBlk][D], sdKm[kBlk][D], sdKt[kBlk][D];
  __shared__ float sX[kBlk][D];           // dW, then dXw
  __shared__ float sT[kBlk][kBlk], sAun[kBlk][kBlk], sdA[kBlk][kBlk], sdAqk[kBlk][kBlk];
  __shared__ float sdbeta[kBlk], sdGC[D];
  __shared__ float sStage[2 * D * (SC + 1)];     // S0 / dS_C column slabs, then W and U
  float (*sS0)[SC + 1] = reinterpret_cast<float (*)[SC + 1]>(sStage);
  float (*sdSC)[SC + 1] = reinterpret_cast<float (*)[SC + 1]>(sStage + D * (SC + 1));
  float (*sWt)[D] = reinterpret_cast<float (*)[D]>(sStage);
  float (*sUt)[D] = reinterpret_cast<float (*)[D]>(sStage + kBlk * D);
  static_assert(2 * kBlk * D <= 2 * D * (SC + 1), "W and U fit where the slabs were");
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
  block_preprocess<D, IO_BF16, NT>(p, io, b, h, s);
  const size_t bh = static_cast<size_t>(blk) * p.H + h;
  const uint8_t* rec = recs + bh * R.bytes;
  const float* gW = reinterpret_cast<const float*>(rec + R.W);
  const float* gU = reinterpret_cast<const float*>(rec + R.U);
  const float* gT = reinterpret_cast<const float*>(rec + R.T);
  const float* geG = reinterpret_cast<const float*>(rec + R.eGC);
  const float* S0 = Sblk + bh * D * D;
  const float* dSC = dSblk + bh * D * D;
  for (int e = tid; e < kBlk * D; e += NT) {
    const int r = e / D, c = e % D;
    sDel[r][c] = Dblk[bh * kBlk * D + e];
    sdDel[r][c] = dDblk[bh * kBlk * D + e];
    sdO[r][c] = r < b.ntok ? ld<DO_BF16>(dO, (static_cast<size_t>(b.tok0 + r) * p.H + h) * D + c) : 0.f;
  }
  for (int e = tid; e < kBlk * kBlk; e += NT) sT[e / kBlk][e % kBlk] = gT[e];
  __syncthreads();

  // ---- products with S0 and dS_C, staged SC state columns at a time:
  //   dQ+ = dO S0^T, dW = -dDelta S0^T, dK~ = Delta dS_C^T, dG_C = e^{G_C} rowsum(dS_C * S0)
  {
    constexpr int RPT = kBlk * D / NT;   // outputs per thread: channel c, rows s0 .. s0 + RPT - 1
    const int c = tid % D, s0 = (tid / D) * RPT;
    float aQ[RPT], aW[RPT], aK[RPT];
    for (int m = 0; m < RPT; ++m) { aQ[m] = 0.f; aW[m] = 0.f; aK[m] = 0.f; }
    float gc = 0.f;
    for (int j0 = 0; j0 < D; j0 += SC) {
      for (int e = tid; e < D * SC; e += NT) {
        const int r = e / SC, jj = e % SC;
        sS0[r][jj] = S0[static_cast<size_t>(r) * D + j0 + jj];
        sdSC[r][jj] = dSC[static_cast<size_t>(r) * D + j0 + jj];
      }
      __syncthreads();
      for (int jj = 0; jj < SC; ++jj) {
        const float s0v = sS0[c][jj], dsv = sdSC[c][jj];
        if (tid < D) gc += s0v * dsv;
        for (int m = 0; m < RPT; ++m) {
          aQ[m] += sdO[s0 + m][j0 + jj] * s0v;
          aW[m] -= sdDel[s0 + m][j0 + jj] * s0v;
          aK[m] += sDel[s0 + m][j0 + jj] * dsv;
        }
      }
      __syncthreads();
    }
    for (int m = 0; m < RPT; ++m) {
      sdQp[s0 + m][c] = aQ[m];
      sX[s0 + m][c] = aW[m];
      sdKt[s0 + m][c] = aK[m];
    }
    if (tid < D) sdGC[c] = geG[c] * gc;
  }
  __syncthreads();
  // ---- dXw = T^T dW (in place through registers), dXu = T^T dDelta (into sdKm as scratch for now: no)
  {
    constexpr int RPT = kBlk * D / NT;
    const int c = tid % D, s0 = (tid / D) * RPT;
    float xw[RPT], xu[RPT];
    for (int m = 0; m < RPT; ++m) {
      float aw = 0.f, au = 0.f;
      const int mm = s0 + m;
      for (int r = mm; r < kBlk; ++r) {
        aw += sT[r][mm] * sX[r][c];
        au += sT[r][mm] * sdDel[r][c];
      }
      xw[m] = aw;
      xu[m] = au;
    }
    __syncthreads();
    for (int m = 0; m < RPT; ++m) {
      sX[s0 + m][c] = xw[m];
      sdKm[s0 + m][c] = xu[m];    // dXu parked in sdKm until dV is formed
    }
  }
  __syncthreads();
  // ---- dA = -strict_lower(dXw W^T + dXu U^T);  A_un = K+ K-^T;  dAqk = lower(dO Delta^T)
  for (int e = tid; e < kBlk * D; e += NT) {
    sWt[e / D][e % D] = gW[e];
    sUt[e / D][e % D] = gU[e];
  }
  __syncthreads();
  if (tid < kBlk * kBlk) {
    const int r = tid / kBlk, i = tid % kBlk;
    float da = 0.f, aun = 0.f, daq = 0.f;
    if (i < r) {
      for (int c = 0; c < D; ++c) {
        da -= sX[r][c] * sWt[i][c] + sdKm[r][c] * sUt[i][c];
        aun += s.k[r][c] * s.eP[r][c] * (s.k[i][c] * s.eM[i][c]);
      }
    }
    if (i <= r)
      for (int c = 0; c < D; ++c) daq += sdO[r][c] * sDel[i][c];
    sdA[r][i] = da;
    sAun[r][i] = aun;
    sdAqk[r][i] = daq;
  }
  __syncthreads();
  // ---- dbeta; dV; dK+ and dK- from X and A; dQ+ and dK- from Aqk
  if (tid < kBlk) {
    const int r = tid;
    float d = 0.f;
    for (int c = 0; c < D; ++c) d += sX[r][c] * s.k[r][c] * s.eP[r][c] + sdKm[r][c] * s.v[r][c];
    for (int i = 0; i < r; ++i) d += sdA[r][i] * sAun[r][i];
    sdbeta[r] = d;
  }
  {
    constexpr int RPT = kBlk * D / NT;
    const int c = tid % D, s0 = (tid / D) * RPT;
    float dKp[RPT], dKm[RPT], dQp[RPT], dV[RPT], gnp[RPT];
    for (int m = 0; m < RPT; ++m) {
      const int r = s0 + m;
      const float be = s.beta[r];
      float kp = be * sX[r][c];                 // Diag(beta) dXw
      float km = 0.f, qp = sdQp[r][c];
      // the decay's gradient through the single-token terms, dO S0^T on Q+ and
      // beta dXw on K+ (the pair terms of A and Aqk are summed separately)
      gnp[m] = qp * s.q[r][c] * s.eP[r][c] + kp * s.k[r][c] * s.eP[r][c];
      for (int i = 0; i < r; ++i) kp += be * sdA[r][i] * s.k[i][c] * s.eM[i][c];            // (beta dA) K-
      for (int r2 = r + 1; r2 < kBlk; ++r2)
        km += s.beta[r2] * sdA[r2][r] * s.k[r2][c] * s.eP[r2][c];                            // (beta dA)^T K+
      for (int i = 0; i <= r; ++i) qp += sdAqk[r][i] * s.k[i][c] * s.eM[i][c];              // dAqk K-
      for (int r2 = r; r2 < kBlk; ++r2) km += sdAqk[r2][r] * s.q[r2][c] * s.eP[r2][c];      // dAqk^T Q+
      dKp[m] = kp;
      dKm[m] = km;
      dQp[m] = qp;
      dV[m] = be * sdKm[r][c];
    }
    __syncthreads();
    for (int m = 0; m < RPT; ++m) {
      const int r = s0 + m;
      sdKp[r][c] = dKp[m];
      sdKm[r][c] = dKm[m];
      sdQp[r][c] = dQp[m];
      sX[r][c] = dV[m];                         // sX now holds dV
      sDel[r][c] = gnp[m];                      // Delta is no longer needed
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
  if (tid < D) {
    const int c = tid;
    float dG[kBlk], dGs[kBlk], P[kBlk];
    for (int r = 0; r < kBlk; ++r) {
      const float eP = s.eP[r][c], eM = s.eM[r][c], eS = s.eS[r][c];
      const float k = s.k[r][c];
      const float dqp = sdQp[r][c], dkp = sdKp[r][c], dkm = sdKm[r][c], dkt = sdKt[r][c];
      dG[r] = sDel[r][c];
      dGs[r] = dkt * k * eS;
      P[r] = 0.f;
      sdQp[r][c] = dqp * eP;                          // d q^
      sdKp[r][c] = dkp * eP + dkm * eM + dkt * eS;    // d k^
    }
    for (int r = 1; r < kBlk; ++r) {
      const float ar = s.beta[r] * s.k[r][c] * s.eP[r][c], br = s.q[r][c] * s.eP[r][c];
      float rp = 0.f;
      for (int t2 = 1; t2 <= r; ++t2) {
        const int i = t2 - 1;
        rp += (sdA[r][i] * ar + sdAqk[r][i] * br) * (s.k[i][c] * s.eM[i][c]);
        P[t2] += rp;
      }
    }
    // dg_t = sum_{r >= t} dG_r + sum_{r < t} dGs_r + dG_C + P_t, for the block's tokens
    const float gc = sdGC[c];
    float suffix = 0.f;
    for (int r = kBlk - 1; r >= 0; --r) {
      suffix += dG[r];
      dG[r] = suffix;
    }
    float prefix = 0.f;
    for (int r = 0; r < kBlk; ++r) {
      sdKm[r][c] = r < b.ntok ? dG[r] + prefix + gc + P[r] : 0.f;   // dg
      prefix += dGs[r];
    }
  }
  __syncthreads();
  // ---- the preprocess in reverse
  // gate: d alpha, and the block's partial sums for d dt_bias and d A_log
  {
    const float a_exp = expf(p.A_log[h]);
    float alog_part = 0.f;
    if (tid < D) {
      const int c = tid;
      const size_t col = static_cast<size_t>(h) * D + c;
      const float dtb = p.dt_bias[col];
      float dtb_part = 0.f;
      for (int r = 0; r < b.ntok; ++r) {
        const float al = ld<IO_BF16>(io.alpha, static_cast<size_t>(b.tok0 + r) * HD + col);
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
    // d A_log: sum over the block's channels (waves 0 and 1 hold them for D = 128)
    __shared__ float sAl[NT / kWave];
    const float wsum = group_sum<kWave>(alog_part);
    if (tid % kWave == 0) sAl[tid / kWave] = wsum;
    __syncthreads();
    if (tid == 0) {
      float tot = 0.f;
      for (int w = 0; w < NT / kWave; ++w) tot += sAl[w];
      pAlog[bh] = tot;
    }
  }
  // beta
  if (tid < b.ntok) {
    const float bb = ld<IO_BF16>(io.b, static_cast<size_t>(b.tok0 + tid) * p.H + h);
    const float sg = sigmoidf_(bb);
    float dbv = sdbeta[tid] * sg * (1.f - sg);
    if (p.flags & KDA_FLAG_BETA_X2) dbv *= 2.f;
    db[static_cast<size_t>(b.tok0 + tid) * p.H + h] = dbv;
  }
  // L2 norm (q with its scale, k): du = (s / n) (dq^ - q^ (q^ . dq^) / s^2)
  __shared__ float sDot[2][kBlk];
  if (tid < 2 * kBlk * 8) {
    const int row = tid / 8, l8 = tid % 8;
    const bool isq = row < kBlk;
    const int r = isq ? row : row - kBlk;
    float dot = 0.f;
    for (int c = l8; c < D; c += 8) dot += isq ? s.q[r][c] * sdQp[r][c] : s.k[r][c] * sdKp[r][c];
    dot += __shfl_xor(dot, 1, 8);
    dot += __shfl_xor(dot, 2, 8);
    dot += __shfl_xor(dot, 4, 8);
    if (l8 == 0) sDot[isq ? 0 : 1][r] = dot;
  }
  __syncthreads();
  // SiLU: dy = du sigmoid(y) (1 + y (1 - sigmoid(y))), with y recomputed from the raw window
  for (int task = tid; task < 3 * D; task += NT) {
    const int role = task / D, ch = task % D;
    const size_t col = static_cast<size_t>(h) * D + ch;
    const void* xin = role == 0 ? io.q : (role == 1 ? io.k : io.v);
    const void* w = role == 0 ? p.wq : (role == 1 ? p.wk : p.wv);
    const float w0 = ld<IO_BF16>(w, col * 4), w1 = ld<IO_BF16>(w, col * 4 + 1);
    const float w2 = ld<IO_BF16>(w, col * 4 + 2), w3 = ld<IO_BF16>(w, col * 4 + 3);
    const int64_t seq0 = b.tok0 - b.tau0;
    float win[3];
    for (int m = 0; m < 3; ++m) {
      const int tau = b.tau0 - 3 + m;
      if (tau >= 0) win[m] = ld<IO_BF16>(xin, static_cast<size_t>(seq0 + tau) * HD + col);
      else if (io.conv_in) win[m] = ld<IO_BF16>(io.conv_in, (static_cast<size_t>(b.seq) * 3 + (3 + tau)) * 3 * HD + role * HD + col);
      else win[m] = 0.f;
    }
    for (int r = 0; r < b.ntok; ++r) {
      const float xt = ld<IO_BF16>(xin, static_cast<size_t>(b.tok0 + r) * HD + col);
      const float y = w0 * win[0] + w1 * win[1] + w2 * win[2] + w3 * xt;
      win[0] = win[1]; win[1] = win[2]; win[2] = xt;
      float du;
      if (role == 0) {
        const float sc = p.scale, n = s.nq[r];
        du = sc / n * (sdQp[r][ch] - s.q[r][ch] * sDot[0][r] / (sc * sc));
      } else if (role == 1) {
        const float n = s.nk[r];
        du = (sdKp[r][ch] - s.k[r][ch] * sDot[1][r]) / n;
      } else {
        du = sX[r][ch];            // dV
      }
      const float sg = sigmoidf_(y);
      dy[static_cast<size_t>(b.tok0 + r) * 3 * HD + role * HD + col] = du * sg * (1.f + y * (1.f - sg));
    }
  }
}

// ---------------------------------------------------------------- conv reverse
// One workgroup per (64-token chunk, head); a thread per (q/k/v, channel)
// walks the chunk's tokens: dx_t = sum_j w[j] dy_{t+3-j} over tokens of the
// same sequence, the history's gradient for the sequence's first chunk, and
// the chunk's partial d w[j] = sum_t dy_t x_{t-3+j}.
template <int D, bool IO_BF16>
__global__ __launch_bounds__(3 * D) void bwd_conv_kernel(Params p, ChunkTable t, PrefillIO io, const float* dy,
                                                          float* dq, float* dk, float* dv, float* dconv,
                                                          float* pdw) {
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
  float wj[4];
  for (int j = 0; j < 4; ++j) wj[j] = ld<IO_BF16>(w, col * 4 + j);
  auto dyat = [&](int tau) {   // dy of sequence position tau, 0 outside the sequence
    return (tau >= 0 && tau < L) ? dy[static_cast<size_t>(seq0 + tau) * 3 * HD + role * HD + col] : 0.f;
  };
  auto xat = [&](int tau) {    // raw input at sequence position tau (the history before 0)
    if (tau >= 0) return ld<IO_BF16>(xin, static_cast<size_t>(seq0 + tau) * HD + col);
    if (io.conv_in) return ld<IO_BF16>(io.conv_in, (static_cast<size_t>(seq) * 3 + (3 + tau)) * 3 * HD + role * HD + col);
    return 0.f;
  };
  // the chunk's window, loaded before any arithmetic: x at positions
  // tau0 - 3 .. tau0 + 63 and dy at tau0 .. tau0 + 66 (zeros outside)
  constexpr int WN = kChunk + 3;
  float xs[WN], dys[WN];
#pragma unroll
  for (int m = 0; m < WN; ++m) {
    xs[m] = (m - 3 < cnt) ? xat(tau0 - 3 + m) : 0.f;
    dys[m] = dyat(tau0 + m);
  }
  float aw[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < kChunk; ++r) {
    if (r < cnt) {
      float g = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) g += wj[j] * dys[r + 3 - j];
      dx[static_cast<size_t>(seq0 + tau0 + r) * HD + col] = g;
#pragma unroll
      for (int j = 0; j < 4; ++j) aw[j] += dys[r] * xs[r + j];
    }
  }
  for (int j = 0; j < 4; ++j) pw[j] = aw[j];
  if (tau0 == 0 && dconv) {
    // history slot m holds position m - 3: dx_{m-3} = sum_j w[j] dy_{m-j}
    for (int m = 0; m < 3; ++m) {
      float g = 0.f;
      for (int j = 0; j <= m; ++j) g += wj[j] * dys[m - j];
      dconv[(static_cast<size_t>(seq) * 3 + m) * 3 * HD + role * HD + col] = g;
    }
  }
}

// ---------------------------------------------------------------- parameter sums
// One thread per parameter gradient element, summing the partials of every
// chunk (conv weights) or block (dt_bias, A_log) in order.
__global__ void bwd_param_reduce_kernel(int H, int D, ChunkTable t, const float* pdw, const float* pdtb,
                                        const float* pAlog, float* dw_q, float* dw_k, float* dw_v, float* ddt_bias,
                                        float* dA_log) {
  const int64_t HD = static_cast<int64_t>(H) * D;
  const int64_t n_w = 3 * HD * 4, n_dtb = HD, n_al = H;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int nchunks = t.chunk0[t.N];
  const int nblocks = nchunks * kBlocksPerChunk;
  if (e < n_w) {
    float acc = 0.f;
    for (int c = 0; c < nchunks; ++c) acc += pdw[static_cast<size_t>(c) * n_w + e];
    const int64_t role = e / (HD * 4), rest = e % (HD * 4);
    float* dst = role == 0 ? dw_q : (role == 1 ? dw_k : dw_v);
    dst[rest] = acc;
  } else if (e < n_w + n_dtb) {
    const int64_t i = e - n_w;
    float acc = 0.f;
    for (int bk = 0; bk < nblocks; ++bk) acc += pdtb[static_cast<size_t>(bk) * HD + i];
    ddt_bias[i] = acc;
  } else if (e < n_w + n_dtb + n_al) {
    const int64_t i = e - n_w - n_dtb;
    float acc = 0.f;
    for (int bk = 0; bk < nblocks; ++bk) acc += pAlog[static_cast<size_t>(bk) * H + i];
    dA_log[i] = acc;
  }
}

// ---------------------------------------------------------------- launchers
namespace {

template <int D>
constexpr int scan_tile() { return D >= 32 ? 32 : D; }

template <int D, bool IO_BF16, bool DO_BF16>
hipError_t launch_backward_d(const Params& p, const ChunkTable& t, const PrefillIO& io, const BackwardIO& g,
                             const BackwardWS& ws, int N, int max_chunks, hipStream_t st) {
  constexpr int VT = scan_tile<D>();
  const unsigned nblk = static_cast<unsigned>(max_chunks) * kBlocksPerChunk * static_cast<unsigned>(p.H);
  bwd_block_prep_kernel<D, IO_BF16><<<nblk, kBT, 0, st>>>(p, t, io, ws.recs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned nscan = static_cast<unsigned>(N) * p.H * (D / VT);
  bwd_state_scan_kernel<D, VT><<<nscan, kBT, 0, st>>>(p, t, io.S0, ws.recs, ws.Sblk, ws.Dblk);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  bwd_adjoint_scan_kernel<D, VT, DO_BF16><<<nscan, kBT, 0, st>>>(p, t, ws.recs, g.dO, g.dS_final, ws.dSblk, ws.dDblk,
                                                                 g.dS_init, g.dconv);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  bwd_block_grad_kernel<D, IO_BF16, DO_BF16><<<nblk, grad_threads<D>(), 0, st>>>(p, t, io, ws.recs, ws.Sblk, ws.dSblk, ws.Dblk,
                                                                   ws.dDblk, g.dO, ws.dy, g.dalpha, g.db, ws.pdtb,
                                                                   ws.pAlog);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  bwd_conv_kernel<D, IO_BF16><<<static_cast<unsigned>(max_chunks) * p.H, 3 * D, 0, st>>>(p, t, io, ws.dy, g.dq, g.dk,
                                                                                       g.dv, g.dconv, ws.pdw);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t n_out = static_cast<int64_t>(p.H) * D * (3 * 4 + 1) + p.H;
  bwd_param_reduce_kernel<<<static_cast<unsigned>((n_out + 255) / 256), 256, 0, st>>>(
      p.H, D, t, ws.pdw, ws.pdtb, ws.pAlog, g.dw_q, g.dw_k, g.dw_v, g.ddt_bias, g.dA_log);
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
