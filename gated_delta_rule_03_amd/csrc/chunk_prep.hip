// Chunk preparation of the chunked KDA prefill: everything that does not
// depend on the recurrent state, for one (chunk of 64 tokens, head) per
// workgroup, fully parallel over the batch.
//
// 1. Preprocess (AliceAI page, section 二; safe gate from the Ling-3.0-flash-VL
//    page, section "KDA 层的安全门"): a lane owns one channel of one input
//    (q, k, v or alpha) and slides the 4-tap causal conv window down the
//    chunk (the three earlier inputs come from the same sequence or from the
//    incoming conv history), then SiLU; q and k are L2-normalised per token;
//    g = max(-e^{A_log} softplus(alpha + dt_bias), lb); beta = sigmoid(b).
//    Rows past a partial chunk's end are zero with g = beta = 0, an exact
//    identity step of the recurrence.
// 2. Chunked form (derived by unrolling the pages' token loop over the chunk;
//    G_r = sum_{i<=r} g_i per key channel):
//      A[r,i]   = beta_r sum_c k_r k_i e^{G_r - G_i}   (i < r)
//      Aqk[r,i] =        sum_c q_r k_i e^{G_r - G_i}   (i <= r)
//      W = (I + A)^-1 Diag(beta)(K * e^G),  U = (I + A)^-1 Diag(beta) V
//      Q+ = Q * e^G,  K~ = K * e^{G_C - G},  e^{G_C}
//    A and Aqk are 16x16 sub-block products on the matrix cores (bf16 pieces,
//    see mfma.h: two for bf16 inputs, three for fp32 inputs).  A sub-block
//    pair (rows in block R, columns in block I <= R) uses the reference point
//    "end of block I-1": row factor e^{G_r - ref} <= 1 and column factor
//    e^{ref - G_i} = e^{-P_i} <= e^{80} (P = in-block prefix sum, each
//    g >= -5), both finite in fp32; every exponent is a short sum.
//    W and U solve (I + A) X = [beta K+ | beta V] block-row by block-row on
//    the matrix cores: X_R = T_R (B_R - A_{R,<R} X_{<R}) with T_R the inverse
//    of the unit lower-triangular 16x16 diagonal block (I + A_RR), found by a
//    short fp32 substitution.
// The results are written as one Record per (chunk, head).
//
// Eight waves: lane t has role t / D (q, k, v, alpha) and channel t % D, so
// every conv task is one lane's, and each SIMD interleaves two waves.
#include "kda_device.h"
#include "kda_internal.h"
#include "mfma.h"

namespace kda {

namespace {

constexpr int kPrepThreads = 512;

__device__ __forceinline__ int pair_index(int I, int R) {
  // (I, R) with I < R: (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
  return I == 0 ? R - 1 : (I == 1 ? R + 1 : 5);
}

}  // namespace

template <int D, bool IO_BF16>
__global__ __launch_bounds__(kPrepThreads) void chunk_prep_kernel(Params p, ChunkTable t, PrefillIO io,
                                                                  uint8_t* records) {
  constexpr int NT = kPrepThreads;
  constexpr int LDR = D + 4;                       // LDS row stride of the fp32 tiles
  constexpr int KP = D < 32 ? 32 : D;              // channel extent in whole 32-wide steps
  constexpr int LA = 68;                           // row stride of A in LDS (16-byte rows)
  constexpr int GSZ = (64 * LDR > 64 * LA) ? 64 * LDR : 64 * LA;
  constexpr int NP = IO_BF16 ? 2 : 3;              // bf16 pieces per operand
  constexpr Record REC = record_layout(D, NP);
  constexpr int LX = kChunk + 4;                   // row stride of X^T in LDS
  static_assert(2 * D * LX <= 3 * 64 * LDR, "X^T must fit where q, k and k e^{-P} were");
  __shared__ __align__(16) float sBig[3 * 64 * LDR];
  float* sQ = sBig;                                // q, then q e^{P}        (A row operand)
  float* sK = sBig + 64 * LDR;                     // k, then k e^{P}        (A row operand)
  float* sC = sBig + 2 * 64 * LDR;                 // k e^{-P}               (A column operand)
  float* sX = sBig;                                // then X^T [2D][LX], the solve's columns
  __shared__ __align__(16) float sG[GSZ];          // g, then A
  __shared__ __align__(16) float sT[4][16][20];    // inverses of the diagonal blocks of I + A
  __shared__ __align__(16) float sE[6][D];         // e^{sum of block totals between I and R}
  __shared__ float sBeta[64];

  // head-fastest order: the resident workgroups cover every head of a few
  // chunks, so each raw token row is read whole while it is open in DRAM
  // one-dimensional grid, head fastest (grid dimension y holds at most 65536)
  const int h = static_cast<int>(blockIdx.x % static_cast<unsigned>(p.H));
  const int c = static_cast<int>(blockIdx.x / static_cast<unsigned>(p.H));
  if (c >= t.chunk0[t.N]) return;
  const int H = p.H;
  const int s = t.chunk_seq[c];
  const int tau0 = t.s0 + (c - t.chunk0[s]) * kChunk;
  const int64_t tok0 = static_cast<int64_t>(t.cu[s]) + tau0;
  const int len = min(kChunk, t.cu[s + 1] - static_cast<int>(tok0));
  const int tid = threadIdx.x;
  const int role = tid / D, ch = tid % D;          // role 0 q, 1 k, 2 v, 3 alpha (4+ idle)
  const size_t HD = static_cast<size_t>(H) * D;
  const size_t Ctot = 3 * HD;
  const size_t col = static_cast<size_t>(h) * D + ch;
  const uint32_t flags = p.flags;
  uint8_t* rec = records + (static_cast<size_t>(c) * H + h) * REC.bytes;

  // ---- 1. conv + SiLU (q, k, v) or gate (alpha): one channel per lane
  float x[kChunk];   // v lanes: v, then beta v;  k lanes: beta K+  (columns of the solve)
  if (role < 3) {
    const void* xin = role == 0 ? io.q : (role == 1 ? io.k : io.v);
    const void* w = role == 0 ? p.wq : (role == 1 ? p.wk : p.wv);
    const float w0 = ld<IO_BF16>(w, col * 4), w1 = ld<IO_BF16>(w, col * 4 + 1);
    const float w2 = ld<IO_BF16>(w, col * 4 + 2), w3 = ld<IO_BF16>(w, col * 4 + 3);
    float hm[3];
#pragma unroll
    for (int m = 0; m < 3; ++m) {
      const int tau = tau0 - 3 + m;
      if (tau >= 0) hm[m] = ld<IO_BF16>(xin, static_cast<size_t>(t.cu[s] + tau) * HD + col);
      else if (io.conv_in) hm[m] = ld<IO_BF16>(io.conv_in, (static_cast<size_t>(s) * 3 + (3 + tau)) * Ctot + role * HD + col);
      else hm[m] = 0.f;
    }
#pragma unroll
    for (int r = 0; r < kChunk; ++r)   // rows past the chunk's end re-read its last row (no branch)
      x[r] = ld<IO_BF16>(xin, static_cast<size_t>(tok0 + min(r, len - 1)) * HD + col);
    // the conv of every row is independent once its inputs are loaded; no
    // branch inside the row loops, so rows overlap in the pipeline
    const bool raw = flags & KDA_FLAG_SKIP_CONV;
    auto conv_row = [&](int r) {
      const float xm3 = r >= 3 ? x[r - 3] : hm[r], xm2 = r >= 2 ? x[r - 2] : hm[r + 1];
      const float xm1 = r >= 1 ? x[r - 1] : hm[2], xt = x[r];
      const float u = raw ? xt : siluf_(w0 * xm3 + w1 * xm2 + w2 * xm1 + w3 * xt);
      return r < len ? u : 0.f;
    };
    if (role < 2) {
      float* dst = role == 0 ? sQ : sK;
#pragma unroll
      for (int r = 0; r < kChunk; ++r) dst[r * LDR + ch] = conv_row(r);
    } else {
      float u[kChunk];
#pragma unroll
      for (int r = 0; r < kChunk; ++r) u[r] = conv_row(r);
#pragma unroll
      for (int r = 0; r < kChunk; ++r) x[r] = u[r];
    }
  } else if (role == 3) {
    const float a_exp = expf(p.A_log[h]);
    const float dtb = p.dt_bias[col];
    float ar[kChunk];
#pragma unroll
    for (int r = 0; r < kChunk; ++r) ar[r] = ld<IO_BF16>(io.alpha, static_cast<size_t>(tok0 + min(r, len - 1)) * HD + col);
#pragma unroll
    for (int r = 0; r < kChunk; ++r) {
      const float g = (flags & KDA_FLAG_RAW_GATE) ? ar[r] : gate_value(ar[r], dtb, a_exp, p.lower_bound);
      sG[r * LDR + ch] = r < len ? g : 0.f;
    }
  }
  if (tid < kChunk) {
    float be = 0.f;
    if (tid < len) {
      const float bb = ld<IO_BF16>(io.b, static_cast<size_t>(tok0 + tid) * H + h);
      be = (flags & KDA_FLAG_RAW_BETA) ? bb : sigmoidf_(bb);
      if (flags & KDA_FLAG_BETA_X2) be *= 2.0f;
    }
    sBeta[tid] = be;
  }
  __syncthreads();

  // ---- L2 norms of q and k: eight lanes per token
  {
    constexpr int CPP = D / 8;
    const int r = tid >> 3, part = tid & 7;
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int i = 0; i < CPP; ++i) {
      const float a = sQ[r * LDR + part * CPP + i], b = sK[r * LDR + part * CPP + i];
      sq += a * a;
      sk += b * b;
    }
    sq = group_sum<8>(sq);
    sk = group_sum<8>(sk);
    const bool norm = !(flags & KDA_FLAG_SKIP_L2NORM);
    const float iq = (norm ? 1.0f / sqrtf(sq + p.eps) : 1.0f) * p.scale;
    const float ik = norm ? 1.0f / sqrtf(sk + p.eps) : 1.0f;
#pragma unroll
    for (int i = 0; i < CPP; ++i) {
      sQ[r * LDR + part * CPP + i] *= iq;
      sK[r * LDR + part * CPP + i] *= ik;
    }
  }
  __syncthreads();

  // ---- 2a. per-channel decays: q lanes and k lanes each rebuild the
  //      in-block prefix sums P of their channel from g; e^{G_r} is formed as
  //      e^{P_r} times the earlier block factors (one rounding per factor)
  if (role < 2) {
    float gc[kChunk];
#pragma unroll
    for (int r = 0; r < kChunk; ++r) gc[r] = sG[r * LDR + ch];
    float Bt[4], eBt[4];
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      float sum = 0.f;
#pragma unroll
      for (int m = 0; m < kSub; ++m) sum += gc[J * kSub + m];
      Bt[J] = sum;
      eBt[J] = exp_precise(sum);
    }
    if (role == 0) {
      __bf16* Qp = reinterpret_cast<__bf16*>(rec + REC.Qp);
      float eBefore = 1.f;
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        float P = 0.f;
#pragma unroll
        for (int m = 0; m < kSub; ++m) {
          const int r = J * kSub + m;
          P += gc[r];
          const float eP = exp_precise(P);
          const float qv = sQ[r * LDR + ch];
          sQ[r * LDR + ch] = qv * eP;
          __bf16 pc[NP];
          split_pieces<NP>(qv * (eP * eBefore), pc);
#pragma unroll
          for (int k = 0; k < NP; ++k) Qp[k * (REC.tile_plane / 2) + frag_index(r, ch, KP)] = pc[k];
        }
        eBefore *= eBt[J];
      }
    } else {
      // K~^T row of this channel first, from the still unscaled k:
      // k e^{Q_r + later block totals}, Q_r = in-block sum of g after token r;
      // built backwards
      // (8 tokens per 16-byte store of each piece plane)
      bf16x8* KT = reinterpret_cast<bf16x8*>(rec + REC.KT);
      {
        float after = 0.f, Qs = 0.f, tmp[8];
#pragma unroll
        for (int r = kChunk - 1; r >= 0; --r) {
          if (r % kSub == kSub - 1) {
            Qs = 0.f;
            if (r < kChunk - 1) after += Bt[(r + 1) / kSub];
          }
          tmp[r % 8] = sK[r * LDR + ch] * exp_precise(Qs + after);
          Qs += gc[r];
          if (r % 8 == 0) {
            const SplitN<NP> sp = splitN<NP>(tmp);
#pragma unroll
            for (int k = 0; k < NP; ++k) KT[k * (REC.tile_plane / 16) + frag_index(ch, r, kChunk) / 8] = sp.v[k];
          }
        }
      }
      float eBefore = 1.f;
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        float P = 0.f;
#pragma unroll
        for (int m = 0; m < kSub; ++m) {
          const int r = J * kSub + m;
          P += gc[r];
          const float eP = exp_precise(P);
          const float kv = sK[r * LDR + ch];
          sK[r * LDR + ch] = kv * eP;
          sC[r * LDR + ch] = kv * rcp_fast(eP);
          x[r] = sBeta[r] * kv * (eP * eBefore);
        }
        eBefore *= eBt[J];
      }
      reinterpret_cast<float*>(rec + REC.eGC)[ch] = eBefore;
      sE[0][ch] = eBt[0];
      sE[1][ch] = eBt[0] * eBt[1];
      sE[2][ch] = eBt[0] * eBt[1] * eBt[2];
      sE[3][ch] = eBt[1];
      sE[4][ch] = eBt[1] * eBt[2];
      sE[5][ch] = eBt[2];
    }
  } else if (role == 2) {
#pragma unroll
    for (int r = 0; r < kChunk; ++r) x[r] = sBeta[r] * x[r];
  }
  __syncthreads();

  // ---- 2b. A and Aqk, one 16x16 sub-block per task on the matrix cores
  float* sA = sG;    // [64][LA]  A (strictly lower, rows scaled by beta); g is consumed
  {
    const int wave = tid / kWave, lane = tid % kWave, ln = lane & 15, q4 = lane >> 4;
    __bf16* Aq = reinterpret_cast<__bf16*>(rec + REC.Aqk);
    for (int task = wave; task < 32; task += NT / kWave) {
      const int mat = task >> 4, R = (task >> 2) & 3, I = task & 3;
      if (I > R) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 16 * R + 4 * q4 + j, i = 16 * I + ln;
          if (mat == 0) {
            sA[r * LA + i] = 0.f;
          } else {
#pragma unroll
            for (int k = 0; k < NP; ++k) Aq[k * (REC.aqk_plane / 2) + frag_index(r, i, kChunk)] = static_cast<__bf16>(0.f);
          }
        }
        continue;
      }
      const float* rows = mat == 0 ? sK : sQ;
      const float* E = I < R ? sE[pair_index(I, R)] : nullptr;
      f32x4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < KP / 32; ++ks) {
        const int ch0 = 32 * ks + 8 * q4;
        float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, b[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (ch0 < D) {   // eight whole channels (dk >= 16 is a multiple of 8)
          const float4* ra = reinterpret_cast<const float4*>(&rows[(16 * R + ln) * LDR + ch0]);
          const float4* cb = reinterpret_cast<const float4*>(&sC[(16 * I + ln) * LDR + ch0]);
          const float4 a0 = ra[0], a1 = ra[1], b0 = cb[0], b1 = cb[1];
          a[0] = a0.x; a[1] = a0.y; a[2] = a0.z; a[3] = a0.w; a[4] = a1.x; a[5] = a1.y; a[6] = a1.z; a[7] = a1.w;
          b[0] = b0.x; b[1] = b0.y; b[2] = b0.z; b[3] = b0.w; b[4] = b1.x; b[5] = b1.y; b[6] = b1.z; b[7] = b1.w;
          if (E) {
            const float4 e0 = *reinterpret_cast<const float4*>(&E[ch0]);
            const float4 e1 = *reinterpret_cast<const float4*>(&E[ch0 + 4]);
            a[0] *= e0.x; a[1] *= e0.y; a[2] *= e0.z; a[3] *= e0.w;
            a[4] *= e1.x; a[5] *= e1.y; a[6] *= e1.z; a[7] *= e1.w;
          }
        }
        acc = mfmaN<NP>(splitN<NP>(a), splitN<NP>(b), acc);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * R + 4 * q4 + j, i = 16 * I + ln;
        if (mat == 0) {
          sA[r * LA + i] = (i < r) ? sBeta[r] * acc[j] : 0.f;
        } else {
          __bf16 pc[NP];
          split_pieces<NP>((i <= r) ? acc[j] : 0.f, pc);
#pragma unroll
          for (int k = 0; k < NP; ++k) Aq[k * (REC.aqk_plane / 2) + frag_index(r, i, kChunk)] = pc[k];
        }
      }
    }
  }
  __syncthreads();

  // ---- 2c. solve (I + A) X = B = [beta K+ | beta V] by 16-row blocks.
  //      The column owners publish B^T; wave 0 inverts the four unit
  //      lower-triangular diagonal blocks (fp32 substitution, lane = column).
  if (role == 1 || role == 2) {
    float4* xr = reinterpret_cast<float4*>(&sX[((role == 1 ? 0 : D) + ch) * LX]);
#pragma unroll
    for (int v4 = 0; v4 < kChunk / 4; ++v4) xr[v4] = make_float4(x[4 * v4], x[4 * v4 + 1], x[4 * v4 + 2], x[4 * v4 + 3]);
  }
  if (tid < 64) {
    const int R = tid >> 4, j = tid & 15;
    float tcol[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float v = (i == j) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < i; ++m) v -= sA[(16 * R + i) * LA + 16 * R + m] * tcol[m];
      tcol[i] = (i < j) ? 0.f : v;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sT[R][i][j] = tcol[i];
  }
  __syncthreads();
  {
    // wave w owns 16-column blocks w, w + 8 of X (2D columns in all); every
    // barrier below is outside the per-wave loops
    constexpr int NCB = 2 * D / 16;
    constexpr int CBPW = (NCB + NT / kWave - 1) / (NT / kWave);
    const int wave = tid / kWave, lane = tid % kWave, ln = lane & 15, q4 = lane >> 4;
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      // Y = B_R - A_{R,<R} X_{<R}, written back over B_R
#pragma unroll
      for (int bi = 0; bi < CBPW; ++bi) {
        const int cb = wave + bi * (NT / kWave);
        if (cb >= NCB) continue;
        float* xc = &sX[(16 * cb + ln) * LX];
        f32x4 acc = zero4();
#pragma unroll
        for (int ks = 0; ks < (R + 1) / 2; ++ks) {
          const int i0 = 32 * ks + 8 * q4;
          const float4 a0 = *reinterpret_cast<const float4*>(&sA[(16 * R + ln) * LA + i0]);
          const float4 a1 = *reinterpret_cast<const float4*>(&sA[(16 * R + ln) * LA + i0 + 4]);
          const float4 b0 = *reinterpret_cast<const float4*>(&xc[i0]);
          const float4 b1 = *reinterpret_cast<const float4*>(&xc[i0 + 4]);
          const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
          const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
          float a[8], xb[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const bool in = i0 + i < 16 * R;          // only the finished blocks I < R
            a[i] = in ? av[i] : 0.f;
            xb[i] = in ? bv[i] : 0.f;
          }
          acc = mfmaN<NP>(splitN<NP>(a), splitN<NP>(xb), acc);
        }
        float4* yr = reinterpret_cast<float4*>(&xc[16 * R + 4 * q4]);
        const float4 bR = *yr;
        *yr = make_float4(bR.x - acc[0], bR.y - acc[1], bR.z - acc[2], bR.w - acc[3]);
      }
      __syncthreads();
      // X_R = T_R Y  (K = 16: lanes of the upper half-wave contribute zeros)
      f32x4 xr[CBPW];
#pragma unroll
      for (int bi = 0; bi < CBPW; ++bi) {
        const int cb = wave + bi * (NT / kWave);
        if (cb >= NCB) continue;
        const float* xc = &sX[(16 * cb + ln) * LX];
        float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, yb[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (q4 < 2) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            a[i] = sT[R][ln][8 * q4 + i];
            yb[i] = xc[16 * R + 8 * q4 + i];
          }
        }
        xr[bi] = mfmaN<NP>(splitN<NP>(a), splitN<NP>(yb), zero4());
      }
      __syncthreads();
#pragma unroll
      for (int bi = 0; bi < CBPW; ++bi) {
        const int cb = wave + bi * (NT / kWave);
        if (cb >= NCB) continue;
        *reinterpret_cast<float4*>(&sX[(16 * cb + ln) * LX + 16 * R + 4 * q4]) =
            make_float4(xr[bi][0], xr[bi][1], xr[bi][2], xr[bi][3]);
      }
      __syncthreads();
    }
  }
  // W and U^T from X^T, in fragment order
  {
    __bf16* W = reinterpret_cast<__bf16*>(rec + REC.W);
    for (int e = tid; e < kChunk * D; e += NT) {
      const int r = e / D, cc = e % D;
      __bf16 pc[NP];
      split_pieces<NP>(sX[cc * LX + r], pc);
#pragma unroll
      for (int k = 0; k < NP; ++k) W[k * (REC.tile_plane / 2) + frag_index(r, cc, KP)] = pc[k];
    }
    float4* UT = reinterpret_cast<float4*>(rec + REC.UT);
    for (int e = tid; e < D * kChunk / 4; e += NT) {
      const int cc = e / (kChunk / 4), v4 = e % (kChunk / 4);
      UT[ut_index(cc, 4 * v4) / 4] = *reinterpret_cast<const float4*>(&sX[(D + cc) * LX + 4 * v4]);
    }
  }
}

template <int D>
static hipError_t launch_prep_d(const Params& p, const ChunkTable& t, const PrefillIO& io, uint8_t* records,
                                int max_chunks, bool io_bf16, hipStream_t st) {
  const int64_t blocks = static_cast<int64_t>(p.H) * max_chunks;
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(blocks));
  if (io_bf16) chunk_prep_kernel<D, true><<<grid, kPrepThreads, 0, st>>>(p, t, io, records);
  else chunk_prep_kernel<D, false><<<grid, kPrepThreads, 0, st>>>(p, t, io, records);
  return hipGetLastError();
}

hipError_t launch_chunk_prep(const Params& p, const ChunkTable& t, const PrefillIO& io, uint8_t* records,
                             int max_chunks, bool io_bf16, hipStream_t st) {
  if (chunk_prep_rows_supported(p, io, io_bf16)) return launch_chunk_prep_rows(p, t, io, records, max_chunks, st);
  switch (p.D) {
    case 16: return launch_prep_d<16>(p, t, io, records, max_chunks, io_bf16, st);
    case 32: return launch_prep_d<32>(p, t, io, records, max_chunks, io_bf16, st);
    case 64: return launch_prep_d<64>(p, t, io, records, max_chunks, io_bf16, st);
    case 128: return launch_prep_d<128>(p, t, io, records, max_chunks, io_bf16, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kda
