// Chunk preparation of the chunked KDA prefill: everything that does not
// depend on the recurrent state, for one (chunk of 64 tokens, head) per
// workgroup, fully parallel over the batch.
//
// 1. Preprocess (AliceAI page, section 二; safe gate from the Ling-3.0-flash-VL
//    page, section "KDA 层的安全门"): each lane owns a channel and slides the
//    4-tap causal conv window down the chunk (the three earlier inputs come
//    from the same sequence or from the incoming conv history), then SiLU;
//    q and k are L2-normalised per token; g = max(-e^{A_log} softplus(alpha +
//    dt_bias), lb); beta = sigmoid(b).  Rows past a partial chunk's end are
//    zero with g = beta = 0, an exact identity step of the recurrence.
// 2. Chunked form (derived by unrolling the pages' token loop over the chunk;
//    G_r = sum_{i<=r} g_i per key channel):
//      A[r,i]   = beta_r sum_c k_r k_i e^{G_r - G_i}   (i < r)
//      Aqk[r,i] =        sum_c q_r k_i e^{G_r - G_i}   (i <= r)
//      W = (I + A)^-1 Diag(beta)(K * e^G),  U = (I + A)^-1 Diag(beta) V
//      Q+ = Q * e^G,  K~ = K * e^{G_C - G},  e^{G_C}
//    A and Aqk are 16x16 sub-block products on the matrix cores (bf16 pieces,
//    see mfma.h: two for bf16 inputs, three for fp32 inputs).
//    A sub-block pair (rows in block R, columns in block I <= R) uses the
//    reference point "end of block I-1": row factor e^{G_r - ref} <= 1 and
//    column factor e^{ref - G_i} = e^{-P_i} <= e^{80} (P = in-block prefix
//    sum, each g >= -5), both finite in fp32; every exponent is a short sum.
//    W and U come from fp32 forward substitution: a lane owns one column of
//    [beta K+ | beta V] in registers and eliminates row by row against A.
// The results are written as one Record per (chunk, head).
#include "kda_device.h"
#include "kda_internal.h"
#include "mfma.h"

namespace kda {

namespace {

__device__ __forceinline__ int pair_index(int I, int R) {
  // (I, R) with I < R: (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
  return I == 0 ? R - 1 : (I == 1 ? R + 1 : 5);
}

}  // namespace

template <int D, bool IO_BF16>
__global__ __launch_bounds__(256) void chunk_prep_kernel(Params p, ChunkTable t, PrefillIO io, uint8_t* records) {
  constexpr int NT = 256;
  constexpr int LDR = D + 4;                       // LDS row stride of the fp32 tiles
  constexpr int KP = D < 32 ? 32 : D;              // channel extent in whole 32-wide steps
  constexpr int LA = 68;                           // row stride of A / Aqk in LDS (16-byte rows)
  constexpr int VSZ = (64 * LDR > 2 * 64 * LA) ? 64 * LDR : 2 * 64 * LA;
  constexpr Record REC = record_layout(D);
  constexpr int NP = IO_BF16 ? 2 : 3;              // bf16 pieces per operand
  __shared__ __align__(16) float sQ[64 * LDR];    // q, then q e^{P}
  __shared__ __align__(16) float sK[64 * LDR];    // k, then k e^{P}
  __shared__ __align__(16) float sG[64 * LDR];    // g, then k e^{-P}
  __shared__ __align__(16) float sV[VSZ];          // v, then A (I + A solve) and Aqk
  __shared__ __align__(16) float sE[6][D];         // e^{sum of block totals between I and R}
  __shared__ float sBeta[64];

  // head-fastest order: the resident workgroups cover every head of a few
  // chunks, so each raw token row is read whole while it is open in DRAM
  const int h = blockIdx.x, c = blockIdx.y;
  if (c >= t.chunk0[t.N]) return;
  const int H = p.H;
  const int s = t.chunk_seq[c];
  const int tau0 = (c - t.chunk0[s]) * kChunk;
  const int64_t tok0 = static_cast<int64_t>(t.cu[s]) + tau0;
  const int len = min(kChunk, t.cu[s + 1] - static_cast<int>(tok0));
  const int tid = threadIdx.x;
  const size_t HD = static_cast<size_t>(H) * D;
  const size_t Ctot = 3 * HD;
  const uint32_t flags = p.flags;
  uint8_t* rec = records + (static_cast<size_t>(c) * H + h) * REC.bytes;

  // ---- 1. conv + SiLU (q, k, v) and gate, one channel per task
  const float a_exp = expf(p.A_log[h]);
  for (int task = tid; task < 4 * D; task += NT) {
    const int grp = task / D, ch = task % D;
    const size_t col = static_cast<size_t>(h) * D + ch;
    if (grp < 3) {
      const void* x = grp == 0 ? io.q : (grp == 1 ? io.k : io.v);
      const void* w = grp == 0 ? p.wq : (grp == 1 ? p.wk : p.wv);
      float* dst = grp == 0 ? sQ : (grp == 1 ? sK : sV);
      const float w0 = ld<IO_BF16>(w, col * 4), w1 = ld<IO_BF16>(w, col * 4 + 1);
      const float w2 = ld<IO_BF16>(w, col * 4 + 2), w3 = ld<IO_BF16>(w, col * 4 + 3);
      float hm[3];
#pragma unroll
      for (int m = 0; m < 3; ++m) {
        const int tau = tau0 - 3 + m;
        if (tau >= 0) hm[m] = ld<IO_BF16>(x, static_cast<size_t>(t.cu[s] + tau) * HD + col);
        else if (io.conv_in) hm[m] = ld<IO_BF16>(io.conv_in, (static_cast<size_t>(s) * 3 + (3 + tau)) * Ctot + grp * HD + col);
        else hm[m] = 0.f;
      }
      float xr[kChunk];   // all loads of the channel in flight at once
#pragma unroll
      for (int r = 0; r < kChunk; ++r)   // rows past the chunk's end re-read its last row (no branch)
        xr[r] = ld<IO_BF16>(x, static_cast<size_t>(tok0 + min(r, len - 1)) * HD + col);
      float h3 = hm[0], h2 = hm[1], h1 = hm[2];
#pragma unroll
      for (int r = 0; r < kChunk; ++r) {
        const float xt = xr[r];
        float u = (flags & KDA_FLAG_SKIP_CONV) ? xt : siluf_(w0 * h3 + w1 * h2 + w2 * h1 + w3 * xt);
        u = r < len ? u : 0.f;
        h3 = h2; h2 = h1; h1 = xt;
        dst[r * LDR + ch] = u;
      }
    } else {
      const float dtb = p.dt_bias[col];
      float ar[kChunk];
#pragma unroll
      for (int r = 0; r < kChunk; ++r) ar[r] = ld<IO_BF16>(io.alpha, static_cast<size_t>(tok0 + min(r, len - 1)) * HD + col);
#pragma unroll
      for (int r = 0; r < kChunk; ++r) {
        float g = (flags & KDA_FLAG_RAW_GATE) ? ar[r] : gate_value(ar[r], dtb, a_exp, p.lower_bound);
        sG[r * LDR + ch] = r < len ? g : 0.f;
      }
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

  // ---- L2 norms of q and k: four lanes per token
  {
    constexpr int CPP = D / 4;
    const int r = tid >> 2, part = tid & 3;
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int i = 0; i < CPP; ++i) {
      const float a = sQ[r * LDR + part * CPP + i], b = sK[r * LDR + part * CPP + i];
      sq += a * a;
      sk += b * b;
    }
    sq = group_sum<4>(sq);
    sk = group_sum<4>(sk);
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

  // ---- 2a. per-channel decays (channel owners) and right-hand sides
  float x[kChunk];   // this lane's column of [beta K+ | beta V]
  if (tid < D) {
    const int ch = tid;
    float gc[kChunk], kc[kChunk];
#pragma unroll
    for (int r = 0; r < kChunk; ++r) { gc[r] = sG[r * LDR + ch]; kc[r] = sK[r * LDR + ch]; }
    float Bt[4];
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      float sum = 0.f;
#pragma unroll
      for (int m = 0; m < kSub; ++m) sum += gc[J * kSub + m];
      Bt[J] = sum;
    }
    float* Qp = reinterpret_cast<float*>(rec + REC.Qp);
    // e^{G_r} = e^{P_r} * e^{sum of earlier block totals}: products of factors
    // that each carry one rounding, never exponentials of long sums
    float eBt[4];
#pragma unroll
    for (int J = 0; J < 4; ++J) eBt[J] = expf(Bt[J]);
    float eBefore = 1.f;
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      float P = 0.f;
#pragma unroll
      for (int m = 0; m < kSub; ++m) {
        const int r = J * kSub + m;
        P += gc[r];
        const float eP = expf(P);
        const float qv = sQ[r * LDR + ch];
        sK[r * LDR + ch] = kc[r] * eP;
        sQ[r * LDR + ch] = qv * eP;
        sG[r * LDR + ch] = kc[r] / eP;
        const float eG = eP * eBefore;
        Qp[r * D + ch] = qv * eG;
        x[r] = sBeta[r] * kc[r] * eG;
      }
      eBefore *= eBt[J];
    }
    // K~^T row of this channel: k e^{Q_r + later block totals}, Q_r = in-block
    // sum of g after token r; built backwards, 4 tokens per 16-byte store
    float4* KT = reinterpret_cast<float4*>(rec + REC.KT) + ch * (kChunk / 4);
    {
      float after = 0.f, Qs = 0.f, tmp[4];
#pragma unroll
      for (int r = kChunk - 1; r >= 0; --r) {
        if (r % kSub == kSub - 1) {
          Qs = 0.f;
          if (r < kChunk - 1) after += Bt[(r + 1) / kSub];
        }
        tmp[r % 4] = kc[r] * expf(Qs + after);
        Qs += gc[r];
        if (r % 4 == 0) KT[r / 4] = make_float4(tmp[0], tmp[1], tmp[2], tmp[3]);
      }
    }
    reinterpret_cast<float*>(rec + REC.eGC)[ch] = eBefore;
    sE[0][ch] = eBt[0];
    sE[1][ch] = eBt[0] * eBt[1];
    sE[2][ch] = eBt[0] * eBt[1] * eBt[2];
    sE[3][ch] = eBt[1];
    sE[4][ch] = eBt[1] * eBt[2];
    sE[5][ch] = eBt[2];
  } else if (tid >= 128 && tid < 128 + D) {
    const int ch = tid - 128;
#pragma unroll
    for (int r = 0; r < kChunk; ++r) x[r] = sBeta[r] * sV[r * LDR + ch];
  }
  __syncthreads();

  // ---- 2b. A and Aqk, one 16x16 sub-block per task on the matrix cores
  float* sA = sV;                 // [64][LA]  A (strictly lower, rows scaled by beta)
  float* sAqk = sV + 64 * LA;     // [64][LA]  Aqk (lower, with diagonal)
  {
    const int wave = tid / kWave, lane = tid % kWave, ln = lane & 15, q4 = lane >> 4;
    for (int task = wave; task < 32; task += NT / kWave) {
      const int mat = task >> 4, R = (task >> 2) & 3, I = task & 3;
      float* dst = mat == 0 ? sA : sAqk;
      if (I > R) {
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[(16 * R + 4 * q4 + j) * LA + 16 * I + ln] = 0.f;
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
          const float4* cb = reinterpret_cast<const float4*>(&sG[(16 * I + ln) * LDR + ch0]);
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
        if (mat == 0) dst[r * LA + i] = (i < r) ? sBeta[r] * acc[j] : 0.f;
        else dst[r * LA + i] = (i <= r) ? acc[j] : 0.f;
      }
    }
  }
  __syncthreads();

  // ---- 2c. forward substitution: x_r -= sum_{i<r} A[r,i] x_i
  if (tid < D || (tid >= 128 && tid < 128 + D)) {
#pragma unroll
    for (int r = 1; r < kChunk; ++r) {
      // four independent partial sums over i (rows of A read 4 at a time)
      float a4[4] = {x[r], 0.f, 0.f, 0.f};
#pragma unroll
      for (int i4 = 0; i4 < (r + 3) / 4; ++i4) {
        const float4 av = *reinterpret_cast<const float4*>(&sA[r * LA + 4 * i4]);
        const float aa[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (4 * i4 + j < r) a4[j] -= aa[j] * x[4 * i4 + j];
      }
      x[r] = (a4[0] + a4[1]) + (a4[2] + a4[3]);
    }
    if (tid < D) {
      float* W = reinterpret_cast<float*>(rec + REC.W);
#pragma unroll
      for (int r = 0; r < kChunk; ++r) W[r * D + tid] = x[r];
    } else {
      float4* UT = reinterpret_cast<float4*>(rec + REC.UT) + (tid - 128) * (kChunk / 4);
#pragma unroll
      for (int v4 = 0; v4 < kChunk / 4; ++v4) UT[v4] = make_float4(x[4 * v4], x[4 * v4 + 1], x[4 * v4 + 2], x[4 * v4 + 3]);
    }
  }
  {
    float4* Aq = reinterpret_cast<float4*>(rec + REC.Aqk);
    for (int e = tid; e < kChunk * kChunk / 4; e += NT) {
      const int r = (4 * e) / kChunk, i = (4 * e) % kChunk;
      Aq[e] = *reinterpret_cast<const float4*>(&sAqk[r * LA + i]);
    }
  }
}

template <int D>
static hipError_t launch_prep_d(const Params& p, const ChunkTable& t, const PrefillIO& io, uint8_t* records,
                                int max_chunks, bool io_bf16, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(p.H), static_cast<unsigned>(max_chunks));
  if (io_bf16) chunk_prep_kernel<D, true><<<grid, 256, 0, st>>>(p, t, io, records);
  else chunk_prep_kernel<D, false><<<grid, 256, 0, st>>>(p, t, io, records);
  return hipGetLastError();
}

hipError_t launch_chunk_prep(const Params& p, const ChunkTable& t, const PrefillIO& io, uint8_t* records,
                             int max_chunks, bool io_bf16, hipStream_t st) {
  switch (p.D) {
    case 16: return launch_prep_d<16>(p, t, io, records, max_chunks, io_bf16, st);
    case 32: return launch_prep_d<32>(p, t, io, records, max_chunks, io_bf16, st);
    case 64: return launch_prep_d<64>(p, t, io, records, max_chunks, io_bf16, st);
    case 128: return launch_prep_d<128>(p, t, io, records, max_chunks, io_bf16, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kda
