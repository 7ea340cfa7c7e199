// Sequential scan of the chunked KDA prefill: inter-chunk state propagation
// fused with the chunk output, on the matrix cores (NP bf16 pieces per fp32
// operand, fp32 accumulate; see mfma.h).
//
// One workgroup of four waves per (sequence, head, tile of DVT value
// columns); the columns of the dk x dv state evolve independently.  For each
// chunk of the sequence, in order, with the chunk's Record from chunk prep:
//   Delta = U - W S                       (the corrected values)
//   O     = Q+ S + Aqk Delta              (cross-chunk read + intra-chunk part)
//   S     = Diag(e^{G_C}) S + K~^T Delta  (the state at the next chunk start)
// The output reads the state updated by the current token, as in the pages'
// loop (AliceAI page, section 二), which is why Aqk keeps its diagonal.
//
// Wave w owns token rows 16w..16w+15 of Delta and O and the state rows
// (key channels) 16(w + 4i)..+15; its A operands come straight from the
// record and are split into pieces in registers.  The state stays in fp32
// accumulators for the whole sequence; its transpose is published once per
// chunk to LDS as NP bf16 planes, the B operand of W S and Q+ S, and Delta
// likewise for Aqk Delta and K~^T Delta.
// Workgroups of the same (sequence, head) sit on the same XCD, so the
// record's second reader finds it in that XCD's L2.
//
// At dk = dv in {64, 128} the launcher takes chunk_scan_split_kernel below
// instead: the same steps with the output on four waves of their own.
#include "kda_device.h"
#include "kda_internal.h"
#include "mfma.h"

namespace kda {

// One wave's record operands for one chunk, already split into bf16 pieces,
// in two halves by when they are used: OpsA before the first barrier of a
// chunk (W S, Q+ S, Delta), OpsB after it (Aqk Delta, K~^T Delta, e^{G_C}).
template <int D, int DVT, int NP>
struct OpsA {
  static constexpr int KS = (D < 32 ? 32 : D) / 32;
  static constexpr int CJ = DVT / 16;
  SplitN<NP> w[KS], q[KS];       // W, Q+ rows of this wave's tokens
  float4 u[CJ];                  // U^T, four tokens of one value column
};

template <int D, int DVT, int NP>
struct OpsB {
  static constexpr int CBW = (D / 16 + 3) / 4;
  SplitN<NP> a[2];               // Aqk rows (two 32-token steps)
  SplitN<NP> kt[CBW][2];         // K~^T rows of this wave's state rows
  float4 e[CBW];                 // e^{G_C} of this lane's four state rows
};

template <int NP>
__device__ __forceinline__ SplitN<NP> load_planes(const uint8_t* base, size_t plane_bytes, size_t elem) {
  SplitN<NP> s;
#pragma unroll
  for (int k = 0; k < NP; ++k) s.v[k] = load_bf16x8(base + k * plane_bytes + elem * 2);
  return s;
}

// Every load below reads the wave's 1 KB fragment block, contiguous.
template <int D, int DVT, int NP>
__device__ __forceinline__ void load_ops_a(OpsA<D, DVT, NP>& o, const uint8_t* rec, int wave, int ln, int q4, int j0) {
  constexpr Record REC = record_layout(D, NP);
  using Ops = OpsA<D, DVT, NP>;
  constexpr int KS = Ops::KS, CJ = Ops::CJ, KPD = 32 * KS;
  const float* UT = reinterpret_cast<const float*>(rec + REC.UT);
  const int r0 = 16 * wave;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int ch0 = 32 * ks + 8 * q4;
    if (ch0 < D) {
      const size_t el = frag_index(r0 + ln, ch0, KPD);
      o.w[ks] = load_planes<NP>(rec + REC.W, REC.tile_plane, el);
      o.q[ks] = load_planes<NP>(rec + REC.Qp, REC.tile_plane, el);
    } else {
      o.w[ks] = o.q[ks] = zero_split<NP>();
    }
  }
#pragma unroll
  for (int cj = 0; cj < CJ; ++cj)
    o.u[cj] = *reinterpret_cast<const float4*>(UT + ut_index(j0 + 16 * cj + ln, r0 + 4 * q4));
}

template <int D, int DVT, int NP>
__device__ __forceinline__ void load_ops_b(OpsB<D, DVT, NP>& o, const uint8_t* rec, int wave, int ln, int q4,
                                           int nks_a) {
  constexpr Record REC = record_layout(D, NP);
  constexpr int CBW = OpsB<D, DVT, NP>::CBW, CB = D / 16;
  const float* eGC = reinterpret_cast<const float*>(rec + REC.eGC);
  const int r0 = 16 * wave;
  // in the order of use: e^{G_C} first
#pragma unroll
  for (int i = 0; i < CBW; ++i) {
    const int cb = wave + 4 * i;
    if (CB % 4 == 0 || cb < CB) o.e[i] = *reinterpret_cast<const float4*>(eGC + 16 * cb + 4 * q4);
  }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    if (ks < nks_a)
      o.a[ks] = load_planes<NP>(rec + REC.Aqk, REC.aqk_plane, frag_index(r0 + ln, 32 * ks + 8 * q4, kChunk));
#pragma unroll
  for (int i = 0; i < CBW; ++i) {
    const int cb = wave + 4 * i;
    if (CB % 4 == 0 || cb < CB) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        o.kt[i][ks] = load_planes<NP>(rec + REC.KT, REC.tile_plane, frag_index(16 * cb + ln, 32 * ks + 8 * q4, kChunk));
    }
  }
}

// gate >= 0: this launch is one of two value-tile widths and runs only when
// the chunk table's choice (chunk0[N+1]) equals gate; its workgroups exit
// at once otherwise.
template <int D, int DVT, int NP, bool OUT_BF16>
__global__ __launch_bounds__(256) void chunk_scan_kernel(Params p, ChunkTable t, PrefillIO io, const uint8_t* records,
                                                         int n_sh, int gate) {
  constexpr int NTILE = D / DVT;
  constexpr int KP = D < 32 ? 32 : D;     // channel extent in whole 32-wide steps
  constexpr int KS = KP / 32;             // k steps over channels
  constexpr int CJ = DVT / 16;            // 16-column blocks of the tile
  constexpr int CB = D / 16;              // 16-row blocks of the state
  constexpr int CBW = (CB + 3) / 4;       // state row blocks per wave
  constexpr int LST = KP + 8;             // row stride of S^T in LDS (bf16)
  constexpr int LDT = kChunk + 8;         // row stride of Delta^T in LDS (bf16)
  constexpr Record REC = record_layout(D, NP);
  constexpr int LO = DVT + 4;              // row stride of a wave's output tile in LDS (fp32)
  __shared__ __align__(16) __bf16 sST[NP][DVT * LST];
  __shared__ __align__(16) __bf16 sDT[NP][DVT * LDT];
  __shared__ __align__(16) float sO[4][16 * LO];   // each wave's 16 output rows, for row-contiguous stores

  const int H = p.H;
  // XCD-aware order: blockIdx = ((sh / 8) * NTILE + tile) * 8 + sh % 8
  const int bx = blockIdx.x;
  const int tile = (bx / 8) % NTILE;
  const int sh = (bx / 8 / NTILE) * 8 + bx % 8;
  if (sh >= n_sh) return;
  if (gate >= 0 && t.chunk0[t.N + 1] != gate) return;
  const int s = t.scan_seq(sh / H), h = sh % H;
  const int j0 = tile * DVT;
  const int tid = threadIdx.x, lane = tid % kWave, ln = lane & 15, q4 = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform: scalar branches
  // every wave owns a state row block in each of its CBW slots when the
  // blocks divide evenly (dk >= 64): then the test below is a constant
  auto owns = [&](int i) { return CB % 4 == 0 || wave + 4 * i < CB; };
  const size_t sbase = (static_cast<size_t>(s) * H + h) * D * D;

  // ---- initial state into the accumulators and S^T into LDS
  f32x4 Sacc[CBW][CJ];
#pragma unroll
  for (int i = 0; i < CBW; ++i) {
    const int cb = wave + 4 * i;
#pragma unroll
    for (int cj = 0; cj < CJ; ++cj) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float v = 0.f;
        if (cb < CB && io.S0) v = io.S0[sbase + static_cast<size_t>(16 * cb + 4 * q4 + j) * D + j0 + 16 * cj + ln];
        Sacc[i][cj][j] = v;
      }
    }
  }
  if constexpr (KP > D) {   // zero channel padding (dk = 16 only)
    for (int e = tid; e < DVT * (KP - D); e += 256) {
      const int col = e / (KP - D), ch = D + e % (KP - D);
#pragma unroll
      for (int k = 0; k < NP; ++k) sST[k][col * LST + ch] = static_cast<__bf16>(0.f);
    }
  }
  auto publish_state = [&]() {
#pragma unroll
    for (int i = 0; i < CBW; ++i) {
      const int cb = wave + 4 * i;
      if (!owns(i)) continue;
#pragma unroll
      for (int cj = 0; cj < CJ; ++cj) {
        // the lane's four consecutive state rows, one 8-byte store per plane
        uint32_t w01[NP], w23[NP];
        split_pair<NP>(Sacc[i][cj][0], Sacc[i][cj][1], w01);
        split_pair<NP>(Sacc[i][cj][2], Sacc[i][cj][3], w23);
        const int idx = (16 * cj + ln) * LST + 16 * cb + 4 * q4;
#pragma unroll
        for (int k = 0; k < NP; ++k) *reinterpret_cast<uint2*>(&sST[k][idx]) = make_uint2(w01[k], w23[k]);
      }
    }
  };
  publish_state();
  __syncthreads();

  const int c_first = t.chunk0[s], c_end = t.chunk0[s + 1];
  const int64_t seq0 = t.cu[s];
  const int seq_len = t.cu[s + 1] - t.cu[s];
  const int r0 = 16 * wave;                         // this wave's token rows
  // k steps of Aqk Delta: both for every wave; the record's Aqk is zero above
  // the diagonal, and the waves that need both set the pace anyway
  constexpr int nks_a = 2;
  // One buffer of each operand half, refilled with chunk c + 1 as soon as
  // chunk c has read it (the A half after the first barrier, the B half at the
  // end of the chunk): each record load has about half a chunk in flight.  A
  // second set of buffers (two chunks ahead) measured slower: it pushes the
  // wave past the register file into copies through the accumulation
  // registers.  The refills are unconditional (past the last chunk they
  // re-read it): the same number of loads on every path lets the compiler
  // wait for exactly the loads an operand needs, where a skipped refill makes
  // it wait for all of them.
  OpsA<D, DVT, NP> A0;
  OpsB<D, DVT, NP> B0;
  auto rec_of = [&](int c) { return records + (static_cast<size_t>(min(c, c_end - 1)) * H + h) * REC.bytes; };
  if (c_first < c_end) {
    load_ops_a<D, DVT, NP>(A0, rec_of(c_first), wave, ln, q4, j0);
    load_ops_b<D, DVT, NP>(B0, rec_of(c_first), wave, ln, q4, nks_a);
  }

  auto chunk_step = [&](int c, OpsA<D, DVT, NP>& A, OpsB<D, DVT, NP>& B) {
    const int tau = t.s0 + (c - c_first) * kChunk;   // the chunk's position in the sequence
    const int len = min(kChunk, seq_len - tau);

    // ---- W S and Q+ S for this wave's 16 token rows.  The S^T pieces of
    //      each (k step, column block) are read one group ahead, so the LDS
    //      latency hides behind the previous group's matrix-core steps.
    f32x4 accW[CJ], accQ[CJ];
#pragma unroll
    for (int cj = 0; cj < CJ; ++cj) { accW[cj] = zero4(); accQ[cj] = zero4(); }
    {
      auto load_s = [&](int g) {
        SplitN<NP> b;
#pragma unroll
        for (int k = 0; k < NP; ++k) b.v[k] = load_bf16x8(&sST[k][(16 * (g % CJ) + ln) * LST + 32 * (g / CJ) + 8 * q4]);
        return b;
      };
      SplitN<NP> bS[2];
      bS[0] = load_s(0);
#pragma unroll
      for (int g = 0; g < KS * CJ; ++g) {
        if (g + 1 < KS * CJ) bS[(g + 1) & 1] = load_s(g + 1);
        mfmaN2<NP>(A.w[g / CJ], A.q[g / CJ], bS[g & 1], accW[g % CJ], accQ[g % CJ]);
      }
    }
    // Delta = U - W S, published transposed for the B operands below
#pragma unroll
    for (int cj = 0; cj < CJ; ++cj) {
      const float4 u = A.u[cj];
      uint32_t w01[NP], w23[NP];
      split_pair<NP>(u.x - accW[cj][0], u.y - accW[cj][1], w01);
      split_pair<NP>(u.z - accW[cj][2], u.w - accW[cj][3], w23);
      const int idx = (16 * cj + ln) * LDT + r0 + 4 * q4;
#pragma unroll
      for (int k = 0; k < NP; ++k) *reinterpret_cast<uint2*>(&sDT[k][idx]) = make_uint2(w01[k], w23[k]);
    }
    load_ops_a<D, DVT, NP>(A, rec_of(c + 1), wave, ln, q4, j0);
    __syncthreads();

    // ---- O = Q+ S + Aqk Delta;  S = e^{G_C} S + K~^T Delta
#pragma unroll
    for (int i = 0; i < CBW; ++i) {
      if (!owns(i)) continue;
      float4 e4 = B.e[i];
      // kept below the barrier: hoisted above it, this scaling would wait
      // for the operand loads of the B half early
      asm volatile("" : "+v"(e4.x), "+v"(e4.y), "+v"(e4.z), "+v"(e4.w));
#pragma unroll
      for (int cj = 0; cj < CJ; ++cj) {
        Sacc[i][cj][0] *= e4.x; Sacc[i][cj][1] *= e4.y; Sacc[i][cj][2] *= e4.z; Sacc[i][cj][3] *= e4.w;
      }
    }
    {
      // Delta pieces one (k step, column block) group ahead, as above; the
      // passes of the group's independent products interleaved
      auto load_d = [&](int g) {
        SplitN<NP> b;
#pragma unroll
        for (int k = 0; k < NP; ++k) b.v[k] = load_bf16x8(&sDT[k][(16 * (g % CJ) + ln) * LDT + 32 * (g / CJ) + 8 * q4]);
        return b;
      };
      SplitN<NP> bD[2];
      bD[0] = load_d(0);
#pragma unroll
      for (int g = 0; g < 2 * CJ; ++g) {
        if (g + 1 < 2 * CJ) bD[(g + 1) & 1] = load_d(g + 1);
        const int ks = g / CJ, cj = g % CJ;
        const SplitN<NP>& b = bD[g & 1];
#pragma unroll
        for (int sum = NP - 1; sum >= 0; --sum)
#pragma unroll
          for (int pi = 0; pi <= sum; ++pi) {
            accQ[cj] = mfma(B.a[ks].v[pi], b.v[sum - pi], accQ[cj]);
#pragma unroll
            for (int i = 0; i < CBW; ++i)
              if (owns(i)) Sacc[i][cj] = mfma(B.kt[i][ks].v[pi], b.v[sum - pi], Sacc[i][cj]);
          }
      }
    }
    load_ops_b<D, DVT, NP>(B, rec_of(c + 1), wave, ln, q4, nks_a);
    // this wave's output rows: through its own LDS tile (LDS operations of a
    // wave run in order), then stored row-contiguous, 8 or 16 bytes per
    // access (few memory operations per chunk leave room for the record
    // loads in flight: a wave may have at most 63 outstanding)
    {
      float* so = sO[wave];
#pragma unroll
      for (int cj = 0; cj < CJ; ++cj)
#pragma unroll
        for (int j = 0; j < 4; ++j) so[(4 * q4 + j) * LO + 16 * cj + ln] = accQ[cj][j];
      asm volatile("" ::: "memory");
      constexpr int LPR = 64 / 16;            // lanes per output row
      constexpr int CPL = DVT / LPR;          // columns per lane
      const int orow = lane / LPR, oc0 = (lane % LPR) * CPL;
      if (r0 + orow < len) {
        const size_t base = (static_cast<size_t>(seq0 + tau + r0 + orow) * H + h) * D + j0 + oc0;
        if constexpr (OUT_BF16) {
#pragma unroll
          for (int c4 = 0; c4 < CPL; c4 += 4) {   // four bf16 per 8-byte store
            const float4 a = *reinterpret_cast<const float4*>(&so[orow * LO + oc0 + c4]);
            const bf16x4 pk = {static_cast<__bf16>(a.x), static_cast<__bf16>(a.y), static_cast<__bf16>(a.z),
                               static_cast<__bf16>(a.w)};   // round to nearest even (v_cvt_pk_bf16_f32)
            *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(io.o) + base + c4) = pk;
          }
        } else {
#pragma unroll
          for (int c4 = 0; c4 < CPL; c4 += 4)
            *reinterpret_cast<float4*>(static_cast<float*>(io.o) + base + c4) =
                *reinterpret_cast<const float4*>(&so[orow * LO + oc0 + c4]);
        }
      }
    }
    // every wave is past its reads of S^T (barrier above): publish the new state
    publish_state();
    __syncthreads();
  };

  for (int c = c_first; c < c_end; ++c) chunk_step(c, A0, B0);

  if (io.S_out) {
#pragma unroll
    for (int i = 0; i < CBW; ++i) {
      const int cb = wave + 4 * i;
      if (!owns(i)) continue;
#pragma unroll
      for (int cj = 0; cj < CJ; ++cj)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          io.S_out[sbase + static_cast<size_t>(16 * cb + 4 * q4 + j) * D + j0 + 16 * cj + ln] = Sacc[i][cj][j];
    }
  }
}

// The same scan with the chunk output on waves of its own (dk = dv in {64,
// 128}): eight waves per workgroup, two per SIMD.  Waves 0-3 carry the state
// chain, S -> Delta = U - W S -> S' = e^{G_C} S + K~^T Delta, and waves 4-7
// form O = Q+ S + Aqk Delta for the same token rows and store it.  The output
// is off the chain: its matrix-core steps and the loads of Q+ and Aqk (a
// third of the record) overlap the chain waves' waits instead of adding to
// them.  Both roles meet at the same two barriers per chunk: after the first,
// Delta is in LDS and the output waves are done reading S; after the second,
// the new S is in LDS and Delta has been read.
template <int D, int DVT, int NP>
struct ChainOps {
  static constexpr int KS = D / 32, CJ = DVT / 16, CBW = D / 64;
  SplitN<NP> w[KS];          // W rows of the wave's tokens
  float4 u[CJ];              // U^T, four tokens of one value column
  float4 e[CBW];             // e^{G_C} of the lane's four state rows
  SplitN<NP> kt[CBW][2];     // K~^T rows of the wave's state rows
};

template <int D, int NP>
struct OutOps {
  static constexpr int KS = D / 32;
  SplitN<NP> q[KS];          // Q+ rows of the wave's tokens
  SplitN<NP> a[2];           // Aqk rows
};

template <int D, int DVT, int NP, bool OUT_BF16>
__global__ __launch_bounds__(512) void chunk_scan_split_kernel(Params p, ChunkTable t, PrefillIO io,
                                                               const uint8_t* records, int n_sh, int gate) {
  static_assert(D == 64 || D == 128, "state row blocks must divide evenly over four waves");
  constexpr int NTILE = D / DVT;
  constexpr int KS = D / 32;              // k steps over channels
  constexpr int CJ = DVT / 16;            // 16-column blocks of the tile
  constexpr int CBW = D / 64;             // state row blocks per chain wave
  constexpr int LST = D + 8;              // row stride of S^T in LDS (bf16)
  constexpr int LDT = kChunk + 8;         // row stride of Delta^T in LDS (bf16)
  constexpr Record REC = record_layout(D, NP);
  constexpr int LO = DVT + 4;             // row stride of an output wave's tile in LDS (fp32)
  static_assert((KS * CJ) % 2 == 0 && (2 * CJ) % 2 == 0, "k-step groups go in pairs");
  __shared__ __align__(16) __bf16 sST[NP][DVT * LST];
  __shared__ __align__(16) __bf16 sDT[NP][DVT * LDT];
  __shared__ __align__(16) float sO[4][16 * LO];

  const int H = p.H;
  const int bx = blockIdx.x;
  const int tile = (bx / 8) % NTILE;
  const int sh = (bx / 8 / NTILE) * 8 + bx % 8;
  if (sh >= n_sh) return;
  if (gate >= 0 && t.chunk0[t.N + 1] != gate) return;
  const int s = t.scan_seq(sh / H), h = sh % H;
  const int j0 = tile * DVT;
  const int tid = threadIdx.x, lane = tid % kWave, ln = lane & 15, q4 = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int rw = wave & 3;                // token row block (both roles) / state row blocks rw + 4i
  const int r0 = 16 * rw;
  const size_t sbase = (static_cast<size_t>(s) * H + h) * D * D;
  const int c_first = t.chunk0[s], c_end = t.chunk0[s + 1];
  const int64_t seq0 = t.cu[s];
  const int seq_len = t.cu[s + 1] - t.cu[s];
  auto rec_of = [&](int c) { return records + (static_cast<size_t>(min(c, c_end - 1)) * H + h) * REC.bytes; };
  // the S^T or Delta^T pieces of one (k step, column block) group
  auto load_s = [&](int g) {
    SplitN<NP> b;
#pragma unroll
    for (int k = 0; k < NP; ++k) b.v[k] = load_bf16x8(&sST[k][(16 * (g % CJ) + ln) * LST + 32 * (g / CJ) + 8 * q4]);
    return b;
  };
  auto load_d = [&](int g) {
    SplitN<NP> b;
#pragma unroll
    for (int k = 0; k < NP; ++k) b.v[k] = load_bf16x8(&sDT[k][(16 * (g % CJ) + ln) * LDT + 32 * (g / CJ) + 8 * q4]);
    return b;
  };

  if (wave < 4) {
    // ================= the state chain
    using Ops = ChainOps<D, DVT, NP>;
    auto load_a = [&](Ops& o, const uint8_t* rec) {
      const float* UT = reinterpret_cast<const float*>(rec + REC.UT);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        o.w[ks] = load_planes<NP>(rec + REC.W, REC.tile_plane, frag_index(r0 + ln, 32 * ks + 8 * q4, D));
#pragma unroll
      for (int cj = 0; cj < CJ; ++cj)
        o.u[cj] = *reinterpret_cast<const float4*>(UT + ut_index(j0 + 16 * cj + ln, r0 + 4 * q4));
    };
    auto load_b = [&](Ops& o, const uint8_t* rec) {
      const float* eGC = reinterpret_cast<const float*>(rec + REC.eGC);
#pragma unroll
      for (int i = 0; i < CBW; ++i) o.e[i] = *reinterpret_cast<const float4*>(eGC + 16 * (rw + 4 * i) + 4 * q4);
#pragma unroll
      for (int i = 0; i < CBW; ++i)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          o.kt[i][ks] = load_planes<NP>(rec + REC.KT, REC.tile_plane,
                                        frag_index(16 * (rw + 4 * i) + ln, 32 * ks + 8 * q4, kChunk));
    };
    f32x4 Sacc[CBW][CJ];
#pragma unroll
    for (int i = 0; i < CBW; ++i)
#pragma unroll
      for (int cj = 0; cj < CJ; ++cj)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          Sacc[i][cj][j] = io.S0 ? io.S0[sbase + static_cast<size_t>(16 * (rw + 4 * i) + 4 * q4 + j) * D + j0 + 16 * cj + ln]
                                 : 0.f;
    auto publish_state = [&]() {
#pragma unroll
      for (int i = 0; i < CBW; ++i)
#pragma unroll
        for (int cj = 0; cj < CJ; ++cj) {
          uint32_t w01[NP], w23[NP];
          split_pair<NP>(Sacc[i][cj][0], Sacc[i][cj][1], w01);
          split_pair<NP>(Sacc[i][cj][2], Sacc[i][cj][3], w23);
          const int idx = (16 * cj + ln) * LST + 16 * (rw + 4 * i) + 4 * q4;
#pragma unroll
          for (int k = 0; k < NP; ++k) *reinterpret_cast<uint2*>(&sST[k][idx]) = make_uint2(w01[k], w23[k]);
        }
    };
    publish_state();
    Ops ops;
    if (c_first < c_end) {
      load_a(ops, rec_of(c_first));
      load_b(ops, rec_of(c_first));
    }
    __syncthreads();
    for (int c = c_first; c < c_end; ++c) {
      // W S for this wave's 16 token rows; S^T pieces one group pair ahead
      f32x4 accW[CJ];
#pragma unroll
      for (int cj = 0; cj < CJ; ++cj) accW[cj] = zero4();
      {
        SplitN<NP> bS[2][2];
        bS[0][0] = load_s(0);
        bS[0][1] = load_s(1);
#pragma unroll
        for (int g = 0; g < KS * CJ; g += 2) {
          const int cur = (g / 2) & 1;
          if (g + 2 < KS * CJ) {
            bS[cur ^ 1][0] = load_s(g + 2);
            bS[cur ^ 1][1] = load_s(g + 3);
          }
          mfmaNx2<NP>(ops.w[g / CJ], bS[cur][0], accW[g % CJ], ops.w[(g + 1) / CJ], bS[cur][1], accW[(g + 1) % CJ]);
        }
      }
      // Delta = U - W S, published transposed
#pragma unroll
      for (int cj = 0; cj < CJ; ++cj) {
        const float4 u = ops.u[cj];
        uint32_t w01[NP], w23[NP];
        split_pair<NP>(u.x - accW[cj][0], u.y - accW[cj][1], w01);
        split_pair<NP>(u.z - accW[cj][2], u.w - accW[cj][3], w23);
        const int idx = (16 * cj + ln) * LDT + r0 + 4 * q4;
#pragma unroll
        for (int k = 0; k < NP; ++k) *reinterpret_cast<uint2*>(&sDT[k][idx]) = make_uint2(w01[k], w23[k]);
      }
      load_a(ops, rec_of(c + 1));
      __syncthreads();
      // S = e^{G_C} S + K~^T Delta
#pragma unroll
      for (int i = 0; i < CBW; ++i) {
        float4 e4 = ops.e[i];
        asm volatile("" : "+v"(e4.x), "+v"(e4.y), "+v"(e4.z), "+v"(e4.w));
#pragma unroll
        for (int cj = 0; cj < CJ; ++cj) {
          Sacc[i][cj][0] *= e4.x; Sacc[i][cj][1] *= e4.y; Sacc[i][cj][2] *= e4.z; Sacc[i][cj][3] *= e4.w;
        }
      }
      {
        SplitN<NP> bD[2];
        bD[0] = load_d(0);
#pragma unroll
        for (int g = 0; g < 2 * CJ; ++g) {
          if (g + 1 < 2 * CJ) bD[(g + 1) & 1] = load_d(g + 1);
          const int ks = g / CJ, cj = g % CJ;
          if constexpr (CBW == 2) {
            mfmaN2<NP>(ops.kt[0][ks], ops.kt[1][ks], bD[g & 1], Sacc[0][cj], Sacc[1][cj]);
          } else {
            Sacc[0][cj] = mfmaN<NP>(ops.kt[0][ks], bD[g & 1], Sacc[0][cj]);
          }
        }
      }
      load_b(ops, rec_of(c + 1));
      publish_state();   // every wave is past its reads of S^T (first barrier)
      __syncthreads();
    }
    if (io.S_out) {
#pragma unroll
      for (int i = 0; i < CBW; ++i)
#pragma unroll
        for (int cj = 0; cj < CJ; ++cj)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            io.S_out[sbase + static_cast<size_t>(16 * (rw + 4 * i) + 4 * q4 + j) * D + j0 + 16 * cj + ln] = Sacc[i][cj][j];
    }
  } else {
    // ================= the output
    using Ops = OutOps<D, NP>;
    auto load_a = [&](Ops& o, const uint8_t* rec) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        o.q[ks] = load_planes<NP>(rec + REC.Qp, REC.tile_plane, frag_index(r0 + ln, 32 * ks + 8 * q4, D));
    };
    // Aqk is zero above the diagonal: token rows 0..31 have nothing past
    // column 31, and the row prep does not write those fragments
    const bool aqk_full = rw >= 2;
    auto load_b = [&](Ops& o, const uint8_t* rec) {
      o.a[0] = load_planes<NP>(rec + REC.Aqk, REC.aqk_plane, frag_index(r0 + ln, 8 * q4, kChunk));
      if (aqk_full) o.a[1] = load_planes<NP>(rec + REC.Aqk, REC.aqk_plane, frag_index(r0 + ln, 32 + 8 * q4, kChunk));
      else o.a[1] = zero_split<NP>();
    };
    Ops ops;
    if (c_first < c_end) {
      load_a(ops, rec_of(c_first));
      load_b(ops, rec_of(c_first));
    }
    __syncthreads();
    for (int c = c_first; c < c_end; ++c) {
      const int tau = t.s0 + (c - c_first) * kChunk;   // the chunk's position in the sequence
      const int len = min(kChunk, seq_len - tau);
      f32x4 accQ[CJ];
#pragma unroll
      for (int cj = 0; cj < CJ; ++cj) accQ[cj] = zero4();
      {
        SplitN<NP> bS[2][2];
        bS[0][0] = load_s(0);
        bS[0][1] = load_s(1);
#pragma unroll
        for (int g = 0; g < KS * CJ; g += 2) {
          const int cur = (g / 2) & 1;
          if (g + 2 < KS * CJ) {
            bS[cur ^ 1][0] = load_s(g + 2);
            bS[cur ^ 1][1] = load_s(g + 3);
          }
          mfmaNx2<NP>(ops.q[g / CJ], bS[cur][0], accQ[g % CJ], ops.q[(g + 1) / CJ], bS[cur][1], accQ[(g + 1) % CJ]);
        }
      }
      load_a(ops, rec_of(c + 1));
      __syncthreads();
      {
        SplitN<NP> bD[2][2];
        bD[0][0] = load_d(0);
        bD[0][1] = load_d(1);
#pragma unroll
        for (int g = 0; g < 2 * CJ; g += 2) {
          const int cur = (g / 2) & 1;
          if (g + 2 < 2 * CJ) {
            bD[cur ^ 1][0] = load_d(g + 2);
            bD[cur ^ 1][1] = load_d(g + 3);
          }
          if (CJ >= 2 && g >= CJ && !aqk_full) continue;   // the zero k step
          mfmaNx2<NP>(ops.a[g / CJ], bD[cur][0], accQ[g % CJ], ops.a[(g + 1) / CJ], bD[cur][1], accQ[(g + 1) % CJ]);
        }
      }
      load_b(ops, rec_of(c + 1));
      // the wave's output rows through its own LDS tile, then row-contiguous stores
      {
        float* so = sO[rw];
#pragma unroll
        for (int cj = 0; cj < CJ; ++cj)
#pragma unroll
          for (int j = 0; j < 4; ++j) so[(4 * q4 + j) * LO + 16 * cj + ln] = accQ[cj][j];
        asm volatile("" ::: "memory");
        constexpr int LPR = 64 / 16;
        constexpr int CPL = DVT / LPR;
        const int orow = lane / LPR, oc0 = (lane % LPR) * CPL;
        if (r0 + orow < len) {
          const size_t base = (static_cast<size_t>(seq0 + tau + r0 + orow) * H + h) * D + j0 + oc0;
          if constexpr (OUT_BF16) {
#pragma unroll
            for (int c4 = 0; c4 < CPL; c4 += 4) {
              const float4 a = *reinterpret_cast<const float4*>(&so[orow * LO + oc0 + c4]);
              const bf16x4 pk = {static_cast<__bf16>(a.x), static_cast<__bf16>(a.y), static_cast<__bf16>(a.z),
                                 static_cast<__bf16>(a.w)};
              *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(io.o) + base + c4) = pk;
            }
          } else {
#pragma unroll
            for (int c4 = 0; c4 < CPL; c4 += 4)
              *reinterpret_cast<float4*>(static_cast<float*>(io.o) + base + c4) =
                  *reinterpret_cast<const float4*>(&so[orow * LO + oc0 + c4]);
          }
        }
      }
      __syncthreads();
    }
  }
}

// Value-tile width: the widest tile that still gives every CU a workgroup.
// (Narrower tiles do not buy a second resident workgroup per CU: the
// prefetched operands keep a wave near the register-file limit.)
static int pick_dvt(int D, int n_sh) {
  for (int dvt : {64, 32, 16})
    if (dvt <= D && static_cast<long>(n_sh) * (D / dvt) >= 256) return dvt;
  return 16;
}

template <int D, int DVT>
static hipError_t launch_scan_dt(const Params& p, const ChunkTable& t, const PrefillIO& io, const uint8_t* records,
                                 bool io_bf16, bool out_bf16, int gate, hipStream_t st) {
  const int n_sh = t.N * p.H;
  const int groups = (n_sh + 7) / 8;
  const dim3 grid(static_cast<unsigned>(groups * 8 * (D / DVT)));
  if constexpr (D == 64 || D == 128) {   // the output on waves of its own
    if (io_bf16) {
      if (out_bf16) chunk_scan_split_kernel<D, DVT, 2, true><<<grid, 512, 0, st>>>(p, t, io, records, n_sh, gate);
      else chunk_scan_split_kernel<D, DVT, 2, false><<<grid, 512, 0, st>>>(p, t, io, records, n_sh, gate);
    } else {
      if (out_bf16) chunk_scan_split_kernel<D, DVT, 3, true><<<grid, 512, 0, st>>>(p, t, io, records, n_sh, gate);
      else chunk_scan_split_kernel<D, DVT, 3, false><<<grid, 512, 0, st>>>(p, t, io, records, n_sh, gate);
    }
    return hipGetLastError();
  }
  if (io_bf16) {
    if (out_bf16) chunk_scan_kernel<D, DVT, 2, true><<<grid, 256, 0, st>>>(p, t, io, records, n_sh, gate);
    else chunk_scan_kernel<D, DVT, 2, false><<<grid, 256, 0, st>>>(p, t, io, records, n_sh, gate);
  } else {
    if (out_bf16) chunk_scan_kernel<D, DVT, 3, true><<<grid, 256, 0, st>>>(p, t, io, records, n_sh, gate);
    else chunk_scan_kernel<D, DVT, 3, false><<<grid, 256, 0, st>>>(p, t, io, records, n_sh, gate);
  }
  return hipGetLastError();
}

template <int D>
static hipError_t launch_scan_d(const Params& p, const ChunkTable& t, const PrefillIO& io, const uint8_t* records,
                                bool io_bf16, bool out_bf16, bool device_choice, hipStream_t st) {
  const int dvt = pick_dvt(D, t.N * p.H);
  if constexpr (D >= 64) {
    if (dvt == 64) {
      if (!device_choice) return launch_scan_dt<D, 64>(p, t, io, records, io_bf16, out_bf16, -1, st);
      // both widths, each running only if the chunk table chose it
      const hipError_t e = launch_scan_dt<D, 64>(p, t, io, records, io_bf16, out_bf16, 0, st);
      if (e != hipSuccess) return e;
      return launch_scan_dt<D, 32>(p, t, io, records, io_bf16, out_bf16, 1, st);
    }
  }
  if constexpr (D >= 32) {
    if (dvt == 32) return launch_scan_dt<D, 32>(p, t, io, records, io_bf16, out_bf16, -1, st);
  }
  return launch_scan_dt<D, 16>(p, t, io, records, io_bf16, out_bf16, -1, st);
}

hipError_t launch_chunk_scan(const Params& p, const ChunkTable& t, const PrefillIO& io, const uint8_t* records,
                             bool io_bf16, bool out_bf16, bool device_choice, hipStream_t st) {
  switch (p.D) {
    case 16: return launch_scan_d<16>(p, t, io, records, io_bf16, out_bf16, device_choice, st);
    case 32: return launch_scan_d<32>(p, t, io, records, io_bf16, out_bf16, device_choice, st);
    case 64: return launch_scan_d<64>(p, t, io, records, io_bf16, out_bf16, device_choice, st);
    case 128: return launch_scan_d<128>(p, t, io, records, io_bf16, out_bf16, device_choice, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kda
