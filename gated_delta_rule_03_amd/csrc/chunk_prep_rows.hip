// Chunk preparation, row-block form: the same Record as chunk_prep.hip (see
// there and kda_internal.h for what it holds and why), computed with a
// different division of labour for the common case of bf16 inputs and
// dk = dv in {64, 128}.
//
// Differences from the general kernel:
//  * Persistent workgroups with a fixed head.  Workgroup (h, grp) walks the
//    chunks grp, grp + G, ... of head h; the raw q/k/v rows (with the three
//    conv rows before the chunk), alpha and b of the NEXT chunk are loaded
//    into registers while the current one is processed, so the input
//    latency is hidden.  The conv weights and dt_bias of the head stay in LDS.
//  * Wave (R, g) owns token rows 16R..16R+15 and key channels CW g ..
//    CW g + CW - 1 (CW = 64 at dk = 128, 32 at dk = 64).  A lane holds one
//    token row r and CW / 4 channels (groups of 8 at 32-channel spacing),
//    which is exactly the A operand of 16x16x32 matrix-core steps, so the
//    row operands of A = beta K K^T and Aqk = Q K^T (with their decays) never
//    leave registers.  The token
//    prefix sums of g inside a 16-row block are DPP scans across the 16
//    lanes of a row, and e^{P} is formed once per element for both q and k.
//    The conv runs as bf16 dot products over tap pairs.
//  * The channel groups' partial sums of A and Aqk meet in LDS: group 1
//    stores and group 0 adds its own on top, in that order.
//  * The solve of (I + A) X = [beta K+ | beta V] forms T = (I + A)^-1 first:
//    the inverses of the four diagonal blocks by forward substitution, then
//    each 16-column block of T on fp32 matrix-core steps.  X = T B is then a
//    plain product on the bf16 matrix cores (pieces as everywhere else), each
//    wave on its own 16-column blocks of X.
// Row R of a wave is chosen so that the two waves sharing a SIMD (w, w + 4)
// own row blocks R and 3 - R: the triangular A work is then even per SIMD.
#include "kda_device.h"
#include "kda_internal.h"
#include "mfma.h"

namespace kda {

namespace {

constexpr int kRawRows = kChunk + 3;   // the chunk's rows and the three conv rows before it
constexpr int kRowsNP = 2;             // bf16 pieces per operand (bf16 inputs)
// Channels per wave: 64 at dk = 128 (8 waves); 32 at dk = 64 (8 waves rather
// than 4).  Measured on the 32K prefill, 16 waves of 32 channels at dk = 128
// were 39% slower than 8 of 64 (128 registers, with spills).
template <int D>
constexpr int rows_cw() { return D == 128 ? 64 : 32; }

// Lane i of each 16-lane row reads lane i - N of the same row; lanes
// shifted in from outside the row read 0.
template <int N>
__device__ __forceinline__ float dpp_row_shr(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + N, 0xf, 0xf, true));
}

// Sums over lanes 0..i of the lane's 16-lane row (inclusive prefixes), for N
// values at once: written step by step across the values, so that each DPP
// step's wait on the previous result is filled by the other values' steps.
template <int N>
__device__ __forceinline__ void row_prefix(float (&x)[N]) {
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] += dpp_row_shr<1>(x[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] += dpp_row_shr<2>(x[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] += dpp_row_shr<4>(x[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] += dpp_row_shr<8>(x[j]);
}


__device__ __forceinline__ uint32_t word(const uint4& v, int j) { return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w)); }

// a.lo b.lo + a.hi b.hi + c over bf16 pairs (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// C += A B over one 16x16x4 fp32 matrix-core step: lane l gives A[l % 16][l / 16]
// and B[l / 16][l % 16]; C is laid out as in the bf16 steps.
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Keeps the compiler from moving memory accesses across this point: the LDS
// hand-offs inside a wave rely on program order (a wave's LDS operations
// execute in order), and it bounds how far loads are hoisted in unrolled
// loops, which keeps the register count in check.
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Pins computed values where they stand: the compiler may otherwise sink
// arithmetic past a barrier to its first use and keep all of its inputs
// alive instead (here, hundreds of registers of raw inputs and conv taps).
// Eight values go through one statement, so that the scheduler may still
// interleave their computations (one statement per value orders them).
template <int N>
__device__ __forceinline__ void pin(float (&a)[N]) {
  static_assert(N % 8 == 0, "pins go in groups of eight");
#pragma unroll
  for (int i = 0; i < N; i += 8)
    asm volatile("" : "+v"(a[i]), "+v"(a[i + 1]), "+v"(a[i + 2]), "+v"(a[i + 3]), "+v"(a[i + 4]), "+v"(a[i + 5]),
                 "+v"(a[i + 6]), "+v"(a[i + 7]));
}

// Position of one chunk in the packed batch.
struct ChunkPos {
  int s, tau0, len;
  int64_t tok0;
};

// The same memory through the constant address space: a load at a uniform
// index from it is a scalar load (its own counter, results in scalar
// registers), where a global load would occupy the vector-memory counter and
// be waited for together with the stores before it.
__device__ __forceinline__ int scalar_load(const int* p, int i) {
  return ((const __attribute__((address_space(4))) int*)(p))[i];
}

__device__ __forceinline__ int4 scalar_load_desc(const int4* d, int i) {
  const int* p = reinterpret_cast<const int*>(d) + 4 * i;
  return make_int4(scalar_load(p, 0), scalar_load(p, 1), scalar_load(p, 2), scalar_load(p, 3));
}

__device__ __forceinline__ ChunkPos chunk_pos(const int4& d) {
  ChunkPos cp;
  cp.s = d.x;
  cp.tau0 = d.y;
  cp.len = d.z;
  cp.tok0 = d.w;
  return cp;
}

// The raw inputs of one chunk for one head, as this thread loads them.  The
// q | k | v staging rows are 3D/8 pieces of 16 bytes wide; thread t stages
// piece column t % (3D/8) of rows t / (3D/8) + SR j (SR staging rows per pass
// of the block), so that its tensor and channels stay fixed.
template <int D, int NT, int KSW>
struct RawChunk {
  static constexpr int kCols = 3 * D / 8;
  static constexpr int kSR = NT / kCols;                       // rows per pass
  static constexpr int kPer = (kRawRows + kSR - 1) / kSR;      // passes
  uint4 x[kPer];      // staging rows, then written to LDS
  uint4 a[KSW];       // alpha of this lane's row and its channels
  uint16_t b;         // b of this lane's row
  uint32_t zero;      // bit j: piece j stands for a missing history row (written as zeros)
};

}  // namespace

// CW: channels per wave (64: 2 waves per SIMD at dk = 128; 32: 4 waves).
// kHooks: compiled with the input hooks (q, k, v already activated; g or beta
// given directly); without them those selects cost nothing.
template <int D, int CW, bool kHooks>
__global__ __launch_bounds__(64 * 4 * (D / CW), 1) void chunk_prep_rows_kernel(Params p, ChunkTable t, PrefillIO io,
                                                                               uint8_t* records) {
  constexpr int CQ = D / CW;            // channel groups
  constexpr int NW = 4 * CQ;            // waves
  constexpr int NT = 64 * NW;
  constexpr int KSW = CW / 32;          // 32-channel matrix-core k steps per wave
  constexpr int CPL = 8 * KSW;          // channels per lane
  constexpr int NP = kRowsNP;
  constexpr Record REC = record_layout(D, NP);
  constexpr int RAWS = 2 * D + 8;       // staging row stride of q | k (bf16)
  constexpr int RAWV = D + 8;           // staging row stride of v (bf16)
  constexpr int KCS = D + 8;            // row stride of the k e^{-P} pieces (bf16)
  constexpr int LX = D == 64 ? kChunk + 8 : kChunk + 4;   // row stride of X^T (fp32)
  constexpr int LA = kChunk + 4;        // row stride of A, Aqk (fp32)
  constexpr int LT = 16 + 4;            // row stride of the diagonal-block inverses (fp32)
  constexpr int NCB = 2 * D / 16;       // 16-column blocks of X
  constexpr int CBPW = NCB / NW;        // ... per wave
  constexpr size_t kRawBytes = static_cast<size_t>(kRawRows) * RAWS * 2;
  constexpr size_t kKcBytes = static_cast<size_t>(NP) * 64 * KCS * 2;
  constexpr size_t kXBytes = static_cast<size_t>(2 * D) * LX * 4;
  constexpr size_t kUBytes = kRawBytes > kKcBytes ? (kRawBytes > kXBytes ? kRawBytes : kXBytes)
                                                  : (kKcBytes > kXBytes ? kKcBytes : kXBytes);
  using Raw = RawChunk<D, NT, KSW>;
  static_assert(CBPW * NW == NCB, "column blocks must divide evenly over the waves");
  static_assert(kKcBytes <= static_cast<size_t>(D) * LX * 4, "the beta V^T rows of X^T must start past the k e^{-P} pieces");

  // sU holds, in turn: the raw staging rows; the k e^{-P} pieces beside the
  // beta V^T rows of X^T (which start past them); X^T
  __shared__ __align__(16) unsigned char sU[kUBytes];
  __shared__ __align__(16) float sA[64 * LA];            // A (rows scaled by beta)
  __shared__ __align__(16) float sAqk[64 * LA];
  // with four channel groups the partial sums of A and Aqk meet in two pairs
  // of buffers (groups 0, 1 and 2, 3); their readers add the pairs
  __shared__ __align__(16) float sA2[CQ > 2 ? 64 * LA : 4];
  __shared__ __align__(16) float sAqk2[CQ > 2 ? 64 * LA : 4];
  __shared__ __align__(16) float sT[4][16 * LT];         // (I + A_RR)^-1, fp32
  // v's staging rows, apart from q | k: v is convolved in phase 4b, by the
  // waves that have no part in forming T there
  __shared__ __align__(16) __bf16 sRawV[kRawRows * RAWV];
  __shared__ __align__(16) uint2 sWb[3][D];              // conv taps of this head (q, k, v), 4 bf16 each
  __shared__ __align__(16) float sDtb[D];
  __shared__ __align__(16) float sBt[4][D];              // in-block totals of g
  __shared__ __align__(16) float sEBt[4][D];             // their exponentials
  __shared__ float sNorm[CQ][64][2];                     // partial sums of q^2, k^2
  __shared__ float sBeta[64];
  __bf16* sRaw = reinterpret_cast<__bf16*>(sU);
  __bf16* sKc = reinterpret_cast<__bf16*>(sU);
  float* sX = reinterpret_cast<float*>(sU);

  const int H = p.H;
  const int h = blockIdx.x % H, grp = blockIdx.x / H, G = gridDim.x / H;
  const int total = scalar_load(t.chunk0, t.N);
  // Lane coordinates.  Inside the chunk loop they are re-derived from a copy
  // of the thread index the compiler cannot see through, so that it does not
  // hoist per-lane addresses out of the loop and keep them in registers for
  // its whole length (that alone would cost about 150 registers).
  // Waves w, w + 4, ... share a SIMD; their row blocks are a permutation of
  // 0..3 when there are four of them, and R, 3 - R for two, so the
  // triangular A work is even per SIMD.
  struct LaneCoords {
    int tid, w, lane, ln, q4, R, cq, r;
  };
  auto coords = [](int t) {
    LaneCoords L;
    L.tid = t;
    L.w = __builtin_amdgcn_readfirstlane(t / kWave);   // wave-uniform: scalar branches and loop counts
    L.lane = t % kWave;
    L.ln = L.lane & 15;
    L.q4 = L.lane >> 4;
    const int s = L.w & 3, k = L.w >> 2;
    const int base = (k & 2) ? ((s + 2) & 3) : s;
    L.R = (k & 1) ? 3 - base : base;   // row block
    L.cq = k;                          // channel group
    L.r = 16 * L.R + L.ln;             // this lane's token row
    return L;
  };
  const int tid = threadIdx.x;
  const size_t HD = static_cast<size_t>(H) * D;
  const size_t Ctot = 3 * HD;
  const uint32_t flags = p.flags;
  const bool raw_conv = kHooks && (flags & KDA_FLAG_SKIP_CONV);
  const bool raw_gate = kHooks && (flags & KDA_FLAG_RAW_GATE);
  const bool raw_beta = kHooks && (flags & KDA_FLAG_RAW_BETA);
  const bool l2 = !(flags & KDA_FLAG_SKIP_L2NORM);
  const float a_exp = expf(p.A_log[h]);

  // ---- the head's conv taps and dt_bias, once
  {
    for (int e = tid; e < 3 * D; e += NT) {
      const int tens = e / D, ch = e % D;
      const uint16_t* w = static_cast<const uint16_t*>(tens == 0 ? p.wq : (tens == 1 ? p.wk : p.wv)) +
                          (static_cast<size_t>(h) * D + ch) * 4;
      sWb[tens][ch] = make_uint2(w[0] | (static_cast<uint32_t>(w[1]) << 16), w[2] | (static_cast<uint32_t>(w[3]) << 16));
    }
    for (int e = tid; e < D; e += NT) sDtb[e] = p.dt_bias[static_cast<size_t>(h) * D + e];
  }

  // Every piece is loaded from a valid address and zeroed where the history
  // has no row (sequence start without a conv history) or past the staging rows.
  auto load_rows = [&](Raw& nx, const ChunkPos& cp, const LaneCoords& L) {
    const int st_col = L.tid % Raw::kCols, st_row0 = L.tid / Raw::kCols;
    const bool stager = L.tid < Raw::kSR * Raw::kCols;
    const int st_tens = st_col / (D / 8), st_ch = 8 * (st_col % (D / 8));
    const uint16_t* st_x = static_cast<const uint16_t*>(st_tens == 0 ? io.q : (st_tens == 1 ? io.k : io.v)) +
                           static_cast<size_t>(h) * D + st_ch;
    const bool have_hist = io.conv_in != nullptr;
    const uint16_t* st_h = static_cast<const uint16_t*>(have_hist ? io.conv_in : io.q) +
                           (have_hist ? static_cast<size_t>(cp.s) * 3 * Ctot + st_tens * HD + static_cast<size_t>(h) * D + st_ch
                                      : 0);
    // (the zeroing is applied when the pieces are written to LDS: a select
    // here would wait for every load, and for every store before it)
    //
    // Staging row sr is token tok0 - 3 + sr of the sequence (rows past the
    // chunk's end re-read its last token); in the sequence's first chunk rows
    // 0..2 come from the conv history instead, or are zeros without one.
    // Those rows can only be a thread's first piece (kSR >= 3), so only that
    // piece's address is a select; written as a branch per piece, the two
    // cases cost a divergent branch each.  Offsets are 32-bit element counts
    // from one 64-bit base.
    static_assert(Raw::kSR >= 3, "the history rows fall in each thread's first piece");
    const uint16_t* row0 = st_x + (cp.tok0 - 3) * static_cast<int64_t>(HD);
    const uint32_t hd = static_cast<uint32_t>(HD);
    const uint32_t off0 = static_cast<uint32_t>(st_row0) * hd, last = static_cast<uint32_t>(cp.len + 2) * hd;
    const bool hist0 = cp.tau0 == 0 && st_row0 < 3;
    const uint16_t* p0 = row0 + min(off0, last);
    if (have_hist) {   // uniform
      p0 = hist0 ? st_h + static_cast<size_t>(st_row0) * Ctot : p0;
      nx.zero = 0u;
    } else {
      p0 = hist0 ? row0 + 3 * hd : p0;   // any valid row for a missing one
      nx.zero = hist0 ? 1u : 0u;
    }
    nx.x[0] = *reinterpret_cast<const uint4*>(p0);
#pragma unroll
    for (int j = 1; j < Raw::kPer; ++j)
      nx.x[j] = *reinterpret_cast<const uint4*>(row0 + min(off0 + static_cast<uint32_t>(Raw::kSR * j) * hd, last));
  };
  // alpha and b of this lane's row: issued apart from the staging rows (in
  // phase 3, which has no memory operations of its own), since a burst of
  // loads this scattered holds up the wave that issues it
  auto load_gate_inputs = [&](Raw& nx, const ChunkPos& cp, const LaneCoords& L) {
    const uint32_t hd = static_cast<uint32_t>(HD);
    const uint16_t* arow = static_cast<const uint16_t*>(io.alpha) + cp.tok0 * static_cast<int64_t>(HD) +
                           static_cast<size_t>(h) * D + CW * L.cq + 8 * L.q4;
    const uint32_t rr = static_cast<uint32_t>(min(L.r, cp.len - 1));
#pragma unroll
    for (int ks = 0; ks < KSW; ++ks) nx.a[ks] = *reinterpret_cast<const uint4*>(arow + rr * hd + 32 * ks);
    nx.b = static_cast<const uint16_t*>(io.b)[(cp.tok0 + rr) * H + h];
  };

  // The loop is rotated: a chunk's raw inputs are loaded at the start of the
  // previous chunk's phase 1 and written to the staging rows at its end, so
  // the wait for them counts only the memory operations of one iteration.
  Raw nxt;
  ChunkPos cur_pos{}, nxt_pos{};
  // the in-block decay sums (prefix sums of the gate over the lane's 16-row
  // block) of this lane's row and channels for the chunk about to run,
  // computed during the previous chunk's phase 5 (its VALU has room there;
  // phase 1 is VALU-bound), from alpha loaded in that chunk's phase 3
  float g_cur[CPL], e_cur[CPL];   // and e^{P_r}
#pragma unroll
  for (int j = 0; j < CPL; ++j) g_cur[j] = e_cur[j] = 0.f;
  uint32_t b_cur = 0u;
  // the descriptor of the chunk after the next (a uniform index: a scalar
  // load, one chunk ahead of its use)
  int4 desc_ahead = make_int4(0, 0, 0, 0);
  auto stage = [&](const LaneCoords& L) {
    const int st_col = L.tid % Raw::kCols, st_row0 = L.tid / Raw::kCols;
    const bool stager = L.tid < Raw::kSR * Raw::kCols;
    const bool st_v = st_col >= 2 * D / 8;   // a piece of v
    __bf16* const st_dst = st_v ? sRawV + 8 * (st_col - 2 * D / 8) : sRaw + 8 * st_col;
    const int st_stride = st_v ? RAWV : RAWS;
#pragma unroll
    for (int j = 0; j < Raw::kPer; ++j) {
      const int sr = st_row0 + Raw::kSR * j;
      if (stager && sr < kRawRows)
        *reinterpret_cast<uint4*>(st_dst + sr * st_stride) =
            (nxt.zero >> j) & 1u ? make_uint4(0u, 0u, 0u, 0u) : nxt.x[j];
    }
    uint32_t bw = nxt.b;
    asm volatile("" : "+v"(bw));   // arrived before the next load goes out
    b_cur = bw;
  };
  // gate (computed for every lane, then selected) of the chunk at cp, from
  // nx's alpha; rows past the chunk's end get 0
  auto gate_of = [&](const Raw& nx, const ChunkPos& cp, const LaneCoords& L, const float* dtb) {
    const bool live = L.r < cp.len;
#pragma unroll
    for (int ks = 0; ks < KSW; ++ks) {
      const int c0 = CW * L.cq + 32 * ks + 8 * L.q4;
      const uint32_t aw[4] = {nx.a[ks].x, nx.a[ks].y, nx.a[ks].z, nx.a[ks].w};
      const float4 d0 = *reinterpret_cast<const float4*>(&dtb[c0]);
      const float4 d1 = *reinterpret_cast<const float4*>(&dtb[c0 + 4]);
      const float dt[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
      float al[8], gc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        al[i] = (i & 1) ? __uint_as_float(aw[i / 2] & 0xffff0000u) : __uint_as_float(aw[i / 2] << 16);
        gc[i] = gate_value(al[i], dt[i], a_exp, p.lower_bound);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) g_cur[8 * ks + i] = live ? (raw_gate ? al[i] : gc[i]) : 0.f;
    }
    // in-block decay sums P_r (through token r): DPP scans over the 16 lanes
    // (token rows) of each row of the wave
    row_prefix(g_cur);
#pragma unroll
    for (int j = 0; j < CPL; ++j) e_cur[j] = exp_fast(g_cur[j]);
    pin(g_cur);   // computed here, not sunk past the next barrier
    pin(e_cur);
  };
  if (grp < total) {
    cur_pos = chunk_pos(scalar_load_desc(t.desc, grp));
    load_rows(nxt, cur_pos, coords(tid));
    load_gate_inputs(nxt, cur_pos, coords(tid));
    desc_ahead = scalar_load_desc(t.desc, min(grp + G, total - 1));
    stage(coords(tid));
    __syncthreads();   // dt_bias is in shared memory
    gate_of(nxt, cur_pos, coords(tid), sDtb);
  }

  for (int c = grp; c < total; c += G) {
    const ChunkPos cp = cur_pos;
    int tid_opaque = tid;
    asm volatile("" : "+v"(tid_opaque));
    const LaneCoords L = coords(tid_opaque);
    const int w = L.w, lane = L.lane, ln = L.ln, q4 = L.q4, R = L.R, cq = L.cq, r = L.r;
    __syncthreads();   // the staging rows are written

    // ---- the next chunk's staging rows go out now, ahead of phase 1: it
    //      issues no memory operations of its own, so the loads leave before
    //      the record stores of phase 2 and do not queue behind them.  Always
    //      issued (after the last chunk they load that chunk again): with the
    //      same loads on every path the compiler waits only for the ones a
    //      value needs.
    nxt_pos = chunk_pos(desc_ahead);
    load_rows(nxt, nxt_pos, L);
    desc_ahead = scalar_load_desc(t.desc, min(c + 2 * G, total - 1));

    uint8_t* rec = records + (static_cast<size_t>(c) * H + h) * REC.bytes;
    const bool live = r < cp.len;
    // The conv taps and dt_bias never change inside this loop; reading them
    // through an offset the compiler cannot see through keeps it from
    // hoisting 200 registers' worth of LDS loads out of the loop.
    int inv = 0;
    asm volatile("" : "+v"(inv));
    const uint2* tapw = &sWb[0][0] + inv;
    const float* dtb = sDtb + inv;

    // ---- 1. conv + SiLU of this lane's row (q, k; v follows in phase 4b),
    //      beta, the norms' partial sums; the gate and its in-block sums came
    //      from the previous chunk's phase 5
    float qv[CPL], kv[CPL];
#pragma unroll
    for (int tens = 0; tens < 2; ++tens) {
#pragma unroll
      for (int ks = 0; ks < KSW; ++ks) {
        const int c0 = CW * cq + 32 * ks + 8 * q4;
        // all eight LDS reads of the group go out together, then the math
        // (left to itself the scheduler waits for each tap read in turn)
        uint4 xm[4], wv[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) xm[m] = *reinterpret_cast<const uint4*>(&sRaw[(r + m) * RAWS + tens * D + c0]);
#pragma unroll
        for (int jw = 0; jw < 4; ++jw) wv[jw] = *reinterpret_cast<const uint4*>(&tapw[tens * D + c0 + 2 * jw]);
        __builtin_amdgcn_sched_barrier(0);
        // bf16 dot products over tap pairs: the inputs and taps are bf16, so
        // every product is exact and only the three additions round
        // SiLU is computed for every lane and then selected: written as a
        // conditional, it becomes a branch per channel with the exponential
        // chains serialised inside
        float uo[8], rawx[8];
#pragma unroll
        for (int jw = 0; jw < 4; ++jw) {   // channels c0 + 2 jw, c0 + 2 jw + 1
          const uint4 wt = wv[jw];
          const uint32_t x0 = word(xm[0], jw), x1 = word(xm[1], jw), x2 = word(xm[2], jw), x3 = word(xm[3], jw);
          const float ye = dot2_bf16(__builtin_amdgcn_perm(x1, x0, 0x05040100u), wt.x,
                                     dot2_bf16(__builtin_amdgcn_perm(x3, x2, 0x05040100u), wt.y, 0.f));
          const float yo = dot2_bf16(__builtin_amdgcn_perm(x1, x0, 0x07060302u), wt.z,
                                     dot2_bf16(__builtin_amdgcn_perm(x3, x2, 0x07060302u), wt.w, 0.f));
          uo[2 * jw] = siluf_(ye);
          uo[2 * jw + 1] = siluf_(yo);
          rawx[2 * jw] = __uint_as_float(x3 << 16);
          rawx[2 * jw + 1] = __uint_as_float(x3 & 0xffff0000u);
        }
        pin(uo);   // this group is computed before the next group's loads
        // Rows past the chunk's end (copies of its last row) are left as they
        // are: their beta and gate are zero, so their rows of A, beta K+,
        // beta V and hence of W, U and the state update are exactly zero.
#pragma unroll
        for (int i = 0; i < 8; ++i) uo[i] = raw_conv ? rawx[i] : uo[i];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (tens == 0) qv[8 * ks + i] = uo[i];
          else kv[8 * ks + i] = uo[i];
        }
        compiler_fence();
      }
    }
    pin(qv);
    pin(kv);
    float beta = 0.f;
    if (live) {
      const float bb = bf16_to_f32(static_cast<uint16_t>(b_cur));
      beta = raw_beta ? bb : sigmoidf_(bb);
      if (flags & KDA_FLAG_BETA_X2) beta *= 2.0f;
    }
    if (cq == 0 && q4 == 0) sBeta[r] = beta;
    {
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        sq += qv[j] * qv[j];
        sk += kv[j] * kv[j];
      }
      sq += __shfl_xor(sq, 16);
      sk += __shfl_xor(sk, 16);
      sq += __shfl_xor(sq, 32);
      sk += __shfl_xor(sk, 32);
      if (q4 == 0) {
        sNorm[cq][r][0] = sq;
        sNorm[cq][r][1] = sk;
      }
    }
    // in-block decay sums P_r (through token r); e^{P_r} through the hardware
    // exponential: its ~1e-5 relative error at |P| ~ 80 is below the bf16
    // pieces' resolution
    float P[CPL], eP[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      P[j] = g_cur[j];
      eP[j] = e_cur[j];
    }
    pin(P);
    pin(eP);
    if (ln == 15) {
#pragma unroll
      for (int ks = 0; ks < KSW; ++ks) {
        const int c0 = CW * cq + 32 * ks + 8 * q4;
        *reinterpret_cast<float4*>(&sBt[R][c0]) = make_float4(P[8 * ks], P[8 * ks + 1], P[8 * ks + 2], P[8 * ks + 3]);
        *reinterpret_cast<float4*>(&sBt[R][c0 + 4]) =
            make_float4(P[8 * ks + 4], P[8 * ks + 5], P[8 * ks + 6], P[8 * ks + 7]);
        *reinterpret_cast<float4*>(&sEBt[R][c0]) =
            make_float4(eP[8 * ks], eP[8 * ks + 1], eP[8 * ks + 2], eP[8 * ks + 3]);
        *reinterpret_cast<float4*>(&sEBt[R][c0 + 4]) =
            make_float4(eP[8 * ks + 4], eP[8 * ks + 5], eP[8 * ks + 6], eP[8 * ks + 7]);
      }
    }
    __syncthreads();

    // ---- 2. norms, decays and the elementwise outputs of this lane's row
    float iq, ik;
    {
      float nq = sNorm[0][r][0], nk = sNorm[0][r][1];
#pragma unroll
      for (int g = 1; g < CQ; ++g) {
        nq += sNorm[g][r][0];
        nk += sNorm[g][r][1];
      }
      // hardware reciprocal square root (~1 ulp): bf16 inputs only here
      iq = (l2 ? __builtin_amdgcn_rsqf(nq + p.eps) : 1.0f) * p.scale;
      ik = l2 ? __builtin_amdgcn_rsqf(nk + p.eps) : 1.0f;
    }
    float qP[CPL], kP[CPL];
    SplitN<NP> kcp[KSW];   // k e^{-P} pieces: the B operand of this lane's diagonal block
    // e^{G before block R} and the sum of the later block totals, per channel
    // (R is uniform over the wave: the branches are scalar; each product and
    // sum starts from its first term, not from 1 or 0)
    auto before_after = [&](int c0, float (&eb)[8], float (&after)[8]) {
      auto load8 = [&](const float* row, float (&x)[8]) {
        const float4 a = *reinterpret_cast<const float4*>(row + c0);
        const float4 b = *reinterpret_cast<const float4*>(row + c0 + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
      };
      if (R == 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) eb[i] = 1.f;
      } else {
        load8(sEBt[0], eb);
#pragma unroll 1
        for (int J = 1; J < R; ++J) {
          float e[8];
          load8(sEBt[J], e);
#pragma unroll
          for (int i = 0; i < 8; ++i) eb[i] *= e[i];
        }
      }
      if (R == 3) {
#pragma unroll
        for (int i = 0; i < 8; ++i) after[i] = 0.f;
      } else {
        load8(sBt[3], after);
#pragma unroll 1
        for (int J = 2; J > R; --J) {
          float b[8];
          load8(sBt[J], b);
#pragma unroll
          for (int i = 0; i < 8; ++i) after[i] += b[i];
        }
      }
    };
    {
      // key side: k e^{P}, k e^{-P} pieces, K~^T, e^{G_C}
      __bf16* KT = reinterpret_cast<__bf16*>(rec + REC.KT);
      float* eGC = reinterpret_cast<float*>(rec + REC.eGC);
      float ebs[KSW][8];   // e^{G before block R}: kept for the query side
      float fas[KSW][8];   // e^{-Bt_R} for an even block R, else 1: kept for the query side
#pragma unroll
      for (int ks = 0; ks < KSW; ++ks) {
        const int c0 = CW * cq + 32 * ks + 8 * q4;
        float (&eb)[8] = ebs[ks];
        float after[8];
        before_after(c0, eb, after);
        const float4 bt0 = *reinterpret_cast<const float4*>(&sBt[R][c0]);
        const float4 bt1 = *reinterpret_cast<const float4*>(&sBt[R][c0 + 4]);
        const float bt[8] = {bt0.x, bt0.y, bt0.z, bt0.w, bt1.x, bt1.y, bt1.z, bt1.w};
        // The operands of A and Aqk take their decays from the middle of the
        // row block pair (2p, 2p + 1), the end of block 2p: row r of block R
        // carries e^{G_r - G_mid}, column s carries e^{G_mid - G_s}.  For an
        // odd block that is e^{P}, e^{-P} (P the in-block sum); for an even
        // block e^{P - Bt_R}, e^{Bt_R - P} (Bt_R its total).  Either way an
        // exponent spans one block, as for in-block references, and the
        // blocks of one pair need no factor between them.
        float fb[8];
        float (&fa)[8] = fas[ks];
        if ((R & 1) == 0) {
          const float4 e0 = *reinterpret_cast<const float4*>(&sEBt[R][c0]);
          const float4 e1 = *reinterpret_cast<const float4*>(&sEBt[R][c0 + 4]);
          const float ev[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            fb[i] = ev[i];
            fa[i] = rcp_fast(ev[i]);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) fa[i] = fb[i] = 1.f;
        }
        float kc[8], kt[8], pk[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int j = 8 * ks + i;
          const float kk = kv[j] * ik;
          pk[i] = kk * (eP[j] * fa[i]);                         // row operand of the A sub-blocks
          kc[i] = kk * (fb[i] * rcp_fast(eP[j]));               // column operand (factor in [e^{Bt_R}, 1])
          kt[i] = kk * exp_fast((bt[i] - P[j]) + after[i]);     // K~ = k e^{G_C - G_r}
        }
        pin(pk);
#pragma unroll
        for (int i = 0; i < 8; ++i) kP[8 * ks + i] = pk[i];
        kcp[ks] = splitN<NP>(kc);
#pragma unroll
        for (int k = 0; k < NP; ++k) *reinterpret_cast<bf16x8*>(&sKc[k * 64 * KCS + r * KCS + c0]) = kcp[ks].v[k];
        // channels c0 .. c0 + 7 lie in one 16-row block of the fragment order
        // (c0 is a multiple of 8), eight elements apart
        const size_t kt0 = frag_index(c0, r, kChunk);
        uint16_t* KT16 = reinterpret_cast<uint16_t*>(KT) + kt0;
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          uint32_t w[NP];
          split_pair<NP>(kt[i], kt[i + 1], w);
#pragma unroll
          for (int k = 0; k < NP; ++k) {
            KT16[k * (REC.tile_plane / 2) + 8 * i] = static_cast<uint16_t>(w[k]);
            KT16[k * (REC.tile_plane / 2) + 8 * (i + 1)] = static_cast<uint16_t>(w[k] >> 16);
          }
        }
        if (R == 3 && ln == 15) {   // e^{G_C} = e^{G before block 3} e^{P_63}
          float eg[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) eg[i] = eP[8 * ks + i] * eb[i];
          *reinterpret_cast<float4*>(eGC + c0) = make_float4(eg[0], eg[1], eg[2], eg[3]);
          *reinterpret_cast<float4*>(eGC + c0 + 4) = make_float4(eg[4], eg[5], eg[6], eg[7]);
        }
        compiler_fence();
      }
      // query side: Q+ = q e^{G_r} out, q e^{P} kept
      __bf16* Qp = reinterpret_cast<__bf16*>(rec + REC.Qp);
#pragma unroll
      for (int ks = 0; ks < KSW; ++ks) {
        const int c0 = CW * cq + 32 * ks + 8 * q4;
        const float (&eb)[8] = ebs[ks];
        const float (&fa)[8] = fas[ks];
        float qo[8], pq[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int j = 8 * ks + i;
          const float qq = qv[j] * iq;
          qo[i] = qq * (eP[j] * eb[i]);
          pq[i] = qq * (eP[j] * fa[i]);
        }
        pin(pq);
#pragma unroll
        for (int i = 0; i < 8; ++i) qP[8 * ks + i] = pq[i];
        const SplitN<NP> qs = splitN<NP>(qo);
#pragma unroll
        for (int k = 0; k < NP; ++k)
          *reinterpret_cast<bf16x8*>(Qp + k * (REC.tile_plane / 2) + frag_index(r, c0, D)) = qs.v[k];
        compiler_fence();
      }
    }
    pin(qP);
    pin(kP);
    __syncthreads();

    load_gate_inputs(nxt, nxt_pos, L);

    // ---- 3. this wave's channel group's part of A and Aqk, sub-blocks
    //      (R, I <= R).  Groups 1 (and 3) store their partial sums, then
    //      groups 0 (and 2) add their own (held in registers) on top: the same
    //      order every time.
    {
      f32x4 keepA[4], keepQ[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) keepA[I] = keepQ[I] = zero4();
      float* const dA = (CQ > 2 && cq >= 2) ? sA2 : sA;
      float* const dQ = (CQ > 2 && cq >= 2) ? sAqk2 : sAqk;
      // Kept sums are indexed by a static slot: 0 the diagonal block (I = R),
      // 1 the other block of the pair (I = R - 1, R odd), 2 and 3 the blocks
      // of the first pair seen from the second (I = 1, 0; R >= 2).  (An index
      // by I would be a dynamic register index.)
      auto finish = [&](int slot, int I, const f32x4& accA, const f32x4& accQ) {
        if (CQ == 1 || (cq & 1)) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int row = 16 * R + 4 * q4 + j, col = 16 * I + ln;
            dA[row * LA + col] = sBeta[row] * accA[j];
            dQ[row * LA + col] = accQ[j];
          }
        } else {
          keepA[slot] = accA;
          keepQ[slot] = accQ;
        }
      };
      auto col_operand = [&](int I, int c0) {   // the column operand of block I
        SplitN<NP> bk;
#pragma unroll
        for (int k = 0; k < NP; ++k)
          bk.v[k] = *reinterpret_cast<const bf16x8*>(&sKc[k * 64 * KCS + (16 * I + ln) * KCS + c0]);
        return bk;
      };
      // the blocks of this wave's own pair: one split of the row operands
      {
        SplitN<NP> sa[KSW], sq[KSW];
#pragma unroll
        for (int ks = 0; ks < KSW; ++ks) {
          float ra[8], rq[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            ra[i] = kP[8 * ks + i];
            rq[i] = qP[8 * ks + i];
          }
          sa[ks] = splitN<NP>(ra);
          sq[ks] = splitN<NP>(rq);
        }
        {
          f32x4 accA = zero4(), accQ = zero4();
#pragma unroll
          for (int ks = 0; ks < KSW; ++ks) mfmaN2<NP>(sa[ks], sq[ks], kcp[ks], accA, accQ);
          finish(0, R, accA, accQ);
        }
        if (R & 1) {
          f32x4 accA = zero4(), accQ = zero4();
#pragma unroll
          for (int ks = 0; ks < KSW; ++ks)
            mfmaN2<NP>(sa[ks], sq[ks], col_operand(R - 1, CW * cq + 32 * ks + 8 * q4), accA, accQ);
          finish(1, R - 1, accA, accQ);
        }
      }
      // the first pair's blocks from the second: the row operands times
      // e^{Bt_2} and then e^{Bt_1}, the decay between the two pairs' middles.
      // One factor at a time: e^{Bt_1 + Bt_2} alone underflows for strong
      // decays where the row operand times it does not (for block 2 the
      // first factor brings the operand back to e^{P} <= 1).
      if (R >= 2) {
        SplitN<NP> sa[KSW], sq[KSW];
#pragma unroll
        for (int ks = 0; ks < KSW; ++ks) {
          const int c0 = CW * cq + 32 * ks + 8 * q4;
          const float4 e0 = *reinterpret_cast<const float4*>(&sEBt[1][c0]);
          const float4 e1 = *reinterpret_cast<const float4*>(&sEBt[1][c0 + 4]);
          const float4 f0 = *reinterpret_cast<const float4*>(&sEBt[2][c0]);
          const float4 f1 = *reinterpret_cast<const float4*>(&sEBt[2][c0 + 4]);
          const float x1[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
          const float x2[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
          float ra[8], rq[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            ra[i] = (kP[8 * ks + i] * x2[i]) * x1[i];
            rq[i] = (qP[8 * ks + i] * x2[i]) * x1[i];
          }
          sa[ks] = splitN<NP>(ra);
          sq[ks] = splitN<NP>(rq);
        }
#pragma unroll
        for (int I = 1; I >= 0; --I) {
          f32x4 accA = zero4(), accQ = zero4();
#pragma unroll
          for (int ks = 0; ks < KSW; ++ks)
            mfmaN2<NP>(sa[ks], sq[ks], col_operand(I, CW * cq + 32 * ks + 8 * q4), accA, accQ);
          finish(3 - I, I, accA, accQ);
        }
      }
      if constexpr (CQ > 1) {
        __syncthreads();
        if ((cq & 1) == 0) {
          // every read goes out before the first add: one LDS round trip
          // for the whole update, not one per element
          float oa[4][4], oq[4][4], bt[4];
          // each slot's block, and whether this wave has one there (unused
          // slots read block 0 and write nothing)
          const int slot_I[4] = {R, (R & 1) ? R - 1 : 0, R >= 2 ? 1 : 0, 0};
          const bool slot_ok[4] = {true, (R & 1) != 0, R >= 2, R >= 2};
#pragma unroll
          for (int j = 0; j < 4; ++j) bt[j] = sBeta[16 * R + 4 * q4 + j];
#pragma unroll
          for (int sl = 0; sl < 4; ++sl) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int row = 16 * R + 4 * q4 + j, col = 16 * slot_I[sl] + ln;
              oa[sl][j] = dA[row * LA + col];
              oq[sl][j] = dQ[row * LA + col];
            }
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int sl = 0; sl < 4; ++sl) {
            if (!slot_ok[sl]) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int row = 16 * R + 4 * q4 + j, col = 16 * slot_I[sl] + ln;
              dA[row * LA + col] = bt[j] * keepA[sl][j] + oa[sl][j];
              dQ[row * LA + col] = keepQ[sl][j] + oq[sl][j];
            }
          }
        }
      }
    }
    __syncthreads();

    // A as its readers see it: with four channel groups, the sum of the pairs
    auto load_a4 = [&](int idx) {
      float4 a4 = *reinterpret_cast<const float4*>(&sA[idx]);
      if constexpr (CQ > 2) {
        const float4 u4 = *reinterpret_cast<const float4*>(&sA2[idx]);
        a4 = make_float4(a4.x + u4.x, a4.y + u4.y, a4.z + u4.z, a4.w + u4.w);
      }
      return a4;
    };

    // ---- 4. Aqk pieces out; the diagonal-block inverses to LDS; beta K+ to X^T
    {
      __bf16* Aq = reinterpret_cast<__bf16*>(rec + REC.Aqk);
      // by waves 1 .. NW - 1 only: wave 0 forms the diagonal-block inverses
      // below, the longest task of this phase.  A fixed trip count, not a
      // loop (a loop here makes the compiler wait for every outstanding
      // load first).  The 8-column groups of token rows 0..31 past column
      // 31 are zero and are not written (the scan does not read them): 384
      // groups, 128 of rows 0..31 then 256 of rows 32..63.
      constexpr int NAQ = NT - kWave;
      constexpr int NGRP = 32 * 4 + 32 * 8;
#pragma unroll
      for (int it = 0; it < (NGRP + NAQ - 1) / NAQ; ++it) {
        const int e = L.tid - kWave + it * NAQ;
        if (w == 0 || e >= NGRP) break;
        const int rw = e < 128 ? e >> 2 : 32 + ((e - 128) >> 3);
        const int i0 = e < 128 ? 8 * (e & 3) : 8 * ((e - 128) & 7);
        float4 q0 = *reinterpret_cast<const float4*>(&sAqk[rw * LA + i0]);
        float4 q1 = *reinterpret_cast<const float4*>(&sAqk[rw * LA + i0 + 4]);
        if constexpr (CQ > 2) {
          const float4 u0 = *reinterpret_cast<const float4*>(&sAqk2[rw * LA + i0]);
          const float4 u1 = *reinterpret_cast<const float4*>(&sAqk2[rw * LA + i0 + 4]);
          q0 = make_float4(q0.x + u0.x, q0.y + u0.y, q0.z + u0.z, q0.w + u0.w);
          q1 = make_float4(q1.x + u1.x, q1.y + u1.y, q1.z + u1.z, q1.w + u1.w);
        }
        const float qa[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
        float qm[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) qm[i] = (i0 + i <= rw) ? qa[i] : 0.f;
        const SplitN<NP> qs = splitN<NP>(qm);
#pragma unroll
        for (int k = 0; k < NP; ++k)
          *reinterpret_cast<bf16x8*>(Aq + k * (REC.aqk_plane / 2) + frag_index(rw, i0, kChunk)) = qs.v[k];
      }
      if (w == 0) {   // lane = (block, column) of the unit lower-triangular inverses
        const int Rb = lane >> 4, j = lane & 15;
        // the strictly lower triangle of the lane's block, all 36 row pieces
        // read before the substitution starts: read row by row inside it,
        // each row's LDS latency sat on the dependent chain
        constexpr int kPieces = 36;   // sum over rows i of ceil(i / 4)
        float4 al[kPieces];
        {
          int k = 0;
#pragma unroll
          for (int i = 0; i < 16; ++i)
#pragma unroll
            for (int q = 0; q < (i + 3) / 4; ++q) al[k++] = load_a4((16 * Rb + i) * LA + 16 * Rb + 4 * q);
        }
        __builtin_amdgcn_sched_barrier(0);
        // forward substitution down the column; each row's sum runs in four
        // partial sums so the dependent chain is the 16 rows, not 120 FMAs
        float tcol[16];
        int k0 = 0;   // the row's first piece in al[]
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float a[16];
#pragma unroll
          for (int q = 0; q < (i + 3) / 4; ++q) {
            const float4 a4 = al[k0 + q];
            a[4 * q] = a4.x; a[4 * q + 1] = a4.y; a[4 * q + 2] = a4.z; a[4 * q + 3] = a4.w;
          }
          k0 += (i + 3) / 4;
          float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int m = 0; m < i; ++m) ps[m & 3] += a[m] * tcol[m];
          const float v = ((i == j) ? 1.f : 0.f) - ((ps[0] + ps[1]) + (ps[2] + ps[3]));
          tcol[i] = (i < j) ? 0.f : v;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sT[Rb][i * LT + j] = tcol[i];
      }
      // beta K+ = beta k e^{G_r}: the row operand times the decay to the
      // middle of its block pair (e^{Bt_0}, or e^{Bt_2} e^{Bt_1} e^{Bt_0}),
      // one factor at a time from the last block back (the product of the
      // factors alone can underflow where the result does not), over the
      // column operand pieces
#pragma unroll
      for (int ks = 0; ks < KSW; ++ks) {
        const int c0 = CW * cq + 32 * ks + 8 * q4;
        const float beta = sBeta[r];
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = beta * kP[8 * ks + i];
#pragma unroll
        for (int J = 2; J >= 0; --J) {
          if (J == 0 || R >= 2) {
            const float4 e0 = *reinterpret_cast<const float4*>(&sEBt[J][c0]);
            const float4 e1 = *reinterpret_cast<const float4*>(&sEBt[J][c0 + 4]);
            const float ev[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] *= ev[i];
          }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) sX[(c0 + i) * LX + r] = v[i];
      }
    }
    __syncthreads();

    // ---- 4b. T = (I + A)^-1, unit lower triangular: wave J < 4 forms its
    //      16-column block by blocked forward substitution on fp32
    //      matrix-core steps (its earlier blocks stay in its registers, laid
    //      out as the B operand of the next steps), and writes it as bf16
    //      pieces in fragment order over the free Aqk area
    __bf16* sTp = reinterpret_cast<__bf16*>(sAqk);
    static_assert(NP * 64 * 64 * 2 <= 64 * LA * 4, "T's pieces fit the Aqk area");
    if (w < 4) {
      const int J = w;
      f32x4 xb[4];
      auto put = [&](int Rs, const f32x4& x) {   // lane holds T[16 Rs + 4 q4 + i][16 J + ln]
        uint32_t w01[NP], w23[NP];
        split_pair<NP>(x[0], x[1], w01);
        split_pair<NP>(x[2], x[3], w23);
        uint16_t* tp = reinterpret_cast<uint16_t*>(sTp);
#pragma unroll
        for (int k = 0; k < NP; ++k) {
          const size_t e = k * 4096 + frag_index(16 * Rs + 4 * q4, 16 * J + ln, 64);
          // rows 4 q4 .. 4 q4 + 3 of one column: eight elements apart
          tp[e] = static_cast<uint16_t>(w01[k]);
          tp[e + 8] = static_cast<uint16_t>(w01[k] >> 16);
          tp[e + 16] = static_cast<uint16_t>(w23[k]);
          tp[e + 24] = static_cast<uint16_t>(w23[k] >> 16);
        }
      };
#pragma unroll
      for (int Rs = 0; Rs < 4; ++Rs) {
        if (Rs < J) {
          // blocks above the diagonal that the products below read as
          // k padding (T_{0,1}, T_{2,3}) are zero
          if ((Rs == 0 && J == 1) || (Rs == 2 && J == 3)) put(Rs, zero4());
          continue;
        }
        if (Rs == J) {   // X_JJ = T_JJ, read as it is
          f32x4 x;
#pragma unroll
          for (int i = 0; i < 4; ++i) x[i] = sT[J][(4 * q4 + i) * LT + ln];
          xb[Rs] = x;
          put(Rs, x);
          continue;
        }
        f32x4 y;
        {                // Y = - A_{Rs, J..Rs-1} X_{J..Rs-1}: k = 4 q4 + s within each block
          f32x4 acc = zero4();
#pragma unroll
          for (int M = 0; M < 3; ++M) {
            if (M < J || M >= Rs) continue;
            const float4 a4 = load_a4((16 * Rs + ln) * LA + 16 * M + 4 * q4);
            acc = mfma_f32(a4.x, xb[M][0], acc);
            acc = mfma_f32(a4.y, xb[M][1], acc);
            acc = mfma_f32(a4.z, xb[M][2], acc);
            acc = mfma_f32(a4.w, xb[M][3], acc);
          }
          y = f32x4{-acc[0], -acc[1], -acc[2], -acc[3]};
        }
        // X_Rs = T_{Rs,Rs} Y: the lane's own rows of Y are its k = 4 q4 + s
        const float4 t4 = *reinterpret_cast<const float4*>(&sT[Rs][ln * LT + 4 * q4]);
        f32x4 x = zero4();
        x = mfma_f32(t4.x, y[0], x);
        x = mfma_f32(t4.y, y[1], x);
        x = mfma_f32(t4.z, y[2], x);
        x = mfma_f32(t4.w, y[3], x);
        xb[Rs] = x;
        put(Rs, x);
      }
    } else {
      // conv + SiLU of v and beta V^T to its rows of X^T (past the k e^{-P}
      // pieces, untouched since phase 2): lane l of wave w takes token row l
      // and a range of 8-channel groups, reads as in phase 1.  At dk = 128
      // waves 4..7 take 3, 4, 4, 5 of the 16 groups: they share their SIMDs
      // with waves 0..3, whose parts of T shrink from column block 0 to 3
      // (measured at 4 groups each, wave 4 took 4.3K cycles and wave 7 2.9K).
      // Rows past the chunk's end have beta 0.
      constexpr int NG = D / 8;
      const int k4 = w - 4;
      const int gs = NG == 16 ? (k4 == 0 ? 0 : (k4 == 1 ? 3 : (k4 == 2 ? 7 : 11))) : k4 * (NG / 4);
      const int ge = NG == 16 ? (k4 == 0 ? 3 : (k4 == 1 ? 7 : (k4 == 2 ? 11 : 16))) : (k4 + 1) * (NG / 4);
      const int row = lane;
      const float bv = sBeta[row];
#pragma unroll
      for (int g8 = 0; g8 < (NG == 16 ? 5 : NG / 4); ++g8) {
        if (gs + g8 >= ge) break;
        const int c0 = 8 * (gs + g8);
        uint4 xm[4], wv[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) xm[m] = *reinterpret_cast<const uint4*>(&sRawV[(row + m) * RAWV + c0]);
#pragma unroll
        for (int jw = 0; jw < 4; ++jw) wv[jw] = *reinterpret_cast<const uint4*>(&tapw[2 * D + c0 + 2 * jw]);
        __builtin_amdgcn_sched_barrier(0);
        float uo[8];
#pragma unroll
        for (int jw = 0; jw < 4; ++jw) {
          const uint4 wt = wv[jw];
          const uint32_t x0 = word(xm[0], jw), x1 = word(xm[1], jw), x2 = word(xm[2], jw), x3 = word(xm[3], jw);
          const float ye = dot2_bf16(__builtin_amdgcn_perm(x1, x0, 0x05040100u), wt.x,
                                     dot2_bf16(__builtin_amdgcn_perm(x3, x2, 0x05040100u), wt.y, 0.f));
          const float yo = dot2_bf16(__builtin_amdgcn_perm(x1, x0, 0x07060302u), wt.z,
                                     dot2_bf16(__builtin_amdgcn_perm(x3, x2, 0x07060302u), wt.w, 0.f));
          const float se = siluf_(ye), so = siluf_(yo);
          uo[2 * jw] = raw_conv ? __uint_as_float(x3 << 16) : se;
          uo[2 * jw + 1] = raw_conv ? __uint_as_float(x3 & 0xffff0000u) : so;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) sX[(D + c0 + i) * LX + row] = bv * uo[i];
        compiler_fence();
      }
    }
    __syncthreads();

    // ---- 5. per wave, on its own column blocks of X^T:
    //      X = T [beta K+ | beta V] (bf16 pieces, k steps up to the diagonal),
    //      then W and U^T out; the next chunk's gate on the side
    {
      gate_of(nxt, nxt_pos, L, dtb);
#pragma unroll
      for (int bi = 0; bi < CBPW; ++bi) {
        const int cb = w + bi * NW;
        float* xc = &sX[(16 * cb + ln) * LX];
        SplitN<NP> bB[2];   // B: tokens 32 ks + 8 q4 .. + 7 of this lane's column
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) bB[ks] = load_split<NP>(xc + 32 * ks + 8 * q4);
        compiler_fence();   // read before this wave overwrites the column below
#pragma unroll
        for (int R = 0; R < 4; ++R) {
          f32x4 acc = zero4();
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            if (ks == 1 && R < 2) continue;   // T_{R, >= 32} = 0 for R < 2
            SplitN<NP> aT;
#pragma unroll
            for (int k = 0; k < NP; ++k) aT.v[k] = load_bf16x8(&sTp[k * 4096 + frag_index(16 * R + ln, 32 * ks + 8 * q4, 64)]);
            acc = mfmaN<NP>(aT, bB[ks], acc);
          }
          *reinterpret_cast<float4*>(&xc[16 * R + 4 * q4]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
      }
      compiler_fence();
      __bf16* W = reinterpret_cast<__bf16*>(rec + REC.W);
      float* UT = reinterpret_cast<float*>(rec + REC.UT);
#pragma unroll
      for (int bi = 0; bi < CBPW; ++bi) {
        const int cb = w + bi * NW;
        if (cb < D / 16) {   // W: 8 channels of one token per lane and step
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            const int u = lane + 64 * k2, tok = u >> 1, c8 = 16 * cb + 8 * (u & 1);
            float xv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) xv[i] = sX[(c8 + i) * LX + tok];
            const SplitN<NP> ws = splitN<NP>(xv);
#pragma unroll
            for (int k = 0; k < NP; ++k)
              *reinterpret_cast<bf16x8*>(W + k * (REC.tile_plane / 2) + frag_index(tok, c8, D)) = ws.v[k];
          }
        } else {             // U^T, fp32
#pragma unroll
          for (int k2 = 0; k2 < 4; ++k2) {
            const int u = lane + 64 * k2, m = u >> 4, t4 = u & 15;
            const int cu = 16 * cb - D + m;
            *reinterpret_cast<float4*>(UT + ut_index(cu, 4 * t4)) =
                *reinterpret_cast<const float4*>(&sX[(16 * cb + m) * LX + 4 * t4]);
          }
        }
      }
    }
    __syncthreads();   // every wave is done with the shared region
    stage(L);
    cur_pos = nxt_pos;
  }
}

template <int D>
static hipError_t launch_rows_d(const Params& p, const ChunkTable& t, const PrefillIO& io, uint8_t* records,
                                int max_chunks, hipStream_t st) {
  int ncu = 0;
  const hipError_t e = device_cus(&ncu);
  if (e != hipSuccess) return e;
  // one resident workgroup per compute unit; each walks the chunks of one head
  int groups = (ncu + p.H - 1) / p.H;
  groups = groups < 1 ? 1 : (groups > max_chunks ? max_chunks : groups);
  const dim3 grid(static_cast<unsigned>(p.H) * static_cast<unsigned>(groups));
  if (p.flags & (KDA_FLAG_SKIP_CONV | KDA_FLAG_RAW_GATE | KDA_FLAG_RAW_BETA))
    chunk_prep_rows_kernel<D, rows_cw<D>(), true><<<grid, 64 * 4 * (D / rows_cw<D>()), 0, st>>>(p, t, io, records);
  else
    chunk_prep_rows_kernel<D, rows_cw<D>(), false><<<grid, 64 * 4 * (D / rows_cw<D>()), 0, st>>>(p, t, io, records);
  return hipGetLastError();
}

bool chunk_prep_rows_supported(const Params& p, const PrefillIO& io, bool io_bf16) {
  if (!io_bf16 || (p.D != 64 && p.D != 128)) return false;
  auto a16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; };
  return a16(io.q) && a16(io.k) && a16(io.v) && a16(io.alpha) && (io.conv_in == nullptr || a16(io.conv_in));
}

hipError_t launch_chunk_prep_rows(const Params& p, const ChunkTable& t, const PrefillIO& io, uint8_t* records,
                                  int max_chunks, hipStream_t st) {
  switch (p.D) {
    case 64: return launch_rows_d<64>(p, t, io, records, max_chunks, st);
    case 128: return launch_rows_d<128>(p, t, io, records, max_chunks, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kda
