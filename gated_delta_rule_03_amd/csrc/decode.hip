// Single-token KDA decode step (the fused recurrent form): one workgroup per
// (sequence, head).  The step is HBM-bound: the fp32 dk x dv state is streamed
// in once and out once, in place.
//
// Per (sequence n, head h), following the delta-rule loop of the AliceAI page
// (section 二) with the conv history of section 四/五:
//   conv over [3 history inputs, new input] -> SiLU -> L2 norm (q, k)
//   g = max(-exp(A_log) softplus(alpha + dt_bias), lb),  beta = sigmoid(b)
//   S~ = Diag(e^g) S;  p = k^T S~;  r = q^T S~;  delta = beta (v - p)
//   o = r + (q.k) delta          (= q^T (S~ + k delta^T), the updated state)
//   S <- S~ + k delta^T;  history <- [h1, h2, x]
// The state loads are issued before anything else so that their latency
// overlaps the preprocess; a wave covers two full state rows per load (512 B
// contiguous each), every lane moves 16 B per access (streamed, non-temporal),
// and the k^T S~ / q^T S~ column sums are reduced across row groups through
// LDS.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

typedef float f32x4v __attribute__((ext_vector_type(4)));

// Eight waves per (sequence, head): a 64 KB in-place tile streams measurably
// faster with 512 threads than with 256 (more bytes in flight per workgroup).
constexpr int kDecodeThreads = 512;
// Threads of the multi-token decode, and the tokens whose inputs it stages at once.
constexpr int kMultiThreads = 256;
constexpr int kMultiGroup = 2;

// With GATED the output row goes through the layer's epilogue before it is
// stored (y = o / sqrt(mean(o^2) + eps) * w * sigmoid(gate), AliceAI page,
// section 三): the workgroup holds the whole row of dv outputs, so the row's
// sum of squares is one reduction over the waves that own it.
template <int D, bool IO_BF16, bool OUT_BF16, bool GATED>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(Params p, DecodeIO io) {
  constexpr int NT = kDecodeThreads;
  constexpr int C4 = D / 4;                  // float4 columns per state row
  constexpr int RPP = NT / C4;               // state rows covered by one pass of the block
  constexpr int RPT = (D + RPP - 1) / RPP;   // passes (rows per thread)
  __shared__ float u_s[3 * D];               // q | k | v after conv + SiLU
  __shared__ float e_s[D];                   // exp(g)
  __shared__ float red[2][RPP][D];           // per-row-group partial k^T S~, q^T S~
  __shared__ float d_s[D];                   // delta
  __shared__ float scal[4];                  // q scale * inv|q|, inv|k|, beta, q.k
  constexpr int OW = (D + kWave - 1) / kWave;  // waves holding the output row
  __shared__ float osum[OW];                 // per-wave sums of o^2 (epilogue)
  static_assert(D <= kDecodeThreads, "one output column per thread");

  const int tid = threadIdx.x;
  const int H = p.H;
  const int n = blockIdx.x / H, h = blockIdx.x % H;
  const size_t Ctot = static_cast<size_t>(3) * H * D;
  const uint32_t flags = p.flags;

  // ---- the small inputs are requested first, all unconditionally (a load
  // under a condition compiles to a branch that waits for it), then the state
  // tile.  The memory counter drains in issue order, so waiting for the small
  // inputs leaves the state's loads in flight behind the preprocess.
  static_assert(3 * D <= NT, "one conv channel per thread");
  const int cc = min(tid, 3 * D - 1);     // this thread's conv channel (threads past 3D: a valid one, unused)
  const int grp = cc / D, ci = cc % D;
  const size_t ch = static_cast<size_t>(grp) * H * D + static_cast<size_t>(h) * D + ci;
  const void* xsrc = grp == 0 ? io.q : (grp == 1 ? io.k : io.v);
  const void* wsrc = grp == 0 ? p.wq : (grp == 1 ? p.wk : p.wv);
  const size_t cb = static_cast<size_t>(n) * 3 * Ctot + ch;
  const size_t wi = (static_cast<size_t>(h) * D + ci) * 4;
  const float xt = ld<IO_BF16>(xsrc, static_cast<size_t>(n) * H * D + static_cast<size_t>(h) * D + ci);
  const float h0 = ld<IO_BF16>(io.conv_state, cb);
  const float h1 = ld<IO_BF16>(io.conv_state, cb + Ctot);
  const float h2 = ld<IO_BF16>(io.conv_state, cb + 2 * Ctot);
  const float w0 = ld<IO_BF16>(wsrc, wi), w1 = ld<IO_BF16>(wsrc, wi + 1);
  const float w2 = ld<IO_BF16>(wsrc, wi + 2), w3 = ld<IO_BF16>(wsrc, wi + 3);
  const int gi = tid % D;                 // this thread's gate / output channel
  const float al = ld<IO_BF16>(io.alpha, (static_cast<size_t>(n) * H + h) * D + gi);
  const float dtb = p.dt_bias[h * D + gi];
  const float bb = ld<IO_BF16>(io.b, static_cast<size_t>(n) * H + h);
  float graw = 0.f, onw = 0.f;            // epilogue operands of this thread's output column
  if constexpr (GATED) {
    graw = ld<IO_BF16>(io.gate, (static_cast<size_t>(n) * H + h) * D + gi);
    onw = io.onw[gi];
  }
  __builtin_amdgcn_sched_barrier(0);
  const int col4 = tid % C4, rg = tid / C4;
  const size_t base = (static_cast<size_t>(n) * H + h) * D * D;
  f32x4v* Sp = reinterpret_cast<f32x4v*>(io.state + base);
  f32x4v Sv[RPT];
#pragma unroll
  for (int rr = 0; rr < RPT; ++rr) {
    const int r = rg + rr * RPP;
    if (r < D) Sv[rr] = __builtin_nontemporal_load(&Sp[static_cast<size_t>(r) * C4 + col4]);
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- preprocess: conv + SiLU for the 3D channels of this head; shift history
  if (tid < 3 * D) {
    u_s[tid] = (flags & KDA_FLAG_SKIP_CONV) ? xt : siluf_(w0 * h0 + w1 * h1 + w2 * h2 + w3 * xt);
    st<IO_BF16>(io.conv_state, cb, h1);
    st<IO_BF16>(io.conv_state, cb + Ctot, h2);
    st<IO_BF16>(io.conv_state, cb + 2 * Ctot, xt);
  }
  const float a_exp = expf(p.A_log[h]);
  if (tid < D) {
    const float g = (flags & KDA_FLAG_RAW_GATE) ? al : gate_value(al, dtb, a_exp, p.lower_bound);
    e_s[tid] = expf(g);
  }
  float gsig = 0.f;
  if constexpr (GATED) gsig = sigmoidf_(graw);
  if (tid == 0) {
    float be = (flags & KDA_FLAG_RAW_BETA) ? bb : sigmoidf_(bb);
    if (flags & KDA_FLAG_BETA_X2) be *= 2.0f;
    scal[2] = be;
  }
  __syncthreads();

  // ---- norms and q.k (waves 0, 1, 2)
  {
    const int wv = tid / kWave, lane = tid % kWave;
    if (wv < 3) {
      float s = 0.0f;
      for (int i = lane; i < D; i += kWave) {
        const float a = u_s[(wv == 1 ? D : 0) + i];
        const float b2 = u_s[(wv == 0 ? 0 : D) + i];
        s += a * b2;
      }
      s = group_sum<kWave>(s);
      if (lane == 0) scal[wv == 2 ? 3 : wv] = s;   // wave 2 stores raw u_q . u_k in slot 3
    }
  }
  __syncthreads();
  if (tid == 0) {
    const bool norm = !(flags & KDA_FLAG_SKIP_L2NORM);
    const float iq = norm ? 1.0f / sqrtf(scal[0] + p.eps) : 1.0f;
    const float ik = norm ? 1.0f / sqrtf(scal[1] + p.eps) : 1.0f;
    scal[3] = scal[3] * iq * ik * p.scale;
    scal[0] = iq * p.scale;
    scal[1] = ik;
  }
  __syncthreads();
  const float qs = scal[0], ks = scal[1], beta = scal[2], qk = scal[3];

  // ---- one pass over the state
  float pk[4] = {0.f, 0.f, 0.f, 0.f}, pq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int rr = 0; rr < RPT; ++rr) {
    const int r = rg + rr * RPP;
    if (r < D) {
      const float e = e_s[r];
      Sv[rr].x *= e; Sv[rr].y *= e; Sv[rr].z *= e; Sv[rr].w *= e;
      const float kr = u_s[D + r] * ks, qr = u_s[r] * qs;
      pk[0] += kr * Sv[rr].x; pk[1] += kr * Sv[rr].y; pk[2] += kr * Sv[rr].z; pk[3] += kr * Sv[rr].w;
      pq[0] += qr * Sv[rr].x; pq[1] += qr * Sv[rr].y; pq[2] += qr * Sv[rr].z; pq[3] += qr * Sv[rr].w;
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    red[0][rg][col4 * 4 + j] = pk[j];
    red[1][rg][col4 * 4 + j] = pq[j];
  }
  __syncthreads();
  float o_j = 0.f;
  if (tid < D) {
    const int j = tid;
    float pp = 0.f, rq = 0.f;
#pragma unroll 8
    for (int g2 = 0; g2 < RPP; ++g2) { pp += red[0][g2][j]; rq += red[1][g2][j]; }
    const float delta = beta * (u_s[2 * D + j] - pp);
    d_s[j] = delta;
    o_j = rq + qk * delta;
    if constexpr (!GATED) st<OUT_BF16>(io.o, (static_cast<size_t>(n) * H + h) * D + j, o_j);
  }
  if constexpr (GATED) {
    if (tid < OW * kWave) {                     // whole waves: lanes past D add 0
      const float ss = group_sum<kWave>(o_j * o_j);
      if ((tid % kWave) == 0) osum[tid / kWave] = ss;
    }
  }
  __syncthreads();
  if constexpr (GATED) {
    if (tid < D) {
      float ss = 0.f;
#pragma unroll
      for (int w = 0; w < OW; ++w) ss += osum[w];
      const float inv = 1.0f / sqrtf(ss * (1.0f / D) + io.oeps);
      st<OUT_BF16>(io.o, (static_cast<size_t>(n) * H + h) * D + tid, o_j * inv * onw * gsig);
    }
  }
  const float d0 = d_s[col4 * 4], d1 = d_s[col4 * 4 + 1], d2 = d_s[col4 * 4 + 2], d3 = d_s[col4 * 4 + 3];
#pragma unroll
  for (int rr = 0; rr < RPT; ++rr) {
    const int r = rg + rr * RPP;
    if (r < D) {
      const float kr = u_s[D + r] * ks;
      f32x4v s = Sv[rr];
      s.x += kr * d0; s.y += kr * d1; s.z += kr * d2; s.w += kr * d3;
      __builtin_nontemporal_store(s, &Sp[static_cast<size_t>(r) * C4 + col4]);
    }
  }
}

// K tokens per sequence (multi-token decode, speculative verify and commit),
// the state and conv history found in pools through a slot per sequence.
// The state is read once; the per-token steps are those of decode_kernel.
// The state after the first `commit` tokens goes back to the pool (none for
// 0), and so does the conv history after them; every token's output is
// written.  GATED: every token's output row goes through the epilogue, as in
// decode_kernel.
// Four waves per (sequence, head), each thread holding 16 state rows of one
// float4 column (at dk = 128): the state is most of a thread's registers, and
// three states fit on a compute unit at once (eight-wave workgroups fit two,
// their other registers costing as much as the state).  Tokens go in groups:
// the conv, SiLU and norms of a group's tokens do not depend on the state and
// are computed for the whole group first, so each token's serial part is the
// pass over the state, one reduction and the update (two barriers).  The
// conv windows of the 3 dk channels live in shared memory.
template <int D, bool IO_BF16, bool OUT_BF16, bool GATED>
__global__ __launch_bounds__(kMultiThreads) __attribute__((amdgpu_waves_per_eu(3)))
void decode_multi_kernel(Params p, DecodeMultiIO io, int K) {
  constexpr int NT = kMultiThreads;
  constexpr int NW = NT / kWave;
  constexpr int C4 = D / 4;
  constexpr int RPP = NT / C4;
  constexpr int RPT = (D + RPP - 1) / RPP;
  constexpr int KG = kMultiGroup;
  constexpr int NC = 3 * D;                        // conv channels
  constexpr int CPT = (NC + NT - 1) / NT;          // ... per thread
  static_assert(D <= NT, "one gate channel per thread");
  __shared__ float u_s[KG][NC];      // ... after conv + SiLU
  __shared__ float eg_s[KG][D];      // exp(g) of the group's tokens
  __shared__ float b_s[KG];          // beta of the group's tokens
  __shared__ float nrm_s[KG][3];     // |u_q|^2, |u_k|^2, u_q . u_k
  __shared__ float win_s[3][NC];     // each channel's last three raw inputs
  __shared__ float kwin_s[3][NC];    // ... after the committed tokens
  __shared__ float red[2][RPP][D];
  __shared__ float d_s[D];
  constexpr int OW = (D + kWave - 1) / kWave;
  __shared__ float osum[OW];

  const int tid = threadIdx.x;
  const int H = p.H;
  const int n = blockIdx.x / H, h = blockIdx.x % H;
  const int slot = io.slots ? io.slots[n] : n;
  if (slot < 0) return;
  const int commit = io.n_commit ? min(max(io.n_commit[n], 0), K) : K;
  const size_t HD = static_cast<size_t>(H) * D;
  const size_t Ctot = 3 * HD;
  const uint32_t flags = p.flags;

  const int col4 = tid % C4, rg = tid / C4;
  // The small inputs go out first, all unconditionally (a load under a
  // condition compiles to a branch that waits for it; lanes without a channel
  // read a valid one and ignore it): the conv taps, the pooled history and the
  // first group's inputs.  Then the state tile: the memory counter drains in
  // issue order, so the first group's preprocess runs while it arrives.
  float wt[CPT][4], hist[CPT][3];
#pragma unroll
  for (int m = 0; m < CPT; ++m) {
    const int c = min(tid + m * NT, NC - 1);
    const int grp = c / D, ci = c % D;
    const size_t cb = static_cast<size_t>(slot) * 3 * Ctot + static_cast<size_t>(grp) * HD +
                      static_cast<size_t>(h) * D + ci;
    const void* w = grp == 0 ? p.wq : (grp == 1 ? p.wk : p.wv);
    const size_t wi = (static_cast<size_t>(h) * D + ci) * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) wt[m][j] = ld<IO_BF16>(w, wi + j);
#pragma unroll
    for (int j = 0; j < 3; ++j) hist[m][j] = ld<IO_BF16>(io.conv_pool, cb + j * Ctot);
  }
  const float dtb = p.dt_bias[h * D + tid % D];
  float onw = 0.f;
  if constexpr (GATED) onw = io.onw[tid % D];
  float xr[KG][CPT], ar[KG], br;           // a group's raw inputs, alphas and this lane's beta input
  auto load_group = [&](int t0, int kg) {
#pragma unroll
    for (int j = 0; j < KG; ++j) {
      const size_t tok = static_cast<size_t>(n) * K + t0 + min(j, kg - 1);
#pragma unroll
      for (int m = 0; m < CPT; ++m) {
        const int c = min(tid + m * NT, NC - 1);
        const int grp = c / D, ci = c % D;
        const void* xsrc = grp == 0 ? io.q : (grp == 1 ? io.k : io.v);
        xr[j][m] = ld<IO_BF16>(xsrc, tok * HD + static_cast<size_t>(h) * D + ci);
      }
      ar[j] = ld<IO_BF16>(io.alpha, tok * HD + static_cast<size_t>(h) * D + tid % D);
    }
    br = ld<IO_BF16>(io.b, (static_cast<size_t>(n) * K + t0 + min(tid, kg - 1)) * H + h);
  };
  if (K > 0) load_group(0, min(KG, K));
  __builtin_amdgcn_sched_barrier(0);
  f32x4v* Sp = reinterpret_cast<f32x4v*>(io.state_pool + (static_cast<size_t>(slot) * H + h) * D * D);
  f32x4v Sv[RPT];
#pragma unroll
  for (int rr = 0; rr < RPT; ++rr) {
    const int r = rg + rr * RPP;
    if (r < D) Sv[rr] = __builtin_nontemporal_load(&Sp[static_cast<size_t>(r) * C4 + col4]);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int m = 0; m < CPT; ++m) {
    const int c = tid + m * NT;
    if (c < NC) {
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        win_s[j][c] = hist[m][j];
        kwin_s[j][c] = hist[m][j];
      }
    }
  }
  const float a_exp = expf(p.A_log[h]);
  const bool norm = !(flags & KDA_FLAG_SKIP_L2NORM);

  for (int t0 = 0; t0 < K; t0 += KG) {
    const int kg = min(KG, K - t0);
    if (t0 > 0) load_group(t0, kg);
    {
      // conv + SiLU of the group's tokens, channel by channel (the window in
      // registers for the group, back in shared memory after it)
#pragma unroll
      for (int m = 0; m < CPT; ++m) {
        const int c = tid + m * NT;
        if (c < NC) {
          float h0 = win_s[0][c], h1 = win_s[1][c], h2 = win_s[2][c];
#pragma unroll
          for (int j = 0; j < KG; ++j) {
            if (j < kg) {
              const float xt = xr[j][m];
              u_s[j][c] = (flags & KDA_FLAG_SKIP_CONV)
                              ? xt : siluf_(wt[m][0] * h0 + wt[m][1] * h1 + wt[m][2] * h2 + wt[m][3] * xt);
              h0 = h1; h1 = h2; h2 = xt;
              if (t0 + j + 1 == commit) {
                kwin_s[0][c] = h0;
                kwin_s[1][c] = h1;
                kwin_s[2][c] = h2;
              }
            }
          }
          win_s[0][c] = h0;
          win_s[1][c] = h1;
          win_s[2][c] = h2;
        }
      }
#pragma unroll
      for (int j = 0; j < KG; ++j) {
        if (tid < D) {
          const float g = (flags & KDA_FLAG_RAW_GATE) ? ar[j] : gate_value(ar[j], dtb, a_exp, p.lower_bound);
          eg_s[j][tid] = expf(g);
        }
      }
      if (tid < kg) {
        float be = (flags & KDA_FLAG_RAW_BETA) ? br : sigmoidf_(br);
        if (flags & KDA_FLAG_BETA_X2) be *= 2.0f;
        b_s[tid] = be;
      }
    }
    __syncthreads();
    // |u_q|^2, |u_k|^2 and u_q . u_k of every token of the group, a wave per task
    {
      const int wv = tid / kWave, lane = tid % kWave;
      for (int task = wv; task < 3 * kg; task += NW) {
        const int j = task / 3, ty = task % 3;
        float sum = 0.0f;
        for (int i = lane; i < D; i += kWave) {
          const float a = u_s[j][(ty == 1 ? D : 0) + i];
          const float b2 = u_s[j][(ty == 0 ? 0 : D) + i];
          sum += a * b2;
        }
        sum = group_sum<kWave>(sum);
        if (lane == 0) nrm_s[j][ty] = sum;
      }
    }
    __syncthreads();

    for (int j = 0; j < kg; ++j) {
      const int t = t0 + j;
      const size_t tok = static_cast<size_t>(n) * K + t;
      const float iq = norm ? 1.0f / sqrtf(nrm_s[j][0] + p.eps) : 1.0f;
      const float ik = norm ? 1.0f / sqrtf(nrm_s[j][1] + p.eps) : 1.0f;
      const float qs = iq * p.scale, ks = ik, beta = b_s[j], qk = nrm_s[j][2] * iq * ik * p.scale;
      float graw = 0.f;   // the epilogue's gate of this token (every lane loads a valid one)
      if constexpr (GATED) graw = ld<IO_BF16>(io.gate, tok * HD + static_cast<size_t>(h) * D + tid % D);

      float pk[4] = {0.f, 0.f, 0.f, 0.f}, pq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int rr = 0; rr < RPT; ++rr) {
        const int r = rg + rr * RPP;
        if (r < D) {
          const float e = eg_s[j][r];
          Sv[rr].x *= e; Sv[rr].y *= e; Sv[rr].z *= e; Sv[rr].w *= e;
          const float kr = u_s[j][D + r] * ks, qr = u_s[j][r] * qs;
          pk[0] += kr * Sv[rr].x; pk[1] += kr * Sv[rr].y; pk[2] += kr * Sv[rr].z; pk[3] += kr * Sv[rr].w;
          pq[0] += qr * Sv[rr].x; pq[1] += qr * Sv[rr].y; pq[2] += qr * Sv[rr].z; pq[3] += qr * Sv[rr].w;
        }
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        red[0][rg][col4 * 4 + jj] = pk[jj];
        red[1][rg][col4 * 4 + jj] = pq[jj];
      }
      __syncthreads();   // red is complete; d_s and osum are free (read before the last barrier)
      float gsig = 0.f;
      if constexpr (GATED) gsig = sigmoidf_(graw);
      float o_c = 0.f;
      if (tid < D) {
        const int c = tid;
        float pp = 0.f, rq = 0.f;
#pragma unroll
        for (int g2 = 0; g2 < RPP; ++g2) { pp += red[0][g2][c]; rq += red[1][g2][c]; }
        const float delta = beta * (u_s[j][2 * D + c] - pp);
        d_s[c] = delta;
        o_c = rq + qk * delta;
        if constexpr (!GATED) st<OUT_BF16>(io.o, tok * HD + static_cast<size_t>(h) * D + c, o_c);
      }
      if constexpr (GATED) {
        if (tid < OW * kWave) {
          const float ss = group_sum<kWave>(o_c * o_c);
          if ((tid % kWave) == 0) osum[tid / kWave] = ss;
        }
      }
      __syncthreads();   // d_s and osum are complete; red is free
      if constexpr (GATED) {
        if (tid < D) {
          float ss = 0.f;
#pragma unroll
          for (int w = 0; w < OW; ++w) ss += osum[w];
          const float inv = 1.0f / sqrtf(ss * (1.0f / D) + io.oeps);
          st<OUT_BF16>(io.o, tok * HD + static_cast<size_t>(h) * D + tid, o_c * inv * onw * gsig);
        }
      }
      const float d0 = d_s[col4 * 4], d1 = d_s[col4 * 4 + 1], d2 = d_s[col4 * 4 + 2], d3 = d_s[col4 * 4 + 3];
#pragma unroll
      for (int rr = 0; rr < RPT; ++rr) {
        const int r = rg + rr * RPP;
        if (r < D) {
          const float kr = u_s[j][D + r] * ks;
          Sv[rr].x += kr * d0; Sv[rr].y += kr * d1; Sv[rr].z += kr * d2; Sv[rr].w += kr * d3;
          if (t + 1 == commit) __builtin_nontemporal_store(Sv[rr], &Sp[static_cast<size_t>(r) * C4 + col4]);
        }
      }
    }
    __syncthreads();   // u_s, eg_s, b_s, nrm_s, d_s and osum are rewritten by the next group
  }
  if (commit > 0) {
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
      const int c = tid + m * NT;
      if (c < NC) {
        const int grp = c / D, ci = c % D;
        const size_t cb = static_cast<size_t>(slot) * 3 * Ctot + static_cast<size_t>(grp) * HD +
                          static_cast<size_t>(h) * D + ci;
#pragma unroll
        for (int j = 0; j < 3; ++j) st<IO_BF16>(io.conv_pool, cb + j * Ctot, kwin_s[j][c]);
      }
    }
  }
}

template <int D, bool GATED>
static hipError_t launch_decode_multi_g(const Params& p, const DecodeMultiIO& io, int N, int K, bool io_bf16,
                                        bool out_bf16, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(N) * p.H), block(kMultiThreads);
  if (io_bf16 && out_bf16) decode_multi_kernel<D, true, true, GATED><<<grid, block, 0, st>>>(p, io, K);
  else if (io_bf16) decode_multi_kernel<D, true, false, GATED><<<grid, block, 0, st>>>(p, io, K);
  else if (out_bf16) decode_multi_kernel<D, false, true, GATED><<<grid, block, 0, st>>>(p, io, K);
  else decode_multi_kernel<D, false, false, GATED><<<grid, block, 0, st>>>(p, io, K);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_decode_multi_d(const Params& p, const DecodeMultiIO& io, int N, int K, bool io_bf16,
                                        bool out_bf16, hipStream_t st) {
  return io.gate ? launch_decode_multi_g<D, true>(p, io, N, K, io_bf16, out_bf16, st)
                 : launch_decode_multi_g<D, false>(p, io, N, K, io_bf16, out_bf16, st);
}

hipError_t launch_decode_multi(const Params& p, const DecodeMultiIO& io, int N, int K, bool io_bf16, bool out_bf16,
                               hipStream_t st) {
  switch (p.D) {
    case 16: return launch_decode_multi_d<16>(p, io, N, K, io_bf16, out_bf16, st);
    case 32: return launch_decode_multi_d<32>(p, io, N, K, io_bf16, out_bf16, st);
    case 64: return launch_decode_multi_d<64>(p, io, N, K, io_bf16, out_bf16, st);
    case 128: return launch_decode_multi_d<128>(p, io, N, K, io_bf16, out_bf16, st);
    default: return hipErrorInvalidValue;
  }
}

template <int D, bool GATED>
static hipError_t launch_decode_g(const Params& p, const DecodeIO& io, int N, bool io_bf16, bool out_bf16,
                                  hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(N) * p.H), block(kDecodeThreads);
  if (io_bf16 && out_bf16) decode_kernel<D, true, true, GATED><<<grid, block, 0, st>>>(p, io);
  else if (io_bf16) decode_kernel<D, true, false, GATED><<<grid, block, 0, st>>>(p, io);
  else if (out_bf16) decode_kernel<D, false, true, GATED><<<grid, block, 0, st>>>(p, io);
  else decode_kernel<D, false, false, GATED><<<grid, block, 0, st>>>(p, io);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_decode_d(const Params& p, const DecodeIO& io, int N, bool io_bf16, bool out_bf16,
                                  hipStream_t st) {
  return io.gate ? launch_decode_g<D, true>(p, io, N, io_bf16, out_bf16, st)
                 : launch_decode_g<D, false>(p, io, N, io_bf16, out_bf16, st);
}

hipError_t launch_decode(const Params& p, const DecodeIO& io, int N, bool io_bf16, bool out_bf16, hipStream_t st) {
  switch (p.D) {
    case 16: return launch_decode_d<16>(p, io, N, io_bf16, out_bf16, st);
    case 32: return launch_decode_d<32>(p, io, N, io_bf16, out_bf16, st);
    case 64: return launch_decode_d<64>(p, io, N, io_bf16, out_bf16, st);
    case 128: return launch_decode_d<128>(p, io, N, io_bf16, out_bf16, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kda
