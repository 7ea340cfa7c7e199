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
// Tokens whose inputs the multi-token decode stages at once.
constexpr int kMultiGroup = 8;

template <int D, bool IO_BF16, bool OUT_BF16>
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

  const int tid = threadIdx.x;
  const int H = p.H;
  const int n = blockIdx.x / H, h = blockIdx.x % H;
  const size_t Ctot = static_cast<size_t>(3) * H * D;
  const uint32_t flags = p.flags;

  // ---- the state tile is requested first: its latency overlaps the preprocess
  const int col4 = tid % C4, rg = tid / C4;
  const size_t base = (static_cast<size_t>(n) * H + h) * D * D;
  f32x4v* Sp = reinterpret_cast<f32x4v*>(io.state + base);
  f32x4v Sv[RPT];
#pragma unroll
  for (int rr = 0; rr < RPT; ++rr) {
    const int r = rg + rr * RPP;
    if (r < D) Sv[rr] = __builtin_nontemporal_load(&Sp[static_cast<size_t>(r) * C4 + col4]);
  }

  // ---- preprocess: conv + SiLU for the 3D channels of this head; shift history
  for (int c = tid; c < 3 * D; c += NT) {
    const int grp = c / D, i = c % D;
    const size_t ch = static_cast<size_t>(grp) * H * D + static_cast<size_t>(h) * D + i;
    const void* x = grp == 0 ? io.q : (grp == 1 ? io.k : io.v);
    const void* w = grp == 0 ? p.wq : (grp == 1 ? p.wk : p.wv);
    const float xt = ld<IO_BF16>(x, static_cast<size_t>(n) * H * D + static_cast<size_t>(h) * D + i);
    const size_t cb = static_cast<size_t>(n) * 3 * Ctot + ch;
    const float h0 = ld<IO_BF16>(io.conv_state, cb);
    const float h1 = ld<IO_BF16>(io.conv_state, cb + Ctot);
    const float h2 = ld<IO_BF16>(io.conv_state, cb + 2 * Ctot);
    float u;
    if (flags & KDA_FLAG_SKIP_CONV) {
      u = xt;
    } else {
      const size_t wi = (static_cast<size_t>(h) * D + i) * 4;
      const float y = ld<IO_BF16>(w, wi) * h0 + ld<IO_BF16>(w, wi + 1) * h1 + ld<IO_BF16>(w, wi + 2) * h2 +
                      ld<IO_BF16>(w, wi + 3) * xt;
      u = siluf_(y);
    }
    st<IO_BF16>(io.conv_state, cb, h1);
    st<IO_BF16>(io.conv_state, cb + Ctot, h2);
    st<IO_BF16>(io.conv_state, cb + 2 * Ctot, xt);
    u_s[c] = u;
  }
  const float a_exp = expf(p.A_log[h]);
  for (int i = tid; i < D; i += NT) {
    const float al = ld<IO_BF16>(io.alpha, (static_cast<size_t>(n) * H + h) * D + i);
    const float g = (flags & KDA_FLAG_RAW_GATE) ? al : gate_value(al, p.dt_bias[h * D + i], a_exp, p.lower_bound);
    e_s[i] = expf(g);
  }
  if (tid == 0) {
    const float bb = ld<IO_BF16>(io.b, static_cast<size_t>(n) * H + h);
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
  for (int j = tid; j < D; j += NT) {
    float pp = 0.f, rq = 0.f;
#pragma unroll 8
    for (int g2 = 0; g2 < RPP; ++g2) { pp += red[0][g2][j]; rq += red[1][g2][j]; }
    const float delta = beta * (u_s[2 * D + j] - pp);
    d_s[j] = delta;
    st<OUT_BF16>(io.o, (static_cast<size_t>(n) * H + h) * D + j, rq + qk * delta);
  }
  __syncthreads();
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
// The state is read once; the per-token steps are those of decode_kernel,
// with the conv window of each channel kept in its thread's registers.  The
// state after the first `commit` tokens goes back to the pool (none for 0),
// and so does the conv history after them; every token's output is written.
template <int D, bool IO_BF16, bool OUT_BF16>
__global__ __launch_bounds__(kDecodeThreads) void decode_multi_kernel(Params p, DecodeMultiIO io, int K) {
  constexpr int NT = kDecodeThreads;
  constexpr int C4 = D / 4;
  constexpr int RPP = NT / C4;
  constexpr int RPT = (D + RPP - 1) / RPP;
  constexpr int KG = kMultiGroup;
  static_assert(3 * D <= NT && D <= NT, "one conv channel and one gate channel per thread");
  __shared__ float x_s[KG][3 * D];   // raw q | k | v of a group of tokens
  __shared__ float eg_s[KG][D];      // exp(g) of the group's tokens
  __shared__ float b_s[KG];          // beta of the group's tokens
  __shared__ float u_s[3 * D];
  __shared__ float red[2][RPP][D];
  __shared__ float d_s[D];
  __shared__ float scal[4];

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
  f32x4v* Sp = reinterpret_cast<f32x4v*>(io.state_pool + (static_cast<size_t>(slot) * H + h) * D * D);
  f32x4v Sv[RPT];
#pragma unroll
  for (int rr = 0; rr < RPT; ++rr) {
    const int r = rg + rr * RPP;
    if (r < D) Sv[rr] = __builtin_nontemporal_load(&Sp[static_cast<size_t>(r) * C4 + col4]);
  }

  // this thread's conv channel (q, k or v) and its window of raw inputs
  const bool conv_lane = tid < 3 * D;
  const int grp = tid / D, ci = tid % D;
  const size_t ch = static_cast<size_t>(grp) * HD + static_cast<size_t>(h) * D + ci;
  const size_t cb = static_cast<size_t>(slot) * 3 * Ctot + ch;
  float w0 = 0.f, w1 = 0.f, w2 = 0.f, w3 = 0.f, h0 = 0.f, h1 = 0.f, h2 = 0.f;
  const void* xsrc = grp == 0 ? io.q : (grp == 1 ? io.k : io.v);
  if (conv_lane) {
    const void* w = grp == 0 ? p.wq : (grp == 1 ? p.wk : p.wv);
    if (!(flags & KDA_FLAG_SKIP_CONV)) {
      const size_t wi = (static_cast<size_t>(h) * D + ci) * 4;
      w0 = ld<IO_BF16>(w, wi); w1 = ld<IO_BF16>(w, wi + 1); w2 = ld<IO_BF16>(w, wi + 2); w3 = ld<IO_BF16>(w, wi + 3);
    }
    h0 = ld<IO_BF16>(io.conv_pool, cb);
    h1 = ld<IO_BF16>(io.conv_pool, cb + Ctot);
    h2 = ld<IO_BF16>(io.conv_pool, cb + 2 * Ctot);
  }
  float k0 = h0, k1 = h1, k2 = h2;   // the window after the committed tokens
  const float a_exp = expf(p.A_log[h]);
  const float dtb = tid < D ? p.dt_bias[h * D + tid] : 0.f;

  for (int t0 = 0; t0 < K; t0 += KG) {
    // the group's raw inputs, gates and betas, all loads issued together (the
    // first group's right behind the state loads); the token loop below then
    // touches global memory only to store outputs
    const int kg = min(KG, K - t0);
    {
      float xr[KG], ar[KG];
      float br = 0.f;
#pragma unroll
      for (int j = 0; j < KG; ++j) {
        const size_t tok = static_cast<size_t>(n) * K + t0 + min(j, kg - 1);
        xr[j] = conv_lane ? ld<IO_BF16>(xsrc, tok * HD + static_cast<size_t>(h) * D + ci) : 0.f;
        ar[j] = tid < D ? ld<IO_BF16>(io.alpha, tok * HD + static_cast<size_t>(h) * D + tid) : 0.f;
      }
      if (tid < kg) br = ld<IO_BF16>(io.b, (static_cast<size_t>(n) * K + t0 + tid) * H + h);
#pragma unroll
      for (int j = 0; j < KG; ++j) {
        if (conv_lane) x_s[j][tid] = xr[j];
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

    for (int j = 0; j < kg; ++j) {
      const int t = t0 + j;
      const size_t tok = static_cast<size_t>(n) * K + t;
      if (conv_lane) {
        const float xt = x_s[j][tid];
        u_s[tid] = (flags & KDA_FLAG_SKIP_CONV) ? xt : siluf_(w0 * h0 + w1 * h1 + w2 * h2 + w3 * xt);
        h0 = h1; h1 = h2; h2 = xt;
        if (t + 1 == commit) { k0 = h0; k1 = h1; k2 = h2; }
      }
      __syncthreads();
      {
        const int wv = tid / kWave, lane = tid % kWave;
        if (wv < 3) {
          float sum = 0.0f;
          for (int i = lane; i < D; i += kWave) {
            const float a = u_s[(wv == 1 ? D : 0) + i];
            const float b2 = u_s[(wv == 0 ? 0 : D) + i];
            sum += a * b2;
          }
          sum = group_sum<kWave>(sum);
          if (lane == 0) scal[wv == 2 ? 3 : wv] = sum;
        }
      }
      __syncthreads();
      const bool norm = !(flags & KDA_FLAG_SKIP_L2NORM);
      const float iq = norm ? 1.0f / sqrtf(scal[0] + p.eps) : 1.0f;
      const float ik = norm ? 1.0f / sqrtf(scal[1] + p.eps) : 1.0f;
      const float qs = iq * p.scale, ks = ik, beta = b_s[j], qk = scal[3] * iq * ik * p.scale;

      float pk[4] = {0.f, 0.f, 0.f, 0.f}, pq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int rr = 0; rr < RPT; ++rr) {
        const int r = rg + rr * RPP;
        if (r < D) {
          const float e = eg_s[j][r];
          Sv[rr].x *= e; Sv[rr].y *= e; Sv[rr].z *= e; Sv[rr].w *= e;
          const float kr = u_s[D + r] * ks, qr = u_s[r] * qs;
          pk[0] += kr * Sv[rr].x; pk[1] += kr * Sv[rr].y; pk[2] += kr * Sv[rr].z; pk[3] += kr * Sv[rr].w;
          pq[0] += qr * Sv[rr].x; pq[1] += qr * Sv[rr].y; pq[2] += qr * Sv[rr].z; pq[3] += qr * Sv[rr].w;
        }
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        red[0][rg][col4 * 4 + jj] = pk[jj];
        red[1][rg][col4 * 4 + jj] = pq[jj];
      }
      __syncthreads();
      for (int c = tid; c < D; c += NT) {
        float pp = 0.f, rq = 0.f;
#pragma unroll 8
        for (int g2 = 0; g2 < RPP; ++g2) { pp += red[0][g2][c]; rq += red[1][g2][c]; }
        const float delta = beta * (u_s[2 * D + c] - pp);
        d_s[c] = delta;
        st<OUT_BF16>(io.o, tok * HD + static_cast<size_t>(h) * D + c, rq + qk * delta);
      }
      __syncthreads();
      const float d0 = d_s[col4 * 4], d1 = d_s[col4 * 4 + 1], d2 = d_s[col4 * 4 + 2], d3 = d_s[col4 * 4 + 3];
#pragma unroll
      for (int rr = 0; rr < RPT; ++rr) {
        const int r = rg + rr * RPP;
        if (r < D) {
          const float kr = u_s[D + r] * ks;
          Sv[rr].x += kr * d0; Sv[rr].y += kr * d1; Sv[rr].z += kr * d2; Sv[rr].w += kr * d3;
          if (t + 1 == commit) __builtin_nontemporal_store(Sv[rr], &Sp[static_cast<size_t>(r) * C4 + col4]);
        }
      }
      __syncthreads();   // u_s, d_s and scal are rewritten by the next token, x_s / eg_s by the next group
    }
  }
  if (conv_lane && commit > 0) {
    st<IO_BF16>(io.conv_pool, cb, k0);
    st<IO_BF16>(io.conv_pool, cb + Ctot, k1);
    st<IO_BF16>(io.conv_pool, cb + 2 * Ctot, k2);
  }
}

template <int D>
static hipError_t launch_decode_multi_d(const Params& p, const DecodeMultiIO& io, int N, int K, bool io_bf16,
                                        bool out_bf16, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(N) * p.H), block(kDecodeThreads);
  if (io_bf16 && out_bf16) decode_multi_kernel<D, true, true><<<grid, block, 0, st>>>(p, io, K);
  else if (io_bf16) decode_multi_kernel<D, true, false><<<grid, block, 0, st>>>(p, io, K);
  else if (out_bf16) decode_multi_kernel<D, false, true><<<grid, block, 0, st>>>(p, io, K);
  else decode_multi_kernel<D, false, false><<<grid, block, 0, st>>>(p, io, K);
  return hipGetLastError();
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

template <int D>
static hipError_t launch_decode_d(const Params& p, const DecodeIO& io, int N, bool io_bf16, bool out_bf16,
                                  hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(N) * p.H), block(kDecodeThreads);
  if (io_bf16 && out_bf16) decode_kernel<D, true, true><<<grid, block, 0, st>>>(p, io);
  else if (io_bf16) decode_kernel<D, true, false><<<grid, block, 0, st>>>(p, io);
  else if (out_bf16) decode_kernel<D, false, true><<<grid, block, 0, st>>>(p, io);
  else decode_kernel<D, false, false><<<grid, block, 0, st>>>(p, io);
  return hipGetLastError();
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
