// Prefill preprocess: depthwise causal conv1d (kernel 4, padding 3, no bias)
// + SiLU for the q, k, v channels, L2 normalisation of q and k per head, the
// per-channel gate g = max(-exp(A_log) softplus(alpha + dt_bias), lb) and
// beta = sigmoid(b) (AliceAI page, section 二; safe-gate bound from the
// Ling-3.0-flash-VL page, section "KDA 层的安全门").
//
// One workgroup per (chunk, head).  Three lane groups of D/2 lanes own the q,
// k and v channels of the head, two adjacent channels per lane, so every raw
// row of a head is read as one contiguous run of D bf16 values.  Each lane
// slides the 4-tap window down the chunk's tokens; the three inputs before
// the chunk come from the same sequence or, at its start, from the incoming
// conv history.  The q and k norms are lane-group shuffle reductions.
// Output tiles are chunk-major, [chunk][head][64][D] fp32; rows past the end
// of a partial chunk are written as zeros (with g = 0 and beta = 0 such a row
// is an exact identity step of the recurrence).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <int D, bool IO_BF16>
__global__ __launch_bounds__(3 * D / 2) void preprocess_kernel(Params p, ChunkTable t, PrefillIO io,
                                                               ChunkBuffers b) {
  constexpr int G = D / 2;  // lanes per channel group
  const int c = blockIdx.x, h = blockIdx.y;
  if (c >= t.chunk0[t.N]) return;
  const int H = p.H;
  const int s = t.chunk_seq[c];
  const int tau0 = (c - t.chunk0[s]) * kChunk;           // chunk offset inside its sequence
  const int64_t tok0 = static_cast<int64_t>(t.cu[s]) + tau0;
  const int len = min(kChunk, t.cu[s + 1] - static_cast<int>(tok0));
  const int tid = threadIdx.x;
  const int grp = tid / G, lane = tid % G;
  const int i = 2 * lane;                                  // first of this lane's two channels
  const size_t HD = static_cast<size_t>(H) * D;
  const size_t Ctot = 3 * HD;
  const void* x = grp == 0 ? io.q : (grp == 1 ? io.k : io.v);
  const void* w = grp == 0 ? p.wq : (grp == 1 ? p.wk : p.wv);
  const size_t col = static_cast<size_t>(h) * D + i;       // column in the [*, H*D] raw row
  const uint32_t flags = p.flags;

  // conv taps of the two channels
  float w0[4], w1[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    w0[j] = ld<IO_BF16>(w, col * 4 + j);
    w1[j] = ld<IO_BF16>(w, (col + 1) * 4 + j);
  }
  // the three inputs before the first token of the chunk
  float2 hm3, hm2, hm1;
  {
    float2 hv[3];
#pragma unroll
    for (int m = 0; m < 3; ++m) {
      const int tau = tau0 - 3 + m;
      if (tau >= 0) {
        hv[m] = ld2<IO_BF16>(x, static_cast<size_t>(t.cu[s] + tau) * HD + col);
      } else if (io.conv_in) {
        const size_t ci = (static_cast<size_t>(s) * 3 + (3 + tau)) * Ctot + grp * HD + col;
        hv[m] = ld2<IO_BF16>(io.conv_in, ci);
      } else {
        hv[m] = make_float2(0.f, 0.f);
      }
    }
    hm3 = hv[0]; hm2 = hv[1]; hm1 = hv[2];
  }
  const float a_exp = expf(p.A_log[h]);
  const float2 dtb = grp == 0 ? *reinterpret_cast<const float2*>(p.dt_bias + col) : make_float2(0.f, 0.f);
  const size_t tile = (static_cast<size_t>(c) * H + h) * kChunk;   // row index of this tile
  float* out = grp == 0 ? b.qh : (grp == 1 ? b.kh : b.vh);

  for (int r = 0; r < kChunk; ++r) {
    float2 u = make_float2(0.f, 0.f);
    if (r < len) {
      const float2 xt = ld2<IO_BF16>(x, static_cast<size_t>(tok0 + r) * HD + col);
      if (flags & KDA_FLAG_SKIP_CONV) {
        u = xt;
      } else {
        const float y0 = w0[0] * hm3.x + w0[1] * hm2.x + w0[2] * hm1.x + w0[3] * xt.x;
        const float y1 = w1[0] * hm3.y + w1[1] * hm2.y + w1[2] * hm1.y + w1[3] * xt.y;
        u = make_float2(siluf_(y0), siluf_(y1));
      }
      hm3 = hm2; hm2 = hm1; hm1 = xt;
    }
    // every group reduces (keeps the shuffles uniform); only q and k use it
    const float ss = group_sum<G>(u.x * u.x + u.y * u.y);
    if (grp < 2 && !(flags & KDA_FLAG_SKIP_L2NORM)) {
      const float inv = 1.0f / sqrtf(ss + p.eps);
      u.x *= inv; u.y *= inv;
    }
    if (grp == 0) { u.x *= p.scale; u.y *= p.scale; }
    *reinterpret_cast<float2*>(out + (tile + r) * D + i) = u;
    if (grp == 0) {
      float2 g = make_float2(0.f, 0.f);
      if (r < len) {
        const float2 al = ld2<IO_BF16>(io.alpha, static_cast<size_t>(tok0 + r) * HD + col);
        if (flags & KDA_FLAG_RAW_GATE) {
          g = al;
        } else {
          g.x = gate_value(al.x, dtb.x, a_exp, p.lower_bound);
          g.y = gate_value(al.y, dtb.y, a_exp, p.lower_bound);
        }
      }
      *reinterpret_cast<float2*>(b.g + (tile + r) * D + i) = g;
      if (lane == 0) {
        float be = 0.f;
        if (r < len) {
          const float bb = ld<IO_BF16>(io.b, static_cast<size_t>(tok0 + r) * H + h);
          be = (flags & KDA_FLAG_RAW_BETA) ? bb : sigmoidf_(bb);
          if (flags & KDA_FLAG_BETA_X2) be *= 2.0f;
        }
        b.beta[tile + r] = be;
      }
    }
  }
}

template <int D>
static hipError_t launch_pre_d(const Params& p, const ChunkTable& t, const PrefillIO& io, const ChunkBuffers& b,
                               int max_chunks, bool io_bf16, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(max_chunks), static_cast<unsigned>(p.H));
  if (io_bf16) preprocess_kernel<D, true><<<grid, 3 * D / 2, 0, st>>>(p, t, io, b);
  else preprocess_kernel<D, false><<<grid, 3 * D / 2, 0, st>>>(p, t, io, b);
  return hipGetLastError();
}

hipError_t launch_preprocess(const Params& p, const ChunkTable& t, const PrefillIO& io, const ChunkBuffers& b,
                             int max_chunks, bool io_bf16, hipStream_t st) {
  switch (p.D) {
    case 16: return launch_pre_d<16>(p, t, io, b, max_chunks, io_bf16, st);
    case 32: return launch_pre_d<32>(p, t, io, b, max_chunks, io_bf16, st);
    case 64: return launch_pre_d<64>(p, t, io, b, max_chunks, io_bf16, st);
    case 128: return launch_pre_d<128>(p, t, io, b, max_chunks, io_bf16, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kda
