// Packed-batch bookkeeping for the chunked prefill.
//
// build_chunks_kernel turns sequence offsets (device cu_seqlens, or B equal
// lengths) into a chunk table without any host synchronisation: chunk0[s] is
// the first 64-token chunk of sequence s (an exclusive scan of ceil(len/64)),
// chunk0[N] the number of chunks, chunk_seq[c] the sequence owning chunk c and
// desc[c] where chunk c lies.  A table may cover a window of positions
// [s0, s0 + span) of every sequence (the prefill run in slabs); its chunks
// keep their positions in the whole sequence.
// Chunks never straddle two sequences; the last chunk of a sequence may be
// partial.  Grids of the chunk kernels are sized by a host upper bound and
// blocks past chunk0[N] exit.
//
// It also picks the scan's value-tile width for packed batches of unequal
// lengths (chunk0[N+1]): the scan's length is that of its longest
// sequences, and when those (the ones with more than half the longest
// one's chunks) cannot give every compute unit a workgroup at the wide tile
// (64 value columns), the narrow one (32) halves the work of each chunk
// step on that critical path.  Measured on eight packed sequences of
// 1K..129K tokens (32 heads, dk = dv = 128), the narrow tile took the varlen
// prefill from 17.2 to 15.3 ms; on four equal 32K sequences it was slower
// (2.81 ms against 2.31 ms for the scan), which the rule leaves wide.
//
// conv_state_out_kernel writes each sequence's conv history for continuation:
// its last three raw inputs per channel (reaching into the incoming history
// when the sequence is shorter than three tokens), oldest first.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

__global__ __launch_bounds__(1024) void build_chunks_kernel(const int32_t* __restrict__ cu_in, int32_t N,
                                                            int32_t T_uniform, int32_t* __restrict__ cu_ws,
                                                            int32_t* __restrict__ chunk0, int32_t long_tiles,
                                                            int32_t ncu, int32_t s0, int32_t span) {
  __shared__ int32_t scan[1024];
  __shared__ int32_t carry_s, max_s, long_s, carry_l, carry_o;
  const int tid = threadIdx.x;
  auto chunks_of = [&](int s) {   // chunks of the sequence's positions [s0, s0 + span)
    const int len = cu_in ? (cu_in[s + 1] - cu_in[s]) : T_uniform;
    const int in = min(max(len - s0, 0), span);
    return (in + kChunk - 1) / kChunk;
  };
  for (int s = tid; s <= N; s += 1024) cu_ws[s] = cu_in ? cu_in[s] : s * T_uniform;
  if (tid == 0) {
    carry_s = 0;
    max_s = 0;
    long_s = 0;
  }
  __syncthreads();
  for (int base = 0; base < N; base += 1024) {
    const int s = base + tid;
    const int nc = s < N ? chunks_of(s) : 0;
    int wmax = nc;   // one shared atomic per wave
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) wmax = max(wmax, __shfl_xor(wmax, m));
    if ((tid & 63) == 0) atomicMax(&max_s, wmax);
    scan[tid] = nc;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int add = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    const int carry = carry_s;
    if (s < N) chunk0[s] = carry + scan[tid] - nc;
    __syncthreads();
    if (tid == 0) carry_s = carry + scan[1023];
    __syncthreads();
  }
  // the value-tile choice: long_tiles = wide tiles per (sequence, head) of
  // the long sequences, summed over them against the compute units
  const int mx = max_s;
  int n_long = 0;
  if (cu_in) {
    for (int s = tid; s < N; s += 1024) n_long += 2 * chunks_of(s) > mx ? 1 : 0;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) n_long += __shfl_xor(n_long, m);
    if ((tid & 63) == 0) atomicAdd(&long_s, n_long);
  } else if (tid == 0) {
    long_s = mx > 0 ? N : 0;   // equal lengths: every sequence is a long one
  }
  __syncthreads();
  if (tid == 0) {
    chunk0[N] = carry_s;
    chunk0[N + 1] = static_cast<int64_t>(long_s) * long_tiles < ncu ? 1 : 0;
  }
  // the scan's dispatch order: the long sequences first, then the others,
  // each in index order (a stable partition; within a block the two counts
  // travel packed in one prefix sum, 16 bits each, a block holding at most
  // 1024 sequences).  Workgroups start in launch order, so a long sequence's
  // serial chain would otherwise wait for the short ones before it.
  const int n_long_total = cu_in ? long_s : N;
  int32_t* order = chunk0 + N + 2;
  if (tid == 0) {
    carry_l = 0;
    carry_o = 0;
  }
  for (int base = 0; base < N; base += 1024) {
    const int s = base + tid;
    const bool lg = s < N && (!cu_in || 2 * chunks_of(s) > mx);
    const int packed = s < N ? (lg ? 1 : 1 << 16) : 0;
    __syncthreads();   // the previous block's reads of scan[] and of the carries are done
    scan[tid] = packed;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int add = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    const int ex = scan[tid] - packed;   // this block's sequences before s, packed
    if (s < N) order[lg ? carry_l + (ex & 0xffff) : n_long_total + carry_o + (ex >> 16)] = s;
    __syncthreads();
    if (tid == 0) {
      carry_l += scan[1023] & 0xffff;
      carry_o += scan[1023] >> 16;
    }
  }
}

// chunk_seq[c] = the last sequence whose first chunk is <= c (empty sequences
// share their successor's first chunk and are skipped this way), and the
// chunk's descriptor (sequence, first token within it, token count, first
// packed token), so that a kernel finds a chunk's place with one load.  A
// separate launch, so that every chunk0 and cu entry written above is visible.
__global__ __launch_bounds__(256) void fill_chunk_seq_kernel(const int32_t* __restrict__ chunk0,
                                                             const int32_t* __restrict__ cu, int32_t N,
                                                             int32_t* __restrict__ chunk_seq, int4* __restrict__ desc,
                                                             int32_t max_chunks, int32_t s0) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= max_chunks || c >= chunk0[N]) return;
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (chunk0[mid] <= c) lo = mid; else hi = mid - 1;
  }
  chunk_seq[c] = lo;
  const int tau0 = s0 + (c - chunk0[lo]) * kChunk;
  const int tok0 = cu[lo] + tau0;
  desc[c] = make_int4(lo, tau0, min(kChunk, cu[lo + 1] - tok0), tok0);
}

// The compute-unit count of the current device, queried on every call (the
// runtime answers from its own device table): the library keeps no state.
hipError_t device_cus(int* ncu) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  return hipDeviceGetAttribute(ncu, hipDeviceAttributeMultiprocessorCount, dev);
}

hipError_t launch_build_chunks(const int32_t* cu_in, int32_t N, int32_t T_uniform, int32_t* cu_ws, int32_t* chunk0,
                               int32_t* chunk_seq, int4* desc, int32_t max_chunks, int32_t H, int32_t D,
                               hipStream_t st, int32_t s0, int32_t span) {
  int ncu = 0;
  hipError_t e0 = device_cus(&ncu);
  if (e0 != hipSuccess) return e0;
  const int long_tiles = H * (D >= 64 ? D / 64 : 1);
  build_chunks_kernel<<<1, 1024, 0, st>>>(cu_in, N, T_uniform, cu_ws, chunk0, long_tiles, ncu, s0, span);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || max_chunks <= 0) return e;
  fill_chunk_seq_kernel<<<(max_chunks + 255) / 256, 256, 0, st>>>(chunk0, cu_ws, N, chunk_seq, desc, max_chunks, s0);
  return hipGetLastError();
}

template <bool IO_BF16>
__global__ __launch_bounds__(256) void conv_state_out_kernel(ChunkTable t, PrefillIO io, int H, int D) {
  // one-dimensional grid: bps blocks of 256 channels per sequence (grid
  // dimension y holds at most 65536 sequences)
  const size_t Ctot = static_cast<size_t>(3) * H * D;
  const unsigned bps = static_cast<unsigned>((Ctot + 255) / 256);
  const int s = static_cast<int>(blockIdx.x / bps);
  const size_t c = static_cast<size_t>(blockIdx.x % bps) * 256 + threadIdx.x;
  if (c >= Ctot) return;
  const int64_t t0 = t.cu[s];
  const int L = t.cu[s + 1] - t.cu[s];
  const int grp = static_cast<int>(c / (static_cast<size_t>(H) * D));
  const size_t cc = c - static_cast<size_t>(grp) * H * D;
  const void* x = grp == 0 ? io.q : (grp == 1 ? io.k : io.v);
  float val[3];
#pragma unroll
  for (int m = 0; m < 3; ++m) {
    const int tt = L - 3 + m;
    if (tt >= 0) val[m] = ld<IO_BF16>(x, static_cast<size_t>(t0 + tt) * H * D + cc);
    else if (io.conv_in) val[m] = ld<IO_BF16>(io.conv_in, (static_cast<size_t>(s) * 3 + (3 + tt)) * Ctot + c);
    else val[m] = 0.0f;
  }
#pragma unroll
  for (int m = 0; m < 3; ++m) st<IO_BF16>(io.conv_out, (static_cast<size_t>(s) * 3 + m) * Ctot + c, val[m]);
}

hipError_t launch_conv_state_out(const Params& p, const ChunkTable& t, const PrefillIO& io, bool io_bf16,
                                 hipStream_t st) {
  const size_t Ctot = static_cast<size_t>(3) * p.H * p.D;
  const int64_t blocks = static_cast<int64_t>((Ctot + 255) / 256) * t.N;
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(blocks));
  if (io_bf16) conv_state_out_kernel<true><<<grid, 256, 0, st>>>(t, io, p.H, p.D);
  else conv_state_out_kernel<false><<<grid, 256, 0, st>>>(t, io, p.H, p.D);
  return hipGetLastError();
}

}  // namespace kda
