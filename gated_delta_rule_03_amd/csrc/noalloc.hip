// kda_varlen_prefill_noalloc: the packed prefill for callers that cannot
// allocate device memory (code under HIP graph capture, serving loops that
// forbid allocation).  Its workspace is a fixed array in the library's own
// device memory, one copy per GPU, held until the process ends; the call
// itself allocates nothing.
#include <mutex>

#include "kda_internal.h"

namespace {

// The scratch array.  In host code its name is only a stand-in for the
// device symbol: host code uses the address hipGetSymbolAddress returns for
// the current device, never the name.
static __device__ __align__(256) uint8_t scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];
hipError_t g_status[kMaxDevices];

// The scratch address on the current device, looked up once per device (with
// that device current) and kept.
hipError_t scratch_address(void** out) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch[dev] = p;
  });
  if (g_status[dev] != hipSuccess) return g_status[dev];
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" kda_status_t kda_varlen_prefill_noalloc(const kda_config_t* cfg, int32_t N, int32_t total_T,
                                                   const int32_t* cu_seqlens, const void* q, const void* k,
                                                   const void* v, const void* alpha, const void* b,
                                                   const float* initial_state, const void* conv_state_in, void* o,
                                                   float* final_state, void* conv_state_out, void* stream) {
  // sizes before any device call: a batch whose workspace exceeds the
  // scratch runs in slabs (chunked form), and is refused when not even a
  // slab of 64 tokens per sequence fits; an invalid configuration or size
  // (query answer 0) and the empty batch take the ordinary entry point's
  // checks and answer
  const size_t need = kda_varlen_workspace_bytes(cfg, N, total_T);
  if (need == 0 || N == 0)
    return kda_varlen_prefill(cfg, N, total_T, cu_seqlens, q, k, v, alpha, b, initial_state, conv_state_in, o,
                              final_state, conv_state_out, nullptr, 0, stream);
  if (need > KDA_NOALLOC_SCRATCH_BYTES) {
    const size_t slab_need = kda_prefill_slab_workspace_bytes(cfg, N, 64);
    if (slab_need == 0 || slab_need > KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_WORKSPACE_TOO_SMALL;
  }
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return KDA_ERR_HIP;
  // every kernel of the prefill writes the scratch bytes it later reads (the
  // chunk table, then the records; in slabs also the carried state, written
  // by the first slab before any later one reads it), so nothing needs
  // clearing between calls
  return kda_varlen_prefill(cfg, N, total_T, cu_seqlens, q, k, v, alpha, b, initial_state, conv_state_in, o,
                            final_state, conv_state_out, ws, KDA_NOALLOC_SCRATCH_BYTES, stream);
}
