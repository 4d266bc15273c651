// noalloc.hip -- srftq_decode_attention_noalloc: decode attention with its
// workspace in a static device array of the library, for callers that cannot
// allocate device memory.
//
// The array `scratch` exists once per GPU the library runs on.  In host code
// its name stands for a host-side shadow, not a device address, so the
// kernels never receive it: on each device's first call its address there is
// looked up with hipGetSymbolAddress (with that device current) and kept per
// device, and only that address reaches the kernels.
#include <hip/hip_runtime.h>

#include <atomic>

#include "launch.h"
#include "srftq.h"

namespace {

static __device__ __align__(256) uint8_t scratch[SRFTQ_ATTENTION_SCRATCH_BYTES];

std::atomic<void*> g_scratch_ptr[64];

// Address of the current device's copy of `scratch` (null on a HIP error).
// Threads racing on a device's first call look up and store the same value.
void* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" srftq_status srftq_decode_attention_noalloc(const srftq_shape* s, int64_t t_cap, int32_t R,
                                                       const uint16_t* q, const srftq_cache_view* k,
                                                       const srftq_cache_view* v, const int32_t* lengths,
                                                       float scale, float* out, void* stream) {
  return srftq::decode_attention_scratch(s, t_cap, R, q, k, v, lengths, scale, out,
                                         SRFTQ_ATTENTION_SCRATCH_BYTES, scratch_ptr, stream);
}
