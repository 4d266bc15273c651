// ones.hip -- a device-resident row of +1 signs, used when the caller passes
// no sign vector (signs == NULL means s = +1), so kernels always read signs
// through one scalar-loaded pointer.  Static device memory: nothing is
// allocated at run time.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace srftq {

__device__ __attribute__((aligned(16))) int8_t g_plus_ones[256] = {
#define SRFTQ_ONE8 1, 1, 1, 1, 1, 1, 1, 1
#define SRFTQ_ONE64 SRFTQ_ONE8, SRFTQ_ONE8, SRFTQ_ONE8, SRFTQ_ONE8, SRFTQ_ONE8, SRFTQ_ONE8, SRFTQ_ONE8, SRFTQ_ONE8
    SRFTQ_ONE64, SRFTQ_ONE64, SRFTQ_ONE64, SRFTQ_ONE64
#undef SRFTQ_ONE64
#undef SRFTQ_ONE8
};

// Address of g_plus_ones on the current device (cached per device; threads
// racing on a device's first call look up and store the same address).
const int8_t* plus_ones_ptr() {
  static std::atomic<void*> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  void* p = cache[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_plus_ones)) != hipSuccess) return nullptr;
    cache[dev].store(p, std::memory_order_release);
  }
  return (const int8_t*)p;
}

}  // namespace srftq
