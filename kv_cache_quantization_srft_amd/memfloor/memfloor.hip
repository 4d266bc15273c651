// memfloor.hip -- memory-path floor kernels for the benchmark (libsrftq_memfloor.so).
//
// These kernels do no arithmetic of the method: they move exactly the bytes
// a quantize or dequantize launch moves (per 64-vector tile: R KiB read,
// W KiB written, contiguous), so their time is what HBM itself allows for
// that read/write mix.  Two launch shapes are timed: one tile per one-wave
// block (the hardware dispatcher refills the CUs), and a persistent grid in
// which every wave walks the tiles with a fixed stride and holds the next
// tile's reads in registers while it writes the current one.  Reads carry
// the streaming hint; writes are plain or nontemporal.  Each written dword
// depends on the tile's reads (an XOR of them), so no read can be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ void put(u32x4 v, u32x4* p) {
  if constexpr (NT)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}

// R, W: KiB read / written per tile (16 bytes per lane per KiB).
template <int R, int W, bool NT>
__global__ __launch_bounds__(64) void floor_kernel(const u32x4* __restrict__ in, u32x4* __restrict__ out,
                                                   int64_t n_tiles) {
  const int l = threadIdx.x;
  int64_t t = blockIdx.x;
  if (t >= n_tiles) return;
  u32x4 r[R];
#pragma unroll
  for (int i = 0; i < R; ++i) r[i] = __builtin_nontemporal_load(in + t * (64 * R) + i * 64 + l);
  while (true) {
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < R; ++i) acc ^= r[i].x ^ r[i].y ^ r[i].z ^ r[i].w;
    const int64_t tn = t + gridDim.x;
    if (tn < n_tiles) {
#pragma unroll
      for (int i = 0; i < R; ++i) r[i] = __builtin_nontemporal_load(in + tn * (64 * R) + i * 64 + l);
    }
    u32x4* dst = out + t * (64 * W);
#pragma unroll
    for (int i = 0; i < W; ++i) put<NT>(u32x4{acc, acc + 1u, acc + 2u, acc + (uint32_t)i}, dst + i * 64 + l);
    if (tn >= n_tiles) break;
    t = tn;
  }
}

template <int R, int W>
hipError_t launch(int nt, const void* in, void* out, int64_t n_tiles, int grid, hipStream_t stream) {
  if (nt)
    floor_kernel<R, W, true><<<grid, 64, 0, stream>>>((const u32x4*)in, (u32x4*)out, n_tiles);
  else
    floor_kernel<R, W, false><<<grid, 64, 0, stream>>>((const u32x4*)in, (u32x4*)out, n_tiles);
  return hipGetLastError();
}

}  // namespace

// mix 0: 16 KiB read, 5 KiB written per tile (quantize at d = 128, int4,
//        group 16: 64 fp16 rows in, 64 code rows + 64 scale rows out);
// mix 1: 5 KiB read, 16 KiB written (dequantize at the same shape);
// mix 2: 16 KiB read, 16 KiB written (copy).
// in must hold n_tiles * R KiB and out n_tiles * W KiB, 16-byte aligned;
// grid in [1, n_tiles] (n_tiles: one tile per block).  Returns a hipError_t
// code; 1 (hipErrorInvalidValue) for a bad mix, size or grid.
extern "C" int srftq_memfloor(int mix, int nontemporal, const void* in, void* out, int64_t n_tiles, int grid,
                              hipStream_t stream) {
  if (n_tiles <= 0 || grid <= 0 || grid > n_tiles || grid > (1 << 30) || in == nullptr || out == nullptr ||
      ((uintptr_t)in & 15) || ((uintptr_t)out & 15))
    return (int)hipErrorInvalidValue;
  switch (mix) {
    case 0: return (int)launch<16, 5>(nontemporal, in, out, n_tiles, grid, stream);
    case 1: return (int)launch<5, 16>(nontemporal, in, out, n_tiles, grid, stream);
    case 2: return (int)launch<16, 16>(nontemporal, in, out, n_tiles, grid, stream);
    default: return (int)hipErrorInvalidValue;
  }
}
