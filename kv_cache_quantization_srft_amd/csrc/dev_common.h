// dev_common.h -- gfx950 device helpers shared by the libsrftq kernels.
//
// Compile-time twiddles, fp16 half extraction, LDS direct loads
// (global_load_lds_dwordx4, gfx950), wait counters and a static loop.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace srftq {

// ----------------------------------------------------------------------------
// Compile-time trigonometry (Taylor series in double; |x| <= pi).
// ----------------------------------------------------------------------------
constexpr double kPi = 3.14159265358979323846264338327950288;

constexpr double csin(double x) {
  double term = x, sum = x;
  for (int n = 1; n < 32; ++n) {
    term *= -x * x / double((2 * n) * (2 * n + 1));
    sum += term;
  }
  return sum;
}

constexpr double ccos(double x) {
  double term = 1.0, sum = 1.0;
  for (int n = 1; n < 32; ++n) {
    term *= -x * x / double((2 * n - 1) * (2 * n));
    sum += term;
  }
  return sum;
}

constexpr double csqrt(double x) {
  double r = x > 1.0 ? x : 1.0;
  for (int i = 0; i < 64; ++i) r = 0.5 * (r + x / r);
  return r;
}

// ----------------------------------------------------------------------------
// Static loop: f(std::integral_constant<int, I>) for I in [0, N).
// ----------------------------------------------------------------------------
template <class F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ----------------------------------------------------------------------------
// fp16 halves of a dword as fp32 (folds into v_fma_mix_f32 / SDWA cvt).
// ----------------------------------------------------------------------------
__device__ __forceinline__ float hlo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float hhi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed fp16 pair, round to nearest even (v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  float2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, half2_t));
}

__device__ __forceinline__ uint32_t as_u32(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }

// ----------------------------------------------------------------------------
// Wait counters (gfx9 s_waitcnt encoding: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8] | vmcnt_hi[15:14]).
// ----------------------------------------------------------------------------
template <int VM>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 0xf) | (0x7 << 4) | (0xf << 8) | ((VM >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(0xf | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
}

typedef __attribute__((address_space(3))) void lds_void_t;

// LDS offset of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Direct global -> LDS load (LDS-DMA) of SIZE bytes per lane: lane l reads
// sbase + voff(l) and its data lands at LDS byte lds + SIZE*l.  sbase and
// lds are wave-uniform.  Issued from inline asm so the compiler neither
// tracks it nor inserts its blanket vmcnt(0) before later LDS reads; the
// kernels order it themselves with wait_vm<>() / wait_lgkm0(), and they
// issue no other vector-memory loads whose results the compiler tracks.
// "s_nop 0" is the one wait state required between writing M0 and an LDS-DMA.
template <int SIZE, bool STREAM = false>
__device__ __forceinline__ void dma_to_lds(const void* sbase_in, uint32_t voff, uint32_t lds_in) {
  static_assert(SIZE == 16 || SIZE == 4 || SIZE == 2, "LDS-DMA size");
  // Both are wave-uniform; readfirstlane tells the compiler so, which keeps
  // them in scalar registers even where it had placed them in VGPRs.
  const uint64_t sb = (uint64_t)(uintptr_t)sbase_in;
  const uint64_t sbu = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(sb >> 32)) << 32) |
                       (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)sb);
  const void* sbase = (const void*)(uintptr_t)sbu;
  const uint32_t lds = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_in);
  if constexpr (SIZE == 16 && STREAM)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :: "v"(voff), "s"(sbase), "s"(lds) : "memory", "m0");
  else if constexpr (SIZE == 16)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(sbase), "s"(lds) : "memory", "m0");
  else if constexpr (SIZE == 4)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 :: "v"(voff), "s"(sbase), "s"(lds) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_ushort %0, %1"
                 :: "v"(voff), "s"(sbase), "s"(lds) : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are in flight
// (loads and stores complete in issue order on this counter).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Compiler-only ordering point for LDS traffic inside one wave (the LDS
// executes one wave's instructions in order, so no hardware barrier is needed
// when a block is a single wave).
__device__ __forceinline__ void wave_fence() { asm volatile("" ::: "memory"); }

// Read-only data addressed through the constant address space: loads with a
// wave-uniform address become scalar (s_load) loads even across barriers.
template <class T>
using const_ptr = const __attribute__((address_space(4))) T*;
template <class T>
__device__ __forceinline__ const_ptr<T> as_const(const T* p) {
  return (const_ptr<T>)(p);
}

// v_permlane32_swap on a register pair (X, Y): lanes 0..31 end with
// (their own X, lane l+32's X), lanes 32..63 with (lane l-32's Y, their own
// Y) -- a 2 x 2 transpose between the wave's halves and the two registers.
__device__ __forceinline__ void swap32(uint32_t& x, uint32_t& y) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, y, false, false);
  x = r[0];
  y = r[1];
}
__device__ __forceinline__ void swap32(float& x, float& y) {
  uint32_t a = as_u32(x), b = as_u32(y);
  swap32(a, b);
  x = as_f32(a);
  y = as_f32(b);
}

// Debug builds only (SRFTQ_LDS_POISON=1): fill an LDS buffer of one
// single-wave block with 0xff bytes (fp16 and fp32 NaN, all-ones codes and
// masks) before the data meant for it is written, so that any read of a
// byte the kernel did not write this time shows in its output.  The fill
// has completed when this returns, so an LDS-DMA issued next lands after it.
#ifndef SRFTQ_LDS_POISON
#define SRFTQ_LDS_POISON 0
#endif
template <int BYTES>
__device__ __forceinline__ void lds_poison([[maybe_unused]] void* buf, [[maybe_unused]] int lane) {
  if constexpr (SRFTQ_LDS_POISON) {
    static_assert(BYTES % 4 == 0, "dword fill");
    uint32_t* w = (uint32_t*)buf;
    for (int i = lane; i < BYTES / 4; i += 64) w[i] = 0xffffffffu;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
}

// Uniform value -> scalar register.
__device__ __forceinline__ int uniform_i32(int v) { return __builtin_amdgcn_readfirstlane(v); }

}  // namespace srftq
