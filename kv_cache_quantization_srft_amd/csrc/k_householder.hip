// Products of Householder reflections, Q = H_1 H_2 ... H_k with
// H_i = I - 2 v_i v_i^T / |v_i|^2: the parametrization of the Householder
// rotations of "When Quantization Is Free", Metodologia 3 (k = d/2 reflectors
// at d = 256).  fp64 on the device, one wave per row of Q
// (row r = e_r^T H_1 ... H_k), rounded to fp32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dev_common.h"
#include "launch.h"

namespace srftq {

// ----------------------------------------------------------------------------
// Q_m = H_1 ... H_k from V_m [k, d] (fp32), in fp64; d <= 256, k <= 1024.
// Block: 4 waves, rows 4 blockIdx.x .. +3 of matrix blockIdx.y.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void householder_kernel(const float* __restrict__ V, float* __restrict__ Qout,
                                                          int d, int k) {
  __shared__ double beta[1024];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const float* Vm = V + (int64_t)blockIdx.y * k * d;
  auto wave_sum = [&](double s) {
    static_for<6>([&](auto ii) { s += __shfl_xor(s, 1 << decltype(ii)::value); });
    return s;
  };
  for (int i = wave; i < k; i += 4) {
    double s = 0.0;
    static_for<4>([&](auto uu) {
      const int c = lane + 64 * decltype(uu)::value;
      if (c < d) {
        const double v = (double)Vm[(int64_t)i * d + c];
        s += v * v;
      }
    });
    s = wave_sum(s);
    if (lane == 0) beta[i] = s > 0.0 ? 2.0 / s : 0.0;
  }
  __syncthreads();
  const int r = (int)blockIdx.x * 4 + wave;
  if (r >= d) return;
  double row[4];
  static_for<4>([&](auto uu) {
    constexpr int u = decltype(uu)::value;
    row[u] = (lane + 64 * u == r) ? 1.0 : 0.0;
  });
  for (int i = 0; i < k; ++i) {
    // row <- row H_i = row - beta_i (row . v_i) v_i
    double v[4];
    double s = 0.0;
    static_for<4>([&](auto uu) {
      constexpr int u = decltype(uu)::value;
      const int c = lane + 64 * u;
      v[u] = c < d ? (double)Vm[(int64_t)i * d + c] : 0.0;
      s += row[u] * v[u];
    });
    const double f = wave_sum(s) * beta[i];
    static_for<4>([&](auto uu) {
      constexpr int u = decltype(uu)::value;
      row[u] -= f * v[u];
    });
  }
  float* out = Qout + ((int64_t)blockIdx.y * d + r) * d;
  static_for<4>([&](auto uu) {
    constexpr int u = decltype(uu)::value;
    const int c = lane + 64 * u;
    if (c < d) out[c] = (float)row[u];
  });
}

hipError_t run_householder(int d, int k, int64_t n, const float* V, float* Q, hipStream_t st) {
  if (n == 0 || d == 0) return hipSuccess;
  hipLaunchKernelGGL(householder_kernel, dim3((unsigned)((d + 3) / 4), (unsigned)n), dim3(256), 0, st, V, Q, d, k);
  return hipGetLastError();
}

}  // namespace srftq
