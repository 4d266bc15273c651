// kernels_lane.h -- quantize / dequantize for head sizes the tiled kernels do
// not cover (d = 96: the SRFT of any even d is defined, "When Quantization Is
// Free", Metodologia 1, and d = 3 * 2^k takes a radix-3 step, xform.h).
//
// One 64-token tile of one (tensor, head) per block, one vector per lane as
// in kernels.h, but each lane loads and stores its own rows directly: the
// LDS row tiles of the streaming kernels assume power-of-two row sizes.  The
// transform, the quantizer tail and the dequantizer head are the same code.
#pragma once

#include "kernels.h"

namespace srftq {

// A row of NB bytes from / to words: 16-byte accesses when the row size
// allows, else dwords, else 2-byte accesses (rows of 2 mod 4 bytes are only
// 2-byte aligned).
template <int NB, int N>
__device__ __forceinline__ void store_row_bytes(uint8_t* dst, const uint32_t (&v)[N]) {
  static_assert(N * 4 >= NB, "row words");
  if constexpr (NB % 16 == 0) {
    static_for<NB / 16>([&](auto ii) {
      constexpr int i = decltype(ii)::value;
      *(uint4*)(dst + 16 * i) = make_uint4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
    });
  } else if constexpr (NB % 4 == 0) {
    static_for<NB / 4>([&](auto ii) { ((uint32_t*)dst)[decltype(ii)::value] = v[decltype(ii)::value]; });
  } else {
    static_for<NB / 2>([&](auto ii) {
      constexpr int i = decltype(ii)::value;
      ((uint16_t*)dst)[i] = (uint16_t)(v[i / 2] >> (16 * (i % 2)));
    });
  }
}
template <int NB, int N>
__device__ __forceinline__ void load_row_bytes(const uint8_t* src, uint32_t (&v)[N]) {
  static_assert(N * 4 >= NB, "row words");
  if constexpr (NB % 16 == 0) {
    static_for<NB / 16>([&](auto ii) {
      constexpr int i = decltype(ii)::value;
      const uint4 q = *(const uint4*)(src + 16 * i);
      v[4 * i] = q.x;
      v[4 * i + 1] = q.y;
      v[4 * i + 2] = q.z;
      v[4 * i + 3] = q.w;
    });
  } else if constexpr (NB % 4 == 0) {
    static_for<NB / 4>([&](auto ii) { v[decltype(ii)::value] = ((const uint32_t*)src)[decltype(ii)::value]; });
  } else {
    static_for<N>([&](auto ii) { v[decltype(ii)::value] = 0u; });
    static_for<NB / 2>([&](auto ii) {
      constexpr int i = decltype(ii)::value;
      v[i / 2] |= (uint32_t)((const uint16_t*)src)[i] << (16 * (i % 2));
    });
  }
}

template <int D, int G, int BITS, int ROT, int VAR, bool LAM>
__global__ __launch_bounds__(64) void quantize_lane_kernel(const uint16_t* __restrict__ x,
                                                           const int8_t* __restrict__ signs,
                                                           const float* __restrict__ lambda,
                                                           uint8_t* __restrict__ codes_out,
                                                           uint16_t* __restrict__ scales_out, Geo a) {
  constexpr int CB = D * BITS / 8;
  constexpr int SB = 2 * D / G;
  const int lane = threadIdx.x;
  const int tile = blockIdx.x;
  const int k = tile / a.BH, bh = tile - k * a.BH;
  const int64_t t = (int64_t)k * 64 + lane;
  if (t >= a.T) return;
  uint32_t w[D / 2];
  load_words<D / 2>((const uint8_t*)x + row_index(a, bh, t) * (2 * D), w);
  const HeadSigns sg(signs + (int64_t)bh * a.sign_stride);
  float y[D];
  forward<D, ROT, VAR>(w, sg, y);
  uint32_t codes[CodeWords<D, BITS>::kWords];
  uint32_t scales[ScaleWords<D, G>::kWords];
  quantize_tail<D, G, BITS, ROT, VAR, LAM>(y, LAM ? lambda + (int64_t)bh * D : nullptr, codes, scales);
  // cache row: token t, or the tensor's append position + t (dropped outside [0, pitch))
  int64_t tc = t;
  if (a.pos) {
    tc += a.pos[bh / a.H];
    if (tc < 0 || tc >= a.pitch) return;
  }
  const int64_t row = cache_row(a, bh, tc);
  store_row_bytes<CB>(codes_out + row * CB, codes);
  store_row_bytes<SB>((uint8_t*)scales_out + row * SB, scales);
}

// Quantize a few tokens per tensor (decode steps: T = 1 .. 8), one vector per
// lane over the flattened (tensor, token, head) index, so every lane of the
// grid is live; the tiled kernels give each (tensor, head) a 64-token tile,
// which for one token leaves 63 of its 64 lanes idle.  Each lane applies its
// own head's signs and lambda; the transform and the quantizer tail are the
// same code.  Cache rows follow the tiled kernels: row pos[b] + t of head
// (b, h) (or t), dropped outside [0, pitch).
template <int D, int G, int BITS, int ROT, int VAR, bool LAM>
__global__ __launch_bounds__(64) void quantize_flat_kernel(const uint16_t* __restrict__ x,
                                                           const int8_t* __restrict__ signs,
                                                           const float* __restrict__ lambda,
                                                           uint8_t* __restrict__ codes_out,
                                                           uint16_t* __restrict__ scales_out, Geo a) {
  constexpr int CB = D * BITS / 8;
  constexpr int SB = 2 * D / G;
  const int64_t v = (int64_t)blockIdx.x * 64 + threadIdx.x;   // ((b*T + t)*H + h)
  if (v >= (int64_t)a.BH * a.T) return;
  const int64_t bt = v / a.H;
  const int h = (int)(v - bt * a.H);
  const int64_t b = bt / a.T;
  const int64_t t = bt - b * a.T;
  const int64_t bh = b * a.H + h;
  uint32_t w[D / 2];
  load_words<D / 2>((const uint8_t*)x + v * (2 * D), w);
  apply_lane_signs<D>(signs + bh * a.sign_stride, w);
  float y[D];
  forward<D, ROT, VAR>(w, NoSigns{}, y);
  uint32_t codes[CodeWords<D, BITS>::kWords];
  uint32_t scales[ScaleWords<D, G>::kWords];
  quantize_tail<D, G, BITS, ROT, VAR, LAM>(y, LAM ? lambda + bh * D : nullptr, codes, scales);
  int64_t tc = t;
  if (a.pos) {
    tc += a.pos[b];
    if (tc < 0 || tc >= a.pitch) return;
  }
  const int64_t row = bh * a.pitch + tc;
  store_row_bytes<CB>(codes_out + row * CB, codes);
  store_row_bytes<SB>((uint8_t*)scales_out + row * SB, scales);
}

template <int D, int G, int BITS, int ROT, int VAR, bool LAM>
__global__ __launch_bounds__(64) void dequantize_lane_kernel(const uint8_t* __restrict__ codes_in,
                                                             const uint16_t* __restrict__ scales_in,
                                                             const int8_t* __restrict__ signs,
                                                             const float* __restrict__ lambda,
                                                             uint16_t* __restrict__ x_out, Geo a) {
  using Sc = Scales<D, ROT, VAR>;
  constexpr int CB = D * BITS / 8;
  constexpr int SB = 2 * D / G;
  __shared__ float lt[LAM ? D : 1];
  const int lane = threadIdx.x;
  const int tile = blockIdx.x;
  const int k = tile / a.BH, bh = tile - k * a.BH;
  if constexpr (LAM) {
    // e_j / lambda_j of the head (e_j the inverse transform's input scale)
    for (int j = lane; j < D; j += 64) {
      const bool edge = Sc::kEdges && (j == 0 || j == D / 2);
      lt[j] = (edge ? (float)Sc::kInvEdge : (float)Sc::kInvBulk) *
              __builtin_amdgcn_rcpf(lambda[(int64_t)bh * D + j]);
    }
    __syncthreads();
  }
  const int64_t t = (int64_t)k * 64 + lane;
  if (t >= a.T) return;
  const int64_t row = cache_row(a, bh, t);
  uint32_t codes[CodeWords<D, BITS>::kWords];
  uint32_t scales[ScaleWords<D, G>::kWords];
  load_row_bytes<CB>(codes_in + row * CB, codes);
  load_row_bytes<SB>((const uint8_t*)scales_in + row * SB, scales);
  float y[D];
  dequantize_head<D, G, BITS, ROT, VAR, LAM>(codes, scales, lt, y);
  float xr[D];
  inverse<D, ROT, VAR>(y, xr);
  const HeadSigns sg(signs + (int64_t)bh * a.sign_stride);
  uint32_t o[D / 2];
  static_for<D / 2>([&](auto mm) {
    constexpr int m = decltype(mm)::value;
    o[m] = pack_f16x2(xr[2 * m], xr[2 * m + 1]) ^ sg.mask(m);
  });
  store_words<D / 2>((uint8_t*)x_out + row_index(a, bh, t) * (2 * D), o);
}

}  // namespace srftq
