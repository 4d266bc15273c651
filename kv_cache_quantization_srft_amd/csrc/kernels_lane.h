// kernels_lane.h -- quantize / dequantize for head sizes the tiled kernels do
// not cover (d = 96: the SRFT of any even d is defined, "When Quantization Is
// Free", Metodologia 1, and d = 3 * 2^k takes a radix-3 step, xform.h).
//
// One 64-token tile of one (tensor, head) per block (one wave), one vector
// per lane as in kernels.h, blocks ordered so that each XCD takes a
// contiguous range of tiles (lane_item).  The fp16 rows (2D bytes, D/8 16-byte chunks;
// 192 bytes at d = 96) pass through LDS so that global memory sees whole
// rows: quantize fetches its tile by LDS-DMA, dequantize writes its output
// tile from LDS.  Chunk c of row v sits at chunk position c ^ ((v >> 2) & 3)
// (the chunk count is a multiple of 4, so this stays inside the row), which
// keeps the 16 rows of a read phase in different banks.  Code and scale rows
// (48 and 6/12/24 bytes at d = 96) are stored per lane.  The transform, the
// quantizer tail and the dequantizer head are the same code.
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

// Chunk position of chunk c of tile row v (and back: the same XOR).
__device__ __forceinline__ int lane_swz(int v) { return (v >> 2) & 3; }

#ifndef SRFTQ_LANE_XCD
#define SRFTQ_LANE_XCD 1
#endif

// Work item of this block out of n when neighbouring items should share an
// XCD: the chip deals consecutive blocks to its 8 XCDs in turn, so block i
// takes item (i mod 8) ceil(n / 8) + i / 8 and each XCD (its own L2) gets a
// contiguous range.  Tiles of neighbouring heads then meet in one L2: at
// d = 96 their 192-byte fp16 rows share 128-byte cache lines.  -1: none.
// Launched on lane_grid(n) blocks.
__device__ __forceinline__ int lane_item(int n) {
  int i = (int)blockIdx.x;
  if constexpr (SRFTQ_LANE_XCD) i = (i & 7) * ((n + 7) >> 3) + (i >> 3);
  return i < n ? i : -1;
}
inline unsigned lane_grid(int n) { return SRFTQ_LANE_XCD ? (unsigned)(8 * ((n + 7) / 8)) : (unsigned)n; }

// Quantize: one tile per block.  The tile's fp16 rows arrive by LDS-DMA;
// every lane then stores its own code and scale row.
template <int D, int G, int BITS, int ROT, int VAR, bool LAM>
__global__ __launch_bounds__(64) void quantize_lane_kernel(const uint16_t* __restrict__ x,
                                                           const int8_t* __restrict__ signs,
                                                           const float* __restrict__ lambda,
                                                           uint8_t* __restrict__ codes_out,
                                                           uint16_t* __restrict__ scales_out, Geo a) {
  constexpr int CB = D * BITS / 8;
  constexpr int SB = 2 * D / G;
  constexpr int CH = 2 * D / 16;   // 16-byte chunks per fp16 row
  static_assert(CH % 4 == 0, "chunk swizzle stays inside the row");
  __shared__ __attribute__((aligned(16))) uint8_t xt[64 * 2 * D];
  const int lane = threadIdx.x;
  const int tile = lane_item(a.n_tiles);
  if (tile < 0) return;
  const int k = tile / a.BH, bh = tile - k * a.BH;
  const int64_t t0 = (int64_t)k * 64;
  const int nv = a.T - t0 < 64 ? (int)(a.T - t0) : 64;
  // the tile by LDS-DMA: slot p = 64 i + lane holds chunk (p % CH) ^ swz of
  // row p / CH (rows past T re-read the last row)
  lds_poison<64 * 2 * D>(xt, lane);
  {
    const uint8_t* base = (const uint8_t*)x + row_index(a, bh, t0) * (2 * D);
    const uint32_t stride = (uint32_t)a.H * (2 * D);
    static_for<CH>([&](auto ii) {
      constexpr int i = decltype(ii)::value;
      const int p = 64 * i + lane;
      const int v = p / CH;
      const int c = (p % CH) ^ lane_swz(v);
      const int vv = v < nv ? v : nv - 1;
      dma_to_lds<16>(base, (uint32_t)vv * stride + 16u * (uint32_t)c, lds_addr(xt) + 1024u * i);
    });
    wait_vm<0>();
    wave_fence();
  }
  uint32_t w[D / 2];
  {
    const int sw = lane_swz(lane);
    static_for<CH>([&](auto cc) {
      constexpr int c = decltype(cc)::value;
      const uint4 q = *(const uint4*)(xt + lane * (2 * D) + 16 * (c ^ sw));
      w[4 * c + 0] = q.x;
      w[4 * c + 1] = q.y;
      w[4 * c + 2] = q.z;
      w[4 * c + 3] = q.w;
    });
  }
  const HeadSigns sg(signs + (int64_t)bh * a.sign_stride);
  float y[D];
  forward<D, ROT, VAR>(w, sg, y);
  uint32_t codes[CodeWords<D, BITS>::kWords];
  uint32_t scales[ScaleWords<D, G>::kWords];
  quantize_tail<D, G, BITS, ROT, VAR, LAM>(y, LAM ? lambda + (int64_t)bh * D : nullptr, codes, scales);
  // cache row r0 + lane for tile row lane, r0 = t0 or the tensor's append
  // position + t0; rows past T, and rows outside [0, pitch), are not written
  int64_t r0 = t0;
  bool ok = lane < nv;
  if (a.pos) {
    r0 += a.pos[bh / a.H];
    ok = ok && r0 + lane >= 0 && r0 + lane < a.pitch;
  }
  if (ok) {
    const int64_t row = cache_row(a, bh, r0) + lane;
    store_row_bytes<CB>(codes_out + row * CB, codes);
    store_row_bytes<SB>((uint8_t*)scales_out + row * SB, scales);
  }
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
  constexpr int CH = 2 * D / 16;   // 16-byte chunks per fp16 row
  static_assert(CH % 4 == 0, "chunk swizzle stays inside the row");
  __shared__ float lt[LAM ? D : 1];
  __shared__ __attribute__((aligned(16))) uint8_t xo[64 * 2 * D];
  const int lane = threadIdx.x;
  const int tile = lane_item(a.n_tiles);
  if (tile < 0) return;
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
  const int64_t t0 = (int64_t)k * 64;
  const int nv = a.T - t0 < 64 ? (int)(a.T - t0) : 64;
  const int64_t t = t0 + lane;
  const bool live = lane < nv;
  const int64_t row = cache_row(a, bh, live ? t : t0);
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
  // the output tile through LDS: lane writes its row, then every lane stores
  // slot p = 64 i + lane (chunk (p % CH) ^ swz of row p / CH), whole rows at a time
  lds_poison<64 * 2 * D>(xo, lane);
  {
    const int sw = lane_swz(lane);
    static_for<CH>([&](auto cc) {
      constexpr int c = decltype(cc)::value;
      *(uint4*)(xo + lane * (2 * D) + 16 * (c ^ sw)) =
          make_uint4(o[4 * c + 0], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]);
    });
    wait_lgkm0();
    wave_fence();
    uint8_t* base = (uint8_t*)x_out + row_index(a, bh, t0) * (2 * D);
    const int64_t stride = (int64_t)a.H * (2 * D);
    static_for<CH>([&](auto ii) {
      constexpr int i = decltype(ii)::value;
      const int p = 64 * i + lane;
      const int v = p / CH;
      const int c = (p % CH) ^ lane_swz(v);
      if (v < nv) {
        const uint4 q = *(const uint4*)(xo + 16 * p);
        typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
        const u32x4_t w = {q.x, q.y, q.z, q.w};
        __builtin_nontemporal_store(w, (u32x4_t*)(base + v * stride + 16 * c));
      }
    });
  }
}

}  // namespace srftq
