// kernels.h -- libsrftq kernels for gfx950, one KV vector per lane.
//
// Work decomposition: a tile is 64 consecutive tokens of one (tensor, head)
// pair, so the head's signs and lambda row are wave-uniform (scalar loads,
// SGPR operands).  Tiles are numbered token-chunk-major, head-minor, so the
// waves resident at any moment cover adjacent rows of the [B,T,H,d] tensors.
// Each block is one wave; the grid is persistent (about the number of
// resident waves) and walks the tiles with a fixed stride.
//
// Input staging (quantize): the next tile's 64 rows are fetched straight into
// LDS with global_load_lds_dwordx4 (one instruction = 1 KiB, fully coalesced)
// while the current tile computes; lanes then read their own row with
// ds_read_b128 through an XOR swizzle that keeps every 8- and 16-lane phase
// on distinct banks.
// Output staging (dequantize): rows go to LDS and leave as 1 KiB coalesced
// global stores.
#pragma once

#include "quant.h"

// Occupancy targets (waves per SIMD) of the two streaming kernels; they cap
// the unified VGPR budget at 512/waves.
#ifndef SRFTQ_QUANT_WAVES
#define SRFTQ_QUANT_WAVES 2
#endif
#ifndef SRFTQ_DEQUANT_WAVES
#define SRFTQ_DEQUANT_WAVES 2
#endif
#define SRFTQ_QUANT_OCC __attribute__((amdgpu_waves_per_eu(SRFTQ_QUANT_WAVES)))
#define SRFTQ_DEQUANT_OCC __attribute__((amdgpu_waves_per_eu(SRFTQ_DEQUANT_WAVES)))

namespace srftq {

// Sizes of a launch.  Data pointers travel as separate __restrict__ kernel
// arguments so the compiler may read signs and lambda through scalar loads;
// `signs` is never null (the host substitutes a row of +1).
struct Geo {
  int64_t T;
  int32_t H;
  int32_t BH;            // B * H
  int32_t tiles_t;       // ceil(T / 64)
  int32_t n_tiles;       // tiles_t * BH
  int32_t sign_stride;   // elements between heads' sign rows: D, or 0 for a shared row
};


// Tile cursor: (token chunk k, head bh), advanced by a fixed stride.
struct Cursor {
  int k, bh;
  __device__ __forceinline__ void init(int tile, int BH) {
    k = tile / BH;
    bh = tile - k * BH;
  }
  __device__ __forceinline__ void advance(int dk, int dbh, int BH) {
    k += dk;
    bh += dbh;
    if (bh >= BH) {
      bh -= BH;
      k += 1;
    }
  }
};

// Row offset (in elements of d) of token t of head bh: ((b*T + t)*H + h).
__device__ __forceinline__ int64_t row_index(const Geo& a, int bh, int64_t t) {
  const int b = bh / a.H, h = bh - b * a.H;
  return ((int64_t)b * a.T + t) * a.H + h;
}

// ----------------------------------------------------------------------------
// fp16 row tile geometry: 64 rows of 2*D bytes, CPR 16-byte chunks per row.
// Chunk c of row v sits at LDS slot position c ^ sw(v).
// ----------------------------------------------------------------------------
template <int D>
struct F16Tile {
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kCpr = kRowBytes / 16;        // chunks per row
  static constexpr int kInst = kCpr;                 // 64*kCpr chunks / 64 lanes
  static constexpr int kRpi = 64 / kCpr;             // rows per instruction
  static constexpr int kBytes = 64 * kRowBytes;
  static_assert(kCpr == 8 || kCpr == 16, "tile geometry");
  // sw depends on the instruction index only through (i mod kPat)
  static constexpr int kPat = kCpr == 16 ? 4 : 2;
  __device__ static __forceinline__ int sw(int v) {
    return kCpr == 16 ? (v & 15) : ((v & 7) ^ ((v >> 3) & 1));
  }
};

// Per-lane byte offsets (relative to the tile's first row) of the DMA
// source for instruction pattern m, rows spaced rsb bytes apart.
template <int D>
__device__ __forceinline__ uint32_t dma_offset(int lane, int i, uint32_t rsb, int nv) {
  using TL = F16Tile<D>;
  int v = i * TL::kRpi + lane / TL::kCpr;
  const int p = lane % TL::kCpr;
  const int c = p ^ TL::sw(v);
  if (v > nv - 1) v = nv - 1;
  return (uint32_t)v * rsb + 16u * (uint32_t)c;
}

template <int D>
struct DmaPlan {
  using TL = F16Tile<D>;
  uint32_t off[TL::kPat];
  __device__ __forceinline__ void init(int lane, uint32_t rsb) {
#pragma unroll
    for (int m = 0; m < TL::kPat; ++m) off[m] = dma_offset<D>(lane, m, rsb, 64);
  }
};

// Issue the 64-row fp16 tile starting at `base` into LDS.
template <int D>
__device__ __forceinline__ void issue_tile(const uint8_t* base, uint32_t rsb, int nv, int lane,
                                           const DmaPlan<D>& plan, uint8_t* lds) {
  using TL = F16Tile<D>;
  if (nv == 64) {
#pragma unroll
    for (int i = 0; i < TL::kInst; ++i) {
      const uint8_t* g = base + (size_t)(i / TL::kPat) * (size_t)(TL::kPat * TL::kRpi) * rsb;
      lds_dma16(g + plan.off[i % TL::kPat], lds + i * 1024);
    }
  } else {
#pragma unroll
    for (int i = 0; i < TL::kInst; ++i) lds_dma16(base + dma_offset<D>(lane, i, rsb, nv), lds + i * 1024);
  }
}

// Read lane `v`'s own row (D/2 dwords) from the staged tile.
template <int D>
__device__ __forceinline__ void read_row(const uint8_t* lds, int v, uint32_t (&w)[D / 2]) {
  using TL = F16Tile<D>;
  const uint8_t* row = lds + v * TL::kRowBytes;
  const int s = TL::sw(v);
  static_for<TL::kCpr>([&](auto cc) {
    constexpr int c = decltype(cc)::value;
    const uint4 q = *(const uint4*)(row + 16 * (c ^ s));
    w[4 * c + 0] = q.x;
    w[4 * c + 1] = q.y;
    w[4 * c + 2] = q.z;
    w[4 * c + 3] = q.w;
  });
}

template <int N>
__device__ __forceinline__ void store_words(uint8_t* dst, const uint32_t (&v)[N]) {
  if constexpr (N % 4 == 0) {
    static_for<N / 4>([&](auto ii) {
      constexpr int i = decltype(ii)::value;
      *(uint4*)(dst + 16 * i) = make_uint4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
    });
  } else if constexpr (N == 2) {
    *(uint2*)dst = make_uint2(v[0], v[1]);
  } else {
    static_assert(N == 1, "word count");
    *(uint32_t*)dst = v[0];
  }
}

template <int N>
__device__ __forceinline__ void load_words(const uint8_t* src, uint32_t (&v)[N]) {
  if constexpr (N % 4 == 0) {
    static_for<N / 4>([&](auto ii) {
      constexpr int i = decltype(ii)::value;
      const uint4 q = *(const uint4*)(src + 16 * i);
      v[4 * i] = q.x;
      v[4 * i + 1] = q.y;
      v[4 * i + 2] = q.z;
      v[4 * i + 3] = q.w;
    });
  } else if constexpr (N == 2) {
    const uint2 q = *(const uint2*)src;
    v[0] = q.x;
    v[1] = q.y;
  } else {
    static_assert(N == 1, "word count");
    v[0] = *(const uint32_t*)src;
  }
}

// Scales of one vector occupy 2*D/G bytes: store / load exactly that.
template <int D, int G>
__device__ __forceinline__ void store_scales(uint8_t* dst, const uint32_t (&s)[ScaleWords<D, G>::kWords]) {
  if constexpr (D / G == 1) {
    *(uint16_t*)dst = (uint16_t)s[0];
  } else {
    store_words<ScaleWords<D, G>::kWords>(dst, s);
  }
}
template <int D, int G>
__device__ __forceinline__ void load_scales(const uint8_t* src, uint32_t (&s)[ScaleWords<D, G>::kWords]) {
  if constexpr (D / G == 1) {
    s[0] = *(const uint16_t*)src;
  } else {
    load_words<ScaleWords<D, G>::kWords>(src, s);
  }
}

// ----------------------------------------------------------------------------
// Quantize: fp16 [B,T,H,D] -> codes + fp16 scales.
// ----------------------------------------------------------------------------
template <int D, int G, int BITS, int ROT, int VAR, bool LAM>
__global__ __launch_bounds__(64) SRFTQ_QUANT_OCC void quantize_kernel(const uint16_t* __restrict__ x,
                                                      const int8_t* __restrict__ signs,
                                                      const float* __restrict__ lambda,
                                                      uint8_t* __restrict__ codes_out,
                                                      uint16_t* __restrict__ scales_out, Geo a) {
  using TL = F16Tile<D>;
  constexpr int CB = D * BITS / 8;        // code bytes per vector
  constexpr int SB = 2 * D / G;           // scale bytes per vector
  __shared__ __attribute__((aligned(16))) uint8_t lds[TL::kBytes];

  const int lane = threadIdx.x;
  const int stride = gridDim.x;
  if ((int)blockIdx.x >= a.n_tiles) return;
  const uint32_t rsb = (uint32_t)a.H * (uint32_t)TL::kRowBytes;   // x row stride, bytes
  DmaPlan<D> plan;
  plan.init(lane, rsb);
  const int dk = stride / a.BH, dbh = stride - dk * a.BH;

  Cursor cur;
  cur.init(blockIdx.x, a.BH);
  int remaining = (a.n_tiles - 1 - (int)blockIdx.x) / stride;     // tiles after this one

  auto tile_base = [&](const Cursor& c, int& nv) {
    const int64_t t0 = (int64_t)c.k * 64;
    const int64_t left = a.T - t0;
    nv = left < 64 ? (int)left : 64;
    return (const uint8_t*)x + row_index(a, c.bh, t0) * (int64_t)TL::kRowBytes;
  };

  int nv;
  issue_tile<D>(tile_base(cur, nv), rsb, nv, lane, plan, lds);

  for (;;) {
    wait_vmcnt<0>();
    __syncthreads();
    uint32_t w[D / 2];
    read_row<D>(lds, lane, w);
    wait_lgkmcnt0();
    __syncthreads();

    const Cursor now = cur;
    const int nv_now = nv;
    if (remaining > 0) {
      cur.advance(dk, dbh, a.BH);
      issue_tile<D>(tile_base(cur, nv), rsb, nv, lane, plan, lds);
    }

    const HeadSigns sg(signs + (int64_t)now.bh * a.sign_stride);
    float y[D];
    forward<D, ROT, VAR>(w, sg, y);
    uint32_t codes[CodeWords<D, BITS>::kWords];
    uint32_t scales[ScaleWords<D, G>::kWords];
    const float* lam = LAM ? lambda + (int64_t)now.bh * D : nullptr;
    quantize_tail<D, G, BITS, ROT, VAR, LAM>(y, lam, codes, scales);

    if (lane < nv_now) {
      const int64_t r0 = row_index(a, now.bh, (int64_t)now.k * 64);   // uniform
      const uint32_t dr = (uint32_t)lane * (uint32_t)a.H;
      store_words<CodeWords<D, BITS>::kWords>(codes_out + r0 * CB + dr * CB, codes);
      store_scales<D, G>((uint8_t*)scales_out + r0 * SB + dr * SB, scales);
    }
    if (remaining == 0) break;
    --remaining;
  }
}

// ----------------------------------------------------------------------------
// Dequantize: codes + scales -> fp16 [B,T,H,D]; rows leave through LDS as
// coalesced 1 KiB stores.  The next tile's codes are prefetched into
// registers while the current one computes.
// ----------------------------------------------------------------------------
template <int D, int G, int BITS, int ROT, int VAR, bool LAM>
__global__ __launch_bounds__(64) SRFTQ_DEQUANT_OCC void dequantize_kernel(const uint8_t* __restrict__ codes_in,
                                                        const uint16_t* __restrict__ scales_in,
                                                        const int8_t* __restrict__ signs,
                                                        const float* __restrict__ lambda,
                                                        uint16_t* __restrict__ x_out, Geo a) {
  using TL = F16Tile<D>;
  using Sc = Scales<D, ROT, VAR>;
  constexpr int CB = D * BITS / 8;
  constexpr int SB = 2 * D / G;
  constexpr int NCW = CodeWords<D, BITS>::kWords;
  constexpr int NSW = ScaleWords<D, G>::kWords;
  __shared__ __attribute__((aligned(16))) uint8_t lds[TL::kBytes];
  __shared__ __attribute__((aligned(16))) float lam_tab[LAM ? D : 4];

  const int lane = threadIdx.x;
  const int stride = gridDim.x;
  if ((int)blockIdx.x >= a.n_tiles) return;
  const uint32_t rsb = (uint32_t)a.H * (uint32_t)TL::kRowBytes;
  const int dk = stride / a.BH, dbh = stride - dk * a.BH;

  Cursor cur;
  cur.init(blockIdx.x, a.BH);
  int remaining = (a.n_tiles - 1 - (int)blockIdx.x) / stride;

  auto fetch = [&](const Cursor& c, uint32_t (&cw)[NCW], uint32_t (&sw)[NSW], int& nv) {
    const int64_t t0 = (int64_t)c.k * 64;
    const int64_t left = a.T - t0;
    nv = left < 64 ? (int)left : 64;
    const int v = lane < nv ? lane : nv - 1;
    const int64_t r0 = row_index(a, c.bh, t0);                         // uniform
    const uint32_t dr = (uint32_t)v * (uint32_t)a.H;
    load_words<NCW>(codes_in + r0 * CB + dr * CB, cw);
    load_scales<D, G>((const uint8_t*)scales_in + r0 * SB + dr * SB, sw);
  };

  uint32_t cw[NCW], sw[NSW];
  int nv;
  fetch(cur, cw, sw, nv);

  for (;;) {
    const Cursor now = cur;
    const int nv_now = nv;
    uint32_t ccw[NCW], csw[NSW];
#pragma unroll
    for (int i = 0; i < NCW; ++i) ccw[i] = cw[i];
#pragma unroll
    for (int i = 0; i < NSW; ++i) csw[i] = sw[i];
    if (remaining > 0) {
      cur.advance(dk, dbh, a.BH);
      fetch(cur, cw, sw, nv);
    }

    if constexpr (LAM) {
      // e_j / lambda_j is uniform per head: computed lane-parallel once per
      // tile and broadcast from LDS.
      const float* lrow = lambda + (int64_t)now.bh * D;
      for (int j = lane; j < D; j += 64)
        lam_tab[j] = (float)(Sc::is_edge(j) ? Sc::kInvEdge : Sc::kInvBulk) * __builtin_amdgcn_rcpf(lrow[j]);
      __syncthreads();
    }
    float y[D];
    dequantize_head<D, G, BITS, ROT, VAR, LAM>(ccw, csw, lam_tab, y);
    float xr[D];
    inverse<D, ROT, VAR>(y, xr);

    // fp16 RNE, then the sign multiply as an XOR on the packed halves
    const HeadSigns sg(signs + (int64_t)now.bh * a.sign_stride);
    uint32_t o[D / 2];
    static_for<D / 2>([&](auto mm) {
      constexpr int m = decltype(mm)::value;
      o[m] = pack_f16x2(xr[2 * m], xr[2 * m + 1]) ^ sg.mask(m);
    });

    // stage the row in LDS (swizzled), then write 64 rows out coalesced
    {
      uint8_t* row = lds + lane * TL::kRowBytes;
      const int s = TL::sw(lane);
      static_for<TL::kCpr>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        *(uint4*)(row + 16 * (c ^ s)) = make_uint4(o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]);
      });
    }
    __syncthreads();
    {
      const int64_t t0 = (int64_t)now.k * 64;
      uint8_t* obase = (uint8_t*)x_out + row_index(a, now.bh, t0) * (int64_t)TL::kRowBytes;
      static_for<TL::kInst>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
        const int v = i * TL::kRpi + lane / TL::kCpr;
        const int p = lane % TL::kCpr;
        const uint4 q = *(const uint4*)(lds + v * TL::kRowBytes + 16 * (p ^ TL::sw(v)));
        if (v < nv_now) *(uint4*)(obase + (size_t)v * rsb + 16 * p) = q;
      });
    }
    __syncthreads();
    if (remaining == 0) break;
    --remaining;
  }
}

// ----------------------------------------------------------------------------
// Rotation alone (fp32 out, scaled) and its inverse (fp32 in, fp16 out).
// One tile per block; these serve parity checks and calibration.
// ----------------------------------------------------------------------------
template <int D, int ROT, int VAR>
__global__ __launch_bounds__(64) void rotate_kernel(const uint16_t* __restrict__ x,
                                                    const int8_t* __restrict__ signs,
                                                    float* __restrict__ y_out, Geo a) {
  using Sc = Scales<D, ROT, VAR>;
  const int tile = blockIdx.x;
  const int k = tile / a.BH, bh = tile - k * a.BH;
  const int64_t t = (int64_t)k * 64 + threadIdx.x;
  if (t >= a.T) return;
  const int64_t r = row_index(a, bh, t);
  uint32_t w[D / 2];
  load_words<D / 2>((const uint8_t*)x + r * (2 * D), w);
  const HeadSigns sg(signs + (int64_t)bh * a.sign_stride);
  float y[D];
  forward<D, ROT, VAR>(w, sg, y);
  uint32_t o[D];
  static_for<D>([&](auto jj) {
    constexpr int j = decltype(jj)::value;
    o[j] = as_u32(y[j] * (float)(Sc::is_edge(j) ? Sc::kFwdEdge : Sc::kFwdBulk));
  });
  store_words<D>((uint8_t*)y_out + r * (4 * D), o);
}

template <int D, int ROT, int VAR>
__global__ __launch_bounds__(64) void unrotate_kernel(const float* __restrict__ y_in,
                                                      const int8_t* __restrict__ signs,
                                                      uint16_t* __restrict__ x_out, Geo a) {
  using Sc = Scales<D, ROT, VAR>;
  const int tile = blockIdx.x;
  const int k = tile / a.BH, bh = tile - k * a.BH;
  const int64_t t = (int64_t)k * 64 + threadIdx.x;
  if (t >= a.T) return;
  const int64_t r = row_index(a, bh, t);
  uint32_t iw[D];
  load_words<D>((const uint8_t*)y_in + r * (4 * D), iw);
  float y[D];
  static_for<D>([&](auto jj) {
    constexpr int j = decltype(jj)::value;
    y[j] = as_f32(iw[j]) * (float)(Sc::is_edge(j) ? Sc::kInvEdge : Sc::kInvBulk);
  });
  float xr[D];
  inverse<D, ROT, VAR>(y, xr);
  const HeadSigns sg(signs + (int64_t)bh * a.sign_stride);
  uint32_t o[D / 2];
  static_for<D / 2>([&](auto mm) {
    constexpr int m = decltype(mm)::value;
    o[m] = pack_f16x2(xr[2 * m], xr[2 * m + 1]) ^ sg.mask(m);
  });
  store_words<D / 2>((uint8_t*)x_out + r * (2 * D), o);
}

// Calibration: accumulate sum_t y^2 per (bh, j) into acc[bh, j] (zeroed
// beforehand), then finalize lambda = 1/sqrt(sum/T) (1 where sum == 0).
template <int D, int ROT, int VAR>
__global__ __launch_bounds__(64) void calib_accum_kernel(const uint16_t* __restrict__ x,
                                                         const int8_t* __restrict__ signs,
                                                         float* __restrict__ acc, Geo a) {
  using Sc = Scales<D, ROT, VAR>;
  __shared__ float part[64][D + 1];
  const int tile = blockIdx.x;
  const int k = tile / a.BH, bh = tile - k * a.BH;
  const int64_t t = (int64_t)k * 64 + threadIdx.x;
  float y[D];
  if (t < a.T) {
    uint32_t w[D / 2];
    load_words<D / 2>((const uint8_t*)x + row_index(a, bh, t) * (2 * D), w);
    const HeadSigns sg(signs + (int64_t)bh * a.sign_stride);
    forward<D, ROT, VAR>(w, sg, y);
  } else {
    static_for<D>([&](auto jj) { y[decltype(jj)::value] = 0.0f; });
  }
  static_for<D>([&](auto jj) {
    constexpr int j = decltype(jj)::value;
    const float v = y[j] * (float)(Sc::is_edge(j) ? Sc::kFwdEdge : Sc::kFwdBulk);
    part[threadIdx.x][j] = v * v;
  });
  __syncthreads();
  float* dst = acc + (int64_t)bh * D;
  for (int j = threadIdx.x; j < D; j += 64) {
    float s = 0.0f;
    for (int r = 0; r < 64; ++r) s += part[r][j];
    atomicAdd(dst + j, s);
  }
}

static __global__ void fill_kernel(float* __restrict__ p, int64_t n, float v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

static __global__ void calib_finalize_kernel(float* __restrict__ p, int64_t n, float inv_T) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    const float ms = p[i] * inv_T;
    p[i] = ms > 0.0f ? 1.0f / sqrtf(ms) : 1.0f;
  }
}

}  // namespace srftq
