// kernels.h -- libsrftq kernels for gfx950, one KV vector per lane.
//
// Work decomposition: a tile is 64 consecutive tokens of one (tensor, head)
// pair, so the head's signs and lambda row are wave-uniform: they arrive by
// LDS-DMA with the tile, the signs are expanded lane-parallel into one XOR
// mask per packed fp16 pair, and both are read back as LDS broadcasts.
// Tiles are numbered token-chunk-major, head-minor, so the waves resident at
// any moment cover adjacent rows of the [B,T,H,d] tensors.
// Each block is one wave and takes Geo::tpb consecutive tiles (one, at
// d <= 128, so that the hardware dispatcher balances the CUs), or, with
// tpb = 0, the grid is persistent and every block walks the tiles with a
// fixed stride (d = 256).  A block with more than one tile fetches the next
// tile while the current one computes.
//
// Input staging: the tile's rows (quantize: 64 fp16 rows; dequantize: code
// and scale rows) go straight into LDS with global_load_lds_dwordx4 (one
// instruction = 1 KiB of whole rows, streaming cache hint); lanes then read
// their own row with ds_read_b128 through an XOR swizzle that keeps every 8-
// and 16-lane phase on distinct banks.
// Output staging (dequantize): rows go to LDS and leave as 1 KiB coalesced
// nontemporal stores.
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
// d = 256 keeps 256 fp32 coordinates per lane: one wave per SIMD, so that
// each lane has the whole 512-register file (arch + accumulation VGPRs).
#define SRFTQ_QUANT_OCC __attribute__((amdgpu_waves_per_eu(D >= 256 ? 1 : SRFTQ_QUANT_WAVES)))
#define SRFTQ_DEQUANT_OCC __attribute__((amdgpu_waves_per_eu(D >= 256 ? 1 : SRFTQ_DEQUANT_WAVES)))

namespace srftq {

// Sizes of a launch.  Data pointers travel as separate __restrict__ kernel
// arguments; `signs` is never null (the host substitutes a row of +1).
struct Geo {
  int64_t T;             // tokens of x (per tensor)
  int64_t pitch;         // cache rows per head (>= T except when appending)
  const int32_t* pos;    // append: first cache row of each tensor's tokens, or null (row t)
  int32_t H;
  int32_t BH;            // B * H
  int32_t tiles_t;       // ceil(T / 64)
  int32_t n_tiles;       // tiles_t * BH
  int32_t sign_stride;   // elements between heads' sign rows: D, or 0 for a shared row
  int32_t tpb;           // streaming kernels: tiles per block (consecutive); 0 = persistent grid;
                         // -1 = one tile per block in XCD-contiguous order
};

// Tiles of one block of a streaming kernel: either tpb consecutive tiles
// starting at blockIdx*tpb, or (tpb == 0) every gridDim-th tile.
struct TileRange {
  int first, step, remaining;   // remaining = tiles after the first
  __device__ __forceinline__ explicit TileRange(const Geo& a) {
    if (a.tpb < 0) {
      // one tile per block, XCD-contiguous: the chip deals consecutive
      // blocks to its 8 XCDs in turn, so block i takes tile
      // (i mod 8) ceil(n / 8) + i / 8 and each XCD walks one contiguous
      // eighth of the tiles (grid 8 ceil(n / 8); tiles past n exit)
      const int per = (a.n_tiles + 7) >> 3;
      first = (int)(blockIdx.x & 7u) * per + (int)(blockIdx.x >> 3);
      step = 1;
      remaining = 0;
    } else if (a.tpb > 0) {
      first = (int)blockIdx.x * a.tpb;
      step = 1;
      const int n = a.n_tiles - first;
      remaining = (n < a.tpb ? n : a.tpb) - 1;
    } else {
      first = (int)blockIdx.x;
      step = (int)gridDim.x;
      remaining = (a.n_tiles - 1 - first) / step;
    }
  }
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

// The sign diagonal applied to a lane's own fp16 words (each lane may belong
// to a different head), before a transform that then takes no signs.
template <int D>
__device__ __forceinline__ void apply_lane_signs(const int8_t* row, uint32_t (&w)[D / 2]) {
  const uint32_t* r = (const uint32_t*)row;   // 4-byte aligned
  static_for<D / 4>([&](auto ii) {
    constexpr int i = decltype(ii)::value;
    const uint32_t sb = r[i];
    w[2 * i] ^= sign_mask_of(sb);
    w[2 * i + 1] ^= sign_mask_of(sb >> 16);
  });
}
struct NoSigns {
  __device__ __forceinline__ uint32_t mask(int) const { return 0u; }
  __device__ __forceinline__ uint4 mask4(int) const { return make_uint4(0u, 0u, 0u, 0u); }
};

// Row of token t of head bh in x [B,T,H,D]: ((b*T + t)*H + h).
__device__ __forceinline__ int64_t row_index(const Geo& a, int bh, int64_t t) {
  const int b = bh / a.H, h = bh - b * a.H;
  return ((int64_t)b * a.T + t) * a.H + h;
}

// Row t of head bh in the head-major quantized cache [B,H,pitch,.]: a tile's
// 64 code and scale rows are one contiguous run.
__device__ __forceinline__ int64_t cache_row(const Geo& a, int bh, int64_t t) {
  return (int64_t)bh * a.pitch + t;
}

// ----------------------------------------------------------------------------
// A tile of 64 rows of ROWB bytes in LDS, filled by LDS-DMA.  Row v starts at
// v*ROWB; for ROWB >= 16 its 16-byte chunk c sits at position c ^ swz(v),
// an XOR swizzle that keeps ds_read_b128 of "chunk c of my own row" free of
// bank conflicts in every 8-lane and 16-lane phase.  Sub-16-byte rows are
// stored unswizzled (lanes then read consecutive addresses).
//
// DMA: instruction i writes LDS bytes [1 KiB * i, 1 KiB * (i+1)) (16 B per
// lane) or, for ROWB < 16, E = min(ROWB, 4) bytes per lane.  Lane l of
// instruction i fetches chunk (l % CPR) ^ swz(v) of row v = i*RPI + l/CPR:
// every instruction reads whole rows, i.e. full cache lines.  The per-lane
// source offsets depend on i only through i mod kPat and are computed once.
// ----------------------------------------------------------------------------
template <int ROWB, int NR = 64>
struct RowTile {
  static_assert(ROWB == 2 || ROWB == 4 || ROWB == 8 || ROWB == 16 || ROWB == 32 || ROWB == 64 ||
                    ROWB == 128 || ROWB == 256 || ROWB == 512,
                "row size");
  static constexpr bool kWide = ROWB >= 16;
  static constexpr int kElem = kWide ? 16 : (ROWB < 4 ? ROWB : 4);   // DMA bytes per lane
  // LDS-DMA writes at least a dword per lane: a 2-byte row occupies a
  // 4-byte LDS slot
  static constexpr int kSlot = kElem < 4 ? 4 : kElem;
  static constexpr int kEpr = ROWB / kElem;                          // DMA elements per row
  static constexpr int kRpi = 64 / kEpr;                             // rows per instruction
  // instructions per tile of NR rows (rows past NR, when one instruction
  // covers more, re-read the tile's last row into slots past the tile)
  static constexpr int kInst = NR * kEpr >= 64 ? NR * kEpr / 64 : 1;
  static constexpr int kRowLds = kEpr * kSlot;                       // LDS bytes per row
  static constexpr int kBytes = (NR > kRpi ? NR : kRpi) * kRowLds;
  static constexpr int kCpr = kWide ? ROWB / 16 : 1;
  static constexpr int kPat = !kWide ? 1 : kCpr <= 4 ? 1 : kCpr == 8 ? 2 : kCpr == 16 ? 4 : 8;

  __device__ static __forceinline__ int swz(int v) {
    if constexpr (!kWide || kCpr == 1) return 0;
    else if constexpr (kCpr == 2) return ((v >> 2) ^ (v >> 3)) & 1;
    else if constexpr (kCpr == 4) return ((v >> 1) & 3) ^ ((v >> 3) & 1);
    else if constexpr (kCpr == 8) return (v & 7) ^ ((v >> 3) & 1);
    else return v & 15;
  }

  // Source byte offset (relative to row 0) of lane `lane` in instruction i;
  // rows beyond nv-1 are clamped to the last valid row.
  __device__ static __forceinline__ uint32_t src_offset(int lane, int i, uint32_t rsb, int nv) {
    int v = i * kRpi + lane / kEpr;
    const int e = lane % kEpr;
    const int c = kWide ? (e ^ swz(v)) : e;
    if (v > nv - 1) v = nv - 1;
    return (uint32_t)v * rsb + (uint32_t)(c * kElem);
  }

  struct Plan {
    uint32_t off[kPat];
    __device__ __forceinline__ void init(int lane, uint32_t rsb) {
#pragma unroll
      for (int m = 0; m < kPat; ++m) off[m] = src_offset(lane, m, rsb, NR);
    }
  };

  // Issue the whole tile (rows 0..nv-1 of the tile starting at `base`,
  // wave-uniform) into LDS at `lds`.
  __device__ static __forceinline__ void issue(const uint8_t* base, uint32_t rsb, int nv, int lane,
                                               const Plan& plan, uint8_t* lds) {
    const uint32_t l0 = lds_addr(lds);
    if (nv == NR) {
#pragma unroll
      for (int i = 0; i < kInst; ++i) {
        const uint8_t* g = base + (size_t)(i / kPat) * (size_t)(kPat * kRpi) * rsb;
        dma_to_lds<kElem, true>(g, plan.off[i % kPat], l0 + i * 64 * kSlot);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kInst; ++i) dma_to_lds<kElem>(base, src_offset(lane, i, rsb, nv), l0 + i * 64 * kSlot);
    }
  }

  // Lane v's own row as ROWB/4 dwords (ROWB >= 4) or one half-dword.
  template <int NW>
  __device__ static __forceinline__ void read_row(const uint8_t* lds, int v, uint32_t (&w)[NW]) {
    const uint8_t* row = lds + v * kRowLds;
    if constexpr (kWide) {
      static_assert(NW == ROWB / 4, "row words");
      int s = swz(v);
      asm("" : "+v"(s));   // keep per-chunk addresses short-lived (not hoisted)
      static_for<kCpr>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        const uint4 q = *(const uint4*)(row + 16 * (c ^ s));
        w[4 * c + 0] = q.x;
        w[4 * c + 1] = q.y;
        w[4 * c + 2] = q.z;
        w[4 * c + 3] = q.w;
      });
    } else if constexpr (ROWB == 8) {
      const uint2 q = *(const uint2*)row;
      w[0] = q.x;
      w[1] = q.y;
    } else if constexpr (ROWB == 4) {
      w[0] = *(const uint32_t*)row;
    } else {
      w[0] = *(const uint16_t*)row;
    }
  }
};

// A D-float row (lambda) fetched by LDS-DMA: lanes 0..D/4-1 move 16 B each.
template <int D>
__device__ __forceinline__ void issue_row_f32(const float* src, int lane, uint8_t* lds) {
  static_assert(D <= 256, "one DMA instruction per row");
  if (D / 4 == 64 || lane < D / 4) dma_to_lds<16>(src, 16u * (uint32_t)lane, lds_addr(lds));
}

// A head's D int8 signs fetched by LDS-DMA: pair m = 64i + l (lane l of
// instruction i, m < D/2) moves bytes 2m, 2m+1 into the low half of LDS
// dword m (a sub-dword DMA fills one 4-byte slot per lane).  The kernel then
// turns slot m into sign mask m in place (build_masks).
template <int D>
struct SignRow {
  static constexpr int kMasks = D / 2;                 // one per packed fp16 pair
  static constexpr int kSlots = kMasks < 64 ? 64 : kMasks;
  static constexpr int kInst = (kMasks + 63) / 64;
};
template <int D>
__device__ __forceinline__ void issue_signs(const int8_t* row, int lane, uint32_t* lds) {
  static_for<SignRow<D>::kInst>([&](auto ii) {
    constexpr int i = decltype(ii)::value;
    if (64 * i + lane < SignRow<D>::kMasks)
      dma_to_lds<2>(row + 128 * i, 2u * (uint32_t)lane, lds_addr(lds + 64 * i));
  });
}
// Raw sign slots of this lane (read before the next DMA reuses the row).
template <int D>
__device__ __forceinline__ void read_sign_slots(const uint32_t* lds, int lane,
                                                uint32_t (&u)[SignRow<D>::kInst]) {
  static_for<SignRow<D>::kInst>([&](auto ii) {
    constexpr int i = decltype(ii)::value;
    u[i] = lds[64 * i + lane];
  });
}
template <int D>
__device__ __forceinline__ void build_masks(uint32_t* lds, int lane, const uint32_t (&u)[SignRow<D>::kInst]) {
  static_for<SignRow<D>::kInst>([&](auto ii) {
    constexpr int i = decltype(ii)::value;
    lds[64 * i + lane] = sign_mask_of(u[i]);
  });
}

// Number of global store instructions store_words<N> / store_scales issue.
template <int N>
constexpr int store_count() {
  return N % 4 == 0 ? N / 4 : 1;
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
// Quantize: fp16 [B,T,H,D] -> codes + fp16 scales, head-major [B,H,pitch,.]
// (pitch = T, or the capacity of an append cache, where token t of tensor b
// goes to row pos[b] + t).
//
// Loop per tile: wait for the tile's LDS-DMA (not for the previous tile's
// stores), read the own row from LDS, issue the next tile's DMA, transform +
// quantize in registers, store.  lambda rows arrive by DMA too, into a
// double-buffered LDS row read with broadcast ds_reads.
// ----------------------------------------------------------------------------
template <int D, int G, int BITS, int ROT, int VAR, bool LAM>
__global__ __launch_bounds__(64) SRFTQ_QUANT_OCC void quantize_kernel(const uint16_t* __restrict__ x,
                                                                      const int8_t* __restrict__ signs,
                                                                      const float* __restrict__ lambda,
                                                                      uint8_t* __restrict__ codes_out,
                                                                      uint16_t* __restrict__ scales_out,
                                                                      Geo a) {
  using XT = RowTile<2 * D>;
  constexpr int CB = D * BITS / 8;        // code bytes per vector
  constexpr int SB = 2 * D / G;           // scale bytes per vector
  constexpr int NCW = CodeWords<D, BITS>::kWords;
  constexpr int NSW = ScaleWords<D, G>::kWords;
  constexpr int NST = store_count<NCW>() + (D / G == 1 ? 1 : store_count<NSW>());   // global stores per tile
  __shared__ __attribute__((aligned(16))) uint8_t lds[XT::kBytes];
  __shared__ __attribute__((aligned(16))) float lam_lds[LAM ? 2 * D : 4];
  constexpr int SM = SignRow<D>::kSlots;
  __shared__ __attribute__((aligned(16))) uint32_t smask[2 * SM];   // sign masks, double-buffered

  const int lane = threadIdx.x;
  const TileRange tr(a);
  if (tr.first >= a.n_tiles) return;
  const int stride = tr.step;
  const uint32_t rsb = (uint32_t)a.H * (uint32_t)(2 * D);   // x row stride, bytes
  typename XT::Plan plan;
  plan.init(lane, rsb);
  const int dk = stride / a.BH, dbh = stride - dk * a.BH;

  Cursor cur;
  cur.init(tr.first, a.BH);
  int remaining = tr.remaining;     // tiles after this one

  auto issue = [&](const Cursor& c, int& nv, int buf) {
    const int64_t t0 = (int64_t)c.k * 64;
    const int64_t left = a.T - t0;
    nv = left < 64 ? (int)left : 64;
    lds_poison<XT::kBytes>(lds, lane);
    if constexpr (LAM) lds_poison<4 * D>(lam_lds + buf * D, lane);
    lds_poison<4 * SM>(smask + buf * SM, lane);
    XT::issue((const uint8_t*)x + row_index(a, c.bh, t0) * (int64_t)(2 * D), rsb, nv, lane, plan, lds);
    if constexpr (LAM) issue_row_f32<D>(lambda + (int64_t)c.bh * D, lane, (uint8_t*)(lam_lds + buf * D));
    issue_signs<D>(signs + (int64_t)c.bh * a.sign_stride, lane, smask + buf * SM);
  };

  int nv, buf = 0;
  issue(cur, nv, 0);

  // One tile: read it from LDS, start the next tile's DMA, compute, store.
  auto body = [&]() {
    wave_fence();
    uint32_t w[D / 2];
    XT::read_row(lds, lane, w);
    const int cb = buf;
    uint32_t su[SignRow<D>::kInst];
    read_sign_slots<D>(smask + cb * SM, lane, su);
    wait_lgkm0();   // the reads are done before the next DMA reuses the tile

    const Cursor now = cur;
    const int nv_now = nv;
    if (remaining > 0) {
      cur.advance(dk, dbh, a.BH);
      buf ^= 1;
      issue(cur, nv, buf);
    }

    build_masks<D>(smask + cb * SM, lane, su);   // in order before the broadcast reads
    float y[D];
    forward<D, ROT, VAR>(w, LdsSigns{smask + cb * SM}, y);
    uint32_t codes[NCW];
    uint32_t scales[NSW];
    quantize_tail<D, G, BITS, ROT, VAR, LAM>(y, lam_lds + cb * D, codes, scales);

    // Cache row of token 0 of the tile (uniform); when appending, tokens
    // start at the tensor's position and rows outside [0, pitch) are dropped.
    int64_t t0 = (int64_t)now.k * 64;
    bool ok = lane < nv_now;
    if (a.pos) {
      t0 += a.pos[now.bh / a.H];
      ok = ok && t0 + lane >= 0 && t0 + lane < a.pitch;
    }
    if (ok) {
      const int64_t r0 = cache_row(a, now.bh, t0);
      store_words<NCW>(codes_out + r0 * CB + (uint32_t)lane * CB, codes);
      store_scales<D, G>((uint8_t*)scales_out + r0 * SB + (uint32_t)lane * SB, scales);
    }
    // with dropped rows a whole wave may skip its stores: then the next
    // wait must not count on them
    return nv_now == 64 && !a.pos;
  };

  // The first tile is peeled so that every entry into the loop has this
  // tile's stores issued after the next tile's DMA: the wait at the top of
  // the loop then covers the DMA only.
  wait_vm<0>();
  bool full = body();
  while (remaining > 0) {
    --remaining;
    // A full tile issued exactly NST stores after the DMA; after a ragged
    // one some stores may have been skipped, so wait for everything.
    if (full)
      wait_vm<NST>();
    else
      wait_vm<0>();
    full = body();
  }
}

// ----------------------------------------------------------------------------
// Dequantize: rows [0, T) of codes + scales [B,H,pitch,.] -> fp16 [B,T,H,D].  Codes, scales and lambda
// arrive by coalesced LDS-DMA (prefetched one tile ahead); output rows are
// staged through LDS half a row at a time and leave as 1 KiB coalesced
// stores.
// ----------------------------------------------------------------------------
template <int D, int G, int BITS, int ROT, int VAR, bool LAM>
__global__ __launch_bounds__(64) SRFTQ_DEQUANT_OCC void dequantize_kernel(const uint8_t* __restrict__ codes_in,
                                                                          const uint16_t* __restrict__ scales_in,
                                                                          const int8_t* __restrict__ signs,
                                                                          const float* __restrict__ lambda,
                                                                          uint16_t* __restrict__ x_out, Geo a) {
  using Sc = Scales<D, ROT, VAR>;
  constexpr int CB = D * BITS / 8;
  constexpr int SB = 2 * D / G;
  constexpr int NCW = CodeWords<D, BITS>::kWords;
  constexpr int NSW = ScaleWords<D, G>::kWords;
  using CT = RowTile<CB>;
  using ST = RowTile<SB>;
  using OT = RowTile<D>;                  // half an fp16 output row (D bytes)
  constexpr int NST = 2 * OT::kInst;      // global stores per tile
  __shared__ __attribute__((aligned(16))) uint8_t ctile[CT::kBytes];
  __shared__ __attribute__((aligned(16))) uint8_t stile[ST::kBytes < 16 ? 16 : ST::kBytes];
  __shared__ __attribute__((aligned(16))) uint8_t otile[OT::kBytes];
  __shared__ __attribute__((aligned(16))) float lam_lds[LAM ? 2 * D : 4];
  constexpr int SM = SignRow<D>::kSlots;
  __shared__ __attribute__((aligned(16))) uint32_t smask[2 * SM];   // sign masks, double-buffered

  const int lane = threadIdx.x;
  const TileRange tr(a);
  if (tr.first >= a.n_tiles) return;
  const int stride = tr.step;
  const uint32_t rsb_c = CB, rsb_s = SB;   // cache rows are contiguous
  const uint32_t rsb_x = (uint32_t)a.H * (uint32_t)(2 * D);
  typename CT::Plan cplan;
  cplan.init(lane, rsb_c);
  typename ST::Plan splan;
  splan.init(lane, rsb_s);
  // output staging: per-lane LDS and global offsets for each store pattern
  uint32_t o_lds[OT::kPat], o_glb[OT::kPat];
#pragma unroll
  for (int m = 0; m < OT::kPat; ++m) {
    const int v = m * OT::kRpi + lane / OT::kCpr;
    const int p = lane % OT::kCpr;
    o_lds[m] = (uint32_t)(v * D + 16 * (p ^ OT::swz(v)));
    o_glb[m] = (uint32_t)v * rsb_x + 16u * (uint32_t)p;
  }
  const int dk = stride / a.BH, dbh = stride - dk * a.BH;

  Cursor cur;
  cur.init(tr.first, a.BH);
  int remaining = tr.remaining;

  auto issue = [&](const Cursor& c, int& nv, int buf) {
    const int64_t t0 = (int64_t)c.k * 64;
    const int64_t left = a.T - t0;
    nv = left < 64 ? (int)left : 64;
    const int64_t r0 = cache_row(a, c.bh, t0);
    lds_poison<CT::kBytes>(ctile, lane);
    lds_poison<sizeof(stile)>(stile, lane);
    if constexpr (LAM) lds_poison<4 * D>(lam_lds + buf * D, lane);
    lds_poison<4 * SM>(smask + buf * SM, lane);
    CT::issue(codes_in + r0 * CB, rsb_c, nv, lane, cplan, ctile);
    ST::issue((const uint8_t*)scales_in + r0 * SB, rsb_s, nv, lane, splan, stile);
    if constexpr (LAM) issue_row_f32<D>(lambda + (int64_t)c.bh * D, lane, (uint8_t*)(lam_lds + buf * D));
    issue_signs<D>(signs + (int64_t)c.bh * a.sign_stride, lane, smask + buf * SM);
  };

  int nv, buf = 0;
  issue(cur, nv, 0);

  auto body = [&]() {
    wave_fence();
    uint32_t cw[NCW], sw[NSW];
    CT::read_row(ctile, lane, cw);
    ST::read_row(stile, lane, sw);
    const int cb = buf;
    {
      uint32_t su[SignRow<D>::kInst];
      read_sign_slots<D>(smask + cb * SM, lane, su);
      build_masks<D>(smask + cb * SM, lane, su);
    }
    if constexpr (LAM) {
      // e_j / lambda_j, computed lane-parallel in place, read back broadcast
      float* lt = lam_lds + cb * D;
      for (int j = lane; j < D; j += 64) {
        const bool edge = Sc::kEdges && (j == 0 || j == D / 2);
        lt[j] = (edge ? (float)Sc::kInvEdge : (float)Sc::kInvBulk) * __builtin_amdgcn_rcpf(lt[j]);
      }
    }
    wait_lgkm0();   // the reads are done before the next DMA reuses the tiles
    wave_fence();

    const Cursor now = cur;
    const int nv_now = nv;
    if (remaining > 0) {
      cur.advance(dk, dbh, a.BH);
      buf ^= 1;
      issue(cur, nv, buf);
    }

    float y[D];
    dequantize_head<D, G, BITS, ROT, VAR, LAM>(cw, sw, lam_lds + cb * D, y);
    // d = 256 fills the register file: keep the scheduler from interleaving
    // the head with the transform, which would need more than 512 registers
    if constexpr (D >= 256) __builtin_amdgcn_sched_barrier(0);
    float xr[D];
    inverse<D, ROT, VAR>(y, xr);

    // fp16 RNE, then the sign multiply as an XOR on the packed halves
    const LdsSigns sg{smask + cb * SM};
    uint32_t o[D / 2];
    static_for<D / 8>([&](auto qq) {
      constexpr int q = decltype(qq)::value;
      const uint4 m4 = sg.mask4(q);
      o[4 * q + 0] = pack_f16x2(xr[8 * q + 0], xr[8 * q + 1]) ^ m4.x;
      o[4 * q + 1] = pack_f16x2(xr[8 * q + 2], xr[8 * q + 3]) ^ m4.y;
      o[4 * q + 2] = pack_f16x2(xr[8 * q + 4], xr[8 * q + 5]) ^ m4.z;
      o[4 * q + 3] = pack_f16x2(xr[8 * q + 6], xr[8 * q + 7]) ^ m4.w;
    });

    uint8_t* obase = (uint8_t*)x_out + row_index(a, now.bh, (int64_t)now.k * 64) * (int64_t)(2 * D);
    static_for<2>([&](auto hh) {
      constexpr int h = decltype(hh)::value;
      lds_poison<OT::kBytes>(otile, lane);
      {
        uint8_t* row = otile + lane * D;
        int s = OT::swz(lane);
        asm("" : "+v"(s));
        static_for<OT::kCpr>([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          constexpr int k = h * OT::kCpr + c;       // chunk of the full row
          *(uint4*)(row + 16 * (c ^ s)) = make_uint4(o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]);
        });
      }
      wave_fence();
      static_for<OT::kInst>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
        constexpr int m = i % OT::kPat;
        // o_lds[m] already holds the rows of pattern m; add whole periods only
        const uint4 q = *(const uint4*)(otile + (i / OT::kPat) * (OT::kPat * OT::kRpi * D) + o_lds[m]);
        uint8_t* dst = obase + (size_t)(i / OT::kPat) * (size_t)(OT::kPat * OT::kRpi) * rsb_x + h * D + o_glb[m];
        if (nv_now == 64 || i * OT::kRpi + lane / OT::kCpr < nv_now) {
          typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
          const u32x4_t v = {q.x, q.y, q.z, q.w};
          __builtin_nontemporal_store(v, (u32x4_t*)dst);
        }
      });
      wave_fence();
    });
    return nv_now == 64;
  };

  // First tile peeled: inside the loop the wait covers the next tile's DMA
  // only, while this tile's stores drain.
  wait_vm<0>();
  bool full = body();
  while (remaining > 0) {
    --remaining;
    // see quantize_kernel: exact store count only after a full tile
    if (full)
      wait_vm<NST>();
    else
      wait_vm<0>();
    full = body();
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
