// dense.h -- quantize / dequantize with a rotation given as a matrix.
//
// "When Quantization Is Free" (gist.science summary), Metodologia 3: besides
// the fixed SRFT, the pages study a learned rotation R (with lambda) and
// Householder rotations, k = d/2 reflectors at d = 256.  Any such rotation is
// an orthogonal d x d matrix Q; the quantizer of Metodologia 2 step 4 is then
// applied to y = Q (s . x), and the inverse is x = s . Q^T yhat.
//
// The product is a dense contraction (2 d^2 flops per vector), so it runs on
// the matrix cores: v_mfma_f32_32x32x16_f16 (the full-rate fp16 shape of
// gfx950), fp32 accumulation.
//
// quantize_dense_kernel  A block of W = D/32 waves works through consecutive
//   64-token tiles of one (tensor, head) at a time.  Wave w owns output rows
//   32w .. 32w+31: it holds 2^10 Q[r, c] s_c for those rows in registers as
//   fp16 hi + lo parts (A operands, D/2 VGPRs; the factor 2^10 keeps both
//   parts normal), so y = Q (s . x) is two MFMAs per 32 x 32 x 16 block (x is
//   exact in fp16), products exact, sums in fp32.  The MFMA result puts rows
//   8m + 4h + e (m, e < 4) of a 32-row tile in lane half h; the A rows are
//   permuted, tile row i -> 32w + 16 ((i/4) % 2) + 4 (i/8) + i%4, so that lane
//   (token j = lane%32, h = lane/32) ends with the 16 contiguous outputs
//   32w + 16h .. +15 of token j.  The quantizer (quant.h's decision rule)
//   runs on them in registers -- a group of 16 is one lane, a group of 32 two
//   (one shuffle) -- and the lane stores its codes and scale directly.  The x
//   tile arrives by LDS-DMA (every wave reads all of it), one tile ahead; its
//   16-byte chunks are XOR-swizzled by row so that the 16 rows one operand
//   read phase touches fall in different banks.
// dequantize_dense_kernel  The same blocks and the same permuted A tiles, now
//   of 2^10 s_i Q[c, i] (Q^T).  The B operand yhat_c = q_c sigma / lambda_c is
//   not exact in fp16: the block first expands each token's codes into
//   u = yhat 2^sh (sh puts the token's largest |u| in [2^14, 2^15)), split
//   into fp16 hi + lo parts in LDS, then takes three MFMAs per block (hi*hi,
//   hi*lo, lo*hi; lo*lo is below 2^-22 relative) and scales each token's
//   outputs back by 2^(-sh-10) (ldexp) before the fp16 store.
#pragma once

#include "launch.h"
#include "quant.h"

namespace srftq {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t w32x4_t __attribute__((ext_vector_type(4)));

struct DenseGeo {
  int64_t T;            // tokens per tensor
  int64_t n_tiles;      // BH * tiles_t
  int64_t q_stride;     // elements between the heads' matrices (0: one shared matrix)
  int32_t H;
  int32_t tiles_t;      // 64-token tiles per head
  int32_t per_block;    // consecutive tiles per block
  int32_t sign_stride;  // D, or 0 (one shared row)
};

__device__ __forceinline__ w32x4_t lds_read128(uint32_t byte_addr) {
  return *(const __attribute__((address_space(3))) w32x4_t*)(uintptr_t)byte_addr;
}
__device__ __forceinline__ void lds_write128(uint32_t byte_addr, w32x4_t v) {
  *(__attribute__((address_space(3))) w32x4_t*)(uintptr_t)byte_addr = v;
}
__device__ __forceinline__ float lds_readf(uint32_t byte_addr) {
  return *(const __attribute__((address_space(3))) float*)(uintptr_t)byte_addr;
}
__device__ __forceinline__ void lds_writef(uint32_t byte_addr, float v) {
  *(__attribute__((address_space(3))) float*)(uintptr_t)byte_addr = v;
}

// Buffer resources (gfx9 raw buffers: stride 0, byte bounds): loads past
// num_records return 0 and stores past it are dropped, which is how the
// kernels handle the rows past the end of a tensor.  Every offset is a per-
// lane 32-bit byte offset (the bounds check applies to it).
typedef uint32_t w32x2_t __attribute__((ext_vector_type(2)));
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kNT = 2;   // cache policy: nontemporal (streamed once)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// Output row of A-tile row i (0..31) of wave w.
__device__ __forceinline__ int dense_row(int w, int i) {
  return 32 * w + 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
}

// fp16 hi + lo parts of 8 fp32 values.
__device__ __forceinline__ void split8(const float (&v)[8], f16x8_t& hi, f16x8_t& lo) {
  static_for<8>([&](auto ee) {
    constexpr int e = decltype(ee)::value;
    const _Float16 h = (_Float16)v[e];
    hi[e] = h;
    lo[e] = (_Float16)(v[e] - (float)h);
  });
}

__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
  static_for<16>([&](auto ee) { z[decltype(ee)::value] = 0.0f; });
  return z;
}

// ----------------------------------------------------------------------------
// y = Q (s . x), then lambda, group absmax and rounding.
// ----------------------------------------------------------------------------
template <int D, int G, int BITS>
__global__ __launch_bounds__(2 * D, 2) void quantize_dense_kernel(const float* __restrict__ Q,
                                                                  const uint16_t* __restrict__ x,
                                                                  const int8_t* __restrict__ signs,
                                                                  const float* __restrict__ lambda,
                                                                  uint8_t* __restrict__ codes,
                                                                  uint16_t* __restrict__ scales,
                                                                  DenseGeo a) {
  static_assert(D == 64 || D == 128 || D == 256, "head size");
  static_assert(G == 8 || G == 16 || G == 32, "a group lies within one wave's 32 rows");
  using QC = QConst<BITS>;
  constexpr int KS = D / 16;              // k-steps of 16 coordinates
  constexpr int ROWB = 2 * D;             // bytes per x row
  constexpr int CH = ROWB / 16;           // 16-byte chunks per row
  constexpr int SWM = CH < 16 ? CH - 1 : 15;   // chunk swizzle mask
  constexpr int TILE = 64 * ROWB;
  constexpr int NT = 2 * D;               // threads
  constexpr int W = D / 32;               // waves
  constexpr int NDMA = 64 * CH / 64 / W;  // 1 KiB LDS-DMA instructions per wave per tile (4)
  constexpr int NST = 4;                  // buffer stores per wave per tile
  constexpr int CB = D * BITS / 8;        // code bytes per token
  constexpr int NG = D / G;
  static_assert(NDMA * W * 1024 == TILE, "the waves' DMA instructions cover the tile");
  // two x tiles, then lambda * 2^-10 of the current head
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * TILE + 4 * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31, hf = lane >> 5;
  const int64_t first = (int64_t)blockIdx.x * a.per_block;
  int64_t last = first + a.per_block;
  last = last < a.n_tiles ? last : a.n_tiles;
  if (first >= last) return;
  const uint32_t lds0 = lds_addr(smem);

  // LDS layout of a tile: row r (token), 16-byte chunk c at r*ROWB + 16 (c ^ (r & SWM)).
  // DMA: instruction i of wave w fills LDS bytes [1 KiB (NDMA w + i), +1 KiB):
  // slot p = 64 (NDMA w + i) + lane holds chunk (p % CH) ^ (row & SWM) of row
  // p / CH, read from that row of the tile (rows past T re-read the last row).
  const uint32_t xstride = (uint32_t)a.H * ROWB;
  auto issue = [&](int bh, int k, int stage) {
    const int64_t t0 = (int64_t)k * 64;
    const int b = bh / a.H, h = bh - b * a.H;
    const int64_t left = a.T - t0;
    const int rows = left < 64 ? (int)left : 64;
    const uint16_t* base = x + (((int64_t)b * a.T + t0) * a.H + h) * D;
    // offsets recomputed per tile from an opaque lane id: a few VALU ops
    // instead of registers held across the loop
    int ln = lane;
    asm volatile("" : "+v"(ln));
    static_for<NDMA>([&](auto ii) {
      constexpr int i = decltype(ii)::value;
      const int p = 64 * (NDMA * wave + i) + ln;
      const int row = p / CH;
      const int c = (p % CH) ^ (row & SWM);
      const int rr = row < rows ? row : rows - 1;
      dma_to_lds<16, true>(base, (uint32_t)rr * xstride + 16u * (uint32_t)c,
                           lds0 + (uint32_t)(stage * TILE + 1024 * (NDMA * wave + i)));
    });
  };

  // A operands of this wave's rows for head bh.
  f16x8_t ahi[KS], alo[KS];
  auto build = [&](int bh) {
    const float* qrow = Q + (int64_t)bh * a.q_stride + (int64_t)dense_row(wave, j) * D;
    const int8_t* sg = signs + (int64_t)bh * a.sign_stride;
    static_for<KS>([&](auto kk) {
      constexpr int ks = decltype(kk)::value;
      const int c0 = 16 * ks + 8 * hf;
      const float4 v0 = *(const float4*)(qrow + c0);
      const float4 v1 = *(const float4*)(qrow + c0 + 4);
      const uint32_t s0 = *(const uint32_t*)(sg + c0), s1 = *(const uint32_t*)(sg + c0 + 4);
      const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      float p[8];
      static_for<8>([&](auto ee) {
        constexpr int e = decltype(ee)::value;
        const uint32_t sb = ((e < 4 ? s0 : s1) >> (8 * (e & 3))) & 0x80u;   // sign bit of int8 -1
        p[e] = as_f32(as_u32(v[e] * 1024.0f) ^ (sb << 24));
      });
      split8(p, ahi[ks], alo[ks]);
      __builtin_amdgcn_sched_barrier(0);   // one block's loads at a time
    });
  };
  // lambda_r 2^-10 of the segment's head (read after the next barrier)
  const uint32_t lam_lds = lds0 + 2 * TILE;
  auto write_lam = [&](int bh) {
    for (int r = tid; r < D; r += NT)
      lds_writef(lam_lds + 4u * (uint32_t)r, (lambda ? lambda[(int64_t)bh * D + r] : 1.0f) * (1.0f / 1024.0f));
  };

  // B operand of lane (j, hf) at k-step ks of 32-token block n: row 32n + j,
  // chunk 2 ks + hf, stored at chunk (2 ks + hf) ^ s = 2 (ks ^ (s >> 1)) +
  // ((hf ^ s) & 1) with s = j & SWM: a lane base plus (32 ks) ^ (32 (s >> 1)).
  const int sj = j & SWM;
  const uint32_t rlane = (uint32_t)(j * ROWB + 16 * ((hf ^ sj) & 1));
  const uint32_t xu = 32u * (uint32_t)(sj >> 1);
  const uint32_t lam_row = lam_lds + 4u * (uint32_t)(32 * wave + 16 * hf);
  const float magic = as_f32(QC::kMagicBits);

  // Tiles first .. last-1 of the block, head by head.  (bh, k): the current
  // tile's head and index within the head, kept as counters.
  int bh = (int)(first / a.tiles_t);
  int k = (int)(first - (int64_t)bh * a.tiles_t);
  issue(bh, k, 0);
  int64_t it = first;
  while (it < last) {
    // new head: every wave is past the previous tile (its lambda reads), then
    // the matrix rows and lambda of this head; all loads waited for here, so
    // nothing issued on this path is pending inside the tile loop
    __syncthreads();
    build(bh);
    write_lam(bh);
    __builtin_amdgcn_s_waitcnt(0);
    const int64_t seg_end = (it - k) + a.tiles_t < last ? (it - k) + a.tiles_t : last;
    for (; it < seg_end; ++it, ++k) {
      const int stage = (int)((it - first) & 1);
      // this wave's part of the tile has landed: after it, only the previous
      // tile's stores were issued
      if (it == first) wait_vm<0>();
      else wait_vm<NST>();
      __syncthreads();   // the whole tile is in LDS; the other stage is no longer read
      if (it + 1 < last) {
        if (k + 1 < a.tiles_t) issue(bh, k + 1, stage ^ 1);
        else issue(bh + 1, 0, stage ^ 1);
      }

      const uint32_t sbase = lds0 + (uint32_t)(stage * TILE) + rlane;
      const int64_t left = a.T - (int64_t)k * 64;
      const uint32_t rows = left < 64 ? (uint32_t)left : 64u;
      const int64_t row0 = (int64_t)bh * a.T + (int64_t)k * 64;
      static_for<2>([&](auto nn) {
        constexpr int n = decltype(nn)::value;
        const uint32_t nb = sbase + (uint32_t)(32 * n * ROWB);
        f32x16_t acc = zero16();
        f16x8_t bx[2];
        bx[0] = __builtin_bit_cast(f16x8_t, lds_read128(nb + (0u ^ xu)));
        static_for<KS>([&](auto kk) {
          constexpr int ks = decltype(kk)::value;
          if constexpr (ks + 1 < KS)
            bx[(ks + 1) & 1] = __builtin_bit_cast(f16x8_t, lds_read128(nb + ((32u * (ks + 1)) ^ xu)));
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[ks], bx[ks & 1], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo[ks], bx[ks & 1], acc, 0, 0, 0);
        });

        // quantize: lane (j, hf) holds outputs 32w + 16hf .. +15 of token 32n + j
        float z[16];
        static_for<4>([&](auto qq) {
          constexpr int q4 = decltype(qq)::value;
          const w32x4_t l4 = lds_read128(lam_row + 16 * q4);
          static_for<4>([&](auto ee) {
            constexpr int e = 4 * q4 + decltype(ee)::value;
            z[e] = acc[e] * as_f32(l4[decltype(ee)::value]);
          });
        });
        constexpr int GL = G < 16 ? G : 16;   // group width within a lane
        uint32_t tb[16];
        uint32_t shv[16 / GL];
        static_for<16 / GL>([&](auto gg) {
          constexpr int g = decltype(gg)::value;
          float m = 0.0f;
          static_for<GL>([&](auto ee) { m = __builtin_fmaxf(m, __builtin_fabsf(z[g * GL + decltype(ee)::value])); });
          if constexpr (G == 32) m = __builtin_fmaxf(m, __shfl_xor(m, 32));
          const float tq = __builtin_fminf(m * QC::kQinv, 65504.0f);
          const uint32_t sh = pack_f16x2(tq, 0.0f) & 0xffffu;
          const float sg = hlo(sh);
          const float r = sg == 0.0f ? 0.0f : recip_f16_value(sg);
          shv[g] = sh;
          static_for<GL>([&](auto ee) {
            constexpr int e = g * GL + decltype(ee)::value;
            // the clamp only acts for fp16-subnormal or saturated scales
            int bi = (int)as_u32(__builtin_fmaf(z[e], r, magic));
            bi = bi < (int)QC::kLo ? (int)QC::kLo : bi;
            bi = bi > (int)QC::kHi ? (int)QC::kHi : bi;
            tb[e] = (uint32_t)bi;
          });
        });
        // rows past T fall outside the resources' bounds and are dropped; one
        // resource per 32-token block, so both blocks share the lane offsets.
        // Exactly two stores per block (NST per tile), unconditionally.
        const int rn = (int)rows - 32 * n;
        const uint32_t nr = rn > 0 ? (uint32_t)rn : 0u;
        const auto crs = make_rsrc(codes + (row0 + 32 * n) * CB, nr * CB);
        const auto srs = make_rsrc(scales + (row0 + 32 * n) * NG, nr * NG * 2);
        const uint32_t c0 = (uint32_t)(32 * wave + 16 * hf);
        if constexpr (BITS == 4) {
          const w32x2_t v = {pack_codes<4>(tb), pack_codes<4>(tb + 8)};
          __builtin_amdgcn_raw_buffer_store_b64(v, crs, (uint32_t)j * CB + c0 / 2, 0, 0);
        } else {
          const w32x4_t v = {pack_codes<8>(tb), pack_codes<8>(tb + 4), pack_codes<8>(tb + 8), pack_codes<8>(tb + 12)};
          __builtin_amdgcn_raw_buffer_store_b128(v, crs, (uint32_t)j * CB + c0, 0, 0);
        }
        // a group of 32 is shared by the two lane halves: both store the same value
        if constexpr (G == 8)
          __builtin_amdgcn_raw_buffer_store_b32(shv[0] | (shv[1] << 16), srs, 2u * ((uint32_t)j * NG + c0 / 8), 0, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)shv[0], srs, 2u * ((uint32_t)j * NG + c0 / G), 0, 0);
        __builtin_amdgcn_sched_barrier(0);   // one block's state live at a time
      });
    }
    ++bh;
    k = 0;
  }
}

// ----------------------------------------------------------------------------
// x = s . Q^T yhat,  yhat_c = q_c sigma_G(c) / lambda_c.
// ----------------------------------------------------------------------------
template <int D, int G, int BITS>
__global__ __launch_bounds__(2 * D, 2) void dequantize_dense_kernel(const float* __restrict__ Q,
                                                                 const uint8_t* __restrict__ codes,
                                                                 const uint16_t* __restrict__ scales,
                                                                 const int8_t* __restrict__ signs,
                                                                 const float* __restrict__ lambda,
                                                                 uint16_t* __restrict__ x_out,
                                                                 DenseGeo a) {
  static_assert(D == 64 || D == 128 || D == 256, "head size");
  static_assert(G == 8 || G == 16 || G == 32, "group");
  constexpr int KS = D / 16;
  constexpr int PITCH = 2 * D + 16;       // LDS row pitch of the B tiles
  constexpr int TILE = 64 * PITCH;
  constexpr int STAGE = 2 * TILE + 256;   // hi tile, lo tile, 64 output exponents
  constexpr int NT = 2 * D;
  constexpr int LPT = D / 32;             // prep lanes per token (32 coordinates each)
  constexpr int CB = D * BITS / 8;
  constexpr int NG = D / G;
  constexpr int GPL = 32 / G;             // groups per prep lane
  constexpr float kOff = BITS == 4 ? 8.0f : 128.0f;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE + 4 * (D + D / 8)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31, hf = lane >> 5;
  const int64_t first = (int64_t)blockIdx.x * a.per_block;
  int64_t last = first + a.per_block;
  last = last < a.n_tiles ? last : a.n_tiles;
  if (first >= last) return;
  const uint32_t lds0 = lds_addr(smem);
  const uint32_t ilam_lds = lds0 + 2 * STAGE;   // 1 / lambda of the current head

  // prep role: token pr (0..63) of the tile, coordinates 32 pp .. +31
  const int pr = tid / LPT, pp = tid % LPT;
  uint32_t cw[BITS];       // this lane's 32 codes: int4 4 dwords, int8 8 dwords
  uint32_t sw[(GPL + 1) / 2];
  // rows past T read 0 (codes 0, scale 0: their outputs are not stored)
  auto load = [&](int bh, int k) {
    const int64_t t0 = (int64_t)k * 64;
    const int64_t left = a.T - t0;
    const uint32_t rows = left < 64 ? (uint32_t)left : 64u;
    const int64_t row0 = (int64_t)bh * a.T + t0;
    const auto crs = make_rsrc(codes + row0 * CB, rows * CB);
    const auto srs = make_rsrc(scales + row0 * NG, rows * NG * 2);
    static_for<BITS / 4>([&](auto ii) {
      constexpr int i = decltype(ii)::value;
      const w32x4_t v = __builtin_bit_cast(
          w32x4_t, __builtin_amdgcn_raw_buffer_load_b128(crs, (uint32_t)(pr * CB + pp * (4 * BITS) + 16 * i), 0, kNT));
      static_for<4>([&](auto ee) { cw[4 * i + decltype(ee)::value] = v[decltype(ee)::value]; });
    });
    const uint32_t soff = 2u * (uint32_t)(pr * NG + pp * GPL);
    if constexpr (GPL == 1) {
      sw[0] = __builtin_amdgcn_raw_buffer_load_b16(srs, soff, 0, 0);
    } else if constexpr (GPL == 2) {
      sw[0] = __builtin_amdgcn_raw_buffer_load_b32(srs, soff, 0, 0);
    } else {
      const w32x2_t v = __builtin_bit_cast(w32x2_t, __builtin_amdgcn_raw_buffer_load_b64(srs, soff, 0, 0));
      sw[0] = v[0], sw[1] = v[1];
    }
  };
  // u = q sigma / lambda 2^sh as fp16 hi + lo into the stage's B tiles
  auto prep = [&](int stage) {
    float u[32];
    float mx = 0.0f;
    static_for<32>([&](auto mm) {
      constexpr int m = decltype(mm)::value;
      constexpr int g = m / G;
      const float sgm = (g % 2 == 0) ? hlo(sw[g / 2]) : hhi(sw[g / 2]);
      float cval;
      if constexpr (BITS == 4) {
        const uint32_t nib = (cw[m / 8] >> (4 * (m % 8))) & 0xFu;
        cval = (float)(nib ^ 8u);              // q + 8
      } else {
        const uint32_t byte = (cw[m / 4] >> (8 * (m % 4))) & 0xFFu;
        cval = (float)(byte ^ 0x80u);          // q + 128
      }
      // q sigma exactly (small integers), then / lambda
      const float v = __builtin_fmaf(cval, sgm, -kOff * sgm);
      u[m] = v * lds_readf(ilam_lds + 4u * (uint32_t)(36 * pp + m));
      mx = __builtin_fmaxf(mx, __builtin_fabsf(u[m]));
    });
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 1));
    if constexpr (LPT > 2) mx = __builtin_fmaxf(mx, __shfl_xor(mx, 2));
    if constexpr (LPT > 4) mx = __builtin_fmaxf(mx, __shfl_xor(mx, 4));
    // ldexp, not a multiply by 2^sh: sh exceeds 127 for tiny scales
    const int sh = mx > 0.0f ? 15 - __builtin_amdgcn_frexp_expf(mx) : 0;
    const uint32_t sb = lds0 + (uint32_t)(stage * STAGE);
    f16x8_t hi[4], lo[4];
    static_for<4>([&](auto cc) {
      constexpr int c = decltype(cc)::value;
      float v[8];
      static_for<8>([&](auto ee) { v[decltype(ee)::value] = __builtin_ldexpf(u[8 * c + decltype(ee)::value], sh); });
      split8(v, hi[c], lo[c]);
    });
    // write k of lane pp stores chunk (k + 2 (pp / 4)) % 4: lanes pp and pp + 4
    // (64 bytes x 4 apart) then hit different banks
    const int rot = 2 * ((pp >> 2) & 1);
    static_for<4>([&](auto kk) {
      constexpr int k = decltype(kk)::value;
      const int c = (k + rot) & 3;
      const uint32_t off = (uint32_t)(pr * PITCH + 16 * (4 * pp + c));
      const f16x8_t vh = rot ? hi[(k + 2) & 3] : hi[k];
      const f16x8_t vl = rot ? lo[(k + 2) & 3] : lo[k];
      lds_write128(sb + off, __builtin_bit_cast(w32x4_t, vh));
      lds_write128(sb + TILE + off, __builtin_bit_cast(w32x4_t, vl));
    });
    if (pp == 0) lds_writef(sb + 2 * TILE + 4u * (uint32_t)pr, __builtin_bit_cast(float, -sh - 10));
  };

  f16x8_t ahi[KS], alo[KS];
  auto build = [&](int bh) {
    const float* Qh = Q + (int64_t)bh * a.q_stride;
    const int8_t* sg = signs + (int64_t)bh * a.sign_stride;
    const int r = dense_row(wave, j);
    const float s = sg[r] < 0 ? -1024.0f : 1024.0f;
    static_for<KS>([&](auto kk) {
      constexpr int ks = decltype(kk)::value;
      const int c0 = 16 * ks + 8 * hf;
      float p[8];
      static_for<8>([&](auto ee) {
        constexpr int e = decltype(ee)::value;
        p[e] = Qh[(int64_t)(c0 + e) * D + r] * s;
      });
      split8(p, ahi[ks], alo[ks]);
      __builtin_amdgcn_sched_barrier(0);   // one block's loads at a time
    });
  };
  // 1/lambda_c at float index c + 4 (c / 32): the 8 prep lanes of a token
  // read coordinates 32 pp + m at once, which this spreads over 8 banks
  auto build_ilam = [&](int bh) {
    for (int c = tid; c < D; c += NT)
      lds_writef(ilam_lds + 4u * (uint32_t)(c + 4 * (c >> 5)), lambda ? 1.0f / lambda[(int64_t)bh * D + c] : 1.0f);
  };

  // Tiles first .. last-1 of the block, head by head; (bh, k) the current
  // tile's head and index within the head, kept as counters.
  int bh = (int)(first / a.tiles_t);
  int k = (int)(first - (int64_t)bh * a.tiles_t);
  // prologue: the first tile's B operands
  build_ilam(bh);
  load(bh, k);
  __syncthreads();
  prep(0);
  const uint32_t xstride = (uint32_t)a.H * (2 * D);
  const uint32_t xlane = (uint32_t)j * xstride + 2u * (uint32_t)(32 * wave + 16 * hf);
  int64_t it = first;
  while (it < last) {
    // the matrix rows of this head; its loads waited for here, so nothing
    // issued on this path is pending inside the tile loop
    build(bh);
    __builtin_amdgcn_s_waitcnt(0);
    const int64_t seg_end = (it - k) + a.tiles_t < last ? (it - k) + a.tiles_t : last;
    for (; it < seg_end; ++it, ++k) {
      const int stage = (int)((it - first) & 1);
      __syncthreads();   // this stage's B tiles are written; the other stage is no longer read
      const bool more = it + 1 < last;
      const bool head_ends = k + 1 == a.tiles_t;
      if (more) load(head_ends ? bh + 1 : bh, head_ends ? 0 : k + 1);

      const uint32_t sb = lds0 + (uint32_t)(stage * STAGE);
      const uint32_t rb = sb + (uint32_t)(j * PITCH + 16 * hf);
      const int64_t t0 = (int64_t)k * 64;
      const int b = bh / a.H, h = bh - b * a.H;
      const int64_t left = a.T - t0;
      const int rows = left < 64 ? (int)left : 64;
      const uint16_t* xbase = x_out + (((int64_t)b * a.T + t0) * a.H + h) * D;
      static_for<2>([&](auto nn) {
        constexpr int n = decltype(nn)::value;
        f32x16_t acc = zero16();
        f16x8_t bhi[2], blo[2];
        bhi[0] = __builtin_bit_cast(f16x8_t, lds_read128(rb + 32 * n * PITCH));
        blo[0] = __builtin_bit_cast(f16x8_t, lds_read128(rb + TILE + 32 * n * PITCH));
        static_for<KS>([&](auto kk) {
          constexpr int ks = decltype(kk)::value;
          if constexpr (ks + 1 < KS) {
            bhi[(ks + 1) & 1] = __builtin_bit_cast(f16x8_t, lds_read128(rb + 32 * n * PITCH + 32 * (ks + 1)));
            blo[(ks + 1) & 1] = __builtin_bit_cast(f16x8_t, lds_read128(rb + TILE + 32 * n * PITCH + 32 * (ks + 1)));
          }
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[ks], bhi[ks & 1], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[ks], blo[ks & 1], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo[ks], bhi[ks & 1], acc, 0, 0, 0);
        });

        // lane (j, hf): outputs 32w + 16hf .. +15 of token 32n + j
        const int tok = 32 * n + j;
        const int ex = __builtin_bit_cast(int, lds_readf(sb + 2 * TILE + 4u * (uint32_t)tok));
        uint32_t o[8];
        static_for<8>([&](auto ee) {
          constexpr int e = decltype(ee)::value;
          o[e] = pack_f16x2(__builtin_ldexpf(acc[2 * e], ex), __builtin_ldexpf(acc[2 * e + 1], ex));
        });
        // rows past T fall outside the resource's bounds and are dropped; one
        // resource per 32-token block, so both share the lane offset
        const int rn = rows - 32 * n;
        const uint32_t nrec = rn > 0 ? (uint32_t)(rn - 1) * xstride + 2 * D : 0u;
        const auto xrs = make_rsrc((const uint8_t*)xbase + (int64_t)(32 * n) * xstride, nrec);
        const w32x4_t v0 = {o[0], o[1], o[2], o[3]}, v1 = {o[4], o[5], o[6], o[7]};
        __builtin_amdgcn_raw_buffer_store_b128(v0, xrs, xlane, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(v1, xrs, xlane + 16, 0, 0);
        __builtin_amdgcn_sched_barrier(0);   // one block's state live at a time
      });

      if (more) {
        if (head_ends) {
          __syncthreads();   // every prep lane is done with this head's 1/lambda
          build_ilam(bh + 1);
          __syncthreads();
        }
        prep(stage ^ 1);
      }
    }
    ++bh;
    k = 0;
  }
}

// ----------------------------------------------------------------------------
// x = s . Q^T yhat for groups of 16 or 32 coordinates, in two MFMA passes.
//   The codes themselves are the B operand (small integers, exact in fp16);
//   1/lambda_c rides in the A operand, 2^sh s_i Q[c, i] / lambda_c (sh per
//   head, putting the largest 1/lambda_c in [2^13, 2^14), so that |A| stays
//   below 2^14 for an orthogonal Q) as fp16 hi + lo parts; each group's
//   partial sum over its one or two 16-wide k-blocks (two MFMAs each, the
//   first with a zero accumulator) is multiplied in fp32 by the token's group
//   scale sigma and added to the output accumulator.  Products are exact and
//   sums fp32, as in the three-pass kernel; only the operand split differs.
// ----------------------------------------------------------------------------
template <int D, int G, int BITS>
__global__ __launch_bounds__(2 * D, 2) void dequantize_dense2_kernel(const float* __restrict__ Q,
                                                                  const uint8_t* __restrict__ codes,
                                                                  const uint16_t* __restrict__ scales,
                                                                  const int8_t* __restrict__ signs,
                                                                  const float* __restrict__ lambda,
                                                                  uint16_t* __restrict__ x_out,
                                                                  DenseGeo a) {
  static_assert(D == 64 || D == 128 || D == 256, "head size");
  static_assert(G == 16 || G == 32, "a group is one or two 16-wide k-blocks");
  constexpr int KS = D / 16;
  constexpr int KPG = G / 16;             // k-blocks per group
  constexpr int PITCH = 2 * D + 16;       // LDS row pitch of the fp16 code tile
  constexpr int TILE = 64 * PITCH;
  constexpr int NG = D / G;
  constexpr int STAGE = TILE + 4 * 64 * NG;   // code tile, then sigma as [group][token] fp32
  constexpr int NT = 2 * D;
  constexpr int LPT = D / 32;             // prep lanes per token (32 coordinates each)
  constexpr int CB = D * BITS / 8;
  constexpr int GPL = 32 / G;             // groups per prep lane
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE + 4 * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31, hf = lane >> 5;
  const int64_t first = (int64_t)blockIdx.x * a.per_block;
  int64_t last = first + a.per_block;
  last = last < a.n_tiles ? last : a.n_tiles;
  if (first >= last) return;
  const uint32_t lds0 = lds_addr(smem);
  const uint32_t ilam_lds = lds0 + 2 * STAGE;   // 1 / lambda of the current head

  // prep role: token pr (0..63) of the tile, coordinates 32 pp .. +31
  // (re-derived in each use, see build)
  uint32_t cw[BITS];       // this lane's 32 codes: int4 4 dwords, int8 8 dwords
  uint32_t sw[1];
  auto prep_ids = [&](int& pr, int& pp) {
    int t = tid;
    asm volatile("" : "+v"(t));
    pr = t / LPT;
    pp = t % LPT;
  };
  // rows past T read 0 (codes 0, scale 0: their outputs are not stored)
  auto load = [&](int bh, int k) {
    int pr, pp;
    prep_ids(pr, pp);
    const int64_t t0 = (int64_t)k * 64;
    const int64_t left = a.T - t0;
    const uint32_t rows = left < 64 ? (uint32_t)left : 64u;
    const int64_t row0 = (int64_t)bh * a.T + t0;
    const auto crs = make_rsrc(codes + row0 * CB, rows * CB);
    const auto srs = make_rsrc(scales + row0 * NG, rows * NG * 2);
    static_for<BITS / 4>([&](auto ii) {
      constexpr int i = decltype(ii)::value;
      const w32x4_t v = __builtin_bit_cast(
          w32x4_t, __builtin_amdgcn_raw_buffer_load_b128(crs, (uint32_t)(pr * CB + pp * (4 * BITS) + 16 * i), 0, kNT));
      static_for<4>([&](auto ee) { cw[4 * i + decltype(ee)::value] = v[decltype(ee)::value]; });
    });
    const uint32_t soff = 2u * (uint32_t)(pr * NG + pp * GPL);
    if constexpr (GPL == 1) sw[0] = __builtin_amdgcn_raw_buffer_load_b16(srs, soff, 0, 0);
    else sw[0] = __builtin_amdgcn_raw_buffer_load_b32(srs, soff, 0, 0);
  };
  // the codes as fp16 integers q into the stage's tile, sigma into its table
  auto prep = [&](int stage) {
    int pr, pp;
    prep_ids(pr, pp);
    const uint32_t sb = lds0 + (uint32_t)(stage * STAGE);
    w32x4_t ch[4];   // 16-byte chunks: coordinates 32 pp + 8 c .. + 7
    if constexpr (BITS == 4) {
      // nibble + 8 (offset binary) into the low mantissa bits of 1024.0h,
      // then - 1032 per half: exact
      static_for<4>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        const uint32_t v = cw[c] ^ 0x88888888u;
        static_for<4>([&](auto kk) {
          constexpr int k = decltype(kk)::value;
          const uint32_t b = v >> (8 * k);
          const uint32_t hw = 0x64006400u | (b & 0xfu) | ((b & 0xf0u) << 12);
          half2_t h = __builtin_bit_cast(half2_t, hw) - half2_t{(_Float16)1032.0f, (_Float16)1032.0f};
          ch[c][k] = __builtin_bit_cast(uint32_t, h);
        });
      });
    } else {
      static_for<4>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        static_for<2>([&](auto ww) {
          constexpr int w = decltype(ww)::value;
          const uint32_t v = cw[2 * c + w] ^ 0x80808080u;
          static_for<2>([&](auto kk) {
            constexpr int k = decltype(kk)::value;
            const uint32_t b = v >> (16 * k);
            const uint32_t hw = 0x64006400u | (b & 0xffu) | ((b & 0xff00u) << 8);
            half2_t h = __builtin_bit_cast(half2_t, hw) - half2_t{(_Float16)1152.0f, (_Float16)1152.0f};
            ch[c][2 * w + k] = __builtin_bit_cast(uint32_t, h);
          });
        });
      });
    }
    // write k of lane pp stores chunk (k + 2 (pp / 4)) % 4: lanes pp and pp + 4
    // (64 bytes x 4 apart) then hit different banks
    const int rot = 2 * ((pp >> 2) & 1);
    static_for<4>([&](auto kk) {
      constexpr int k = decltype(kk)::value;
      const int c = (k + rot) & 3;
      lds_write128(sb + (uint32_t)(pr * PITCH + 16 * (4 * pp + c)), rot ? ch[(k + 2) & 3] : ch[k]);
    });
    static_for<GPL>([&](auto gg) {
      constexpr int gi = decltype(gg)::value;
      const int g = pp * GPL + gi;
      lds_writef(sb + TILE + 4u * (uint32_t)(g * 64 + pr), gi == 0 ? hlo(sw[0]) : hhi(sw[0]));
    });
  };

  f16x8_t ahi[KS], alo[KS];
  int sh = 0;   // this head's A scaling exponent
  auto build = [&](int bh) {
    // lane indices re-derived here: the addresses built from them are not
    // held in registers through the tile loop
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int jb = ln & 31, hb = ln >> 5;
    // sh from the largest 1/lambda of the head (every wave computes it)
    float m = 0.0f;
    static_for<D / 64>([&](auto ii) {
      m = __builtin_fmaxf(m, lds_readf(ilam_lds + 4u * (uint32_t)(ln + 64 * decltype(ii)::value)));
    });
    static_for<6>([&](auto ii) { m = __builtin_fmaxf(m, __shfl_xor(m, 1 << decltype(ii)::value)); });
    sh = __builtin_amdgcn_readfirstlane(m > 0.0f ? 14 - __builtin_amdgcn_frexp_expf(m) : 0);
    const float* Qh = Q + (int64_t)bh * a.q_stride;
    const int8_t* sg = signs + (int64_t)bh * a.sign_stride;
    const int r = dense_row(wave, jb);
    const float s = __builtin_ldexpf(sg[r] < 0 ? -1.0f : 1.0f, sh);
    static_for<KS>([&](auto kk) {
      constexpr int ks = decltype(kk)::value;
      const int c0 = 16 * ks + 8 * hb;
      const w32x4_t l0 = lds_read128(ilam_lds + 4u * (uint32_t)c0);
      const w32x4_t l1 = lds_read128(ilam_lds + 4u * (uint32_t)(c0 + 4));
      float p[8];
      static_for<8>([&](auto ee) {
        constexpr int e = decltype(ee)::value;
        const float il = as_f32(e < 4 ? l0[e] : l1[e - 4]);
        p[e] = Qh[(int64_t)(c0 + e) * D + r] * il * s;
      });
      split8(p, ahi[ks], alo[ks]);
      __builtin_amdgcn_sched_barrier(0);   // one block's loads at a time
    });
  };
  auto build_ilam = [&](int bh) {
    for (int c = tid; c < D; c += NT)
      lds_writef(ilam_lds + 4u * (uint32_t)c, lambda ? 1.0f / lambda[(int64_t)bh * D + c] : 1.0f);
  };

  // Tiles first .. last-1 of the block, head by head; (bh, k) the current
  // tile's head and index within the head, kept as counters.
  int bh = (int)(first / a.tiles_t);
  int k = (int)(first - (int64_t)bh * a.tiles_t);
  // prologue: the first tile's B operands
  build_ilam(bh);
  load(bh, k);
  __syncthreads();
  prep(0);
  const uint32_t xstride = (uint32_t)a.H * (2 * D);
  const uint32_t xlane = (uint32_t)j * xstride + 2u * (uint32_t)(32 * wave + 16 * hf);
  int64_t it = first;
  while (it < last) {
    // the matrix rows of this head; its loads waited for here, so nothing
    // issued on this path is pending inside the tile loop
    build(bh);
    __builtin_amdgcn_s_waitcnt(0);
    const int64_t seg_end = (it - k) + a.tiles_t < last ? (it - k) + a.tiles_t : last;
    for (; it < seg_end; ++it, ++k) {
      const int stage = (int)((it - first) & 1);
      __syncthreads();   // this stage's tile is written; the other stage is no longer read
      const bool more = it + 1 < last;
      const bool head_ends = k + 1 == a.tiles_t;
      if (more) load(head_ends ? bh + 1 : bh, head_ends ? 0 : k + 1);

      const uint32_t sb = lds0 + (uint32_t)(stage * STAGE);
      const uint32_t rb = sb + (uint32_t)(j * PITCH + 16 * hf);
      const int64_t t0 = (int64_t)k * 64;
      const int b = bh / a.H, h = bh - b * a.H;
      const int64_t left = a.T - t0;
      const int rows = left < 64 ? (int)left : 64;
      const uint16_t* xbase = x_out + (((int64_t)b * a.T + t0) * a.H + h) * D;
      static_for<2>([&](auto nn) {
        constexpr int n = decltype(nn)::value;
        const int tok = 32 * n + j;
        f32x16_t acc = zero16();
        f32x16_t part[2];
        // software-pipelined by group: group gs's MFMAs are issued before
        // group gs - 1's sigma scaling, so the VALU work overlaps the matrix
        // cores; a scheduling barrier per step keeps the zero-accumulator
        // MFMAs of later groups from being hoisted (each would hold 16 more
        // registers)
        constexpr int NGK = KS / KPG;
        // B operands one group ahead, sigma one step ahead: the LDS reads'
        // latency is covered by the step before their use
        f16x8_t bq[2][KPG];
        float sgm[2];
        auto read_b = [&](auto gc) {
          constexpr int gb = decltype(gc)::value;
          static_for<KPG>([&](auto qq) {
            constexpr int q = decltype(qq)::value;
            bq[gb & 1][q] = __builtin_bit_cast(f16x8_t, lds_read128(rb + 32 * n * PITCH + 32 * (gb * KPG + q)));
          });
        };
        read_b(std::integral_constant<int, 0>{});
        static_for<NGK + 1>([&](auto gg) {
          constexpr int gs = decltype(gg)::value;
          if constexpr (gs + 1 < NGK) read_b(std::integral_constant<int, gs + 1>{});
          if constexpr (gs < NGK) {
            sgm[gs & 1] = lds_readf(sb + TILE + 4u * (uint32_t)(gs * 64 + tok));
            static_for<KPG>([&](auto qq) {
              constexpr int q = decltype(qq)::value;
              constexpr int ks = gs * KPG + q;
              if constexpr (q == 0)
                part[gs & 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[ks], bq[gs & 1][q], zero16(), 0, 0, 0);
              else
                part[gs & 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[ks], bq[gs & 1][q], part[gs & 1], 0, 0, 0);
              part[gs & 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo[ks], bq[gs & 1][q], part[gs & 1], 0, 0, 0);
            });
          }
          if constexpr (gs > 0) {
            constexpr int g = gs - 1;
            static_for<16>([&](auto ee) {
              constexpr int e = decltype(ee)::value;
              acc[e] = __builtin_fmaf(sgm[g & 1], part[g & 1][e], acc[e]);
            });
            // the sums stay here: sunk to the end, every group's partial
            // would be live at once
            asm volatile("" : "+v"(acc));
          }
          __builtin_amdgcn_sched_barrier(0);
        });

        // lane (j, hf): outputs 32w + 16hf .. +15 of token 32n + j
        uint32_t o[8];
        static_for<8>([&](auto ee) {
          constexpr int e = decltype(ee)::value;
          o[e] = pack_f16x2(__builtin_ldexpf(acc[2 * e], -sh), __builtin_ldexpf(acc[2 * e + 1], -sh));
        });
        // rows past T fall outside the resource's bounds and are dropped; one
        // resource per 32-token block, so both share the lane offset
        const int rn = rows - 32 * n;
        const uint32_t nrec = rn > 0 ? (uint32_t)(rn - 1) * xstride + 2 * D : 0u;
        const auto xrs = make_rsrc((const uint8_t*)xbase + (int64_t)(32 * n) * xstride, nrec);
        const w32x4_t v0 = {o[0], o[1], o[2], o[3]}, v1 = {o[4], o[5], o[6], o[7]};
        __builtin_amdgcn_raw_buffer_store_b128(v0, xrs, xlane, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(v1, xrs, xlane + 16, 0, 0);
        __builtin_amdgcn_sched_barrier(0);   // one block's state live at a time
      });

      if (more) {
        if (head_ends) {
          __syncthreads();   // every wave has built this head's A operands
          build_ilam(bh + 1);
          __syncthreads();
        }
        prep(stage ^ 1);
      }
    }
    ++bh;
    k = 0;
  }
}

}  // namespace srftq
