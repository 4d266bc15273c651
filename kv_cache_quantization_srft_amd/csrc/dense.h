// dense.h -- quantize / dequantize with a rotation given as a matrix.
//
// "When Quantization Is Free" (gist.science summary), Metodologia 3: besides
// the fixed SRFT, the pages study a learned rotation R (with lambda) and
// Householder rotations, k = d/2 reflectors at d = 256.  Any such rotation is
// an orthogonal d x d matrix Q; the quantizer of Metodologia 2 step 4 is then
// applied to y = Q (s . x), and the inverse is x = s . Q^T yhat.
//
// The product is a dense contraction (2 d^2 flops per vector), so it runs on
// the matrix cores: v_mfma_f32_16x16x32_f16, fp32 accumulation.
//
// quantize_dense_kernel  A block of W = D/32 waves works through consecutive
//   64-token tiles of one (tensor, head) at a time.  Wave w owns output rows
//   32w .. 32w+31: it holds 2^10 Q[r, c] s_c for those rows in registers as
//   fp16 hi + lo parts (A operands, D/2 VGPRs: 2^10 keeps both parts normal),
//   so y = Q (s . x) is two MFMAs per 16 x 16 x 32 block (x is exact in fp16)
//   with products exact and sums in fp32.  The rows of each 16-row A tile are
//   permuted, row i of tile t -> 32w + 8(i/4) + 4t + i%4, so that lane
//   (token j = lane%16, q = lane/16) ends with the 8 contiguous outputs
//   32w + 8q .. +7 of token j: the quantizer (quant.h's decision rule) runs on
//   them in registers, groups of 16 / 32 span 2 / 4 lanes (one shuffle each),
//   and the lane stores its codes and scale directly.  The x tile is staged
//   through LDS (read by every wave), prefetched a tile ahead in registers;
//   its 16-byte chunks are XOR-swizzled by row so that the 16 rows one MFMA
//   operand read touches fall in different banks.
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
typedef float f32x4_t __attribute__((ext_vector_type(4)));
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

// Output row of A-tile row i (0..15) in tile t (0, 1) of wave w.
__device__ __forceinline__ int dense_row(int w, int t, int i) { return 32 * w + 8 * (i >> 2) + 4 * t + (i & 3); }

// LDS byte offset of 16-byte chunk ch of row `row` in a tile of ROWB-byte rows.
template <int ROWB>
__device__ __forceinline__ uint32_t swz(int row, int ch) {
  return (uint32_t)(row * ROWB + 16 * (ch ^ (row & 7)));
}

// The MFMA operand reads of lane (j, q): chunk 4 kb + q of rows 16 n + j.
// With s = j & 7, (4 kb + q) ^ s = 4 (kb ^ (s >> 2)) + (q ^ (s & 3)), and
// kb ^ (s >> 2) is kb + (s >> 2) for even kb and kb - (s >> 2) for odd kb:
// two per-lane bases plus compile-time offsets.
template <int ROWB>
struct SwzReader {
  uint32_t base[2];
  __device__ __forceinline__ SwzReader(uint32_t tile, int j, int q) {
    const int s = j & 7;
    const uint32_t b = tile + (uint32_t)(j * ROWB + 16 * (q ^ (s & 3)));
    base[0] = b + 64u * (uint32_t)(s >> 2);
    base[1] = b - 64u * (uint32_t)(s >> 2);
  }
  template <int N, int KB>
  __device__ __forceinline__ uint32_t at() const {
    return base[KB & 1] + (uint32_t)(16 * N * ROWB + 64 * KB);
  }
};

// fp16 hi + lo parts of 8 fp32 values.
__device__ __forceinline__ void split8(const float (&v)[8], f16x8_t& hi, f16x8_t& lo) {
  static_for<8>([&](auto ee) {
    constexpr int e = decltype(ee)::value;
    const _Float16 h = (_Float16)v[e];
    hi[e] = h;
    lo[e] = (_Float16)(v[e] - (float)h);
  });
}

// ----------------------------------------------------------------------------
// y = Q (s . x), then lambda, group absmax and rounding.
// ----------------------------------------------------------------------------
template <int D, int G, int BITS>
__global__ __launch_bounds__(2 * D) void quantize_dense_kernel(const float* __restrict__ Q,
                                                               const uint16_t* __restrict__ x,
                                                               const int8_t* __restrict__ signs,
                                                               const float* __restrict__ lambda,
                                                               uint8_t* __restrict__ codes,
                                                               uint16_t* __restrict__ scales,
                                                               DenseGeo a) {
  static_assert(D == 64 || D == 128 || D == 256, "head size");
  static_assert(G == 8 || G == 16 || G == 32, "a group lies within one wave's 32 rows");
  using QC = QConst<BITS>;
  constexpr int KS = D / 32;              // k-steps of 32 coordinates
  constexpr int ROWB = 2 * D;             // bytes per x row
  constexpr int CH = ROWB / 16;           // 16-byte chunks per row
  constexpr int TILE = 64 * ROWB;
  constexpr int NT = 2 * D;               // threads
  constexpr int LD = 64 * CH / NT;        // chunks per thread per tile (4)
  constexpr int CB = D * BITS / 8;        // code bytes per token
  constexpr int NG = D / G;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, q = lane >> 4;
  const int64_t first = (int64_t)blockIdx.x * a.per_block;
  int64_t last = first + a.per_block;
  last = last < a.n_tiles ? last : a.n_tiles;
  if (first >= last) return;
  const uint32_t lds0 = lds_addr(smem);

  // Global loads of one tile into registers (rows past T re-read row T-1).
  w32x4_t pre[LD];
  auto load = [&](int64_t tile) {
    const int bh = (int)(tile / a.tiles_t);
    const int64_t t0 = (tile - (int64_t)bh * a.tiles_t) * 64;
    const int b = bh / a.H, h = bh - b * a.H;
    static_for<LD>([&](auto ii) {
      constexpr int i = decltype(ii)::value;
      const int c = tid + NT * i;
      const int row = c / CH, ch = c % CH;
      int64_t t = t0 + row;
      t = t < a.T ? t : a.T - 1;
      const uint16_t* src = x + (((int64_t)b * a.T + t) * a.H + h) * D + 8 * ch;
      pre[i] = __builtin_nontemporal_load((const w32x4_t*)src);
    });
  };
  auto write = [&](int stage) {
    static_for<LD>([&](auto ii) {
      constexpr int i = decltype(ii)::value;
      const int c = tid + NT * i;
      lds_write128(lds0 + (uint32_t)(stage * TILE) + swz<ROWB>(c / CH, c % CH), pre[i]);
    });
  };

  // A operands of this wave's rows for head bh; lambda of the lane's 8 outputs.
  f16x8_t ahi[2][KS], alo[2][KS];
  float lamr[8];
  auto build = [&](int bh) {
    const float* Qh = Q + (int64_t)bh * a.q_stride;
    const int8_t* sg = signs + (int64_t)bh * a.sign_stride;
    static_for<2>([&](auto tt) {
      constexpr int t = decltype(tt)::value;
      const float* qrow = Qh + (int64_t)dense_row(wave, t, j) * D;
      static_for<KS>([&](auto kk) {
        constexpr int kb = decltype(kk)::value;
        const int c0 = 32 * kb + 8 * q;
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
        split8(p, ahi[t][kb], alo[t][kb]);
        __builtin_amdgcn_sched_barrier(0);   // one block's loads at a time
      });
    });
    const int r0 = 32 * wave + 8 * q;
    static_for<8>([&](auto ee) {
      constexpr int e = decltype(ee)::value;
      lamr[e] = (lambda ? lambda[(int64_t)bh * D + r0 + e] : 1.0f) * (1.0f / 1024.0f);
    });
  };

  load(first);
  write(0);
  int cur_bh = -1;
  for (int64_t it = first; it < last; ++it) {
    const int stage = (int)((it - first) & 1);
    const int bh = (int)(it / a.tiles_t);
    if (bh != cur_bh) {
      build(bh);
      cur_bh = bh;
    }
    __syncthreads();   // this stage is written; the other one is no longer read
    if (it + 1 < last) load(it + 1);

    const SwzReader<ROWB> rd(lds0 + (uint32_t)(stage * TILE), j, q);
    const int64_t t0 = (it - (int64_t)bh * a.tiles_t) * 64;
    const float magic = as_f32(QC::kMagicBits);
    // two halves of two 16-token blocks each; B operands one k-step ahead
    static_for<2>([&](auto hh) {
      constexpr int h2 = decltype(hh)::value;
      f32x4_t acc[2][2];
      static_for<2>([&](auto nn) {
        static_for<2>([&](auto tt) { acc[decltype(nn)::value][decltype(tt)::value] = (f32x4_t){0.f, 0.f, 0.f, 0.f}; });
      });
      f16x8_t bx[2][2];
      auto fetch = [&](auto kc) {
        constexpr int kb = decltype(kc)::value;
        static_for<2>([&](auto nn) {
          constexpr int n = decltype(nn)::value;
          bx[kb & 1][n] = __builtin_bit_cast(f16x8_t, lds_read128(rd.template at<2 * h2 + n, kb>()));
        });
      };
      fetch(std::integral_constant<int, 0>{});
      static_for<KS>([&](auto kk) {
        constexpr int kb = decltype(kk)::value;
        constexpr int cb = kb & 1;
        if constexpr (kb + 1 < KS) fetch(std::integral_constant<int, kb + 1>{});
        static_for<2>([&](auto nn) {
          constexpr int n = decltype(nn)::value;
          static_for<2>([&](auto tt) {
            constexpr int t = decltype(tt)::value;
            acc[n][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[t][kb], bx[cb][n], acc[n][t], 0, 0, 0);
          });
        });
        static_for<2>([&](auto nn) {
          constexpr int n = decltype(nn)::value;
          static_for<2>([&](auto tt) {
            constexpr int t = decltype(tt)::value;
            acc[n][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[t][kb], bx[cb][n], acc[n][t], 0, 0, 0);
          });
        });
        __builtin_amdgcn_sched_barrier(0);
      });

      // quantize: lane (j, q) holds outputs 32w + 8q .. +7 of token 16n + j
      static_for<2>([&](auto nn) {
        constexpr int n = decltype(nn)::value;
        float z[8];
        static_for<4>([&](auto ee) {
          constexpr int e = decltype(ee)::value;
          z[e] = acc[n][0][e] * lamr[e];
          z[4 + e] = acc[n][1][e] * lamr[4 + e];
        });
        float m = 0.0f;
        static_for<8>([&](auto ee) { m = __builtin_fmaxf(m, __builtin_fabsf(z[decltype(ee)::value])); });
        if constexpr (G >= 16) m = __builtin_fmaxf(m, __shfl_xor(m, 16));
        if constexpr (G >= 32) m = __builtin_fmaxf(m, __shfl_xor(m, 32));
        const float tq = __builtin_fminf(m * QC::kQinv, 65504.0f);
        const uint32_t sh = pack_f16x2(tq, 0.0f) & 0xffffu;
        const float sg = hlo(sh);
        const float r = sg == 0.0f ? 0.0f : recip_f16_value(sg);
        uint32_t tb[8];
        static_for<8>([&](auto ee) {
          constexpr int e = decltype(ee)::value;
          // the clamp only acts for fp16-subnormal or saturated scales
          int bi = (int)as_u32(__builtin_fmaf(z[e], r, magic));
          bi = bi < (int)QC::kLo ? (int)QC::kLo : bi;
          bi = bi > (int)QC::kHi ? (int)QC::kHi : bi;
          tb[e] = (uint32_t)bi;
        });
        const int64_t t = t0 + 16 * (2 * h2 + n) + j;
        if (t < a.T) {
          const int64_t row = (int64_t)bh * a.T + t;
          const int c0 = 32 * wave + 8 * q;
          if constexpr (BITS == 4) {
            *(uint32_t*)(codes + row * CB + c0 / 2) = pack_codes<4>(tb);
          } else {
            *(uint2*)(codes + row * CB + c0) = make_uint2(pack_codes<8>(tb), pack_codes<8>(tb + 4));
          }
          if (c0 % G == 0) scales[row * NG + c0 / G] = (uint16_t)sh;
        }
      });
    });

    if (it + 1 < last) write(stage ^ 1);
  }
}

// ----------------------------------------------------------------------------
// x = s . Q^T yhat,  yhat_c = q_c sigma_G(c) / lambda_c.
// ----------------------------------------------------------------------------
template <int D, int G, int BITS>
__global__ __launch_bounds__(2 * D) void dequantize_dense_kernel(const float* __restrict__ Q,
                                                                 const uint8_t* __restrict__ codes,
                                                                 const uint16_t* __restrict__ scales,
                                                                 const int8_t* __restrict__ signs,
                                                                 const float* __restrict__ lambda,
                                                                 uint16_t* __restrict__ x_out,
                                                                 DenseGeo a) {
  static_assert(D == 64 || D == 128 || D == 256, "head size");
  static_assert(G == 8 || G == 16 || G == 32, "group");
  constexpr int KS = D / 32;
  constexpr int ROWB = 2 * D;             // bytes per B row (fp16)
  constexpr int TILE = 64 * ROWB;
  constexpr int STAGE = 2 * TILE + 256;   // hi tile, lo tile, 64 output multipliers
  constexpr int NT = 2 * D;
  constexpr int LPT = D / 32;             // prep lanes per token (32 coordinates each)
  constexpr int CB = D * BITS / 8;
  constexpr int NG = D / G;
  constexpr int GPL = 32 / G;             // groups per prep lane
  constexpr float kOff = BITS == 4 ? 8.0f : 128.0f;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE + 4 * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, q = lane >> 4;
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
  auto load = [&](int64_t tile) {
    const int bh = (int)(tile / a.tiles_t);
    int64_t t = (tile - (int64_t)bh * a.tiles_t) * 64 + pr;
    t = t < a.T ? t : a.T - 1;
    const int64_t row = (int64_t)bh * a.T + t;
    const w32x4_t* src = (const w32x4_t*)(codes + row * CB + pp * (4 * BITS));
    static_for<BITS / 4>([&](auto ii) {
      constexpr int i = decltype(ii)::value;
      const w32x4_t v = __builtin_nontemporal_load(src + i);
      static_for<4>([&](auto ee) { cw[4 * i + decltype(ee)::value] = v[decltype(ee)::value]; });
    });
    const uint16_t* srow = scales + row * NG + pp * GPL;
    if constexpr (GPL == 1) sw[0] = srow[0];
    else if constexpr (GPL == 2) sw[0] = *(const uint32_t*)srow;
    else {
      const uint2 v = *(const uint2*)srow;
      sw[0] = v.x, sw[1] = v.y;
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
      u[m] = v * lds_readf(ilam_lds + 4u * (uint32_t)(32 * pp + m));
      mx = __builtin_fmaxf(mx, __builtin_fabsf(u[m]));
    });
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 1));
    if constexpr (LPT > 2) mx = __builtin_fmaxf(mx, __shfl_xor(mx, 2));
    if constexpr (LPT > 4) mx = __builtin_fmaxf(mx, __shfl_xor(mx, 4));
    // ldexp, not a multiply by 2^sh: sh exceeds 127 for tiny scales
    const int sh = mx > 0.0f ? 15 - __builtin_amdgcn_frexp_expf(mx) : 0;
    const uint32_t sb = lds0 + (uint32_t)(stage * STAGE);
    static_for<4>([&](auto cc) {
      constexpr int c = decltype(cc)::value;
      float v[8];
      static_for<8>([&](auto ee) { v[decltype(ee)::value] = __builtin_ldexpf(u[8 * c + decltype(ee)::value], sh); });
      f16x8_t hi, lo;
      split8(v, hi, lo);
      const uint32_t off = swz<ROWB>(pr, 4 * pp + c);
      lds_write128(sb + off, __builtin_bit_cast(w32x4_t, hi));
      lds_write128(sb + TILE + off, __builtin_bit_cast(w32x4_t, lo));
    });
    if (pp == 0) lds_writef(sb + 2 * TILE + 4u * (uint32_t)pr, __builtin_bit_cast(float, -sh - 10));
  };

  f16x8_t ahi[2][KS], alo[2][KS];
  auto build = [&](int bh) {
    const float* Qh = Q + (int64_t)bh * a.q_stride;
    const int8_t* sg = signs + (int64_t)bh * a.sign_stride;
    static_for<2>([&](auto tt) {
      constexpr int t = decltype(tt)::value;
      const int r = dense_row(wave, t, j);
      const float s = sg[r] < 0 ? -1024.0f : 1024.0f;
      static_for<KS>([&](auto kk) {
        constexpr int kb = decltype(kk)::value;
        const int c0 = 32 * kb + 8 * q;
        float p[8];
        static_for<8>([&](auto ee) {
          constexpr int e = decltype(ee)::value;
          p[e] = Qh[(int64_t)(c0 + e) * D + r] * s;
        });
        split8(p, ahi[t][kb], alo[t][kb]);
        __builtin_amdgcn_sched_barrier(0);   // one block's loads at a time
      });
    });
  };
  auto build_ilam = [&](int bh) {
    for (int c = tid; c < D; c += NT)
      lds_writef(ilam_lds + 4u * (uint32_t)c, lambda ? 1.0f / lambda[(int64_t)bh * D + c] : 1.0f);
  };

  // prologue: the first tile's B operands
  int cur_bh = (int)(first / a.tiles_t);
  build_ilam(cur_bh);
  load(first);
  __syncthreads();
  prep(0);
  build(cur_bh);

  for (int64_t it = first; it < last; ++it) {
    const int stage = (int)((it - first) & 1);
    const int bh = (int)(it / a.tiles_t);
    if (bh != cur_bh) {
      build(bh);
      cur_bh = bh;
    }
    __syncthreads();   // this stage's B tiles are written; the other stage is no longer read
    const bool more = it + 1 < last;
    const int nbh = more ? (int)((it + 1) / a.tiles_t) : bh;
    if (more) load(it + 1);

    const uint32_t sb = lds0 + (uint32_t)(stage * STAGE);
    const SwzReader<ROWB> rd(sb, j, q);
    const int64_t t0 = (it - (int64_t)bh * a.tiles_t) * 64;
    const int b = bh / a.H, h = bh - b * a.H;
    static_for<2>([&](auto hh) {
      constexpr int h2 = decltype(hh)::value;
      f32x4_t acc[2][2];
      static_for<2>([&](auto nn) {
        static_for<2>([&](auto tt) { acc[decltype(nn)::value][decltype(tt)::value] = (f32x4_t){0.f, 0.f, 0.f, 0.f}; });
      });
      f16x8_t bhi[2][2], blo[2][2];
      auto fetch = [&](auto kc) {
        constexpr int kb = decltype(kc)::value;
        static_for<2>([&](auto nn) {
          constexpr int n = decltype(nn)::value;
          const uint32_t off = rd.template at<2 * h2 + n, kb>();
          bhi[kb & 1][n] = __builtin_bit_cast(f16x8_t, lds_read128(off));
          blo[kb & 1][n] = __builtin_bit_cast(f16x8_t, lds_read128(off + TILE));
        });
      };
      fetch(std::integral_constant<int, 0>{});
      static_for<KS>([&](auto kk) {
        constexpr int kb = decltype(kk)::value;
        constexpr int cb = kb & 1;
        if constexpr (kb + 1 < KS) fetch(std::integral_constant<int, kb + 1>{});
        static_for<2>([&](auto nn) {
          constexpr int n = decltype(nn)::value;
          static_for<2>([&](auto tt) {
            constexpr int t = decltype(tt)::value;
            acc[n][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[t][kb], bhi[cb][n], acc[n][t], 0, 0, 0);
          });
        });
        static_for<2>([&](auto nn) {
          constexpr int n = decltype(nn)::value;
          static_for<2>([&](auto tt) {
            constexpr int t = decltype(tt)::value;
            acc[n][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[t][kb], blo[cb][n], acc[n][t], 0, 0, 0);
          });
        });
        static_for<2>([&](auto nn) {
          constexpr int n = decltype(nn)::value;
          static_for<2>([&](auto tt) {
            constexpr int t = decltype(tt)::value;
            acc[n][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[t][kb], bhi[cb][n], acc[n][t], 0, 0, 0);
          });
        });
        __builtin_amdgcn_sched_barrier(0);
      });

      // lane (j, q): outputs 32w + 8q .. +7 of token 16n + j
      static_for<2>([&](auto nn) {
        constexpr int n = decltype(nn)::value;
        const int tok = 16 * (2 * h2 + n) + j;
        const int ex = __builtin_bit_cast(int, lds_readf(sb + 2 * TILE + 4u * (uint32_t)tok));
        const int64_t t = t0 + tok;
        if (t < a.T) {
          float o8[8];
          static_for<4>([&](auto ee) {
            constexpr int e = decltype(ee)::value;
            o8[e] = __builtin_ldexpf(acc[n][0][e], ex);
            o8[4 + e] = __builtin_ldexpf(acc[n][1][e], ex);
          });
          const uint4 o = make_uint4(pack_f16x2(o8[0], o8[1]), pack_f16x2(o8[2], o8[3]),
                                     pack_f16x2(o8[4], o8[5]), pack_f16x2(o8[6], o8[7]));
          *(uint4*)(x_out + (((int64_t)b * a.T + t) * a.H + h) * D + 32 * wave + 8 * q) = o;
        }
      });
    });

    if (more) {
      if (nbh != bh) {
        __syncthreads();   // every prep lane is done with this head's 1/lambda
        build_ilam(nbh);
        __syncthreads();
      }
      prep(stage ^ 1);
    }
  }
}

}  // namespace srftq
