// kernels2.h -- quantize / dequantize with two lanes per vector.
//
// One lane cannot hold a 256-value vector in registers at more than one wave
// per SIMD, and a 64-token tile of 512-byte rows fills the LDS of a CU at
// four waves.  Here a wave takes a tile of 32 tokens and each token's vector
// is split over lanes t and t + 32 (role p = 0, 1), so every lane holds d/2
// values and two waves share each SIMD.  Written for any power-of-two d; the
// library runs it for d = 256 and for the rotation-free quantizer.
//
// SRFT ("When Quantization Is Free", Metodologia 1 and 2): decimation in
// time by two.  Lane p takes the samples x[2m + p] and computes their
// 128-point real DFT (E for p = 0, O for p = 1) with the in-register
// radix-2 code of the 128-point transform; the last radix-2 stage
//   X_k = E_k + W^k O_k,  X_{N-k} = conj(E_k - W^k O_k),  W = e^{-2 pi i / d},
// is split so that both lanes run the same instructions: lane 1 first
// multiplies its O_k by W^k, then v_permlane32_swap exchanges register pairs
// (h[k], h[N-k]) as a 2 x 2 transpose between the lane halves, after which
// lane 0 holds (Re E_k, Re W^k O_k) and lane 1 (Im E_k, Im W^k O_k), and one
// sum and one difference per k give lane 0 the real parts Re X_k (packed
// coordinates 0..127) and lane 1 the imaginary parts (coordinates 128..255,
// those from 192 on negated).  Each lane then owns whole groups, half the
// code row and half the scale row.
//
// SRHT: H_256 [a; b] = [H_128 (a + b); H_128 (a - b)], so lane p transforms
// a + (-1)^p b (the sign flip folded into its sign masks) and owns packed
// coordinates 128p .. 128p + 127.  No rotation: lane p owns its half row.
//
// The inverse runs the same steps backwards (the swap is its own inverse).
#pragma once

#include "kernels.h"

#ifndef SRFTQ_QUANT2_WAVES
#define SRFTQ_QUANT2_WAVES 2
#endif
#ifndef SRFTQ_DEQUANT2_WAVES
#define SRFTQ_DEQUANT2_WAVES 2
#endif

namespace srftq {

// Per-coordinate scales of one lane's L = D/2 coordinates: the packed
// coordinates 0 and D/2 of the SRFT (the edges) are local coordinate 0 of
// lanes 0 and 1.
template <int D, int ROT>
struct HalfScales {
  static constexpr bool kEdges = (ROT == ROT_SRFT);
  static constexpr double kFwdBulk = Scales<D, ROT, VAR_REAL>::kFwdBulk;
  static constexpr double kFwdEdge = Scales<D, ROT, VAR_REAL>::kFwdEdge;
  static constexpr double kInvBulk = Scales<D, ROT, VAR_REAL>::kInvBulk;
  static constexpr double kInvEdge = Scales<D, ROT, VAR_REAL>::kInvEdge;
  static constexpr bool is_edge(int i) { return kEdges && i == 0; }
};

// Sign masks of one head for the two-lane kernels: table[q][m], q = role,
// m < D/2 the packed fp16 pair (elements 2m, 2m+1).  Role 1 of the SRHT has
// the masks of the bottom half (m >= D/4) flipped, so that its pair sums
// are a - b.  Built lane-parallel from the raw sign row (D bytes in LDS).
template <int D, int ROT>
__device__ __forceinline__ void build_masks2(const uint32_t* raw, uint32_t* table, int lane) {
  static_assert(D / 4 <= 64 * 2, "sign dwords per lane");
  for (int i = lane; i < D / 4; i += 64) {
    const uint32_t u = raw[i];                // sign bytes 4i .. 4i+3
    const uint32_t m0 = sign_mask_of(u), m1 = sign_mask_of(u >> 16);
    table[2 * i] = m0;
    table[2 * i + 1] = m1;
    if constexpr (ROT == ROT_SRHT) {
      const uint32_t f = (2 * i >= D / 4) ? 0x80008000u : 0u;
      table[D / 2 + 2 * i] = m0 ^ f;
      table[D / 2 + 2 * i + 1] = m1 ^ f;
    }
  }
}

// Chunk c (16 bytes) of row v of a swizzled RowTile, c < kCpr.
template <class RT>
__device__ __forceinline__ uint4 tile_chunk(const uint8_t* lds, int v, int c) {
  return *(const uint4*)(lds + v * RT::kRowLds + 16 * (c ^ RT::swz(v)));
}

// ----------------------------------------------------------------------------
// Quantize, two lanes per vector, one 32-token tile per block.
// ----------------------------------------------------------------------------
template <int D, int G, int BITS, int ROT, bool LAM>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(SRFTQ_QUANT2_WAVES)))
void quantize2_kernel(const uint16_t* __restrict__ x, const int8_t* __restrict__ signs,
                      const float* __restrict__ lambda, uint8_t* __restrict__ codes_out,
                      uint16_t* __restrict__ scales_out, Geo a) {
  constexpr int L = D / 2;                  // coordinates per lane
  using Sc = HalfScales<D, ROT>;
  using XT = RowTile<2 * D, 32>;
  constexpr bool XL = G > L;                          // one group over both lanes (G = D)
  constexpr int GL = XL ? L : G;                      // group width inside a lane
  constexpr int CB = D * BITS / 8, CBL = CB / 2;     // code bytes per vector / per lane
  constexpr int SB = 2 * D / G, SBL = XL ? SB : SB / 2;   // scale bytes per vector / per lane
  constexpr int NCW = CodeWords<L, BITS>::kWords;
  constexpr int NSW = ScaleWords<L, GL>::kWords;
  static_assert(G <= L || G == D, "groups stay inside one lane, or span the vector");
  __shared__ __attribute__((aligned(16))) uint8_t lds[XT::kBytes];
  __shared__ __attribute__((aligned(16))) float lam_lds[LAM ? D : 4];
  __shared__ __attribute__((aligned(16))) uint32_t sraw[D / 4];
  __shared__ __attribute__((aligned(16))) uint32_t smask[ROT == ROT_SRHT ? D : D / 2];

  const int lane = threadIdx.x;
  const int t = lane & 31, p = lane >> 5;
  const int tile = (int)blockIdx.x;
  if (tile >= a.n_tiles) return;
  const int k = tile / a.BH, bh = tile - k * a.BH;
  const int64_t t0 = (int64_t)k * 32;
  const int64_t left = a.T - t0;
  const int nv = left < 32 ? (int)left : 32;
  const uint32_t rsb = (uint32_t)a.H * (uint32_t)(2 * D);

  {
    typename XT::Plan plan;
    plan.init(lane, rsb);
    XT::issue((const uint8_t*)x + row_index(a, bh, t0) * (int64_t)(2 * D), rsb, nv, lane, plan, lds);
  }
  if constexpr (LAM) issue_row_f32<D>(lambda + (int64_t)bh * D, lane, (uint8_t*)lam_lds);
  if (lane < D / 4) dma_to_lds<4>(signs + (int64_t)bh * a.sign_stride, 4u * (uint32_t)lane, lds_addr(sraw));
  wait_vm<0>();
  wave_fence();
  build_masks2<D, ROT>(sraw, smask, lane);
  wave_fence();

  float h[L];
  if constexpr (ROT == ROT_SRFT) {
    // own half row: dwords 64p .. 64p+63 (elements 128p ..), signs applied
    uint32_t dw[L / 2];
    const uint32_t* mrow = smask + (L / 2) * p;
    static_for<L / 8>([&](auto cc) {
      constexpr int c = decltype(cc)::value;
      const uint4 q = tile_chunk<XT>(lds, t, (L / 8) * p + c);
      const uint4 m = *(const uint4*)(mrow + 4 * c);
      dw[4 * c + 0] = q.x ^ m.x;
      dw[4 * c + 1] = q.y ^ m.y;
      dw[4 * c + 2] = q.z ^ m.z;
      dw[4 * c + 3] = q.w ^ m.w;
    });
    // w[m] = (x[4m + p], x[4m + 2 + p]): the fp16 pairs of the lane's
    // subsequence y_m = x[2m + p], split out of the halves and exchanged
    uint32_t w[L / 2];
    static_for<L / 4>([&](auto mm) {
      constexpr int m = decltype(mm)::value;
      uint32_t e = __builtin_amdgcn_perm(dw[2 * m + 1], dw[2 * m], 0x05040100u);
      uint32_t o = __builtin_amdgcn_perm(dw[2 * m + 1], dw[2 * m], 0x07060302u);
      swap32(e, o);
      w[m] = e;
      w[m + L / 4] = o;
    });
    float p0[L / 2], p1[L / 2];
    pair_sums<L>(w, NoSigns{}, p0, p1);
    rdft<L, 1, 0, L>(p0, p1, h);
    // lane 1: O_k <- W^k O_k
    if (p) {
      static_for<L / 2 - 1>([&](auto kk) {
        constexpr int q = decltype(kk)::value + 1;
        constexpr float c = (float)ccos(2.0 * kPi * q / D), s = (float)csin(2.0 * kPi * q / D);
        const float Or = h[q], Oi = h[L - q];
        h[q] = __builtin_fmaf(c, Or, s * Oi);
        h[L - q] = __builtin_fmaf(c, Oi, -s * Or);
      });
    }
    const float sgn = p ? -1.0f : 1.0f;
    {
      float X = h[0], Y = h[0];
      swap32(X, Y);                     // both lanes: X = E_0, Y = O_0
      h[0] = __builtin_fmaf(sgn, Y, X);  // X_0 (lane 0), X_{d/2} (lane 1)
    }
    static_for<L / 2 - 1>([&](auto kk) {
      constexpr int q = decltype(kk)::value + 1;
      float u = h[q], v = h[L - q];
      swap32(u, v);
      h[q] = u + v;
      h[L - q] = u - v;
    });
    // h[L/2]: lane 0 keeps E_{L/2} = Re X_{L/2}; lane 1 keeps O_{L/2}, which
    // is -Im X_{L/2}, in its negated upper half.  The negation folds into
    // the rounding of those groups, or (a group spanning both halves) is
    // undone here.
    constexpr bool kFold = G <= L / 2;
    if constexpr (!kFold) {
      static_for<L / 2>([&](auto ii) { h[L / 2 + decltype(ii)::value] *= sgn; });
    }
    uint32_t codes[NCW];
    uint32_t scales[NSW];
    quantize_tail<L, GL, BITS, ROT, VAR_REAL, LAM, Sc, (kFold ? L / 2 : L), XL>(h, lam_lds + L * p, codes, scales,
                                                                             sgn);
    // stores
    int64_t tt0 = t0;
    bool ok = t < nv;
    if (a.pos) {
      tt0 += a.pos[bh / a.H];
      ok = ok && tt0 + t >= 0 && tt0 + t < a.pitch;
    }
    if (ok) {
      const int64_t r0 = cache_row(a, bh, tt0) + t;
      store_words<NCW>(codes_out + r0 * CB + CBL * p, codes);
      if (!XL || p == 0) store_scales<L, GL>((uint8_t*)scales_out + r0 * SB + (XL ? 0 : SBL * p), scales);
    }
  } else {
    if constexpr (ROT == ROT_SRHT) {
      // pair sums a + (-1)^p b of the top and bottom halves
      const uint32_t* mrow = smask + D / 2 * p;
      float one = 1.0f;
      asm("" : "+s"(one));
      static_for<L / 8>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        const uint4 qa = tile_chunk<XT>(lds, t, c);
        const uint4 qb = tile_chunk<XT>(lds, t, L / 8 + c);
        const uint4 ma = *(const uint4*)(smask + 4 * c);
        const uint4 mb = *(const uint4*)(mrow + L / 2 + 4 * c);
        const uint32_t wa[4] = {qa.x ^ ma.x, qa.y ^ ma.y, qa.z ^ ma.z, qa.w ^ ma.w};
        const uint32_t wb[4] = {qb.x ^ mb.x, qb.y ^ mb.y, qb.z ^ mb.z, qb.w ^ mb.w};
        static_for<4>([&](auto ii) {
          constexpr int i = decltype(ii)::value;
          h[8 * c + 2 * i] = __builtin_fmaf(hlo(wb[i]), one, hlo(wa[i]));
          h[8 * c + 2 * i + 1] = __builtin_fmaf(hhi(wb[i]), one, hhi(wa[i]));
        });
      });
      wht<L>(h);
    } else {
      const uint32_t* mrow = smask + (L / 2) * p;
      static_for<L / 8>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        const uint4 q = tile_chunk<XT>(lds, t, (L / 8) * p + c);
        const uint4 m = *(const uint4*)(mrow + 4 * c);
        const uint32_t wv[4] = {q.x ^ m.x, q.y ^ m.y, q.z ^ m.z, q.w ^ m.w};
        static_for<4>([&](auto ii) {
          constexpr int i = decltype(ii)::value;
          h[8 * c + 2 * i] = hlo(wv[i]);
          h[8 * c + 2 * i + 1] = hhi(wv[i]);
        });
      });
    }
    uint32_t codes[NCW];
    uint32_t scales[NSW];
    quantize_tail<L, GL, BITS, ROT, VAR_REAL, LAM, Sc, L, XL>(h, lam_lds + L * p, codes, scales, 1.0f);
    int64_t tt0 = t0;
    bool ok = t < nv;
    if (a.pos) {
      tt0 += a.pos[bh / a.H];
      ok = ok && tt0 + t >= 0 && tt0 + t < a.pitch;
    }
    if (ok) {
      const int64_t r0 = cache_row(a, bh, tt0) + t;
      store_words<NCW>(codes_out + r0 * CB + CBL * p, codes);
      if (!XL || p == 0) store_scales<L, GL>((uint8_t*)scales_out + r0 * SB + (XL ? 0 : SBL * p), scales);
    }
  }
}

// ----------------------------------------------------------------------------
// Dequantize, two lanes per vector, one 32-token tile per block.
// Output rows are staged in LDS (over the code and scale tiles, which are
// read into registers first) and leave as 1 KiB nontemporal stores.
// ----------------------------------------------------------------------------
template <int D, int G, int BITS, int ROT, bool LAM>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(SRFTQ_DEQUANT2_WAVES)))
void dequantize2_kernel(const uint8_t* __restrict__ codes_in, const uint16_t* __restrict__ scales_in,
                        const int8_t* __restrict__ signs, const float* __restrict__ lambda,
                        uint16_t* __restrict__ x_out, Geo a) {
  constexpr int L = D / 2;
  using Sc = HalfScales<D, ROT>;
  constexpr bool XL = G > L;                          // one group over both lanes (G = D)
  constexpr int GL = XL ? L : G;
  constexpr int CB = D * BITS / 8, CBL = CB / 2;
  constexpr int SB = 2 * D / G, SBL = XL ? SB : SB / 2;   // both lanes read the one scale
  constexpr int NCW = CodeWords<L, BITS>::kWords;
  constexpr int NSW = ScaleWords<L, GL>::kWords;
  static_assert(G <= L || G == D, "groups stay inside one lane, or span the vector");
  using CT = RowTile<CB, 32>;
  using ST = RowTile<SB, 32>;
  using OT = RowTile<2 * D, 32>;
  static_assert(CT::kBytes + (ST::kBytes < 16 ? 16 : ST::kBytes) <= OT::kBytes, "tiles fit the output staging");
  __shared__ __attribute__((aligned(16))) uint8_t lds[OT::kBytes];
  uint8_t* const ctile = lds;
  uint8_t* const stile = lds + CT::kBytes;
  __shared__ __attribute__((aligned(16))) float lam_lds[LAM ? D : 4];
  __shared__ __attribute__((aligned(16))) uint32_t sraw[D / 4];
  __shared__ __attribute__((aligned(16))) uint32_t smask[D / 2];

  const int lane = threadIdx.x;
  const int t = lane & 31, p = lane >> 5;
  const int tile = (int)blockIdx.x;
  if (tile >= a.n_tiles) return;
  const int k = tile / a.BH, bh = tile - k * a.BH;
  const int64_t t0 = (int64_t)k * 32;
  const int64_t left = a.T - t0;
  const int nv = left < 32 ? (int)left : 32;
  const uint32_t rsb_x = (uint32_t)a.H * (uint32_t)(2 * D);

  {
    const int64_t r0 = cache_row(a, bh, t0);
    typename CT::Plan cplan;
    cplan.init(lane, CB);
    CT::issue(codes_in + r0 * CB, CB, nv, lane, cplan, ctile);
    typename ST::Plan splan;
    splan.init(lane, SB);
    ST::issue((const uint8_t*)scales_in + r0 * SB, SB, nv, lane, splan, stile);
  }
  if constexpr (LAM) issue_row_f32<D>(lambda + (int64_t)bh * D, lane, (uint8_t*)lam_lds);
  if (lane < D / 4) dma_to_lds<4>(signs + (int64_t)bh * a.sign_stride, 4u * (uint32_t)lane, lds_addr(sraw));
  wait_vm<0>();
  wave_fence();
  build_masks2<D, ROT_SRFT>(sraw, smask, lane);   // plain masks (no SRHT flip on the way out)
  if constexpr (LAM) {
    // e_j / lambda_j, lane-parallel, read back per lane
    for (int j = lane; j < D; j += 64) {
      const bool edge = Sc::kEdges && (j % L == 0);
      lam_lds[j] = (edge ? (float)Sc::kInvEdge : (float)Sc::kInvBulk) * __builtin_amdgcn_rcpf(lam_lds[j]);
    }
    wave_fence();
  }
  // this lane's half code row and half scale row
  uint32_t cw[NCW], sw[NSW];
  {
    if constexpr (CBL >= 16) {
      static_for<CBL / 16>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        const uint4 q = tile_chunk<CT>(ctile, t, (CBL / 16) * p + c);
        cw[4 * c] = q.x;
        cw[4 * c + 1] = q.y;
        cw[4 * c + 2] = q.z;
        cw[4 * c + 3] = q.w;
      });
    }
    if constexpr (SBL >= 16) {
      static_for<SBL / 16>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        const uint4 q = tile_chunk<ST>(stile, t, (SBL / 16) * p + c);
        sw[4 * c] = q.x;
        sw[4 * c + 1] = q.y;
        sw[4 * c + 2] = q.z;
        sw[4 * c + 3] = q.w;
      });
    } else {
      // rows of 2, 4 or 8 bytes per lane-half: within one 16-byte chunk of
      // the row (position swizzled), or unswizzled sub-16-byte rows
      const uint8_t* row = stile + t * ST::kRowLds;
      if constexpr (ST::kWide) {
        const uint8_t* src = row + 16 * (0 ^ ST::swz(t)) + (XL ? 0 : SBL * p);
        if constexpr (SBL == 8) {
          const uint2 q = *(const uint2*)src;
          sw[0] = q.x;
          sw[1] = q.y;
        } else if constexpr (SBL == 4) {
          sw[0] = *(const uint32_t*)src;
        } else {
          sw[0] = *(const uint16_t*)src;
        }
      } else {
        // ST::kElem-byte elements, each in a kSlot-byte slot
        static_assert(SBL % 2 == 0, "scale bytes per lane");
        if constexpr (XL) {
          sw[0] = *(const uint16_t*)row;
        } else if constexpr (ST::kElem >= SBL) {
          const uint8_t* src = row + SBL * p;
          if constexpr (SBL == 4) sw[0] = *(const uint32_t*)src;
          else sw[0] = *(const uint16_t*)src;
        } else {
          // 2-byte elements in 4-byte slots: element p of the row
          sw[0] = *(const uint16_t*)(row + ST::kSlot * p);
        }
      }
    }
  }
  wait_lgkm0();
  wave_fence();   // the tiles are read: the output staging may overwrite them

  const float sgn = p ? -1.0f : 1.0f;
  // SRFT: lane 1's upper half is carried negated (as the forward leaves it)
  constexpr bool kFold = ROT == ROT_SRFT && G <= L / 2;
  float h[L];
  dequantize_head<L, GL, BITS, ROT, VAR_REAL, LAM, Sc, (kFold ? L / 2 : L)>(cw, sw, lam_lds + L * p, h, sgn);
  if constexpr (ROT == ROT_SRFT && !kFold) {
    static_for<L / 2>([&](auto ii) { h[L / 2 + decltype(ii)::value] *= sgn; });
  }
  uint32_t o[L / 2];   // this lane's output dwords, in the order it stages them
  if constexpr (ROT == ROT_SRFT) {
    static_for<L / 2 - 1>([&](auto kk) {
      constexpr int q = decltype(kk)::value + 1;
      float u = h[q] + h[L - q], v = h[q] - h[L - q];
      swap32(u, v);
      h[q] = u;
      h[L - q] = v;
    });
    {
      float X = h[0], Y = h[0];
      swap32(X, Y);
      h[0] = __builtin_fmaf(sgn, Y, X);
    }
    if (p) {   // lane 1: O_k <- conj(W^k) O_k
      static_for<L / 2 - 1>([&](auto kk) {
        constexpr int q = decltype(kk)::value + 1;
        constexpr float c = (float)ccos(2.0 * kPi * q / D), s = (float)csin(2.0 * kPi * q / D);
        const float Or = h[q], Oi = h[L - q];
        h[q] = __builtin_fmaf(c, Or, -s * Oi);
        h[L - q] = __builtin_fmaf(c, Oi, s * Or);
      });
    }
    float xr[L];
    irdft<L, 1, 0, L, 2>(h, xr);        // x[2m + p]
    uint32_t pk[L / 2];
    static_for<L / 2>([&](auto mm) {
      constexpr int m = decltype(mm)::value;
      pk[m] = pack_f16x2(xr[2 * m], xr[2 * m + 1]);   // (x[4m + p], x[4m + 2 + p])
    });
    static_for<L / 4>([&](auto mm) {
      constexpr int m = decltype(mm)::value;
      uint32_t X = pk[m], Y = pk[m + L / 4];
      swap32(X, Y);   // lane 0: pairs m of both lanes; lane 1: pairs m + L/4
      o[2 * m] = __builtin_amdgcn_perm(Y, X, 0x05040100u);
      o[2 * m + 1] = __builtin_amdgcn_perm(Y, X, 0x07060302u);
    });
  } else if constexpr (ROT == ROT_SRHT) {
    wht<L>(h);
    float top[L / 2], bot[L / 2];
    static_for<L / 2>([&](auto ii) {
      constexpr int i = decltype(ii)::value;
      float X = h[i], Y = h[i + L / 2];
      swap32(X, Y);   // lane 0: (H a)_i, (H b)_i; lane 1: the same for i + L/2
      top[i] = X + Y;
      bot[i] = X - Y;
    });
    static_for<L / 4>([&](auto mm) {
      constexpr int m = decltype(mm)::value;
      o[m] = pack_f16x2(top[2 * m], top[2 * m + 1]);
      o[L / 4 + m] = pack_f16x2(bot[2 * m], bot[2 * m + 1]);
    });
  } else {
    static_for<L / 2>([&](auto mm) {
      constexpr int m = decltype(mm)::value;
      o[m] = pack_f16x2(h[2 * m], h[2 * m + 1]);
    });
  }

  // Output dwords of lane p: SRFT and none: dwords 64p .. 64p+63 of the row;
  // SRHT: dwords 32p .. 32p+31 (top) and 64 + 32p .. (bottom).  Apply the
  // signs and stage the row in LDS (16-byte chunks, swizzled).
  {
    uint8_t* row = lds + t * OT::kRowLds;
    static_for<L / 8>([&](auto cc) {
      constexpr int c = decltype(cc)::value;   // the lane's c-th chunk
      int chunk;
      if constexpr (ROT == ROT_SRHT)
        chunk = (c < L / 16) ? (L / 16) * p + c : L / 8 + (L / 16) * p + (c - L / 16);
      else
        chunk = (L / 8) * p + c;
      const uint4 m = *(const uint4*)(smask + 4 * chunk);
      *(uint4*)(row + 16 * (chunk ^ OT::swz(t))) =
          make_uint4(o[4 * c] ^ m.x, o[4 * c + 1] ^ m.y, o[4 * c + 2] ^ m.z, o[4 * c + 3] ^ m.w);
    });
  }
  wave_fence();
  {
    uint8_t* obase = (uint8_t*)x_out + row_index(a, bh, t0) * (int64_t)(2 * D);
    static_for<OT::kInst>([&](auto ii) {
      constexpr int i = decltype(ii)::value;
      const int v = i * OT::kRpi + lane / OT::kCpr;
      const int c = lane % OT::kCpr;
      if (v < nv) {
        const uint4 q = *(const uint4*)(lds + v * OT::kRowLds + 16 * (c ^ OT::swz(v)));
        typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
        const u32x4_t val = {q.x, q.y, q.z, q.w};
        __builtin_nontemporal_store(val, (u32x4_t*)(obase + (int64_t)v * rsb_x + 16 * c));
      }
    });
  }
}

}  // namespace srftq
