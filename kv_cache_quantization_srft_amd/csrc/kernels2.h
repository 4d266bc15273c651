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
  static_assert(D / 4 <= 64, "one sign dword per lane");
  if (D / 4 == 64 || lane < D / 4) {
    const int i = lane;
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
// Balanced last step of the two-lane SRFT, for groups of at most Q = D/8
// coordinates (or one group over the whole vector).
//
// After the per-lane transforms lane 0 holds E (the spectrum of x[2m]) and
// lane 1 holds O (of x[2m+1]), halfcomplex of length L = D/2.  Bin kappa =
// k + Q p (0 < k < Q) of the half spectra goes to lane p: two
// v_permlane32_swap bring it E_kappa and O_kappa, and it forms
//   X_kappa = E + W^kappa O,  X_{D/2-kappa} = conj(E - W^kappa O),
// W = e^{-2 pi i / D}, with its own twiddle read from an LDS table.  Bins 0,
// Q and 2Q are exchanged on their own.  Lane p then owns four runs of Q
// packed coordinates, starting at Seg2<D>::base(s, p) and held in its local
// slots [sQ, (s+1)Q): both lanes run the same instructions (no lane idles
// through a twiddle), and no group crosses lanes.  The inverse runs the same
// steps backwards.
// ----------------------------------------------------------------------------
template <int D>
struct Seg2 {
  static constexpr int Q = D / 8;
  static constexpr int kBase[4] = {0, 3 * Q, 4 * Q, 7 * Q};   // run starts of lane 0
  static constexpr int kDir[4] = {1, -1, 1, -1};              // run start change per unit of p, in Q
  __device__ static __forceinline__ int base(int s, int p) { return kBase[s] + kDir[s] * Q * p; }
};

// Every coordinate of the two-lane SRFT at the bulk scale: the two edge
// coordinates (packed 0 and D/2, both in lane 0) are rescaled by the
// combine step itself.
struct NoEdges {
  static constexpr bool kEdges = false;
  static constexpr bool is_edge(int) { return false; }
};
template <int D>
struct BulkScales : NoEdges {
  static constexpr double kFwdBulk = Scales<D, ROT_SRFT, VAR_REAL>::kFwdBulk;
  static constexpr double kFwdEdge = kFwdBulk;
  static constexpr double kInvBulk = Scales<D, ROT_SRFT, VAR_REAL>::kInvBulk;
  static constexpr double kInvEdge = kInvBulk;
};

// lambda entries of a lane's runs: plus = lam + Q p, minus = lam - Q p.
template <int D>
struct SegLam {
  const float* plus;
  const float* minus;
};
template <int D>
__device__ __forceinline__ const float* lam_at(const SegLam<D>& l, int j) {
  constexpr int Q = Seg2<D>::Q;
  const int s = j / Q;
  return ((s & 1) ? l.minus : l.plus) + Seg2<D>::kBase[s] + (j - s * Q);
}

// (cos, sin)(2 pi l / D) for l < D/4: the twiddles of the balanced step
// (lane p uses entries Q p .. Q p + Q - 1).
template <int D>
struct QuarterTwiddles {
  float v[D / 2];
  constexpr QuarterTwiddles() : v() {
    for (int l = 0; l < D / 4; ++l) {
      v[2 * l] = (float)ccos(2.0 * kPi * l / D);
      v[2 * l + 1] = (float)csin(2.0 * kPi * l / D);
    }
  }
};
template <int D>
__device__ __forceinline__ void build_twiddles2(float2* tw, int lane) {
  static constexpr QuarterTwiddles<D> kT{};
  static_assert(D / 4 <= 64, "one twiddle per lane");
  if (D / 4 == 64 || lane < D / 4) tw[lane] = make_float2(kT.v[2 * lane], kT.v[2 * lane + 1]);
}

// Forward: h (E in lane 0, O in lane 1) -> y, this lane's runs.  twl: the
// lane's twiddles (LDS), odd: lane 1, rho: kFwdEdge / kFwdBulk, applied to
// X_0 and X_{D/2}.
template <int D>
__device__ __forceinline__ void srft2_forward(const float (&h)[D / 2], float (&y)[D / 2], const float2* twl,
                                              bool odd, float rho) {
  constexpr int L = D / 2, Q = D / 8, M = 2 * Q;
  constexpr float r2 = 0.70710678118654752440f;
  const float sg = odd ? 1.0f : -1.0f;
  // bins 0 and M: lane 0 gets (E_0, O_0), lane 1 (E_M, O_M)
  float u = h[0], v = h[M];
  swap32(u, v);
  // bin Q of both half spectra, to both lanes
  float er = h[Q], orr = h[Q];
  swap32(er, orr);
  float ei = h[L - Q], oi = h[L - Q];
  swap32(ei, oi);
  // W^Q O_Q, W^Q = (1 - i) / sqrt 2: lane 1 forms X_Q, lane 0 X_{D/2-Q}
  const float pr = (orr + oi) * r2, pi = (oi - orr) * r2;
  const float R = __builtin_fmaf(sg, pr, er), I = __builtin_fmaf(sg, ei, pi);
  y[0] = odd ? R : (u + v) * rho;          // Re X_Q          | X_0
  y[Q] = odd ? u : R;                      // Re X_M = E_M    | Re X_{D/2-Q}
  y[2 * Q] = odd ? I : (u - v) * rho;      // Im X_Q          | X_{D/2}
  y[3 * Q] = odd ? -v : I;                 // Im X_M = -O_M   | Im X_{D/2-Q}
  static_for<Q - 1>([&](auto kk) {
    constexpr int k = decltype(kk)::value + 1;
    float er_ = h[k], or_ = h[k + Q];
    swap32(er_, or_);   // Re E_kappa, Re O_kappa
    float ei_ = h[L - k], oi_ = h[L - Q - k];
    swap32(ei_, oi_);   // Im E_kappa, Im O_kappa
    const float2 w = twl[k];
    const float xr = __builtin_fmaf(w.y, oi_, __builtin_fmaf(w.x, or_, er_));
    const float xi = __builtin_fmaf(-w.y, or_, __builtin_fmaf(w.x, oi_, ei_));
    y[k] = xr;                                      // Re X_kappa
    y[2 * Q + k] = xi;                              // Im X_kappa
    y[2 * Q - k] = __builtin_fmaf(2.0f, er_, -xr);  // Re X_{D/2-kappa}
    y[4 * Q - k] = __builtin_fmaf(-2.0f, ei_, xi);  // Im X_{D/2-kappa}
  });
}

// Inverse: this lane's runs y -> h (E' in lane 0, O' in lane 1, as the
// inverse half transforms take them: E'_k = X_k + conj X_{D/2-k}, O'_k =
// conj(W^k) (X_k - conj X_{D/2-k}), bin M carrying its pending factor 2).
// rho: kInvEdge / kInvBulk where the scales have not yet been applied per
// coordinate, else 1.
template <int D>
__device__ __forceinline__ void srft2_inverse(const float (&y)[D / 2], float (&h)[D / 2], const float2* twl,
                                              bool odd, float rho) {
  constexpr int L = D / 2, Q = D / 8, M = 2 * Q;
  constexpr float r2 = 0.70710678118654752440f;
  {
    // bins 0 and M: lane 0 has X_0 = y[0], X_{D/2} = y[2Q]; lane 1 has X_M
    float t1 = odd ? y[Q] : (y[0] + y[2 * Q]) * rho;
    float t2 = odd ? -y[3 * Q] : (y[0] - y[2 * Q]) * rho;
    swap32(t1, t2);   // lane 0: (E'_0, E'_M); lane 1: (O'_0, O'_M)
    h[0] = t1;
    h[M] = t2;
  }
  {
    // bin Q: lane 1 has X_Q = (y[0], y[2Q]), lane 0 X_{D/2-Q} = (y[Q], y[3Q])
    float vr = odd ? y[0] : y[Q], vr2 = vr;
    swap32(vr, vr2);   // both lanes: Re X_{D/2-Q}, Re X_Q
    float vi = odd ? y[2 * Q] : y[3 * Q], vi2 = vi;
    swap32(vi, vi2);   // both lanes: Im X_{D/2-Q}, Im X_Q
    const float pr = vr2 - vr, pi = vi2 + vi;   // X_Q - conj X_{D/2-Q}
    h[Q] = odd ? (pr - pi) * r2 : vr2 + vr;
    h[L - Q] = odd ? (pr + pi) * r2 : vi2 - vi;
  }
  static_for<Q - 1>([&](auto kk) {
    constexpr int k = decltype(kk)::value + 1;
    const float ar = y[k], ai = y[2 * Q + k];          // X_kappa
    const float br = y[2 * Q - k], bi = y[4 * Q - k];  // X_{D/2-kappa}
    const float2 w = twl[k];
    const float pr = ar - br, pi = ai + bi;             // X_kappa - conj X_{D/2-kappa}
    float er = ar + br, orr = __builtin_fmaf(w.x, pr, -w.y * pi);
    float ei = ai - bi, oi = __builtin_fmaf(w.x, pi, w.y * pr);
    swap32(er, orr);   // lane 0: (E'_k, E'_{k+Q}); lane 1: (O'_k, O'_{k+Q})
    swap32(ei, oi);
    h[k] = er;
    h[k + Q] = orr;
    h[L - k] = ei;
    h[L - Q - k] = oi;
  });
}

// ----------------------------------------------------------------------------
// Quantize, two lanes per vector, 32-token tiles.  A block walks the tiles
// of its TileRange; each tile's rows are read from LDS into registers, then
// the next tile's LDS-DMA is issued (into the same LDS, with its lambda and
// sign rows into the other half of their double buffers) and runs while
// this tile computes and stores.
// ----------------------------------------------------------------------------
template <int D, int G, int BITS, int ROT, bool LAM>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(SRFTQ_QUANT2_WAVES)))
void quantize2_kernel(const uint16_t* __restrict__ x, const int8_t* __restrict__ signs,
                      const float* __restrict__ lambda, uint8_t* __restrict__ codes_out,
                      uint16_t* __restrict__ scales_out, Geo a) {
  constexpr int L = D / 2;                  // coordinates per lane
  using Sc = HalfScales<D, ROT>;
  using XT = RowTile<2 * D, 32>;
  // SRFT: the balanced layout (runs of Q = D/8 coordinates); SRHT and none:
  // lane p owns the half row [pL, pL + L)
  constexpr bool kBal = ROT == ROT_SRFT;
  constexpr int Q = D / 8;
  // groups larger than what one lane holds of them continue in the partner
  // lane, each lane holding half of every group
  constexpr bool XL = kBal ? G > Q : G > L;
  constexpr int GL = XL ? G / 2 : G;                  // group width inside a lane
  constexpr int CB = D * BITS / 8, CBL = CB / 2;     // code bytes per vector / per lane
  constexpr int SB = 2 * D / G, SBL = XL ? SB : SB / 2;   // scale bytes per vector / per lane
  constexpr int NCW = CodeWords<L, BITS>::kWords;
  constexpr int NSW = ScaleWords<L, GL>::kWords;
  constexpr int SEGW = Q * BITS / 32;                 // code words per run (balanced layout)
  // global store instructions per tile (every lane issues the same ones)
  constexpr int NST = kBal ? 4 * store_count<SEGW>() + (XL ? 1 : 4)
                           : store_count<NCW>() + (L / GL == 1 ? 1 : store_count<NSW>());
  // raw dwords a lane reads from the tile: its half row, or (SRHT) the row
  constexpr int NRAW = ROT == ROT_SRHT ? D / 2 : L / 2;
  static_assert(kBal || G <= L || G == D, "groups stay inside one lane, or span the vector");
  __shared__ __attribute__((aligned(16))) uint8_t lds[XT::kBytes];
  __shared__ __attribute__((aligned(16))) float lam_lds[LAM ? 2 * D : 4];
  __shared__ __attribute__((aligned(16))) uint32_t sraw[2 * (D / 4)];
  __shared__ __attribute__((aligned(16))) uint32_t smask[ROT == ROT_SRHT ? D : D / 2];
  __shared__ __attribute__((aligned(16))) float2 tw2[kBal ? D / 4 : 1];

  const int lane_id = threadIdx.x;
  const TileRange tr(a);
  if (tr.first >= a.n_tiles) return;
  if constexpr (kBal) build_twiddles2<D>(tw2, lane_id);
  const uint32_t rsb = (uint32_t)a.H * (uint32_t)(2 * D);
  const int dk = tr.step / a.BH, dbh = tr.step - dk * a.BH;
  Cursor cur;
  cur.init(tr.first, a.BH);
  int remaining = tr.remaining;

  auto issue = [&](const Cursor& c, int& nv, int buf, int lane) {
    const int64_t t0 = (int64_t)c.k * 32;
    const int64_t left = a.T - t0;
    nv = left < 32 ? (int)left : 32;
    lds_poison<XT::kBytes>(lds, lane);
    if constexpr (LAM) lds_poison<4 * D>(lam_lds + buf * D, lane);
    lds_poison<D>(sraw + buf * (D / 4), lane);
    // the DMA offsets are recomputed per tile rather than held in registers
    typename XT::Plan plan;
    plan.init(lane, rsb);
    XT::issue((const uint8_t*)x + row_index(a, c.bh, t0) * (int64_t)(2 * D), rsb, nv, lane, plan, lds);
    if constexpr (LAM) issue_row_f32<D>(lambda + (int64_t)c.bh * D, lane, (uint8_t*)(lam_lds + buf * D));
    if (D / 4 == 64 || lane < D / 4)
      dma_to_lds<4>(signs + (int64_t)c.bh * a.sign_stride, 4u * (uint32_t)lane, lds_addr(sraw + buf * (D / 4)));
  };

  int nv, buf = 0;
  issue(cur, nv, 0, lane_id);
  bool full = false;   // the previous tile issued exactly NST stores after this tile's DMA
  for (;;) {
    // lane indices re-derived each tile: the addresses built from them are
    // recomputed per tile instead of being held in registers across tiles
    int lane = lane_id;
    asm volatile("" : "+v"(lane));
    const int t = lane & 31, p = lane >> 5;
    // wait for this tile's DMA; a full previous tile's stores may still drain
    if (full)
      wait_vm<NST>();
    else
      wait_vm<0>();
    wave_fence();
    const int cb = buf;
    build_masks2<D, ROT>(sraw + cb * (D / 4), smask, lane);
    wave_fence();

    float h[L];
    uint32_t raw[ROT == ROT_NONE ? 1 : NRAW];
    if constexpr (ROT == ROT_NONE) {
      // the own half row, signs applied, straight to fp32
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
    } else {
      static_for<NRAW / 4>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        // SRFT: chunks of the own half row; SRHT: the whole row
        const uint4 q = ROT == ROT_SRHT ? tile_chunk<XT>(lds, t, c) : tile_chunk<XT>(lds, t, (L / 8) * p + c);
        raw[4 * c + 0] = q.x;
        raw[4 * c + 1] = q.y;
        raw[4 * c + 2] = q.z;
        raw[4 * c + 3] = q.w;
      });
    }
    wait_lgkm0();   // the tile is in registers: the next DMA may overwrite it
    wave_fence();

    const Cursor now = cur;
    const int nv_now = nv;
    const bool more = remaining > 0;
    if (more) {
      cur.advance(dk, dbh, a.BH);
      buf ^= 1;
      issue(cur, nv, buf, lane);
    }

    if constexpr (ROT == ROT_SRFT) {
      // own half row (elements 128p ..), signs applied
      const uint32_t* mrow = smask + (L / 2) * p;
      uint32_t dw[L / 2];
      static_for<L / 8>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        const uint4 m = *(const uint4*)(mrow + 4 * c);
        dw[4 * c + 0] = raw[4 * c + 0] ^ m.x;
        dw[4 * c + 1] = raw[4 * c + 1] ^ m.y;
        dw[4 * c + 2] = raw[4 * c + 2] ^ m.z;
        dw[4 * c + 3] = raw[4 * c + 3] ^ m.w;
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
      float hs[L];
      rdft<L, 1, 0, L>(p0, p1, hs);
      srft2_forward<D>(hs, h, tw2 + Q * p, p != 0, (float)(Sc::kFwdEdge / Sc::kFwdBulk));
    } else if constexpr (ROT == ROT_SRHT) {
      // pair sums a + (-1)^p b of the top and bottom halves
      const uint32_t* mrow = smask + D / 2 * p;
      float one = 1.0f;
      asm("" : "+s"(one));
      static_for<L / 8>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        const uint4 ma = *(const uint4*)(smask + 4 * c);
        const uint4 mb = *(const uint4*)(mrow + L / 2 + 4 * c);
        const uint32_t wa[4] = {raw[4 * c] ^ ma.x, raw[4 * c + 1] ^ ma.y, raw[4 * c + 2] ^ ma.z,
                                raw[4 * c + 3] ^ ma.w};
        const uint32_t wb[4] = {raw[L / 2 + 4 * c] ^ mb.x, raw[L / 2 + 4 * c + 1] ^ mb.y,
                                raw[L / 2 + 4 * c + 2] ^ mb.z, raw[L / 2 + 4 * c + 3] ^ mb.w};
        static_for<4>([&](auto ii) {
          constexpr int i = decltype(ii)::value;
          h[8 * c + 2 * i] = __builtin_fmaf(hlo(wb[i]), one, hlo(wa[i]));
          h[8 * c + 2 * i + 1] = __builtin_fmaf(hhi(wb[i]), one, hhi(wa[i]));
        });
      });
      wht<L>(h);
    }
    uint32_t codes[NCW];
    uint32_t scales[NSW];
    float* const lt = lam_lds + cb * D;
    if constexpr (kBal)
      quantize_tail<L, GL, BITS, ROT, VAR_REAL, LAM, BulkScales<D>, L, XL>(h, SegLam<D>{lt + Q * p, lt - Q * p},
                                                                         codes, scales, 1.0f);
    else
      quantize_tail<L, GL, BITS, ROT, VAR_REAL, LAM, Sc, L, XL>(h, lt + L * p, codes, scales, 1.0f);

    // Cache row of token 0 of the tile (uniform); when appending, tokens
    // start at the tensor's position and rows outside [0, pitch) are dropped.
    int64_t t0 = (int64_t)now.k * 32;
    bool ok = t < nv_now;
    if (a.pos) {
      t0 += a.pos[now.bh / a.H];
      ok = ok && t0 + t >= 0 && t0 + t < a.pitch;
    }
    if (ok) {
      const int64_t r0 = cache_row(a, now.bh, t0) + t;
      if constexpr (kBal) {
        // run s of this lane: SEGW code words and Q/G scales
        static_for<4>([&](auto ss) {
          constexpr int sidx = decltype(ss)::value;
          const int cbase = Seg2<D>::base(sidx, p);
          uint32_t cwd[SEGW];
          static_for<SEGW>([&](auto ii) { cwd[decltype(ii)::value] = codes[sidx * SEGW + decltype(ii)::value]; });
          store_words<SEGW>(codes_out + r0 * CB + cbase * BITS / 8, cwd);
          if constexpr (!XL) {
            constexpr int GPS = Q / G;   // groups per run
            uint8_t* sdst = (uint8_t*)scales_out + r0 * SB + (cbase / G) * 2;
            if constexpr (GPS == 4)
              *(uint2*)sdst = make_uint2(scales[2 * sidx], scales[2 * sidx + 1]);
            else if constexpr (GPS == 2)
              *(uint32_t*)sdst = scales[sidx];
            else
              *(uint16_t*)sdst = (uint16_t)(scales[sidx / 2] >> (16 * (sidx % 2)));
          }
        });
        if constexpr (XL) {
          if (p == 0) store_scales<L, GL>((uint8_t*)scales_out + r0 * SB, scales);
        }
      } else {
        store_words<NCW>(codes_out + r0 * CB + CBL * p, codes);
        if (!XL || p == 0) store_scales<L, GL>((uint8_t*)scales_out + r0 * SB + (XL ? 0 : SBL * p), scales);
      }
    }
    // with dropped rows a whole wave may skip its stores: then the next
    // wait must not count on them
    full = nv_now == 32 && !a.pos;
    if (!more) break;
    --remaining;
  }
}

// ----------------------------------------------------------------------------
// Dequantize, two lanes per vector, 32-token tiles walked as in quantize:
// each tile's code and scale rows are read into registers, then the next
// tile's LDS-DMA is issued and runs while this tile computes.  Output rows
// leave through LDS in two rounds of half rows, each as 1 KiB nontemporal
// stores.
// ----------------------------------------------------------------------------
template <int D, int G, int BITS, int ROT, bool LAM>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(SRFTQ_DEQUANT2_WAVES)))
void dequantize2_kernel(const uint8_t* __restrict__ codes_in, const uint16_t* __restrict__ scales_in,
                        const int8_t* __restrict__ signs, const float* __restrict__ lambda,
                        uint16_t* __restrict__ x_out, Geo a) {
  constexpr int L = D / 2;
  using Sc = HalfScales<D, ROT>;
  // layouts and groups as in quantize2_kernel
  constexpr bool kBal = ROT == ROT_SRFT;
  constexpr int Q = D / 8;
  constexpr bool XL = kBal ? G > Q : G > L;
  constexpr int GL = XL ? G / 2 : G;
  constexpr int CB = D * BITS / 8, CBL = CB / 2;
  constexpr int SB = 2 * D / G, SBL = XL ? SB : SB / 2;   // shared groups: both lanes read every scale
  constexpr int NCW = CodeWords<L, BITS>::kWords;
  constexpr int NSW = ScaleWords<L, GL>::kWords;
  static_assert(kBal || G <= L || G == D, "groups stay inside one lane, or span the vector");
  constexpr int SEGW = Q * BITS / 32;                 // code words per run (balanced layout)
  using CT = RowTile<CB, 32>;
  using ST = RowTile<SB, 32>;
  // output staging in NR rounds (two at d = 256, where whole rows would not
  // fit the LDS of two waves per SIMD), CPR chunks per lane and round
  constexpr int NR = D >= 256 ? 2 : 1;
  constexpr int CPR = L / 8 / NR;
  using OT = RowTile<2 * D / NR, 32>;    // a round's share of the 32 rows
  constexpr int NST = NR * OT::kInst;    // global stores per tile
  __shared__ __attribute__((aligned(16))) uint8_t ctile[CT::kBytes];
  __shared__ __attribute__((aligned(16))) uint8_t stile[ST::kBytes < 16 ? 16 : ST::kBytes];
  __shared__ __attribute__((aligned(16))) uint8_t otile[OT::kBytes];
  __shared__ __attribute__((aligned(16))) float lam_lds[LAM ? 2 * D : 4];
  __shared__ __attribute__((aligned(16))) uint32_t sraw[2 * (D / 4)];
  __shared__ __attribute__((aligned(16))) uint32_t smask[D / 2];
  __shared__ __attribute__((aligned(16))) float2 tw2[kBal ? D / 4 : 1];

  const int lane_id = threadIdx.x;
  const TileRange tr(a);
  if (tr.first >= a.n_tiles) return;
  if constexpr (kBal) build_twiddles2<D>(tw2, lane_id);
  const uint32_t rsb_x = (uint32_t)a.H * (uint32_t)(2 * D);
  const int dk = tr.step / a.BH, dbh = tr.step - dk * a.BH;
  Cursor cur;
  cur.init(tr.first, a.BH);
  int remaining = tr.remaining;

  auto issue = [&](const Cursor& c, int& nv, int buf, int lane) {
    const int64_t t0 = (int64_t)c.k * 32;
    const int64_t left = a.T - t0;
    nv = left < 32 ? (int)left : 32;
    const int64_t r0 = cache_row(a, c.bh, t0);
    lds_poison<CT::kBytes>(ctile, lane);
    lds_poison<sizeof(stile)>(stile, lane);
    if constexpr (LAM) lds_poison<4 * D>(lam_lds + buf * D, lane);
    lds_poison<D>(sraw + buf * (D / 4), lane);
    typename CT::Plan cplan;
    cplan.init(lane, CB);
    typename ST::Plan splan;
    splan.init(lane, SB);
    CT::issue(codes_in + r0 * CB, CB, nv, lane, cplan, ctile);
    ST::issue((const uint8_t*)scales_in + r0 * SB, SB, nv, lane, splan, stile);
    if constexpr (LAM) issue_row_f32<D>(lambda + (int64_t)c.bh * D, lane, (uint8_t*)(lam_lds + buf * D));
    if (D / 4 == 64 || lane < D / 4)
      dma_to_lds<4>(signs + (int64_t)c.bh * a.sign_stride, 4u * (uint32_t)lane, lds_addr(sraw + buf * (D / 4)));
  };

  int nv, buf = 0;
  issue(cur, nv, 0, lane_id);
  bool full = false;   // the previous tile issued exactly NST stores after this tile's DMA
  for (;;) {
    // lane indices re-derived each tile: the addresses built from them are
    // recomputed per tile instead of being held in registers across tiles
    int lane = lane_id;
    asm volatile("" : "+v"(lane));
    const int t = lane & 31, p = lane >> 5;
    if (full)
      wait_vm<NST>();
    else
      wait_vm<0>();
    wave_fence();
    const int cb = buf;
    float* const lt = lam_lds + cb * D;
    build_masks2<D, ROT_SRFT>(sraw + cb * (D / 4), smask, lane);   // plain masks (no SRHT flip on the way out)
    if constexpr (LAM) {
      // e_j / lambda_j, lane-parallel in place, read back per lane
      static_assert(D % 64 == 0, "lambda entries per lane");
      static_for<D / 64>([&](auto ii) {
        const int j = lane + 64 * decltype(ii)::value;
        const bool edge = Sc::kEdges && (j % L == 0);
        lt[j] = (edge ? (float)Sc::kInvEdge : (float)Sc::kInvBulk) * __builtin_amdgcn_rcpf(lt[j]);
      });
    }
    wave_fence();
    // this lane's half code row and half scale row (balanced SRFT: its runs)
    uint32_t cw[NCW], sw[NSW];
    if constexpr (kBal) {
      static_for<4>([&](auto ss) {
        constexpr int sidx = decltype(ss)::value;
        const int cbase = Seg2<D>::base(sidx, p);
        static_for<SEGW / 4>([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          const uint4 qv = tile_chunk<CT>(ctile, t, cbase * BITS / 128 + c);
          cw[sidx * SEGW + 4 * c] = qv.x;
          cw[sidx * SEGW + 4 * c + 1] = qv.y;
          cw[sidx * SEGW + 4 * c + 2] = qv.z;
          cw[sidx * SEGW + 4 * c + 3] = qv.w;
        });
        if constexpr (!XL) {
          constexpr int GPS = Q / G;   // groups per run
          const int so = (cbase / G) * 2;
          const uint8_t* src = stile + t * ST::kRowLds + 16 * ((so >> 4) ^ ST::swz(t)) + (so & 15);
          if constexpr (GPS == 4) {
            const uint2 v2 = *(const uint2*)src;
            sw[2 * sidx] = v2.x;
            sw[2 * sidx + 1] = v2.y;
          } else if constexpr (GPS == 2) {
            sw[sidx] = *(const uint32_t*)src;
          } else {
            const uint32_t v1 = *(const uint16_t*)src;
            if constexpr (sidx % 2 == 0) sw[sidx / 2] = v1;
            else sw[sidx / 2] |= v1 << 16;
          }
        }
      });
      if constexpr (XL) {
        // the whole scale row (1, 2 or 4 scales, unswizzled)
        const uint8_t* row = stile + t * ST::kRowLds;
        if constexpr (SB == 8) {
          const uint2 v2 = *(const uint2*)row;
          sw[0] = v2.x;
          sw[1] = v2.y;
        } else if constexpr (SB == 4) {
          sw[0] = *(const uint32_t*)row;
        } else {
          sw[0] = *(const uint16_t*)row;
        }
      }
    } else {
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
    wait_lgkm0();   // the tiles are in registers: the next DMA may overwrite them
    wave_fence();

    const Cursor now = cur;
    const int nv_now = nv;
    const bool more = remaining > 0;
    if (more) {
      cur.advance(dk, dbh, a.BH);
      buf ^= 1;
      issue(cur, nv, buf, lane);
    }

    float h[L];
    if constexpr (kBal) {
      float yb[L];
      dequantize_head<L, GL, BITS, ROT, VAR_REAL, LAM, BulkScales<D>, L>(cw, sw, SegLam<D>{lt + Q * p, lt - Q * p},
                                                                        yb, 1.0f);
      srft2_inverse<D>(yb, h, tw2 + Q * p, p != 0, LAM ? 1.0f : (float)(Sc::kInvEdge / Sc::kInvBulk));
    } else {
      dequantize_head<L, GL, BITS, ROT, VAR_REAL, LAM, Sc, L>(cw, sw, lt + L * p, h, 1.0f);
    }
    uint32_t o[L / 2];   // this lane's output dwords, in the order it stages them
    if constexpr (ROT == ROT_SRFT) {
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

    // Output dwords of lane p: SRFT and none: dwords 64p .. 64p+63 of the
    // row (L/2 = D/4 in general); SRHT: dwords 32p .. 32p+31 (top) and
    // 64 + 32p .. (bottom); gchunk(c, p) is the row chunk of the lane's
    // chunk c.  They leave in NR rounds: in round r every lane stages its
    // chunks r CPR .. (r+1) CPR - 1, signs applied, into LDS row t (role 0's
    // then role 1's), and the wave stores the staged rows (at d = 256 a
    // round's pieces are 128-byte halves of the lanes' half rows, whole
    // cache lines).
    auto gchunk = [&](int c, int role) {
      if constexpr (ROT == ROT_SRHT)
        return (c < L / 16) ? (L / 16) * role + c : L / 8 + (L / 16) * role + (c - L / 16);
      else
        return (L / 8) * role + c;
    };
    uint8_t* const obase = (uint8_t*)x_out + row_index(a, now.bh, (int64_t)now.k * 32) * (int64_t)(2 * D);
    // the staging and store addresses are built here, not held through the
    // transform
    int lane_o = lane;
    asm volatile("" : "+v"(lane_o));
    const uint32_t t_o = (uint32_t)lane_o & 31u, p_o = (uint32_t)lane_o >> 5;
    const uint32_t wrow = t_o * OT::kRowLds, wswz = (uint32_t)OT::swz((int)t_o);
    // stores: lane l moves chunk jl = l % kCpr of the staged rows v0 + i kRpi,
    // which belongs to role jl / CPR; g0 is its byte offset in round 0
    const uint32_t v0 = (uint32_t)lane_o / OT::kCpr, jl = (uint32_t)lane_o % OT::kCpr;
    const uint32_t g0 = v0 * rsb_x + 16u * (uint32_t)gchunk((int)(jl % CPR), (int)(jl / CPR));
    // bytes between a chunk's rounds (two rounds: CPR = L/16)
    constexpr uint32_t kRoundStep = ROT == ROT_SRHT ? 2 * L : L;
    static_for<NR>([&](auto rr) {
      constexpr int r = decltype(rr)::value;
      lds_poison<OT::kBytes>(otile, lane_o);
      static_for<CPR>([&](auto jj) {
        constexpr int j = decltype(jj)::value;
        constexpr int c = r * CPR + j;
        const uint4 m = *(const uint4*)(smask + 4 * gchunk(c, (int)p_o));
        *(uint4*)(otile + wrow + 16 * ((CPR * p_o + j) ^ wswz)) =
            make_uint4(o[4 * c] ^ m.x, o[4 * c + 1] ^ m.y, o[4 * c + 2] ^ m.z, o[4 * c + 3] ^ m.w);
      });
      wave_fence();
      static_for<OT::kInst>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
        const uint32_t v = v0 + i * OT::kRpi;
        const uint4 q = *(const uint4*)(otile + v * OT::kRowLds + 16 * (jl ^ (uint32_t)OT::swz((int)v)));
        if (nv_now == 32 || (int)v < nv_now) {
          typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
          const u32x4_t val = {q.x, q.y, q.z, q.w};
          uint8_t* const rows = obase + (size_t)(i * OT::kRpi) * rsb_x;   // uniform
          __builtin_nontemporal_store(val, (u32x4_t*)(rows + (g0 + r * kRoundStep)));
        }
      });
      wait_lgkm0();   // round r's rows are read before round r + 1 overwrites them
      wave_fence();
    });
    full = nv_now == 32;
    if (!more) break;
    --remaining;
  }
}

}  // namespace srftq
