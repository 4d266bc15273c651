// quant.h -- per-lane quantizer tail and dequantizer head.
//
// "When Quantization Is Free" (gist.science summary), "Metodologia" 2 step 4
// (per-channel lambda rescale, per-group absmax, rounding to signed
// int4/int8) and step 5 (two int4 per byte), with "Metodologia" 3
// (per-channel + per-group scaling).  Decision rule (fp32):
//   z = lambda * y;  a = max_G |z|;  sigma = fp16(min(a * fp32(1/qmax), 65504));
//   r = fp32(1/sigma) correctly rounded;
//   q = clamp(rne(z * r), -qmax, qmax) with the product exact  (q = 0 when
//   sigma == 0).
//
// Implementation notes (gfx950):
//   - The transform leaves y unscaled; the per-coordinate scale c_j is
//     uniform inside a group except at SRFT coordinates 0 and d/2, so the
//     absmax is taken on unscaled values and scaled once per group (fp32
//     rounding is monotonic, so max(fl(c|y|)) = fl(c max|y|)), and c is
//     folded into the per-group reciprocal.
//   - rne(z * r) is one FMA with the magic constant 1.5*2^23 + 2^(bits-1):
//     the fp32 add rounds to the nearest integer (ties to even) and leaves
//     q + 2^(bits-1) in the low bits, so codes are offset-binary until one
//     XOR per dword flips them to two's complement.
//   - Every group with a normal fp16 sigma below 65504 has |z / sigma| <=
//     7.0035 (resp. 127.07), so rounding alone stays in range; the clamp is
//     only needed for fp16-subnormal or saturated scales and runs on a
//     separate, wave-uniform path.
#pragma once

#include "xform.h"

namespace srftq {

// Byte K of a dword as fp32: one v_cvt_f32_ubyteK (register-only asm; the
// compiler would otherwise extract the byte first when it knows the upper
// bits of each byte are clear).
template <int K>
__device__ __forceinline__ float ubyte_f32(uint32_t v) {
  float r;
  if constexpr (K == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(v));
  else if constexpr (K == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(v));
  else if constexpr (K == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(v));
  else asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(v));
  return r;
}

template <int BITS>
struct QConst {
  static constexpr int kQmax = BITS == 4 ? 7 : 127;
  static constexpr float kQinv = (float)(1.0 / kQmax);
  static constexpr uint32_t kMagicBits = 0x4b400000u + (BITS == 4 ? 8u : 128u);
  static constexpr uint32_t kLo = kMagicBits - (uint32_t)kQmax;   // bits of q = -qmax
  static constexpr uint32_t kHi = kMagicBits + (uint32_t)kQmax;   // bits of q = +qmax
};

// fp32(1/sigma), correctly rounded, for sigma an fp16 value.  1/sigma =
// 2^-e / m with an integer m < 2^11 is never within 2^-36 (relative) of an
// fp32 rounding midpoint, so an fp64 reciprocal (plus one Newton step) rounded
// to fp32 is the correctly rounded fp32 reciprocal.  One per group.
__device__ __forceinline__ float recip_f16_value(float sigma) {
  const double s = (double)sigma;
  double r = __builtin_amdgcn_rcp(s);
  r = __builtin_fma(r, __builtin_fma(-s, r, 1.0), r);
  return (float)r;
}

// Codes of one vector: int4 -> D/8 dwords, int8 -> D/4 dwords.
template <int D, int BITS>
struct CodeWords {
  static constexpr int kWords = D * BITS / 32;
};

// Scales of one vector, fp16, packed two per dword (last dword half-used
// when D/G is odd, i.e. D/G == 1).
template <int D, int G>
struct ScaleWords {
  static constexpr int kGroups = D / G;
  static constexpr int kWords = (kGroups + 1) / 2;
};

// Pack rounded magic-biased values t[0..7] (int4) or t[0..3] (int8) of
// coordinates 8i.. (resp. 4i..) into one code dword.
template <int BITS>
__device__ __forceinline__ uint32_t pack_codes(const uint32_t* t) {
  if constexpr (BITS == 4) {
    const uint32_t b0 = (t[1] << 4) | t[0];     // low byte: nibbles q0+8, q1+8
    const uint32_t b1 = (t[3] << 4) | t[2];
    const uint32_t b2 = (t[5] << 4) | t[4];
    const uint32_t b3 = (t[7] << 4) | t[6];
    const uint32_t p01 = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
    const uint32_t p23 = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);
    return __builtin_amdgcn_perm(p23, p01, 0x05040100u) ^ 0x88888888u;
  } else {
    const uint32_t p01 = __builtin_amdgcn_perm(t[1], t[0], 0x0c0c0400u);
    const uint32_t p23 = __builtin_amdgcn_perm(t[3], t[2], 0x0c0c0400u);
    return __builtin_amdgcn_perm(p23, p01, 0x05040100u) ^ 0x80808080u;
  }
}

// Quantize one vector.  y: unscaled transform output (packed order).
// lam: the head's lambda row in LDS (read broadcast) or unused.
template <int D, int G, int BITS, int ROT, int VAR, bool LAM>
__device__ __forceinline__ void quantize_tail(float (&y)[D], const float* __restrict__ lam,
                                              uint32_t (&codes)[CodeWords<D, BITS>::kWords],
                                              uint32_t (&scales)[ScaleWords<D, G>::kWords]) {
  using Sc = Scales<D, ROT, VAR>;
  using Q = QConst<BITS>;
  constexpr int NG = D / G;
  constexpr float cB = (float)Sc::kFwdBulk;
  constexpr float cE = (float)Sc::kFwdEdge;

  if constexpr (LAM) {
    // z = lambda * y group by group; the next group's lambda (LDS
    // broadcast) is requested before this group's multiplies, so the LDS
    // latency overlaps them instead of stalling each read.
    static_assert(G % 4 == 0, "lambda groups are read four floats at a time");
    float lc[G], ln[G];
    auto fetch = [&](float (&dst)[G], int g) {
      static_for<G / 4>([&](auto qq) {
        constexpr int q = decltype(qq)::value;
        const float4 v = *(const float4*)(lam + g * G + 4 * q);
        dst[4 * q + 0] = v.x;
        dst[4 * q + 1] = v.y;
        dst[4 * q + 2] = v.z;
        dst[4 * q + 3] = v.w;
      });
    };
    fetch(lc, 0);
    static_for<NG>([&](auto gg) {
      constexpr int g = decltype(gg)::value;
      if constexpr (g + 1 < NG) fetch(ln, g + 1);
      static_for<G>([&](auto kk) {
        constexpr int k = decltype(kk)::value;
        y[g * G + k] = y[g * G + k] * lc[k];
      });
      if constexpr (g + 1 < NG) {
        static_for<G>([&](auto kk) { lc[decltype(kk)::value] = ln[decltype(kk)::value]; });
      }
    });
  }

  float rB[NG], rE[NG];
  uint32_t need_clamp = 0;
  static_for<(NG + 1) / 2>([&](auto pp) {
    constexpr int g0 = 2 * decltype(pp)::value;
    float t[2];
    static_for<(g0 + 1 < NG ? 2 : 1)>([&](auto ii) {
      constexpr int g = g0 + decltype(ii)::value;
      float mb = 0.0f, me = 0.0f;
      static_for<G>([&](auto kk) {
        constexpr int j = g * G + decltype(kk)::value;
        if constexpr (Sc::is_edge(j))
          me = __builtin_fmaxf(me, __builtin_fabsf(y[j]));
        else
          mb = __builtin_fmaxf(mb, __builtin_fabsf(y[j]));
      });
      float a = mb * cB;
      constexpr bool has_edge = Sc::is_edge(g * G) || (Sc::kEdges && (g * G <= D / 2) && (D / 2 < (g + 1) * G));
      if constexpr (has_edge) a = __builtin_fmaxf(a, me * cE);
      const float tt = a * Q::kQinv;
      need_clamp |= (tt > 65504.0f) ? 1u : 0u;
      t[decltype(ii)::value] = __builtin_fminf(tt, 65504.0f);
    });
    uint32_t sw;
    if constexpr (g0 + 1 < NG) {
      sw = pack_f16x2(t[0], t[1]);
    } else {
      sw = pack_f16x2(t[0], 0.0f) & 0xffffu;
    }
    scales[g0 / 2] = sw;
    static_for<(g0 + 1 < NG ? 2 : 1)>([&](auto ii) {
      constexpr int g = g0 + decltype(ii)::value;
      const float sg = ii == 0 ? hlo(sw) : hhi(sw);
      // sigma subnormal (and nonzero): rounding alone may leave the range
      need_clamp |= (sg != 0.0f && sg < 6.103515625e-05f) ? 1u : 0u;
      const float r = sg == 0.0f ? 0.0f : recip_f16_value(sg);
      rB[g] = r * cB;
      rE[g] = r * cE;
    });
  });

  const float magic = as_f32(Q::kMagicBits);
  auto emit = [&](auto clampc) {
    constexpr bool CLAMP = decltype(clampc)::value;
    constexpr int PER = BITS == 4 ? 8 : 4;
    static_for<D / PER>([&](auto ww) {
      constexpr int w = decltype(ww)::value;
      uint32_t t[PER];
      static_for<PER>([&](auto ii) {
        constexpr int j = w * PER + decltype(ii)::value;
        constexpr int g = j / G;
        const float r = Sc::is_edge(j) ? rE[g] : rB[g];
        uint32_t b = as_u32(__builtin_fmaf(y[j], r, magic));
        if constexpr (CLAMP) {
          // signed compare: huge negative products give negative bit patterns
          int bi = (int)b;
          bi = bi < (int)Q::kLo ? (int)Q::kLo : bi;
          bi = bi > (int)Q::kHi ? (int)Q::kHi : bi;
          b = (uint32_t)bi;
        }
        t[decltype(ii)::value] = b;
      });
      codes[w] = pack_codes<BITS>(t);
    });
  };
  if (__builtin_amdgcn_ballot_w64(need_clamp != 0) == 0) {
    emit(std::integral_constant<bool, false>{});
  } else {
    emit(std::integral_constant<bool, true>{});
  }
}

// Dequantizer head: codes + scales of one vector -> coordinates multiplied
// by sigma_G * e_j / lambda_j, where e_j is the inverse transform's input
// scale.  lam: table of e_j / lambda_j for the head (LAM) or unused.
template <int D, int G, int BITS, int ROT, int VAR, bool LAM>
__device__ __forceinline__ void dequantize_head(const uint32_t (&codes)[CodeWords<D, BITS>::kWords],
                                                const uint32_t (&scales)[ScaleWords<D, G>::kWords],
                                                const float* __restrict__ lam, float (&y)[D]) {
  using Sc = Scales<D, ROT, VAR>;
  constexpr int NG = D / G;
  constexpr float eB = (float)Sc::kInvBulk;
  constexpr float eE = (float)Sc::kInvEdge;
  constexpr float off = BITS == 4 ? 8.0f : 128.0f;

  float sg[NG];
  static_for<NG>([&](auto gg) {
    constexpr int g = decltype(gg)::value;
    sg[g] = (g % 2 == 0) ? hlo(scales[g / 2]) : hhi(scales[g / 2]);
  });

  // u = q + off as fp32, exactly: bytes of (codes ^ bias) -> v_cvt_f32_ubyteN
  float u[D];
  if constexpr (BITS == 4) {
    static_for<D / 8>([&](auto ww) {
      constexpr int w = decltype(ww)::value;
      const uint32_t v = codes[w] ^ 0x88888888u;
      const uint32_t lo = v & 0x0f0f0f0fu;          // coordinates 8w + 0, 2, 4, 6
      const uint32_t hi = (v >> 4) & 0x0f0f0f0fu;   // coordinates 8w + 1, 3, 5, 7
      u[8 * w + 0] = ubyte_f32<0>(lo);
      u[8 * w + 2] = ubyte_f32<1>(lo);
      u[8 * w + 4] = ubyte_f32<2>(lo);
      u[8 * w + 6] = ubyte_f32<3>(lo);
      u[8 * w + 1] = ubyte_f32<0>(hi);
      u[8 * w + 3] = ubyte_f32<1>(hi);
      u[8 * w + 5] = ubyte_f32<2>(hi);
      u[8 * w + 7] = ubyte_f32<3>(hi);
    });
  } else {
    static_for<D / 4>([&](auto ww) {
      constexpr int w = decltype(ww)::value;
      const uint32_t v = codes[w] ^ 0x80808080u;
      u[4 * w + 0] = ubyte_f32<0>(v);
      u[4 * w + 1] = ubyte_f32<1>(v);
      u[4 * w + 2] = ubyte_f32<2>(v);
      u[4 * w + 3] = ubyte_f32<3>(v);
    });
  }

  if constexpr (LAM) {
    // q*sigma exactly (fma of small integers), then * (e_j / lambda_j),
    // the latter precomputed per head in lam[].
    static_for<NG>([&](auto gg) {
      constexpr int g = decltype(gg)::value;
      const float s = sg[g], ns = -off * sg[g];
      static_for<G>([&](auto kk) {
        constexpr int j = g * G + decltype(kk)::value;
        y[j] = __builtin_fmaf(u[j], s, ns) * lam[j];
      });
      // d = 256 fills the register file: one group's table reads at a time
      if constexpr (D >= 256) __builtin_amdgcn_sched_barrier(0);
    });
  } else {
    static_for<NG>([&](auto gg) {
      constexpr int g = decltype(gg)::value;
      const float kb = sg[g] * eB, nkb = -off * kb;
      const float ke = sg[g] * eE, nke = -off * ke;
      static_for<G>([&](auto kk) {
        constexpr int j = g * G + decltype(kk)::value;
        y[j] = Sc::is_edge(j) ? __builtin_fmaf(u[j], ke, nke) : __builtin_fmaf(u[j], kb, nkb);
      });
    });
  }
}

}  // namespace srftq
