// xform.h -- register-resident rotations of one KV vector per lane.
//
// The rotation is SRFT(x) = pack(F diag(s) x) ("When Quantization Is Free",
// gist.science summary, "Metodologia" 1; fused pipeline steps 1-3 in
// "Metodologia" 2), or the normalized Walsh-Hadamard transform for the SRHT
// variant.  Every lane owns one whole d-vector, so all butterflies are
// in-register with compile-time indices and compile-time twiddles: no
// cross-lane traffic and no twiddle loads.
//
// Two SRFT organisations compute the same orthonormal map:
//   VAR_REAL   real-input radix-2 decimation in time.  Its first log2(d/2)
//              passes compute the d/2-point DFTs of the even and odd samples
//              (the real and imaginary parts of the paired sequence
//              z_m = x_2m + i x_2m+1); its last pass is the Hermitian unpack
//              X_k = E_k + W_d^k O_k.  Each pass keeps only the
//              non-redundant half of every Hermitian sub-spectrum, which
//              saves a quarter of the arithmetic of VAR_PAIRED.
//   VAR_PAIRED the pages' organisation: pair z_m = x_2m + i x_2m+1, run a
//              d/2-point complex radix-2 FFT, unpack the Hermitian symmetry.
//
// Spectra are held "halfcomplex": for a real sequence of length L,
// h[k] = Re X_k (0 <= k <= L/2) and h[L-k] = Im X_k (0 < k < L/2).
// The packed output order is y = [h[0..N], h[d-1], h[d-2], ..., h[N+1]], i.e.
// [Re X_0..Re X_N, Im X_1..Im X_{N-1}] with N = d/2, before the per-coordinate
// scale (1/sqrt(d) for X_0, X_N and sqrt(2/d) for the rest).
#pragma once

#include "dev_common.h"

namespace srftq {

enum : int { ROT_SRFT = 0, ROT_SRHT = 1, ROT_NONE = 2 };
enum : int { VAR_REAL = 1, VAR_PAIRED = 2 };

// Per-coordinate scale of the unscaled transform outputs (forward) and of
// the inputs of the unscaled inverse.  Coordinates 0 and d/2 of the SRFT
// ("edges") carry a different scale from the rest ("bulk").
template <int D, int ROT, int VAR>
struct Scales {
  static constexpr bool kEdges = (ROT == ROT_SRFT);
  static constexpr double kFwdBulk = ROT == ROT_NONE ? 1.0
                                   : ROT == ROT_SRHT ? 1.0 / csqrt(D)
                                   : VAR == VAR_REAL ? csqrt(2.0 / D)
                                                     : 1.0 / csqrt(2.0 * D);
  static constexpr double kFwdEdge = ROT == ROT_SRFT ? 1.0 / csqrt(D) : kFwdBulk;
  static constexpr double kInvBulk = ROT == ROT_NONE ? 1.0
                                   : ROT == ROT_SRHT ? 1.0 / csqrt(D)
                                                     : 1.0 / csqrt(2.0 * D);
  static constexpr double kInvEdge = ROT == ROT_SRFT ? 1.0 / csqrt(D) : kInvBulk;
  static constexpr bool is_edge(int j) { return kEdges && (j == 0 || j == D / 2); }
};

// Sign sources.  mask(m) is the XOR mask that flips the fp16 sign bits of
// elements 2m and 2m+1 where s = -1 (bit 15 and bit 31); mask4(q) returns
// masks 4q .. 4q+3.
//
// HeadSigns: the int8 +-1 row read as 4-byte words through scalar loads
// (wave-uniform, 4-byte aligned row pointer); masks built on the scalar unit.
struct HeadSigns {
  const_ptr<uint32_t> p;
  __device__ __forceinline__ explicit HeadSigns(const int8_t* row)
      : p(as_const((const uint32_t*)row)) {}
  // bit 7 of sign byte j
  __device__ __forceinline__ uint32_t sbit(int j) const { return (p[j >> 2] >> (8 * (j & 3) + 7)) & 1u; }
  __device__ __forceinline__ uint32_t mask(int m) const {
    uint32_t v = (sbit(2 * m) << 15) | (sbit(2 * m + 1) << 31);
    asm("" : "+s"(v));   // keep the mask whole in an SGPR: one v_xor per use
    return v;
  }
  __device__ __forceinline__ uint4 mask4(int q) const {
    return make_uint4(mask(4 * q), mask(4 * q + 1), mask(4 * q + 2), mask(4 * q + 3));
  }
};

// LdsSigns: the masks of one head already expanded in LDS (D/2 dwords,
// built lane-parallel by the streaming kernels); every lane reads the same
// address, so each ds_read_b128 is a broadcast.
struct LdsSigns {
  const uint32_t* row;
  __device__ __forceinline__ uint32_t mask(int m) const { return row[m]; }
  __device__ __forceinline__ uint4 mask4(int q) const { return *(const uint4*)(row + 4 * q); }
};

// Mask of elements 2m, 2m+1 from their two sign bytes (low 16 bits of u):
// bit 7 of each byte is set exactly for -1.
__device__ __forceinline__ uint32_t sign_mask_of(uint32_t u) {
  return ((u & 0x80u) << 8) | ((u & 0x8000u) << 16);
}

// ----------------------------------------------------------------------------
// Pass 1 from fp16: s (.) x, converted, and the pair sums of elements r and
// r + d/2:  p0[r] = x'_r + x'_{r+d/2},  p1[r] = x'_r - x'_{r+d/2}.
// Every rotation starts with exactly these (radix-2 split on the top index
// bit); the sign multiply is one XOR per packed pair and each sum one
// v_fma_mix_f32 from the packed halves.
// ----------------------------------------------------------------------------
template <int D, class S>
__device__ __forceinline__ void pair_sums(const uint32_t (&w)[D / 2], const S& sg,
                                          float (&p0)[D / 2], float (&p1)[D / 2]) {
  static_assert(D % 16 == 0, "pair_sums reads masks four at a time");
  // an opaque 1.0 keeps the sums as fma_mix (fp16 sources, fp32 result)
  float one = 1.0f;
  asm("" : "+s"(one));
  static_for<D / 16>([&](auto qq) {
    constexpr int q = decltype(qq)::value;
    const uint4 ma4 = sg.mask4(q), mb4 = sg.mask4(D / 16 + q);
    const uint32_t ma[4] = {ma4.x, ma4.y, ma4.z, ma4.w};
    const uint32_t mb[4] = {mb4.x, mb4.y, mb4.z, mb4.w};
    static_for<4>([&](auto ii) {
      constexpr int i = decltype(ii)::value;
      constexpr int m = 4 * q + i;
      const uint32_t wa = w[m] ^ ma[i];              // elements 2m, 2m+1
      const uint32_t wb = w[D / 4 + m] ^ mb[i];      // elements d/2+2m, d/2+2m+1
      p0[2 * m] = __builtin_fmaf(hlo(wb), one, hlo(wa));
      p1[2 * m] = __builtin_fmaf(hlo(wb), -one, hlo(wa));
      p0[2 * m + 1] = __builtin_fmaf(hhi(wb), one, hhi(wa));
      p1[2 * m + 1] = __builtin_fmaf(hhi(wb), -one, hhi(wa));
    });
  });
}

// ----------------------------------------------------------------------------
// VAR_REAL forward: halfcomplex combine of two length-L spectra E, O (of the
// even / odd subsequences) into the length-2L spectrum:
//   X_k = E_k + W^k O_k,  X_{L-k} = conj(E_k - W^k O_k),  W = e^{-i pi/L}.
// Six FMAs per k (the second output reuses the first: 2E - (E + WO)).
// ----------------------------------------------------------------------------
template <int L>
__device__ __forceinline__ void hc_combine(const float (&E)[L], const float (&O)[L], float (&X)[2 * L]) {
  X[0] = E[0] + O[0];
  X[L] = E[0] - O[0];
  if constexpr (L >= 2) {
    X[L / 2] = E[L / 2];
    X[2 * L - L / 2] = -O[L / 2];
  }
  static_for<(L >= 4 ? L / 2 - 1 : 0)>([&](auto kk) {
    constexpr int k = decltype(kk)::value + 1;
    constexpr float c = (float)ccos(kPi * k / L);
    constexpr float s = (float)csin(kPi * k / L);
    const float Er = E[k], Ei = E[L - k], Or = O[k], Oi = O[L - k];
    const float xr = __builtin_fmaf(s, Oi, __builtin_fmaf(c, Or, Er));
    const float xi = __builtin_fmaf(-s, Or, __builtin_fmaf(c, Oi, Ei));
    X[k] = xr;
    X[2 * L - k] = xi;
    X[L - k] = __builtin_fmaf(2.0f, Er, -xr);
    X[L + k] = __builtin_fmaf(-2.0f, Ei, xi);
  });
}

// Halfcomplex DFT of the subsequence x[OFF + m*S], m < L (L*S = D).
template <int L, int S, int OFF, int D>
__device__ __forceinline__ void rdft(const float (&p0)[D / 2], const float (&p1)[D / 2], float (&X)[L]) {
  if constexpr (L == 2) {
    X[0] = p0[OFF];
    X[1] = p1[OFF];
  } else {
    float E[L / 2], O[L / 2];
    rdft<L / 2, 2 * S, OFF, D>(p0, p1, E);
    rdft<L / 2, 2 * S, OFF + S, D>(p0, p1, O);
    hc_combine<L / 2>(E, O, X);
  }
}

// ----------------------------------------------------------------------------
// d = 3L (L a power of two): the halfcomplex spectrum X of length 3L from the
// spectra Y_r of the three subsequences x[3m + r] (decimation in time by 3):
//   X_{k + Ls} = sum_r W^{r(k + Ls)} Y_r,k = A + wb^s B + wb^{2s} C,
//   A = Y_0,k,  B = W^k Y_1,k,  C = W^{2k} Y_2,k,  W = e^{-2 pi i / 3L},
//   wb = e^{-2 pi i / 3};
// for 0 <= k <= L/2 this gives X_k, X_{k+L} and X_{k+2L} = conj X_{L-k}, which
// together cover bins 0 .. 3L/2.
// ----------------------------------------------------------------------------
template <int L>
__device__ __forceinline__ void hc_combine3(const float (&Y0)[L], const float (&Y1)[L], const float (&Y2)[L],
                                            float (&X)[3 * L]) {
  constexpr int D = 3 * L, N = D / 2;
  constexpr float h3 = (float)(0.86602540378443864676);   // sqrt(3) / 2
  static_for<L / 2 + 1>([&](auto kk) {
    constexpr int k = decltype(kk)::value;
    constexpr bool real = (k == 0 || k == L / 2);            // Y_r,k is real at DC and Nyquist
    constexpr float c1 = (float)ccos(2.0 * kPi * k / D), s1 = (float)csin(2.0 * kPi * k / D);
    constexpr float c2 = (float)ccos(4.0 * kPi * k / D), s2 = (float)csin(4.0 * kPi * k / D);
    const float ar = Y0[k], ai = real ? 0.0f : Y0[L - k];
    const float y1r = Y1[k], y1i = real ? 0.0f : Y1[L - k];
    const float y2r = Y2[k], y2i = real ? 0.0f : Y2[L - k];
    // B = (c1 - i s1) Y1,  C = (c2 - i s2) Y2
    const float br = __builtin_fmaf(c1, y1r, s1 * y1i), bi = __builtin_fmaf(c1, y1i, -s1 * y1r);
    const float cr = __builtin_fmaf(c2, y2r, s2 * y2i), ci = __builtin_fmaf(c2, y2i, -s2 * y2r);
    const float sr = br + cr, si = bi + ci;
    const float dr = br - cr, di = bi - ci;
    const float tr = __builtin_fmaf(-0.5f, sr, ar), ti = __builtin_fmaf(-0.5f, si, ai);
    // X_k = A + S
    X[k] = ar + sr;
    if constexpr (k > 0) X[D - k] = ai + si;
    // X_{k+L} = T - i h3 Dd
    X[k + L] = __builtin_fmaf(h3, di, tr);
    if constexpr (k + L < N) X[D - k - L] = __builtin_fmaf(-h3, dr, ti);
    // X_{k+2L} = T + i h3 Dd = conj X_{L-k}: skip the bins already written (k = 0, L/2)
    if constexpr (k > 0 && L - k != k) {
      X[L - k] = __builtin_fmaf(-h3, di, tr);
      X[D - L + k] = -__builtin_fmaf(h3, dr, ti);
    }
  });
}

// ----------------------------------------------------------------------------
// VAR_PAIRED forward: complex radix-2 DIT FFT of z_m = x'_2m + i x'_2m+1.
// Butterfly X_k = E_k + W O_k, X_{k+L/2} = E_k - W O_k in six FMAs.
// ----------------------------------------------------------------------------
template <int L, int S, int OFF, int D, bool INV>
__device__ __forceinline__ void cfft(const float (&p0)[D / 2], const float (&p1)[D / 2],
                                     float (&Xr)[L], float (&Xi)[L]);

template <int L, bool INV>
__device__ __forceinline__ void c_butterflies(const float (&Er)[L / 2], const float (&Ei)[L / 2],
                                              const float (&Or)[L / 2], const float (&Oi)[L / 2],
                                              float (&Xr)[L], float (&Xi)[L]) {
  static_for<L / 2>([&](auto kk) {
    constexpr int k = decltype(kk)::value;
    if constexpr (k == 0) {
      Xr[0] = Er[0] + Or[0];
      Xi[0] = Ei[0] + Oi[0];
      Xr[L / 2] = Er[0] - Or[0];
      Xi[L / 2] = Ei[0] - Oi[0];
    } else if constexpr (4 * k == L) {
      // W = -i (forward) or +i (inverse)
      const float wr = INV ? -Oi[k] : Oi[k];
      const float wi = INV ? Or[k] : -Or[k];
      Xr[k] = Er[k] + wr;
      Xi[k] = Ei[k] + wi;
      Xr[k + L / 2] = Er[k] - wr;
      Xi[k + L / 2] = Ei[k] - wi;
    } else {
      constexpr float c = (float)ccos(2.0 * kPi * k / L);
      constexpr float s = INV ? -(float)csin(2.0 * kPi * k / L) : (float)csin(2.0 * kPi * k / L);
      // W = c - i s:  W O = (c Or + s Oi) + i (c Oi - s Or)
      const float xr = __builtin_fmaf(s, Oi[k], __builtin_fmaf(c, Or[k], Er[k]));
      const float xi = __builtin_fmaf(-s, Or[k], __builtin_fmaf(c, Oi[k], Ei[k]));
      Xr[k] = xr;
      Xi[k] = xi;
      Xr[k + L / 2] = __builtin_fmaf(2.0f, Er[k], -xr);
      Xi[k + L / 2] = __builtin_fmaf(2.0f, Ei[k], -xi);
    }
  });
}

template <int L, int S, int OFF, int D, bool INV>
__device__ __forceinline__ void cfft(const float (&p0)[D / 2], const float (&p1)[D / 2],
                                     float (&Xr)[L], float (&Xi)[L]) {
  if constexpr (L == 2) {
    Xr[0] = p0[2 * OFF];
    Xi[0] = p0[2 * OFF + 1];
    Xr[1] = p1[2 * OFF];
    Xi[1] = p1[2 * OFF + 1];
  } else {
    float Er[L / 2], Ei[L / 2], Or[L / 2], Oi[L / 2];
    cfft<L / 2, 2 * S, OFF, D, INV>(p0, p1, Er, Ei);
    cfft<L / 2, 2 * S, OFF + S, D, INV>(p0, p1, Or, Oi);
    c_butterflies<L, INV>(Er, Ei, Or, Oi, Xr, Xi);
  }
}

// Hermitian unpack of Z (d/2-point spectrum of z) into the halfcomplex
// spectrum of x, bins 1..N-1 doubled (their scale absorbs the 1/2):
//   2E_k = Z_k + conj Z_{N-k},  2O_k = (Z_k - conj Z_{N-k}) / i,
//   2X_k = 2E_k + W_d^k 2O_k,  2X_{N-k} = conj(2E_k - W_d^k 2O_k).
template <int D>
__device__ __forceinline__ void hermitian_unpack(const float (&Zr)[D / 2], const float (&Zi)[D / 2],
                                                 float (&h)[D]) {
  constexpr int N = D / 2;
  h[0] = Zr[0] + Zi[0];
  h[N] = Zr[0] - Zi[0];
  h[N / 2] = 2.0f * Zr[N / 2];
  h[D - N / 2] = -2.0f * Zi[N / 2];
  static_for<N / 2 - 1>([&](auto kk) {
    constexpr int k = decltype(kk)::value + 1;
    constexpr float c = (float)ccos(2.0 * kPi * k / D);
    constexpr float s = (float)csin(2.0 * kPi * k / D);
    const float A = Zr[k] + Zr[N - k];
    const float B = Zi[k] - Zi[N - k];
    const float C = Zi[k] + Zi[N - k];
    const float Dm = Zr[N - k] - Zr[k];
    const float xr = __builtin_fmaf(s, Dm, __builtin_fmaf(c, C, A));
    const float xi = __builtin_fmaf(-s, C, __builtin_fmaf(c, Dm, B));
    h[k] = xr;
    h[D - k] = xi;
    h[N - k] = __builtin_fmaf(2.0f, A, -xr);
    h[N + k] = __builtin_fmaf(-2.0f, B, xi);
  });
}

// In-place natural-order (Sylvester) Walsh-Hadamard transform of the M
// values v[OFF .. OFF+M) (unnormalized), depth first:
// H_M [a; b] = [H a + H b; H a - H b], so each half is finished before the
// combining stage, which keeps few temporaries live at d = 256.
template <int M, int OFF = 0, int LEN>
__device__ __forceinline__ void wht(float (&v)[LEN]) {
  if constexpr (M > 1) {
    wht<M / 2, OFF>(v);
    wht<M / 2, OFF + M / 2>(v);
    static_for<M / 2>([&](auto ii) {
      constexpr int i = OFF + decltype(ii)::value;
      const float a = v[i], b = v[i + M / 2];
      v[i] = a + b;
      v[i + M / 2] = a - b;
    });
  }
}

// ----------------------------------------------------------------------------
// Forward rotation of one vector given as D/2 packed fp16 dwords.  Output y
// is in packed order and unscaled (multiply by Scales<>::kFwd*).
// ----------------------------------------------------------------------------
template <int D, int ROT, int VAR, class S>
__device__ __forceinline__ void forward(const uint32_t (&w)[D / 2], const S& sg, float (&y)[D]) {
  if constexpr (ROT == ROT_NONE) {
    static_for<D / 2>([&](auto mm) {
      constexpr int m = decltype(mm)::value;
      const uint32_t v = w[m] ^ sg.mask(m);
      y[2 * m] = hlo(v);
      y[2 * m + 1] = hhi(v);
    });
  } else {
    float p0[D / 2], p1[D / 2];
    pair_sums<D>(w, sg, p0, p1);
    if constexpr (ROT == ROT_SRHT) {
      wht<D / 2>(p0);
      wht<D / 2>(p1);
      static_for<D / 2>([&](auto kk) {
        constexpr int k = decltype(kk)::value;
        y[k] = p0[k];
        y[D / 2 + k] = p1[k];
      });
    } else {
      constexpr int N = D / 2;
      float h[D];
      if constexpr (VAR == VAR_PAIRED) {
        float Zr[N], Zi[N];
        cfft<N, 1, 0, D, false>(p0, p1, Zr, Zi);
        hermitian_unpack<D>(Zr, Zi, h);
      } else if constexpr (D % 3 == 0) {
        constexpr int L = D / 3;
        float Y0[L], Y1[L], Y2[L];
        rdft<L, 3, 0, D>(p0, p1, Y0);
        rdft<L, 3, 1, D>(p0, p1, Y1);
        rdft<L, 3, 2, D>(p0, p1, Y2);
        hc_combine3<L>(Y0, Y1, Y2, h);
      } else {
        rdft<D, 1, 0, D>(p0, p1, h);
      }
      static_for<N + 1>([&](auto jj) {
        constexpr int j = decltype(jj)::value;
        y[j] = h[j];
      });
      static_for<N - 1>([&](auto kk) {
        constexpr int k = decltype(kk)::value + 1;
        y[N + k] = h[D - k];
      });
    }
  }
}

// ----------------------------------------------------------------------------
// Inverse rotation.  Input: packed coordinates already multiplied by
// Scales<>::kInv* (and by the dequantization scale).  Output: x' = M^T y,
// natural order, before the sign multiply.
// ----------------------------------------------------------------------------

// Split a halfcomplex length-2M spectrum X (whose Nyquist entry X[M] carries a
// pending factor NYQ) into the spectra of its even / odd samples:
//   E_k = X_k + conj X_{M-k},  O_k = conj(W^k) (X_k - conj X_{M-k}),
//   W = e^{-i pi/M}.
// The Nyquist entries of E and O come out with pending factors 2 and -2.
template <int M, int NYQ>
__device__ __forceinline__ void hc_split(const float (&X)[2 * M], float (&E)[M], float (&O)[M]) {
  constexpr float f = (float)NYQ;
  E[0] = __builtin_fmaf(f, X[M], X[0]);
  O[0] = __builtin_fmaf(-f, X[M], X[0]);
  if constexpr (M >= 2) {
    E[M / 2] = X[M / 2];
    O[M / 2] = X[2 * M - M / 2];
  }
  static_for<(M >= 4 ? M / 2 - 1 : 0)>([&](auto kk) {
    constexpr int k = decltype(kk)::value + 1;
    constexpr float c = (float)ccos(kPi * k / M);
    constexpr float s = (float)csin(kPi * k / M);
    const float Pr = X[k], Pi = X[2 * M - k];
    const float Qr = X[M - k], Qi = -X[M + k];
    const float Er = Pr + Qr, Ei = Pi + Qi;
    const float Dr = Pr - Qr, Di = Pi - Qi;
    // conj(W) D = (c + i s)(Dr + i Di)
    E[k] = Er;
    E[M - k] = Ei;
    O[k] = __builtin_fmaf(c, Dr, -s * Di);
    O[M - k] = __builtin_fmaf(c, Di, s * Dr);
  });
}

// Inverse of rdft: the subsequence x[OFF + m*S] from its halfcomplex spectrum.
template <int L, int S, int OFF, int D, int NYQ>
__device__ __forceinline__ void irdft(const float (&X)[L], float (&x)[D]) {
  if constexpr (L == 2) {
    constexpr float f = (float)NYQ;
    x[OFF] = __builtin_fmaf(f, X[1], X[0]);
    x[OFF + S] = __builtin_fmaf(-f, X[1], X[0]);
  } else {
    float E[L / 2], O[L / 2];
    hc_split<L / 2, NYQ>(X, E, O);
    irdft<L / 2, 2 * S, OFF, D, 2>(E, x);
    irdft<L / 2, 2 * S, OFF + S, D, -2>(O, x);
  }
}

// Inverse complex DIT FFT (e^{+}) of Z[OFF + k*S], natural-order output.
template <int L, int S, int OFF, int NN>
__device__ __forceinline__ void icfft(const float (&Zr)[NN], const float (&Zi)[NN], float (&zr)[L], float (&zi)[L]) {
  if constexpr (L == 2) {
    zr[0] = Zr[OFF] + Zr[OFF + S];
    zi[0] = Zi[OFF] + Zi[OFF + S];
    zr[1] = Zr[OFF] - Zr[OFF + S];
    zi[1] = Zi[OFF] - Zi[OFF + S];
  } else {
    float Er[L / 2], Ei[L / 2], Or[L / 2], Oi[L / 2];
    icfft<L / 2, 2 * S, OFF, NN>(Zr, Zi, Er, Ei);
    icfft<L / 2, 2 * S, OFF + S, NN>(Zr, Zi, Or, Oi);
    c_butterflies<L, true>(Er, Ei, Or, Oi, zr, zi);
  }
}

// d = 3L: decimation in frequency by 3 of the real inverse
//   x_n = h_0 + (-1)^n h_{3L/2} + 2 sum_{0<k<3L/2} Re((h_k + i h_{3L-k}) e^{2 pi i k n / 3L}):
// with G the full Hermitian spectrum, x_{3m+r} is the length-L real inverse of
//   Z_r,k = W^{-kr} (G_k + w^r G_{k+L} + w^{2r} G_{k+2L}),  w = e^{2 pi i / 3},
// where G_{k+L} = H_{k+L} and G_{k+2L} = conj H_{L-k} for 0 <= k <= L/2.
template <int L>
__device__ __forceinline__ void hc_split3(const float (&h)[3 * L], float (&Z0)[L], float (&Z1)[L], float (&Z2)[L]) {
  constexpr int D = 3 * L, N = D / 2;
  constexpr float h3 = (float)(0.86602540378443864676);
  static_for<L / 2 + 1>([&](auto kk) {
    constexpr int k = decltype(kk)::value;
    constexpr float c1 = (float)ccos(2.0 * kPi * k / D), s1 = (float)csin(2.0 * kPi * k / D);
    constexpr float c2 = (float)ccos(4.0 * kPi * k / D), s2 = (float)csin(4.0 * kPi * k / D);
    const float gar = h[k], gai = (k == 0) ? 0.0f : h[D - k];
    const float gbr = h[k + L], gbi = (k + L == N) ? 0.0f : h[D - k - L];
    const float gcr = h[L - k], gci = (k == L) ? 0.0f : -h[D - L + k];   // conj H_{L-k}
    const float sr = gbr + gcr, si = gbi + gci;
    const float dr = gbr - gcr, di = gbi - gci;
    const float tr = __builtin_fmaf(-0.5f, sr, gar), ti = __builtin_fmaf(-0.5f, si, gai);
    // T1 = T + i h3 Dd, T2 = T - i h3 Dd
    const float t1r = __builtin_fmaf(-h3, di, tr), t1i = __builtin_fmaf(h3, dr, ti);
    const float t2r = __builtin_fmaf(h3, di, tr), t2i = __builtin_fmaf(-h3, dr, ti);
    // Z0 = G_a + S;  Z1 = (c1 + i s1) T1;  Z2 = (c2 + i s2) T2
    const float z0r = gar + sr, z0i = gai + si;
    const float z1r = __builtin_fmaf(c1, t1r, -s1 * t1i), z1i = __builtin_fmaf(c1, t1i, s1 * t1r);
    const float z2r = __builtin_fmaf(c2, t2r, -s2 * t2i), z2i = __builtin_fmaf(c2, t2i, s2 * t2r);
    Z0[k] = z0r;
    Z1[k] = z1r;
    Z2[k] = z2r;
    if constexpr (k > 0 && k < L / 2) {
      Z0[L - k] = z0i;
      Z1[L - k] = z1i;
      Z2[L - k] = z2i;
    }
  });
}

template <int D, int ROT, int VAR>
__device__ __forceinline__ void inverse(const float (&y)[D], float (&x)[D]) {
  constexpr int N = D / 2;
  if constexpr (ROT == ROT_NONE) {
    static_for<D>([&](auto jj) {
      constexpr int j = decltype(jj)::value;
      x[j] = y[j];
    });
  } else if constexpr (ROT == ROT_SRHT) {
    // in place in x: the two half-length transforms, then the top-bit stage
    static_for<D>([&](auto jj) {
      constexpr int j = decltype(jj)::value;
      x[j] = y[j];
    });
    wht<N, 0>(x);
    wht<N, N>(x);
    static_for<N>([&](auto rr) {
      constexpr int r = decltype(rr)::value;
      const float u = x[r], v = x[r + N];
      x[r] = u + v;
      x[r + N] = u - v;
    });
  } else if constexpr (VAR == VAR_PAIRED) {
    // Re-pair: Z_k = E_k + i O_k with 2E_k = X_k + conj X_{N-k},
    // 2O_k = (X_k - conj X_{N-k}) conj(W_d^k); then z = IDFT_N(Z).
    float Zr[N], Zi[N];
    Zr[0] = y[0] + y[N];
    Zi[0] = y[0] - y[N];
    Zr[N / 2] = 2.0f * y[N / 2];
    Zi[N / 2] = -2.0f * y[N + N / 2];
    static_for<N / 2 - 1>([&](auto kk) {
      constexpr int k = decltype(kk)::value + 1;
      constexpr float c = (float)ccos(2.0 * kPi * k / D);
      constexpr float s = (float)csin(2.0 * kPi * k / D);
      const float Pr = y[k], Pi = y[N + k];           // X_k
      const float Qr = y[N - k], Qi = -y[D - k];      // conj X_{N-k}
      const float Er = Pr + Qr, Ei = Pi + Qi;
      const float Dr = Pr - Qr, Di = Pi - Qi;
      const float Or = __builtin_fmaf(c, Dr, -s * Di);
      const float Oi = __builtin_fmaf(c, Di, s * Dr);
      Zr[k] = Er - Oi;
      Zi[k] = Ei + Or;
      Zr[N - k] = Er + Oi;
      Zi[N - k] = Or - Ei;
    });
    float zr[N], zi[N];
    icfft<N, 1, 0, N>(Zr, Zi, zr, zi);
    static_for<N>([&](auto mm) {
      constexpr int m = decltype(mm)::value;
      x[2 * m] = zr[m];
      x[2 * m + 1] = zi[m];
    });
  } else {
    float h[D];
    static_for<N + 1>([&](auto jj) {
      constexpr int j = decltype(jj)::value;
      h[j] = y[j];
    });
    static_for<N - 1>([&](auto kk) {
      constexpr int k = decltype(kk)::value + 1;
      h[D - k] = y[N + k];
    });
    if constexpr (D % 3 == 0) {
      constexpr int L = D / 3;
      float Z0[L], Z1[L], Z2[L];
      hc_split3<L>(h, Z0, Z1, Z2);
      irdft<L, 3, 0, D, 1>(Z0, x);
      irdft<L, 3, 1, D, 1>(Z1, x);
      irdft<L, 3, 2, D, 1>(Z2, x);
    } else {
      irdft<D, 1, 0, D, 1>(h, x);
    }
  }
}

}  // namespace srftq
