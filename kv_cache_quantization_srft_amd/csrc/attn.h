// attn.h -- decode attention that reads the quantized cache directly.
//
// For one new query token per tensor b and query head r of KV head h (R query
// heads share a KV head):
//   o_r = sum_{t < len_b} softmax_t(scale * q_r . k^_t) v^_t,
// where k^_t, v^_t are the exact reconstructions s (.) M^T y^ of the cached
// codes, y^_j = c_j sigma_G(j) / lambda_j (the dequantizer of the pages'
// int4 KV cache, "When Quantization Is Free", Metodologia 1-2, before any fp16
// rounding).  M is orthonormal, so q . k^ = (M (s_k . q)) . y^: the scores are
// taken in the rotated domain against the codes themselves, the output is
// accumulated there as well, and each query head is unrotated once at the end:
//   o_r = s_v (.) M^T ( sum_t p_t c^v_t sigma^v_t / lambda_v ).
//
// Kernels (one launch each):
//   attn_qprep_kernel    u_r = M (s_k . q_r) * scale * log2(e) / lambda_k,
//                        stored as 2^-e_r u_r with e_r putting max |u_r| in
//                        [2^10, 2^11) (so that its fp16 parts neither
//                        overflow nor go subnormal) plus the factor 2^e_r
//                        (one wave per query head).
//   attn_partial_kernel  one block of 4 waves per chunk of one (tensor, KV
//                        head) (the tensor's 16-token blocks split evenly
//                        over its chunks' waves); per 16-token block a wave
//                        computes the scores of 16 query heads (R used, the
//                        rest zero) with v_mfma_f32_16x16x16_f16 -- the codes
//                        are exact in fp16 (A), the query coordinates are
//                        split into fp16 hi + lo parts (B, two MFMAs) -- and
//                        scales each group's fp32 partial by its sigma; keeps
//                        an online softmax in base 2; accumulates P.V with a
//                        second MFMA whose A operand is fp16(c_v * sigma_v)
//                        and whose B operand is fp16(2^14 p) (p <= 1 after
//                        the running max, so the terms that matter stay
//                        normal fp16 numbers; the 2^14 cancels against the
//                        softmax sum, accumulated from the same values):
//                        two roundings to fp16 per term, the only steps
//                        beyond fp32 in the path.  The 4 waves merge through
//                        LDS and write one (max, sum, accumulator) per query
//                        head and chunk.
//   attn_combine_kernel  merges the chunks of one query head, divides by the
//                        softmax sum and lambda_v, unrotates and signs.
//
// Staging: every 16-token block's K codes (whole rows), V codes (transposed
// by dword: [dword][token], so that a lane's four tokens of one coordinate
// are one 16-byte LDS read) and both scale rows arrive by LDS-DMA into a
// ring of NS stages per wave, NS - 1 blocks ahead; rows past the tensor's length are
// never read (their lanes re-read the last valid row, whose finite values
// the softmax masks).
#pragma once

#include "kernels.h"
#include "launch.h"

namespace srftq {

// A rotation given as a matrix (learned or Householder, row-major fp32
// [d, d] per (tensor, KV head)): the query rotation and the unrotation are
// dense products; the scoring kernel is the same for every rotation.
enum : int { ROT_DENSE = 3 };

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Byte sizes of the per-wave staging and of the merge area of attn_partial_kernel.
template <int D, int G, int BITS>
struct AttnTile {
  static constexpr int RB = D * BITS / 8;       // code bytes per token
  static constexpr int NG = D / G;              // groups per token
  static constexpr int SRB = 2 * NG;            // scale bytes per token
  static constexpr int NB = D / 16;             // MFMA k-blocks per token
  static constexpr int CT = 16 * RB;            // code bytes of a 16-token block
  static constexpr int ST = 16 * SRB;           // scale bytes of a block
  static constexpr int KC_INST = (CT + 1023) / 1024;   // K codes: 16 B per lane
  static constexpr int KC_BYTES = 1024 * KC_INST;
  static constexpr int VC_INST = CT / 256;             // V codes: 4 B per lane, transposed
  // scale rows move in 4-byte pieces when a row is a whole number of dwords,
  // else in 2-byte pieces (d = 96, group 32: 6-byte rows)
  static constexpr int SE = SRB % 4 == 0 ? 4 : 2;
  // LDS-DMA fills a whole dword slot per lane: 2-byte pieces sit 4 bytes apart
  static constexpr int SSLOT = SE < 4 ? 4 : SE;
  static constexpr int S_INST = (ST + 64 * SE - 1) / (64 * SE);
  static constexpr int S_BYTES = 64 * SSLOT * S_INST;
  static constexpr int OFF_VC = KC_BYTES;
  static constexpr int OFF_KS = OFF_VC + CT;
  static constexpr int OFF_VS = OFF_KS + S_BYTES;
  static constexpr int STAGE = OFF_VS + S_BYTES;       // one buffer
  static constexpr int NDMA = KC_INST + VC_INST + 2 * S_INST;   // DMA instructions per block
  // blocks in flight per wave: enough bytes outstanding to cover HBM latency,
  // within the 6-bit vmcnt counter
  static constexpr int NS = 1 + 63 / NDMA < 4 ? 1 + 63 / NDMA : 4;
  static constexpr int WAVE_BYTES = NS * STAGE;
  static constexpr int MERGE_ACC = 4 * NB * 64 * 16;   // [wave][kb][lane] float4
  static constexpr int MERGE_BYTES = MERGE_ACC + 4 * 16 * 8;
  static constexpr int LDS_BYTES = 4 * WAVE_BYTES > MERGE_BYTES ? 4 * WAVE_BYTES : MERGE_BYTES;
  static_assert(G >= 16 && G % 16 == 0, "a group spans whole MFMA k-blocks");
  static_assert(CT % 256 == 0, "V codes move in 256-byte DMA instructions");
  static_assert(BITS != 4 || NB % 2 == 0, "int4 V codes unpack in blocks of 32 coordinates");
  static_assert(NS >= 2 && (NS - 1) * NDMA <= 63, "the blocks in flight fit the vmcnt counter");
};

__device__ __forceinline__ uint32_t lds_u32(uint32_t byte_addr) {
  return *(const __attribute__((address_space(3))) uint32_t*)(uintptr_t)byte_addr;
}
__device__ __forceinline__ u32x4_t lds_u32x4(uint32_t byte_addr) {
  return *(const __attribute__((address_space(3))) u32x4_t*)(uintptr_t)byte_addr;
}
__device__ __forceinline__ uint32_t lds_u16(uint32_t byte_addr) {
  return *(const __attribute__((address_space(3))) uint16_t*)(uintptr_t)byte_addr;
}
typedef const __attribute__((address_space(3))) uint32_t* lds_u32p;
typedef const __attribute__((address_space(3))) u32x4_t* lds_u32x4p;
__device__ __forceinline__ lds_u32p lds_ptr32(uint32_t byte_addr) { return (lds_u32p)(uintptr_t)byte_addr; }
__device__ __forceinline__ lds_u32x4p lds_ptr128(uint32_t byte_addr) { return (lds_u32x4p)(uintptr_t)byte_addr; }

// ((z ^ 0x00080008) & 0x000F000F) | 0x64006400: the nibbles at bits 0-3 and
// 16-19 of z, offset by 8 (two's complement -> 0..15), as the fp16 pair
// 1024 + n (one v_bitop3).
__device__ __forceinline__ uint32_t nib_f16x2(uint32_t z) {
  return ((z ^ 0x00080008u) & 0x000F000Fu) | 0x64006400u;
}
// ((z ^ 0x00800080) & 0x00F000F0) | 0x54005400: the nibbles at bits 4-7 and
// 20-23, offset by 8, as the fp16 pair 64 + n without a shift: they fill
// mantissa bits 4-7, where one unit is worth 2^(6-10+4) = 1 (one v_bitop3).
__device__ __forceinline__ uint32_t nib_hi_f16x2(uint32_t z) {
  return ((z ^ 0x00800080u) & 0x00F000F0u) | 0x54005400u;
}

// v (own) and v of lane l ^ 16 / l ^ 32, as the two halves of a
// v_permlane16_swap / v_permlane32_swap of (v, v): each lane keeps its own
// value in one result and receives its partner's in the other, so one VALU
// exchange (no LDS round trip) serves a butterfly reduction over 16 / 32.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(as_u32(v), as_u32(v), false, false);
  return __builtin_fmaxf(as_f32(r[0]), as_f32(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(as_u32(v), as_u32(v), false, false);
  return __builtin_fmaxf(as_f32(r[0]), as_f32(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(as_u32(v), as_u32(v), false, false);
  return as_f32(r[0]) + as_f32(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(as_u32(v), as_u32(v), false, false);
  return as_f32(r[0]) + as_f32(r[1]);
}

// Wait until at most k * N vector-memory operations are in flight, k < NS.
template <int N, int NS>
__device__ __forceinline__ void wait_blocks(int k) {
  static_for<NS>([&](auto kk) {
    constexpr int i = decltype(kk)::value;
    if (k == i) wait_vm<i * N>();
  });
}

// Two fp16 lanes holding 0x6400 | n (= 1024 + n), minus the bias: exact small
// integers.
__device__ __forceinline__ uint32_t f16x2_minus(uint32_t w, float bias) {
  half2_t h = __builtin_bit_cast(half2_t, w);
  h = h - (half2_t){(_Float16)bias, (_Float16)bias};
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ uint32_t f16x2_mul(uint32_t a, uint32_t b) {
  const half2_t h = __builtin_bit_cast(half2_t, a) * __builtin_bit_cast(half2_t, b);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ half4_t half4_of(uint32_t lo, uint32_t hi) {
  const uint2 v = make_uint2(lo, hi);
  return __builtin_bit_cast(half4_t, v);
}

// fp16 value of a scale: half `hi` of a dword.
__device__ __forceinline__ float f16_half(uint32_t w, int hi) { return hi ? hhi(w) : hlo(w); }

// Scale sigma of group g of row `row` in an LDS scale tile: rows of SRB
// bytes back to back when SRB is a multiple of 4, else moved in 2-byte
// pieces that sit in 4-byte slots (scale (row, g) is piece row SRB/2 + g).
template <int SRB>
__device__ __forceinline__ float tile_scale(uint32_t tile, int row, int g) {
  if constexpr (SRB % 4 == 0) {
    const uint32_t w = lds_u32(tile + (uint32_t)(row * SRB + 4 * (g >> 1)));
    return f16_half(w, g & 1);
  } else {
    return hlo(lds_u16(tile + (uint32_t)(2 * row * SRB + 4 * g)));
  }
}

// The fp16 scales of group g of rows `row` and `row + 1`, packed (low, high).
template <int SRB>
__device__ __forceinline__ uint32_t scale_pair(uint32_t tile, int row, int g) {
  if constexpr (SRB % 4 == 0) {
    const uint32_t w0 = lds_u32(tile + (uint32_t)(row * SRB + 4 * (g >> 1)));
    const uint32_t w1 = lds_u32(tile + (uint32_t)((row + 1) * SRB + 4 * (g >> 1)));
    return __builtin_amdgcn_perm(w1, w0, (g & 1) ? 0x07060302u : 0x05040100u);
  } else {
    return lds_u16(tile + (uint32_t)(2 * row * SRB + 4 * g)) |
           (lds_u16(tile + (uint32_t)(2 * (row + 1) * SRB + 4 * g)) << 16);
  }
}

// The same for group 2j + h (groups of 16, scale rows a whole number of
// dwords): half h of dword j of each row; h may differ between lanes.
template <int SRB>
__device__ __forceinline__ uint32_t scale_pair_g16(uint32_t tile, int row, int j, int h) {
  static_assert(SRB % 4 == 0, "scale rows of whole dwords");
  const uint32_t w0 = lds_u32(tile + (uint32_t)(row * SRB + 4 * j));
  const uint32_t w1 = lds_u32(tile + (uint32_t)((row + 1) * SRB + 4 * j));
  return __builtin_amdgcn_perm(w1, w0, h ? 0x07060302u : 0x05040100u);
}

// ----------------------------------------------------------------------------
// Transforms of single vectors spread over a wave (the query rotation and the
// output unrotation, one vector per query head): cooperative, so that their
// latency is a few hundred instructions rather than a whole transform on one
// lane.
// ----------------------------------------------------------------------------

// (cos, -sin)(2 pi m / D) for m in [0, D), interleaved: the DFT kernel
// exp(-2 pi i m / D) rounded to fp32 from the compile-time series.
template <int D>
struct DftTwiddles {
  float v[2 * D];
  constexpr DftTwiddles() : v{} {
    for (int m = 0; m < D; ++m) {
      const int mm = 2 * m <= D ? m : m - D;   // angle in (-pi, pi]
      const double ang = 2.0 * kPi * mm / D;
      v[2 * m] = (float)ccos(ang);
      v[2 * m + 1] = -(float)csin(ang);
    }
  }
};
template <int D>
__device__ __forceinline__ const float* dft_twiddles() {
  static constexpr DftTwiddles<D> kTab{};
  return kTab.v;
}

// Query head of this block for the per-query-head kernels, launched on
// xcd_grid(n) blocks: the chip deals consecutive blocks to its 8 XCDs in
// turn, so block i takes head (i mod 8) ceil(n / 8) + i / 8 and each XCD
// (its own L2) gets a contiguous range of heads -- the R heads of a KV head
// read that head's matrix through one L2 instead of eight.  -1: no head.
__device__ __forceinline__ int64_t xcd_head(int64_t n) {
  const int64_t per = (n + 7) / 8;
  const int64_t v = (int64_t)(blockIdx.x % 8u) * per + blockIdx.x / 8u;
  return v < n ? v : -1;
}
inline unsigned xcd_grid(int64_t n) { return (unsigned)(8 * ((n + 7) / 8)); }

// Orthonormal scale of rotated coordinate j: the transforms run unscaled,
// a matrix is orthonormal as given.
template <int D, int ROT>
__device__ __forceinline__ float coord_scale(int j) {
  if constexpr (ROT == ROT_DENSE) {
    return 1.0f;
  } else {
    using Sc = Scales<D, ROT, VAR_REAL>;
    return (float)(Sc::is_edge(j) ? Sc::kFwdEdge : Sc::kFwdBulk);
  }
}

// i mod D for 0 <= i < 2D
template <int D>
__device__ __forceinline__ int wrap(int i) {
  if constexpr ((D & (D - 1)) == 0)
    return i & (D - 1);
  else
    return i >= D ? i - D : i;
}

__device__ __forceinline__ float wave_sum(float v) {
  static_for<6>([&](auto ii) { v += __shfl_xor(v, 1 << decltype(ii)::value); });
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  static_for<6>([&](auto ii) { v = __builtin_fmaxf(v, __shfl_xor(v, 1 << decltype(ii)::value)); });
  return v;
}

// A d-vector spread over one wave: lane l holds elements P l .. P l + P - 1
// (d = 64: lanes 0..31 hold two each, the rest none).
template <int D>
struct WaveVec {
  static constexpr int P = D >= 128 ? D / 64 : 2;
  static constexpr int NL = D / P;   // lanes holding elements
};

// Unnormalized Walsh-Hadamard transform in natural (Sylvester) order,
// y_j = sum_m (-1)^popcount(j & m) x_m, of a vector laid out as in WaveVec:
// butterflies over the in-lane index bits, then over the lane bits through
// lane exchanges.
template <int D>
__device__ __forceinline__ void wave_fwht(float (&x)[WaveVec<D>::P], int lane) {
  constexpr int P = WaveVec<D>::P, NL = WaveVec<D>::NL;
  static_for<P>([&](auto hh) {
    constexpr int h = decltype(hh)::value;
    static_for<P>([&](auto tt) {
      constexpr int t = decltype(tt)::value;
      if constexpr ((h & (h - 1)) == 0 && h > 0 && (t & h) == 0 && t + h < P) {
        const float a = x[t], b = x[t + h];
        x[t] = a + b;
        x[t + h] = a - b;
      }
    });
  });
  static_for<6>([&](auto bb) {
    constexpr int msk = 1 << decltype(bb)::value;
    if constexpr (msk < NL) {
      static_for<P>([&](auto tt) {
        constexpr int t = decltype(tt)::value;
        const float o = __shfl_xor(x[t], msk);
        x[t] = (lane & msk) ? o - x[t] : x[t] + o;
      });
    }
  });
}

// ----------------------------------------------------------------------------
// u = M (s_k . q) * scale * log2(e) / lambda_k for one query head per block
// of four waves, v = b*H*R + h*R + r (KV head bh = v / R).  SRFT: lane k
// accumulates the DFT bin X_k = sum_m x_m exp(-2 pi i k m / d) from the LDS
// copy of x and the twiddle table (two bins per lane at d = 256), each wave
// over a quarter of m, and the bin X_{d/2} is the alternating sum of x; the
// packed coordinates are Re X_0..Re X_{d/2}, Im X_1..Im X_{d/2-1} with the
// orthonormal scales.  Matrix: lane j forms rows j, j + 64, ... of Q with x,
// each wave over a quarter of the columns.  Wave 0 adds the quarters and
// finishes; SRHT and no rotation run on wave 0 alone (wave_fwht).
// ----------------------------------------------------------------------------
template <int D, int ROT>
__global__ __launch_bounds__(256) void attn_qprep_kernel(const uint16_t* __restrict__ q,
                                                         const int8_t* __restrict__ signs_k,
                                                         const float* __restrict__ lam_k,
                                                         const float* __restrict__ Qk, int64_t q_stride,
                                                         float* __restrict__ uq,
                                                         float* __restrict__ uexp, AttnGeo a) {
  constexpr int P = WaveVec<D>::P, NL = WaveVec<D>::NL;
  constexpr int N = D / 2;
  constexpr int KPL = N >= 64 ? N / 64 : 1;                   // SRFT bins per lane
  constexpr int NO = ROT == ROT_SRFT    ? 2 * KPL              // outputs per lane
                   : ROT == ROT_DENSE ? (D + 63) / 64          // matrix rows lane + 64 o
                                      : P;
  constexpr int MQ = D / 4;                                    // sum terms per wave (SRFT, matrix)
  constexpr bool kSplit = ROT == ROT_SRFT || ROT == ROT_DENSE;
  __shared__ __attribute__((aligned(16))) float xs[kSplit ? D : 4];
  __shared__ __attribute__((aligned(16))) float tw[ROT == ROT_SRFT ? 2 * D : 4];
  __shared__ __attribute__((aligned(16))) float red[ROT == ROT_SRFT ? 4 * NO * 64 : 4];   // [wave][o][lane]
  __shared__ float usum[ROT == ROT_DENSE ? D : 1];                                 // matrix rows' sums
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t v = xcd_head((int64_t)a.BH * a.R);
  if (v < 0) return;
  const int64_t bh = v / a.R;

  // wave 0: x = s_k (.) q, elements P lane .. P lane + P - 1
  float x[P];
  static_for<P>([&](auto tt) { x[decltype(tt)::value] = 0.0f; });
  if (wave == 0 && lane < NL) {
    const uint16_t* src = q + v * D + P * lane;
    if constexpr (P == 2) {
      const uint32_t w = *(const uint32_t*)src;
      x[0] = hlo(w), x[1] = hhi(w);
    } else {
      static_for<P / 4>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
        const uint2 w = *(const uint2*)(src + 4 * i);
        x[4 * i] = hlo(w.x), x[4 * i + 1] = hhi(w.x), x[4 * i + 2] = hlo(w.y), x[4 * i + 3] = hhi(w.y);
      });
    }
    const int8_t* sg = signs_k + bh * a.sign_stride_k + P * lane;
    static_for<P>([&](auto tt) {
      constexpr int t = decltype(tt)::value;
      if (sg[t] < 0) x[t] = -x[t];
    });
  }

  int jo[NO];   // coordinate of each output of a wave-0 lane, -1 where it has none
  static_for<NO>([&](auto oo) {
    constexpr int o = decltype(oo)::value;
    if constexpr (ROT == ROT_SRFT) {
      const int k = lane + 64 * (o / 2);
      jo[o] = k >= N ? -1 : (o & 1) ? (k == 0 ? N : N + k) : k;
    } else if constexpr (ROT == ROT_DENSE) {
      jo[o] = lane + 64 * o < D ? lane + 64 * o : -1;
    } else {
      jo[o] = lane < NL ? P * lane + o : -1;
    }
  });
  // 1 / lambda_k of the outputs, loaded before the transform
  float rl[NO];
  static_for<NO>([&](auto oo) {
    constexpr int o = decltype(oo)::value;
    rl[o] = (wave == 0 && lam_k && jo[o] >= 0) ? __builtin_amdgcn_rcpf(lam_k[bh * D + jo[o]]) : 1.0f;
  });

  float y[NO];
  static_for<NO>([&](auto oo) { y[decltype(oo)::value] = 0.0f; });
  if constexpr (kSplit) {
    // the four waves split the sum over m into quarters; wave 0 adds them up
    if (wave == 0 && lane < NL) static_for<P>([&](auto tt) { xs[P * lane + decltype(tt)::value] = x[decltype(tt)::value]; });
    if constexpr (ROT == ROT_SRFT) {
      const float* twg = dft_twiddles<D>();
      for (int i = (int)threadIdx.x; i < 2 * D; i += 256) tw[i] = twg[i];
    }
    __syncthreads();
    const int m0 = wave * MQ;
    float part[NO];   // SRFT: this wave's quarter of each bin
    if constexpr (ROT == ROT_SRFT) {
      static_for<KPL>([&](auto kk) {
        constexpr int i = decltype(kk)::value;
        const int k = lane + 64 * i;
        float re[4] = {0.f, 0.f, 0.f, 0.f}, im[4] = {0.f, 0.f, 0.f, 0.f};
        if (k < N) {
          int idx = (k * m0) % D;   // k m mod d
#pragma unroll 4
          for (int m = m0; m < m0 + MQ; m += 4) {
            const float4 xv = *(const float4*)&xs[m];
            const float xe[4] = {xv.x, xv.y, xv.z, xv.w};
            static_for<4>([&](auto ee) {
              constexpr int e = decltype(ee)::value;
              const float2 w = *(const float2*)&tw[2 * idx];
              re[e] = __builtin_fmaf(xe[e], w.x, re[e]);
              im[e] = __builtin_fmaf(xe[e], w.y, im[e]);
              idx = wrap<D>(idx + k);
            });
          }
        }
        part[2 * i] = (re[0] + re[1]) + (re[2] + re[3]);
        part[2 * i + 1] = (im[0] + im[1]) + (im[2] + im[3]);
      });
    } else {
      // u_j = sum_m Q[j][m] x_m.  Wave w takes rows [w d/4, (w + 1) d/4).  A
      // load instruction covers RPI whole rows, LPR lanes of 16 bytes each
      // (1 KiB contiguous), so each lane holds one 4-column partial per
      // instruction; a transposing butterfly over the LPR lanes of a row
      // (halving the values at each step) leaves row i of the wave's rows on
      // lanes lr = i SPL .. i SPL + SPL - 1 of each group.
      constexpr int LPR = D / 4, RPI = 64 / LPR, NI = D * D / 1024, SPL = LPR / NI;
      constexpr int BATCH = NI < 16 ? NI : 16;
      const int lr = lane % LPR, grp = lane / LPR;
      const float4 xv = *(const float4*)&xs[4 * lr];
      const float4* src = (const float4*)(Qk + bh * q_stride) + (int64_t)wave * (D / 4) * LPR + lane;
      float pv[NI];
      static_for<NI / BATCH>([&](auto bb) {
        constexpr int b0 = decltype(bb)::value * BATCH;
        float4 w[BATCH];
        static_for<BATCH>([&](auto ii) { w[decltype(ii)::value] = src[(b0 + decltype(ii)::value) * 64]; });
        static_for<BATCH>([&](auto ii) {
          constexpr int i = decltype(ii)::value;
          pv[b0 + i] = __builtin_fmaf(w[i].x, xv.x, w[i].y * xv.y) + __builtin_fmaf(w[i].z, xv.z, w[i].w * xv.w);
        });
      });
      static_for<6>([&](auto ss) {
        constexpr int st = decltype(ss)::value;
        constexpr int half = NI >> (st + 1), mask = LPR >> (st + 1);
        if constexpr (half >= 1) {
          const bool up = (lane & mask) != 0;
          static_for<half>([&](auto kk) {
            constexpr int k = decltype(kk)::value;
            const float send = up ? pv[k] : pv[k + half];
            const float keep = up ? pv[k + half] : pv[k];
            pv[k] = keep + __shfl_xor(send, mask);
          });
        }
      });
      static_for<6>([&](auto ss) {
        constexpr int mask = SPL >> (decltype(ss)::value + 1);
        if constexpr (mask >= 1) pv[0] += __shfl_xor(pv[0], mask);
      });
      if (lr % SPL == 0) usum[wave * (D / 4) + (lr / SPL) * RPI + grp] = pv[0];
    }
    if constexpr (ROT == ROT_SRFT) {
      static_for<NO>([&](auto oo) {
        constexpr int o = decltype(oo)::value;
        red[(wave * NO + o) * 64 + lane] = part[o];
      });
    }
    __syncthreads();
    if (wave != 0) return;
    static_for<NO>([&](auto oo) {
      constexpr int o = decltype(oo)::value;
      if constexpr (ROT == ROT_DENSE)
        y[o] = jo[o] >= 0 ? usum[jo[o]] : 0.0f;
      else
        y[o] = (red[o * 64 + lane] + red[(NO + o) * 64 + lane]) +
               (red[(2 * NO + o) * 64 + lane] + red[(3 * NO + o) * 64 + lane]);
    });
    if constexpr (ROT == ROT_SRFT) {
      // X_{d/2} = sum_m (-1)^m x_m (P is even: element P l + t has the sign of t)
      float alt = 0.0f;
      static_for<P>([&](auto tt) {
        constexpr int t = decltype(tt)::value;
        alt += (t & 1) ? -x[t] : x[t];
      });
      alt = wave_sum(alt);
      if (lane == 0) y[1] = alt;   // bin 0 has no imaginary part: its slot holds X_{d/2}
    }
  } else {
    if (wave != 0) return;
    if constexpr (ROT == ROT_SRHT) wave_fwht<D>(x, lane);
    static_for<P>([&](auto tt) { y[decltype(tt)::value] = x[decltype(tt)::value]; });
  }

  // wave 0: scales, the power-of-two normalization, the stores
  float mx = 0.0f;
  static_for<NO>([&](auto oo) {
    constexpr int o = decltype(oo)::value;
    const int j = jo[o];
    if (j >= 0) {
      float u = y[o] * coord_scale<D, ROT>(j) * a.scale_log2e;
      if (lam_k) u = u * rl[o];
      y[o] = u;
      mx = __builtin_fmaxf(mx, __builtin_fabsf(u));
    }
  });
  mx = wave_max(mx);
  // power of two 2^e with max |u| / 2^e in [2^10, 2^11) (e = 0 for u = 0)
  const int e = mx > 0.0f ? __builtin_amdgcn_frexp_expf(mx) - 11 : 0;
  const float down = __builtin_ldexpf(1.0f, -e);
  static_for<NO>([&](auto oo) {
    constexpr int o = decltype(oo)::value;
    if (jo[o] >= 0) uq[v * D + jo[o]] = y[o] * down;
  });
  if (lane == 0) uexp[v] = __builtin_ldexpf(1.0f, e);
}

// ----------------------------------------------------------------------------
// Partial attention of one chunk of one (tensor, KV head).
// Lane roles in a wave: jl = lane & 15, q = lane >> 4.
//   score MFMA  D[token][head]:  A = K codes, lane holds token jl, coordinates
//               16kb + 4q + {0,2,1,3} (int4) or {0,1,2,3} (int8); B = u, lane
//               holds head jl at the same coordinates; D: tokens 4q+e, head jl.
//   P.V MFMA    D[coord][head]:  A = V codes of tokens 4q+e, lane holds
//               coordinate 16kb + jl (int8) or, per block j of 32
//               coordinates, 32j + 2jl in acc[2j] and 32j + 2jl + 1 in
//               acc[2j + 1] (int4: both nibbles of byte jl); B = fp16(p *
//               sigma_v), tokens 4q+e, head jl (the score layout); D: those
//               coordinates of rows 4q + e, head jl.
// ----------------------------------------------------------------------------
template <int D, int G, int BITS>
__global__ __launch_bounds__(256) void attn_partial_kernel(const uint8_t* __restrict__ codes_k,
                                                           const uint16_t* __restrict__ scales_k,
                                                           const uint8_t* __restrict__ codes_v,
                                                           const uint16_t* __restrict__ scales_v,
                                                           const int32_t* __restrict__ lengths,
                                                           const float* __restrict__ uq,
                                                           const float* __restrict__ uexp,
                                                           float* __restrict__ ws_ml,
                                                           float* __restrict__ ws_acc, AttnGeo a) {
  using Tl = AttnTile<D, G, BITS>;
  constexpr int RB = Tl::RB, SRB = Tl::SRB, NB = Tl::NB, CT = Tl::CT;
  constexpr int KB_PER_G = G / 16;
  constexpr float kBias = BITS == 4 ? 1032.0f : 1152.0f;   // 1024 + offset of the code
  constexpr float kPScale = 14.0f;                          // B = fp16(2^14 p)
  __shared__ __attribute__((aligned(16))) uint8_t smem[Tl::LDS_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int c = (int)(blockIdx.x % (unsigned)a.n_chunks);
  const int bh = (int)(blockIdx.x / (unsigned)a.n_chunks);
  const int b = bh / a.H;
  const int jl = lane & 15, q = lane >> 4;

  int64_t len = a.T;
  if (lengths) {
    const int64_t lb = lengths[b];
    len = lb < 0 ? 0 : (lb < a.T ? lb : a.T);
  }
  // this tensor's 16-token blocks split evenly over the 4 * n_chunks waves of
  // (tensor, KV head): wave w takes blocks [w nb / nw, (w + 1) nb / nw)
  const int64_t nb16 = (len + 15) / 16, nw = 4 * (int64_t)a.n_chunks, w = (int64_t)c * 4 + wave;
  const int64_t t_begin = 16 * (w * nb16 / nw);
  int64_t t_end = 16 * ((w + 1) * nb16 / nw);
  t_end = t_end < len ? t_end : len;
  const int nblk = t_end > t_begin ? (int)((t_end - t_begin + 15) / 16) : 0;

  const int64_t row0 = (int64_t)bh * a.pitch;
  const uint8_t* kc = codes_k + row0 * RB;
  const uint8_t* vc = codes_v + row0 * RB;
  const uint8_t* ks = (const uint8_t*)scales_k + row0 * SRB;
  const uint8_t* vs = (const uint8_t*)scales_v + row0 * SRB;
  const uint32_t lds_wave = lds_addr(smem) + (uint32_t)wave * Tl::WAVE_BYTES;

  // B operands of the scores: u of head jl, hi and lo fp16 parts.
  half4_t bhi[NB], blo[NB];
  const float uscale = uexp[(int64_t)bh * a.R + (jl < a.R ? jl : 0)];
  {
    const bool live = jl < a.R;
    const float* u = uq + ((int64_t)bh * a.R + (live ? jl : 0)) * D;
    static_for<NB>([&](auto kk) {
      constexpr int kb = decltype(kk)::value;
      float4 v = *(const float4*)(u + 16 * kb + 4 * q);
      if (!live) v = make_float4(0.f, 0.f, 0.f, 0.f);
      const float e[4] = {v.x, BITS == 4 ? v.z : v.y, BITS == 4 ? v.y : v.z, v.w};
      static_for<4>([&](auto ee) {
        constexpr int i = decltype(ee)::value;
        const _Float16 h = (_Float16)e[i];
        bhi[kb][i] = h;
        blo[kb][i] = (_Float16)(e[i] - (float)h);
      });
    });
  }

  auto issue = [&](int blk, int buf) {
    const int64_t t0 = t_begin + 16 * (int64_t)blk;
    const int64_t left = t_end - t0;
    const int nv = left < 16 ? (int)left : 16;
    const uint32_t base = lds_wave + (uint32_t)buf * Tl::STAGE;
    const uint8_t* kcb = kc + t0 * RB;
    const uint8_t* vcb = vc + t0 * RB;
    const uint8_t* ksb = ks + t0 * SRB;
    const uint8_t* vsb = vs + t0 * SRB;
    // K codes, whole rows; offsets past the valid rows re-read the last valid chunk
    const uint32_t klim = (uint32_t)(nv * RB - 16);
    static_for<Tl::KC_INST>([&](auto ii) {
      constexpr int i = decltype(ii)::value;
      uint32_t off = (uint32_t)(1024 * i + 16 * lane);
      off = off < klim ? off : klim;
      dma_to_lds<16, true>(kcb, off, base + 1024 * i);
    });
    // V codes transposed: LDS dword 64i + lane holds dword w = 4i + lane/16 of row lane%16
    const int rr = (lane & 15) < nv ? (lane & 15) : nv - 1;
    static_for<Tl::VC_INST>([&](auto ii) {
      constexpr int i = decltype(ii)::value;
      const uint32_t off = (uint32_t)(rr * RB + 4 * (4 * i + (lane >> 4)));
      dma_to_lds<4>(vcb, off, base + Tl::OFF_VC + 256 * i);
    });
    // scale rows
    const uint32_t slim = (uint32_t)(nv * SRB - Tl::SE);
    static_for<Tl::S_INST>([&](auto ii) {
      constexpr int i = decltype(ii)::value;
      uint32_t off = (uint32_t)(64 * Tl::SE * i + Tl::SE * lane);
      off = off < slim ? off : slim;
      dma_to_lds<Tl::SE>(ksb, off, base + Tl::OFF_KS + 64 * Tl::SSLOT * i);
      dma_to_lds<Tl::SE>(vsb, off, base + Tl::OFF_VS + 64 * Tl::SSLOT * i);
    });
  };

  float4_t acc[NB];
  static_for<NB>([&](auto kk) { acc[decltype(kk)::value] = (float4_t){0.f, 0.f, 0.f, 0.f}; });
  float m_run = -__builtin_inff();
  float l_part = 0.0f;

  // per-lane constant selectors
  const uint32_t ksel = (q & 1) ? 0x0C030C02u : 0x0C010C00u;            // K int4: half q&1 of the dword
  // V: byte jl & 3 of a dword (int4: byte jl of a 32-coordinate block,
  // both of its nibbles; int8: the coordinate's byte)
  const uint32_t vsel = 0x0C000C00u | (uint32_t)(jl & 3) | ((4u + (uint32_t)(jl & 3)) << 16);

  constexpr int NS = Tl::NS;
  for (int i = 0; i < NS - 1 && i < nblk; ++i) issue(i, i);
  for (int blk = 0; blk < nblk; ++blk) {
    const int cur = blk % NS;
    wait_lgkm0();   // the stage about to be refilled has been read
    wave_fence();
    const int nxt = blk + NS - 1;
    if (nxt < nblk) issue(nxt, nxt % NS);
    const int rest = nblk - 1 - blk;
    wait_blocks<Tl::NDMA, NS>(rest < NS - 1 ? rest : NS - 1);   // this block has landed
    wave_fence();
    const uint32_t base = lds_wave + (uint32_t)cur * Tl::STAGE;
    const int64_t t0 = t_begin + 16 * (int64_t)blk;
    const int nv = (t_end - t0) < 16 ? (int)(t_end - t0) : 16;

    // ---- scores: S[e] = sum_G sigma_k(4q+e, G) * sum_{k in G} c_k u_k ----
    float S[4] = {0.f, 0.f, 0.f, 0.f};
    float4_t dg = (float4_t){0.f, 0.f, 0.f, 0.f};
    // this lane's K code dwords: row jl, dword 2kb + q/2 (int4) or 4kb + q (int8)
    const lds_u32p krow = lds_ptr32(base + (uint32_t)(jl * RB + 4 * (BITS == 4 ? (q >> 1) : q)));
    static_for<NB>([&](auto kk) {
      constexpr int kb = decltype(kk)::value;
      half4_t A;
      if constexpr (BITS == 4) {
        const uint32_t z = __builtin_amdgcn_perm(0u, krow[2 * kb], ksel);
        const uint32_t a0 = f16x2_minus(nib_f16x2(z), kBias);
        const uint32_t a1 = f16x2_minus(nib_hi_f16x2(z), 72.0f);   // 64 + offset of the code
        A = half4_of(a0, a1);
      } else {
        const uint32_t x = krow[4 * kb];
        const uint32_t a0 = f16x2_minus(__builtin_amdgcn_perm(0u, x, 0x0C010C00u) ^ 0x64806480u, kBias);
        const uint32_t a1 = f16x2_minus(__builtin_amdgcn_perm(0u, x, 0x0C030C02u) ^ 0x64806480u, kBias);
        A = half4_of(a0, a1);
      }
      if constexpr (kb % KB_PER_G == 0)
        dg = __builtin_amdgcn_mfma_f32_16x16x16f16(A, bhi[kb], (float4_t){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      else
        dg = __builtin_amdgcn_mfma_f32_16x16x16f16(A, bhi[kb], dg, 0, 0, 0);
      dg = __builtin_amdgcn_mfma_f32_16x16x16f16(A, blo[kb], dg, 0, 0, 0);
      if constexpr (kb % KB_PER_G == KB_PER_G - 1) {
        constexpr int g = kb / KB_PER_G;
        static_for<4>([&](auto ee) {
          constexpr int e = decltype(ee)::value;
          S[e] += tile_scale<SRB>(base + Tl::OFF_KS, 4 * q + e, g) * dg[e];
        });
      }
    });

    // ---- online softmax (base 2) over the block's valid tokens ----
    static_for<4>([&](auto ee) {
      constexpr int e = decltype(ee)::value;
      S[e] = 4 * q + e < nv ? S[e] * uscale : -__builtin_inff();
    });
    float mx = __builtin_fmaxf(__builtin_fmaxf(S[0], S[1]), __builtin_fmaxf(S[2], S[3]));
    mx = max_xor32(max_xor16(mx));   // over the block's 16 tokens (lanes 16 apart)
    if (__builtin_amdgcn_ballot_w64(mx > m_run)) {
      const float m_new = __builtin_fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_part *= alpha;
      static_for<NB>([&](auto kk) {
        constexpr int kb = decltype(kk)::value;
        acc[kb] *= alpha;
      });
      m_run = m_new;
    }
    float p[4];   // 2^14 * softmax numerator, <= 2^14
    static_for<4>([&](auto ee) {
      constexpr int e = decltype(ee)::value;
      p[e] = __builtin_amdgcn_exp2f(S[e] - (m_run - kPScale));
    });
    l_part += (p[0] + p[1]) + (p[2] + p[3]);

    // ---- P.V: acc[coord][head] += sum_t fp16(c_v(t, coord) sigma_v(t, G)) fp16(2^14 p_t) ----
    const half4_t Bv = half4_of(pack_f16x2(p[0], p[1]), pack_f16x2(p[2], p[3]));
    if constexpr (BITS == 4) {
      // Block j of 32 coordinates: lane jl takes byte jl of each token's 16
      // code bytes, i.e. coordinates 32j + 2jl (low nibble, into acc[2j]) and
      // 32j + 2jl + 1 (high nibble, into acc[2j + 1]), so both nibbles unpack
      // without a shift.  Transposed V tile: dword w of tokens 4q..4q+3 at
      // 16-byte index 4w + q; the lane's byte sits in dword 4j + jl/4.
      const lds_u32x4p vcol = lds_ptr128(base + Tl::OFF_VC) + (uint32_t)(4 * (jl >> 2) + q);
      uint32_t sv01 = 0, sv23 = 0;   // sigma_v of the lane's tokens (4q, 4q+1), (4q+2, 4q+3)
      static_for<NB / 2>([&](auto jj) {
        constexpr int j = decltype(jj)::value;
        if constexpr (G == 16) {
          // the lane's group 2j + jl/8: its pair of scales is dword j of the
          // row, half jl/8
          sv01 = scale_pair_g16<SRB>(base + Tl::OFF_VS, 4 * q, j, jl >> 3);
          sv23 = scale_pair_g16<SRB>(base + Tl::OFF_VS, 4 * q + 2, j, jl >> 3);
        } else if constexpr ((32 * j) % G == 0) {
          constexpr int g = 32 * j / G;
          sv01 = scale_pair<SRB>(base + Tl::OFF_VS, 4 * q, g);
          sv23 = scale_pair<SRB>(base + Tl::OFF_VS, 4 * q + 2, g);
        }
        const u32x4_t x = vcol[16 * j];
        const uint32_t z01 = __builtin_amdgcn_perm(x.y, x.x, vsel);
        const uint32_t z23 = __builtin_amdgcn_perm(x.w, x.z, vsel);
        const uint32_t e0 = f16x2_mul(f16x2_minus(nib_f16x2(z01), kBias), sv01);
        const uint32_t e1 = f16x2_mul(f16x2_minus(nib_f16x2(z23), kBias), sv23);
        const uint32_t o0 = f16x2_mul(f16x2_minus(nib_hi_f16x2(z01), 72.0f), sv01);
        const uint32_t o1 = f16x2_mul(f16x2_minus(nib_hi_f16x2(z23), 72.0f), sv23);
        acc[2 * j] = __builtin_amdgcn_mfma_f32_16x16x16f16(half4_of(e0, e1), Bv, acc[2 * j], 0, 0, 0);
        acc[2 * j + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(half4_of(o0, o1), Bv, acc[2 * j + 1], 0, 0, 0);
      });
    } else {
      // lane jl takes coordinate 16kb + jl, the byte jl & 3 of dword 4kb + jl/4
      const lds_u32x4p vcol = lds_ptr128(base + Tl::OFF_VC) + (uint32_t)(4 * (jl >> 2) + q);
      uint32_t sv01 = 0, sv23 = 0;
      static_for<NB>([&](auto kk) {
        constexpr int kb = decltype(kk)::value;
        if constexpr (kb % KB_PER_G == 0) {
          constexpr int g = kb / KB_PER_G;
          sv01 = scale_pair<SRB>(base + Tl::OFF_VS, 4 * q, g);
          sv23 = scale_pair<SRB>(base + Tl::OFF_VS, 4 * q + 2, g);
        }
        const u32x4_t x = vcol[16 * kb];
        uint32_t a0 = f16x2_minus(__builtin_amdgcn_perm(x.y, x.x, vsel) ^ 0x64806480u, kBias);
        uint32_t a1 = f16x2_minus(__builtin_amdgcn_perm(x.w, x.z, vsel) ^ 0x64806480u, kBias);
        a0 = f16x2_mul(a0, sv01);
        a1 = f16x2_mul(a1, sv23);
        acc[kb] = __builtin_amdgcn_mfma_f32_16x16x16f16(half4_of(a0, a1), Bv, acc[kb], 0, 0, 0);
      });
    }
  }

  // softmax sum of head jl over the wave's tokens
  const float l_w = sum_xor32(sum_xor16(l_part));

  // ---- merge the 4 waves through LDS (the staging area is reused) ----
  __syncthreads();
  const uint32_t macc = lds_addr(smem);
  const uint32_t mml = macc + Tl::MERGE_ACC;
  static_for<NB>([&](auto kk) {
    constexpr int kb = decltype(kk)::value;
    *(__attribute__((address_space(3))) float4_t*)(uintptr_t)(macc + 16u * ((uint32_t)(wave * NB + kb) * 64u + lane)) = acc[kb];
  });
  if (q == 0) {
    *(__attribute__((address_space(3))) float2_t*)(uintptr_t)(mml + 8u * (uint32_t)(wave * 16 + jl)) = (float2_t){m_run, l_w};
  }
  __syncthreads();

  float mw[4], fw[4];
  float m = -__builtin_inff();
  static_for<4>([&](auto ww) {
    constexpr int w = decltype(ww)::value;
    mw[w] = (*(const __attribute__((address_space(3))) float2_t*)(uintptr_t)(mml + 8u * (uint32_t)(w * 16 + jl)))[0];
    m = __builtin_fmaxf(m, mw[w]);
  });
  static_for<4>([&](auto ww) {
    constexpr int w = decltype(ww)::value;
    fw[w] = mw[w] == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(mw[w] - m);
  });
  const int64_t slot = ((int64_t)bh * a.n_chunks + c) * a.R + jl;   // valid for jl < R
  auto merged = [&](int kb) {   // acc[kb] of this lane summed over the 4 waves
    float4_t s = (float4_t){0.f, 0.f, 0.f, 0.f};
    static_for<4>([&](auto ww) {
      constexpr int w = decltype(ww)::value;
      const float4_t v = *(const __attribute__((address_space(3))) float4_t*)(uintptr_t)(macc + 16u * ((uint32_t)(w * NB + kb) * 64u + lane));
      s += fw[w] * v;
    });
    return s;
  };
  if constexpr (BITS == 4) {
    // acc[2j] element e holds coordinate 32j + 8q + 2e, acc[2j + 1] the next
    static_for<NB / 2>([&](auto jj) {
      constexpr int j = decltype(jj)::value;
      if (j % 4 == wave) {
        const float4_t se = merged(2 * j), so = merged(2 * j + 1);
        if (jl < a.R) {
          float* dst = ws_acc + slot * D + 32 * j + 8 * q;
          *(float4_t*)dst = (float4_t){se[0], so[0], se[1], so[1]};
          *(float4_t*)(dst + 4) = (float4_t){se[2], so[2], se[3], so[3]};
        }
      }
    });
  } else {
    static_for<NB>([&](auto kk) {
      constexpr int kb = decltype(kk)::value;
      if (kb % 4 == wave) {
        const float4_t s = merged(kb);
        if (jl < a.R) *(float4_t*)(ws_acc + slot * D + 16 * kb + 4 * q) = s;
      }
    });
  }
  if (wave == 0 && q == 0 && jl < a.R) {
    float l = 0.0f;
    static_for<4>([&](auto ww) {
      constexpr int w = decltype(ww)::value;
      l += fw[w] * (*(const __attribute__((address_space(3))) float2_t*)(uintptr_t)(mml + 8u * (uint32_t)(w * 16 + jl)))[1];
    });
    *(float2_t*)(ws_ml + 2 * slot) = (float2_t){m, l};
  }
}

// ----------------------------------------------------------------------------
// One query head: merge its chunks, w = acc / (l * lambda_v), o = s_v . M^T w.
// Block = (tensor, query head), 4 waves: the threads split the chunks for
// the maxima and sums, each wave accumulates every fourth chunk with its
// lanes splitting the coordinates, the waves add up through LDS, and the
// unrotation runs on all threads: SRFT one output coordinate per thread (a
// direct inverse DFT from the LDS twiddle table), SRHT wave_fwht on wave 0.
// ----------------------------------------------------------------------------
template <int D, int ROT>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ ws_ml,
                                                           const float* __restrict__ ws_acc,
                                                           const int8_t* __restrict__ signs_v,
                                                           const float* __restrict__ lam_v,
                                                           const float* __restrict__ Qv, int64_t q_stride,
                                                           float* __restrict__ out, AttnGeo a) {
  constexpr int PER = (D + 63) / 64;   // coordinates lane + 64 k per lane (d = 96: the second for lanes < 32)
  __shared__ __attribute__((aligned(16))) float part[4][D];
  __shared__ __attribute__((aligned(16))) float tw[ROT == ROT_SRFT ? 2 * D : 4];
  __shared__ __attribute__((aligned(16))) float pacc[ROT == ROT_DENSE ? 1024 : 4];   // matrix: [part][d]
  __shared__ float red[2][4];
  const int64_t v = xcd_head((int64_t)a.BH * a.R);   // b*H*R + h*R + r
  if (v < 0) return;
  const int bh = (int)(v / a.R);
  const int r = (int)(v - (int64_t)bh * a.R);
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int NC = a.n_chunks;
  const int64_t s0 = (int64_t)bh * NC * a.R + r;   // slot of chunk 0; chunk c at s0 + c*R
  if constexpr (ROT == ROT_SRFT) {
    const float* twg = dft_twiddles<D>();
    for (int i = t; i < 2 * D; i += 256) tw[i] = twg[i];   // read after the barriers below
  }
  constexpr int JPT = (D + 255) / 256;   // coordinates j = t + 256 i per thread
  float rlv[JPT];
  static_for<JPT>([&](auto ii) {
    const int j = t + 256 * decltype(ii)::value;
    rlv[decltype(ii)::value] = (lam_v && j < D) ? __builtin_amdgcn_rcpf(lam_v[(int64_t)bh * D + j]) : 1.0f;
  });

  // largest chunk maximum and the weighted sum of the chunk sums
  float m = -__builtin_inff();
  for (int ch = t; ch < NC; ch += 256) m = __builtin_fmaxf(m, ws_ml[2 * (s0 + (int64_t)ch * a.R)]);
  static_for<6>([&](auto ii) { m = __builtin_fmaxf(m, __shfl_xor(m, 1 << decltype(ii)::value)); });
  if (lane == 0) red[0][wave] = m;
  __syncthreads();
  m = __builtin_fmaxf(__builtin_fmaxf(red[0][0], red[0][1]), __builtin_fmaxf(red[0][2], red[0][3]));
  auto weight = [&](float mc) { return mc == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(mc - m); };
  float l = 0.0f;
  for (int ch = t; ch < NC; ch += 256) {
    const int64_t s = s0 + (int64_t)ch * a.R;
    l += weight(ws_ml[2 * s]) * ws_ml[2 * s + 1];
  }
  static_for<6>([&](auto ii) { l += __shfl_xor(l, 1 << decltype(ii)::value); });
  if (lane == 0) red[1][wave] = l;

  // accumulators: wave w takes chunks w, w + 4, ...
  float w[PER];
  static_for<PER>([&](auto kk) { w[decltype(kk)::value] = 0.0f; });
#pragma unroll 4
  for (int ch = wave; ch < NC; ch += 4) {
    const int64_t s = s0 + (int64_t)ch * a.R;
    const float f = weight(ws_ml[2 * s]);          // wave-uniform (scalar load)
    const float* src = ws_acc + s * D + lane;
    static_for<PER>([&](auto kk) {
      constexpr int k = decltype(kk)::value;
      if (D % 64 == 0 || lane + 64 * k < D) w[k] += f * src[64 * k];
    });
  }
  static_for<PER>([&](auto kk) {
    constexpr int k = decltype(kk)::value;
    if (D % 64 == 0 || lane + 64 * k < D) part[wave][lane + 64 * k] = w[k];
  });
  __syncthreads();
  l = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
  const float inv_l = l > 0.0f ? 1.0f / l : 0.0f;
  // z_j = acc_j / (l lambda_j) times the orthonormal scale of coordinate j:
  // x = M^T (acc / (l lambda)) below takes the unscaled transform of z
  static_for<JPT>([&](auto ii) {
    const int j = t + 256 * decltype(ii)::value;
    if (j < D) {
      float y = ((part[0][j] + part[1][j]) + (part[2][j] + part[3][j])) * inv_l;
      if (lam_v) y = y * rlv[decltype(ii)::value];
      part[0][j] = y * coord_scale<D, ROT>(j);
    }
  });
  __syncthreads();
  const int8_t* sg = signs_v + (int64_t)bh * a.sign_stride_v;
  float* dst = out + v * D;
  if constexpr (ROT == ROT_SRFT) {
    // x_m = z_0 + (-1)^m z_{d/2} + sum_{0<k<d/2} (cos(2 pi k m/d) z_k - sin(2 pi k m/d) z_{d/2+k}),
    // one output per thread
    constexpr int N = D / 2;
    if (t < D) {
      const int m = t;
      const float* z = part[0];
      float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
      int idx = 0;   // k m mod d
#pragma unroll 2
      for (int k = 0; k < N; k += 4) {
        const float4 zr = *(const float4*)&z[k];
        const float4 zi = *(const float4*)&z[N + k];
        float2 w = *(const float2*)&tw[2 * idx];
        s0 = __builtin_fmaf(zr.x, w.x, s0);
        s0 = __builtin_fmaf(zi.x, w.y, s0);
        idx = wrap<D>(idx + m);
        w = *(const float2*)&tw[2 * idx];
        s1 = __builtin_fmaf(zr.y, w.x, s1);
        s1 = __builtin_fmaf(zi.y, w.y, s1);
        idx = wrap<D>(idx + m);
        w = *(const float2*)&tw[2 * idx];
        s2 = __builtin_fmaf(zr.z, w.x, s2);
        s2 = __builtin_fmaf(zi.z, w.y, s2);
        idx = wrap<D>(idx + m);
        w = *(const float2*)&tw[2 * idx];
        s3 = __builtin_fmaf(zr.w, w.x, s3);
        s3 = __builtin_fmaf(zi.w, w.y, s3);
        idx = wrap<D>(idx + m);
      }
      // the k = 0 term above is z_0 (its sine is 0)
      float xm = ((s0 + s1) + (s2 + s3)) + ((m & 1) ? -z[N] : z[N]);
      if (sg[m] < 0) xm = -xm;
      dst[m] = xm;
    }
  } else if constexpr (ROT == ROT_DENSE) {
    // x_m = sum_j Q[j][m] z_j: thread t takes columns 4c .. 4c + 3 (c = t mod
    // d/4) over rows [p JR, (p + 1) JR) (p = t / (d/4); NP = 1024/d parts of
    // JR = d/NP rows), reading 16-byte pieces of the rows; the parts add up
    // through LDS
    constexpr int C4 = D / 4, NP = 256 / C4, JR = D / NP, JB = JR < 16 ? JR : 16;
    const int c = t % C4, pr = t / C4;
    const float* Qh = Qv + (int64_t)bh * q_stride + 4 * c;
    const float* z = part[0];
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = pr * JR; j0 < (pr + 1) * JR; j0 += JB) {
      float4 w[JB];
      static_for<JB>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
        w[i] = *(const float4*)(Qh + (int64_t)(j0 + i) * D);
      });
      static_for<JB>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
        const float zj = z[j0 + i];
        acc.x = __builtin_fmaf(w[i].x, zj, acc.x);
        acc.y = __builtin_fmaf(w[i].y, zj, acc.y);
        acc.z = __builtin_fmaf(w[i].z, zj, acc.z);
        acc.w = __builtin_fmaf(w[i].w, zj, acc.w);
      });
    }
    *(float4*)&pacc[pr * D + 4 * c] = acc;
    __syncthreads();
    if (t < D) {
      const int m = t;
      float xm = 0.0f;
      static_for<NP>([&](auto pp) { xm += pacc[decltype(pp)::value * D + m]; });
      if (sg[m] < 0) xm = -xm;
      dst[m] = xm;
    }
  } else if constexpr (ROT == ROT_SRHT) {
    constexpr int P = WaveVec<D>::P, NL = WaveVec<D>::NL;
    if (wave == 0) {
      float x[P];
      static_for<P>([&](auto tt) {
        constexpr int i = decltype(tt)::value;
        x[i] = lane < NL ? part[0][P * lane + i] : 0.0f;
      });
      wave_fwht<D>(x, lane);
      if (lane < NL) {
        static_for<P>([&](auto tt) {
          constexpr int i = decltype(tt)::value;
          const int m = P * lane + i;
          dst[m] = sg[m] < 0 ? -x[i] : x[i];
        });
      }
    }
  } else {
    for (int m = t; m < D; m += 256) dst[m] = sg[m] < 0 ? -part[0][m] : part[0][m];
  }
}

}  // namespace srftq
