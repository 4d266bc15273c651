// launch.h -- host-side dispatch from a runtime srftq_shape to the compiled
// kernel instance, and persistent-grid sizing.
#pragma once

#include <hip/hip_runtime.h>

#include "srftq.h"

namespace srftq {

enum class Op : int { Quantize = 0, Dequantize = 1, Rotate = 2, Unrotate = 3, Calibrate = 4 };

struct Ptrs {
  const void* x;         // quantize / rotate / calibrate input (fp16)
  const float* y_in;     // unrotate input (fp32)
  const uint8_t* codes_in;
  const uint16_t* scales_in;
  const int8_t* signs;   // never null: a shared +1 row when the caller passes none
  bool signs_shared;     // true: one row for every head (stride 0)
  const float* lambda;
  uint8_t* codes_out;
  uint16_t* scales_out;
  uint16_t* x_out;
  float* y_out;
  float* lambda_out;
  int64_t pitch;          // cache rows per head; 0 = T (the cache holds exactly x's tokens)
  const int32_t* pos;     // append positions [B] (device) or null
};

// Per-d entry points (one translation unit per d, direction and rotation
// selector r: 0 = SRFT real-input, 1 = SRFT paired, 2 = SRHT, 3 = none).
using RunFn = hipError_t (*)(const srftq_shape&, const Ptrs&, hipStream_t);
#define SRFTQ_DECL_RUN(d)                                                         \
  hipError_t run_quantize_d##d##_r0(const srftq_shape&, const Ptrs&, hipStream_t);   \
  hipError_t run_quantize_d##d##_r1(const srftq_shape&, const Ptrs&, hipStream_t);   \
  hipError_t run_quantize_d##d##_r2(const srftq_shape&, const Ptrs&, hipStream_t);   \
  hipError_t run_quantize_d##d##_r3(const srftq_shape&, const Ptrs&, hipStream_t);   \
  hipError_t run_dequantize_d##d##_r0(const srftq_shape&, const Ptrs&, hipStream_t); \
  hipError_t run_dequantize_d##d##_r1(const srftq_shape&, const Ptrs&, hipStream_t); \
  hipError_t run_dequantize_d##d##_r2(const srftq_shape&, const Ptrs&, hipStream_t); \
  hipError_t run_dequantize_d##d##_r3(const srftq_shape&, const Ptrs&, hipStream_t); \
  hipError_t run_misc_d##d(Op op, const srftq_shape&, const Ptrs&, hipStream_t);
SRFTQ_DECL_RUN(64)
SRFTQ_DECL_RUN(128)
SRFTQ_DECL_RUN(256)
#undef SRFTQ_DECL_RUN
// Head sizes served by the per-lane kernels (kernels_lane.h).
hipError_t run_quantize_d96(const srftq_shape&, const Ptrs&, hipStream_t);
hipError_t run_dequantize_d96(const srftq_shape&, const Ptrs&, hipStream_t);
hipError_t run_misc_d96(Op op, const srftq_shape&, const Ptrs&, hipStream_t);

inline int rot_selector(const srftq_shape& s) {
  if (s.rot == SRFTQ_ROT_SRFT) return s.variant == 2 ? 1 : 0;
  return s.rot == SRFTQ_ROT_SRHT ? 2 : 3;
}

// Decode attention over the quantized cache (attn.h).
struct AttnGeo {
  int64_t T;             // tokens attended at most (lengths are clamped to it)
  int64_t pitch;         // cache rows per head
  int32_t H;             // KV heads per tensor
  int32_t R;             // query heads per KV head, 1..16
  int32_t BH;            // B * H
  int32_t n_chunks;      // chunks per (tensor, KV head), 4 waves each; a tensor's
                         // 16-token blocks are split evenly over its 4 * n_chunks waves
  int32_t sign_stride_k; // elements between K heads' sign rows: d, or 0 (shared row)
  int32_t sign_stride_v;
  float scale_log2e;     // softmax scale * log2(e)
};

struct AttnArgs {
  AttnGeo geo;
  int rot, group, bits;
  bool dense;              // rotation given as matrices Qk, Qv (rot ignored)
  const float* Qk;         // [., d, d] fp32, matrix of head bh at Qk + bh * q_stride
  const float* Qv;
  int64_t q_stride;
  const uint16_t* q;
  const uint8_t* codes_k;
  const uint16_t* scales_k;
  const int8_t* signs_k;   // never null (shared +1 row when the caller passes none)
  const float* lam_k;
  const uint8_t* codes_v;
  const uint16_t* scales_v;
  const int8_t* signs_v;
  const float* lam_v;
  const int32_t* lengths;
  float* out;
  float* uq;       // workspace: rotated queries [B*H*R, d], normalized by a power of two
  float* uexp;     // workspace: that power of two per query head [B*H*R]
  float* ws_ml;    // workspace: per (head, chunk, query head) max and sum
  float* ws_acc;   // workspace: per (head, chunk, query head) accumulator [d]
};
using RunAttnFn = hipError_t (*)(const AttnArgs&, hipStream_t);
hipError_t run_attention_d64(const AttnArgs&, hipStream_t);
hipError_t run_attention_d96(const AttnArgs&, hipStream_t);
hipError_t run_attention_d128(const AttnArgs&, hipStream_t);
hipError_t run_attention_d256(const AttnArgs&, hipStream_t);

// Quantize / dequantize with a rotation given as a matrix (dense.h).
struct DenseArgs {
  bool quantize;
  int group, bits;
  int64_t T;
  int32_t H, BH;
  const float* Q;          // [., d, d] fp32, matrix of head bh at Q + bh * q_stride
  int64_t q_stride;
  const int8_t* signs;     // never null (shared +1 row when the caller passes none)
  int32_t sign_stride;     // d, or 0
  const float* lambda;     // [B, H, d] or null
  const uint16_t* x;
  uint8_t* codes_out;
  uint16_t* scales_out;
  const uint8_t* codes_in;
  const uint16_t* scales_in;
  uint16_t* x_out;
};
using RunDenseFn = hipError_t (*)(const DenseArgs&, hipStream_t);
hipError_t run_dense_d64(const DenseArgs&, hipStream_t);
hipError_t run_dense_d128(const DenseArgs&, hipStream_t);
hipError_t run_dense_d256(const DenseArgs&, hipStream_t);
// Q_m = H_1 ... H_k from V [n, k, d] into Q [n, d, d] (d <= 256, k <= 1024).
hipError_t run_householder(int d, int k, int64_t n, const float* V, float* Q, hipStream_t st);

// Decode attention with its workspace in the library's per-device scratch
// array (srftq_decode_attention_noalloc): every argument is checked first,
// then `scratch` returns the current device's array address (null on a HIP
// error); scratch_bytes is the array's size.
using ScratchFn = void* (*)();
srftq_status decode_attention_scratch(const srftq_shape* s, int64_t t_cap, int32_t R, const uint16_t* q,
                                      const srftq_cache_view* k, const srftq_cache_view* v,
                                      const int32_t* lengths, float scale, float* out, size_t scratch_bytes,
                                      ScratchFn scratch, void* stream);

// Number of compute units of the current device (cached per device).
int device_cu_count();

// Resident blocks per CU of a kernel at a block size (cached per kernel).
int blocks_per_cu(const void* kernel, int block);

// Tiles per block of the streaming kernels (0 = persistent grid, -1 = one
// tile per block in XCD-contiguous order).  One tile per block lets the
// hardware dispatcher balance the load across CUs (waves of a persistent
// grid finish up to 40 % apart); at d = 256, with one wave per SIMD, the
// persistent grid's one-tile-ahead prefetch hides more latency.  With four
// or more heads a token's rows of all heads lie within a few KB, and the
// XCD-contiguous order keeps them on one XCD (its own L2).
int tiles_per_block(int d, int H);

// Persistent grid: at most (resident blocks per CU) x CUs, at least 1.
inline int persistent_grid(const void* kernel, int n_tiles, int block) {
  long g = (long)blocks_per_cu(kernel, block) * (long)device_cu_count();
  if (g > n_tiles) g = n_tiles;
  return g < 1 ? 1 : (int)g;
}

// Launch sizes derived from a validated shape.
struct GeoH {
  int64_t T;
  int32_t H, BH, tiles_t, n_tiles;
};
inline GeoH make_geo(const srftq_shape& s) {
  GeoH g;
  g.T = s.T;
  g.H = s.H;
  g.BH = (int32_t)(s.B * s.H);
  g.tiles_t = (int32_t)((s.T + 63) / 64);
  g.n_tiles = g.tiles_t * g.BH;
  return g;
}

}  // namespace srftq
