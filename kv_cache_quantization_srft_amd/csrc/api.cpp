// api.cpp -- the C ABI of libsrftq (include/srftq.h): argument validation on
// the host, then dispatch to the per-head-size kernel translation units.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdlib>
#include <mutex>
#include <unordered_map>

#include "launch.h"
#include "srftq.h"

namespace srftq {

// Per-device cache; concurrent first calls from several host threads may
// both query the device, and store the same value.
int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
  int n = cache[dev].load(std::memory_order_acquire);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 1;
    cache[dev].store(n, std::memory_order_release);
  }
  return n;
}

const int8_t* plus_ones_ptr();   // defined with the device array in ones.hip

int tiles_per_block(int d, int H) { return d >= 256 ? 0 : H >= 4 ? -1 : 1; }

int blocks_per_cu(const void* kernel, int block) {
  static std::mutex mu;
  static std::unordered_map<const void*, int> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(kernel);
  if (it != cache.end()) return it->second;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, block, 0) != hipSuccess || nb <= 0) nb = 1;
  cache.emplace(kernel, nb);
  return nb;
}

}  // namespace srftq

namespace {

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

srftq_status validate(const srftq_shape* s) {
  if (!s) return SRFTQ_ERR_NULL;
  if (s->B < 0 || s->T < 0 || s->H < 1) return SRFTQ_ERR_SHAPE;
  if (s->d != 64 && s->d != 96 && s->d != 128 && s->d != 256) return SRFTQ_ERR_UNSUPPORTED;
  if (s->bits != 4 && s->bits != 8) return SRFTQ_ERR_UNSUPPORTED;
  if (!is_pow2(s->group) || s->group < 8 || s->group > s->d || s->d % s->group != 0)
    return SRFTQ_ERR_UNSUPPORTED;
  if (s->rot != SRFTQ_ROT_SRFT && s->rot != SRFTQ_ROT_SRHT && s->rot != SRFTQ_ROT_NONE)
    return SRFTQ_ERR_UNSUPPORTED;
  if (s->variant < 0 || s->variant > 2) return SRFTQ_ERR_UNSUPPORTED;
  // d = 96: the SRFT's real-input transform with a radix-3 step, or no rotation
  // (the Walsh-Hadamard matrix and the paired complex FFT need a power of two)
  if (s->d == 96 && (s->rot == SRFTQ_ROT_SRHT || (s->rot == SRFTQ_ROT_SRFT && s->variant == 2)))
    return SRFTQ_ERR_UNSUPPORTED;
  // 32-bit tile counters and per-lane byte offsets; every product below is
  // bounded before it is formed (B*H < 2^31, so B*H*d < 2^39)
  if (s->H > 65535) return SRFTQ_ERR_SHAPE;
  if (s->B > (int64_t)0x7fffffff / s->H) return SRFTQ_ERR_SHAPE;
  const int64_t BH = s->B * (int64_t)s->H;
  const int64_t tiles_t = s->T / 32 + (s->T % 32 != 0);   // the smallest tiles (d = 256)
  if (BH > 0 && tiles_t > (int64_t)0x7fffffff / BH) return SRFTQ_ERR_SHAPE;
  if (BH > 0 && s->T > (int64_t)0x7fffffffffffLL / (BH * s->d)) return SRFTQ_ERR_SHAPE;
  return SRFTQ_OK;
}

int64_t nvec(const srftq_shape* s) { return s->B * s->T * (int64_t)s->H; }

srftq_status from_hip(hipError_t e) { return e == hipSuccess ? SRFTQ_OK : SRFTQ_ERR_HIP; }

const srftq::RunFn kQuantize[3][4] = {
    {srftq::run_quantize_d64_r0, srftq::run_quantize_d64_r1, srftq::run_quantize_d64_r2,
     srftq::run_quantize_d64_r3},
    {srftq::run_quantize_d128_r0, srftq::run_quantize_d128_r1, srftq::run_quantize_d128_r2,
     srftq::run_quantize_d128_r3},
    {srftq::run_quantize_d256_r0, srftq::run_quantize_d256_r1, srftq::run_quantize_d256_r2,
     srftq::run_quantize_d256_r3}};
const srftq::RunFn kDequantize[3][4] = {
    {srftq::run_dequantize_d64_r0, srftq::run_dequantize_d64_r1, srftq::run_dequantize_d64_r2,
     srftq::run_dequantize_d64_r3},
    {srftq::run_dequantize_d128_r0, srftq::run_dequantize_d128_r1, srftq::run_dequantize_d128_r2,
     srftq::run_dequantize_d128_r3},
    {srftq::run_dequantize_d256_r0, srftq::run_dequantize_d256_r1, srftq::run_dequantize_d256_r2,
     srftq::run_dequantize_d256_r3}};

// The kernel for a validated shape: the tiled kernels of d = 64, 128, 256
// (table), or the per-lane kernels of d = 96 (lane96).
srftq::RunFn pick(const srftq::RunFn (&table)[3][4], srftq::RunFn lane96, const srftq_shape* s) {
  if (s->d == 96) return lane96;
  const int di = s->d == 64 ? 0 : s->d == 128 ? 1 : s->d == 256 ? 2 : -1;
  if (di < 0) return nullptr;
  return table[di][srftq::rot_selector(*s)];
}

srftq_status check_side(const int8_t* signs, const float* lambda) {
  if (signs && !aligned4(signs)) return SRFTQ_ERR_ALIGN;
  if (lambda && !aligned4(lambda)) return SRFTQ_ERR_ALIGN;
  return SRFTQ_OK;
}

// A cache of t_cap rows per head must keep byte offsets within int64 range
// (the same bound validate() puts on T).
srftq_status validate_cache(const srftq_shape* s, int64_t t_cap) {
  if (t_cap < 0) return SRFTQ_ERR_SHAPE;
  if (s->B > (int64_t)0x7fffffff / s->H) return SRFTQ_ERR_SHAPE;   // as validate(): B*H < 2^31
  if (s->B > 0 && t_cap > (int64_t)0x7fffffffffffLL / (s->B * (int64_t)s->H * s->d)) return SRFTQ_ERR_SHAPE;
  return SRFTQ_OK;
}

srftq_status quantize_into(const srftq_shape* s, int64_t pitch, const int32_t* pos, const uint16_t* x,
                           const int8_t* signs, const float* lambda, uint8_t* codes, uint16_t* scales,
                           void* stream) {
  srftq_status st;
  if (!x || !codes || !scales) return SRFTQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return SRFTQ_ERR_ALIGN;
  if (pos && !aligned4(pos)) return SRFTQ_ERR_ALIGN;
  if ((st = check_side(signs, lambda)) != SRFTQ_OK) return st;
  srftq::Ptrs p = {};
  p.x = x;
  p.signs = signs ? signs : srftq::plus_ones_ptr();
  p.signs_shared = (signs == nullptr);
  if (!p.signs) return SRFTQ_ERR_HIP;
  p.lambda = lambda;
  p.codes_out = codes;
  p.scales_out = scales;
  p.pitch = pitch;
  p.pos = pos;
  const srftq::RunFn fn = pick(kQuantize, srftq::run_quantize_d96, s);
  return fn ? from_hip(fn(*s, p, (hipStream_t)stream)) : SRFTQ_ERR_UNSUPPORTED;
}

srftq_status dequantize_from(const srftq_shape* s, int64_t pitch, const uint8_t* codes,
                             const uint16_t* scales, const int8_t* signs, const float* lambda,
                             uint16_t* x_out, void* stream) {
  srftq_status st;
  if (!codes || !scales || !x_out) return SRFTQ_ERR_NULL;
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(x_out)) return SRFTQ_ERR_ALIGN;
  if ((st = check_side(signs, lambda)) != SRFTQ_OK) return st;
  srftq::Ptrs p = {};
  p.codes_in = codes;
  p.scales_in = scales;
  p.signs = signs ? signs : srftq::plus_ones_ptr();
  p.signs_shared = (signs == nullptr);
  if (!p.signs) return SRFTQ_ERR_HIP;
  p.lambda = lambda;
  p.x_out = x_out;
  p.pitch = pitch;
  const srftq::RunFn fn = pick(kDequantize, srftq::run_dequantize_d96, s);
  return fn ? from_hip(fn(*s, p, (hipStream_t)stream)) : SRFTQ_ERR_UNSUPPORTED;
}

// Decode attention: the number of chunks per (tensor, KV head), and the
// workspace carve-up.  The partial kernel is VALU-bound with four 256-thread
// blocks resident per CU (1024 on the chip); a grid of at most one resident
// round, with every wave's share of tokens equal, avoids a final round of a
// few blocks that cannot keep the SIMDs busy (measured at 28 layers x 2 KV
// heads x 32768 tokens: 18 chunks 82 us, 37 chunks 90 us).  Each wave keeps
// at least four 16-token blocks so that its load pipeline fills.
struct AttnPlan {
  int n_chunks = 1;
  size_t off_exp = 0, off_ml = 0, off_acc = 0, bytes = 0;
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

bool attn_plan(const srftq_shape* s, int32_t R, AttnPlan* p) {
  if (validate(s) != SRFTQ_OK || R < 1 || R > 16 || s->group < 16) return false;
  if (s->d != 64 && s->d != 96 && s->d != 128 && s->d != 256) return false;
  const int64_t BH = s->B * (int64_t)s->H;
  constexpr int64_t kResidentBlocks = 1024;
  const int64_t blocks16 = (s->T + 15) / 16;
  int64_t nc = BH > 0 ? kResidentBlocks / BH : 1;
  if (nc > blocks16 / 16) nc = blocks16 / 16;
  if (nc < 1) nc = 1;
  if (BH * nc > 0x7fffffffLL || BH * R > 0x7ffffff0LL) return false;   // grids of up to BH * R + 7 blocks
  p->n_chunks = (int)nc;
  const size_t uq = (size_t)BH * R * s->d * 4;
  const size_t ml = (size_t)BH * nc * R * 2 * 4;
  const size_t acc = (size_t)BH * nc * R * s->d * 4;
  p->off_exp = align256(uq);
  p->off_ml = p->off_exp + align256((size_t)BH * R * 4);
  p->off_acc = p->off_ml + align256(ml);
  p->bytes = p->off_acc + align256(acc);
  return true;
}

const srftq::RunAttnFn kAttention[4] = {srftq::run_attention_d64, srftq::run_attention_d96,
                                        srftq::run_attention_d128, srftq::run_attention_d256};

// Rotation given as a matrix: the sizes of validate(); d in {64, 128, 256},
// group in {8, 16, 32}; rot and variant are not used.  q_stride 0 (one
// matrix) or at least d*d, a multiple of 4 (16-byte aligned matrices).
srftq_status validate_dense(const srftq_shape* s, int64_t q_stride) {
  if (!s) return SRFTQ_ERR_NULL;
  srftq_shape t = *s;
  t.rot = SRFTQ_ROT_NONE;
  t.variant = 0;
  srftq_status st = validate(&t);
  if (st != SRFTQ_OK) return st;
  if (s->d != 64 && s->d != 128 && s->d != 256) return SRFTQ_ERR_UNSUPPORTED;
  if (s->group != 8 && s->group != 16 && s->group != 32) return SRFTQ_ERR_UNSUPPORTED;
  if (q_stride < 0 || (q_stride != 0 && (q_stride < (int64_t)s->d * s->d || q_stride % 4 != 0)))
    return SRFTQ_ERR_SHAPE;
  if (q_stride > 0 && s->B * (int64_t)s->H > (int64_t)0x7fffffffffffLL / q_stride) return SRFTQ_ERR_SHAPE;
  return SRFTQ_OK;
}

const srftq::RunDenseFn kDense[3] = {srftq::run_dense_d64, srftq::run_dense_d128, srftq::run_dense_d256};

srftq_status run_dense(srftq::DenseArgs& a, const srftq_shape* s, const int8_t* signs, void* stream) {
  a.group = s->group;
  a.bits = s->bits;
  a.T = s->T;
  a.H = s->H;
  a.BH = (int32_t)(s->B * s->H);
  a.signs = signs ? signs : srftq::plus_ones_ptr();
  a.sign_stride = signs ? s->d : 0;
  if (!a.signs) return SRFTQ_ERR_HIP;
  const int di = s->d == 64 ? 0 : s->d == 128 ? 1 : 2;
  return from_hip(kDense[di](a, (hipStream_t)stream));
}

// The kernels read a sign row for every head: the shared +1 row where the
// caller passes none (a device lookup, so after every argument check).
srftq_status set_plus_ones(srftq::AttnArgs& a) {
  if (a.signs_k && a.signs_v) return SRFTQ_OK;
  const int8_t* ones = srftq::plus_ones_ptr();
  if (!ones) return SRFTQ_ERR_HIP;
  if (!a.signs_k) a.signs_k = ones;
  if (!a.signs_v) a.signs_v = ones;
  return SRFTQ_OK;
}

// The workspace carve-up of an attention plan (see AttnPlan).
void set_workspace(srftq::AttnArgs& a, void* workspace, const AttnPlan& plan) {
  a.uq = (float*)workspace;
  a.uexp = (float*)((char*)workspace + plan.off_exp);
  a.ws_ml = (float*)((char*)workspace + plan.off_ml);
  a.ws_acc = (float*)((char*)workspace + plan.off_acc);
}

// Checks and launch arguments shared by the decode-attention entry points
// (the shape already validated); `empty` when there is nothing to launch.
// With `deferred`, the workspace is the library's own scratch array, looked
// up after every check (it needs a device): only its size is checked here,
// and a problem too large for it is SRFTQ_ERR_CAPACITY.
srftq_status attention_args(const srftq_shape* s, int64_t t_cap, int32_t R, const uint16_t* q,
                            const srftq_cache_view* k, const srftq_cache_view* v, const int32_t* lengths,
                            float scale, float* out, void* workspace, size_t workspace_bytes,
                            srftq::AttnArgs& a, bool& empty, bool deferred = false) {
  srftq_status st;
  if (R < 1 || R > 16) return SRFTQ_ERR_SHAPE;
  if (s->group < 16) return SRFTQ_ERR_UNSUPPORTED;
  if ((st = validate_cache(s, t_cap)) != SRFTQ_OK) return st;
  if (t_cap < s->T) return SRFTQ_ERR_SHAPE;
  if (!(scale == scale) || scale > 3.0e38f || scale < -3.0e38f) return SRFTQ_ERR_SHAPE;
  AttnPlan plan;
  if (!attn_plan(s, R, &plan)) return SRFTQ_ERR_SHAPE;
  empty = s->B * (int64_t)s->H == 0;
  if (empty) return SRFTQ_OK;
  if (deferred && workspace_bytes < plan.bytes) return SRFTQ_ERR_CAPACITY;
  if (!q || !k || !v || !out || (!workspace && !deferred)) return SRFTQ_ERR_NULL;
  if (!k->codes || !k->scales || !v->codes || !v->scales) return SRFTQ_ERR_NULL;
  if (!aligned16(q) || !aligned16(out) || (!deferred && !aligned16(workspace)) || !aligned16(k->codes) ||
      !aligned16(k->scales) || !aligned16(v->codes) || !aligned16(v->scales))
    return SRFTQ_ERR_ALIGN;
  if (lengths && !aligned4(lengths)) return SRFTQ_ERR_ALIGN;
  if ((st = check_side(k->signs, k->lambda)) != SRFTQ_OK) return st;
  if ((st = check_side(v->signs, v->lambda)) != SRFTQ_OK) return st;
  if (workspace_bytes < plan.bytes) return SRFTQ_ERR_SHAPE;
  a.geo.T = s->T;
  a.geo.pitch = t_cap;
  a.geo.H = s->H;
  a.geo.R = R;
  a.geo.BH = (int32_t)(s->B * s->H);
  a.geo.n_chunks = plan.n_chunks;
  a.geo.sign_stride_k = k->signs ? s->d : 0;
  a.geo.sign_stride_v = v->signs ? s->d : 0;
  a.geo.scale_log2e = (float)((double)scale * 1.4426950408889634);
  a.group = s->group;
  a.bits = s->bits;
  a.q = q;
  a.codes_k = k->codes;
  a.scales_k = k->scales;
  a.signs_k = k->signs;   // NULL: the shared +1 row, set by set_plus_ones
  a.lam_k = k->lambda;
  a.codes_v = v->codes;
  a.scales_v = v->scales;
  a.signs_v = v->signs;
  a.lam_v = v->lambda;
  a.lengths = lengths;
  a.out = out;
  set_workspace(a, workspace, plan);
  return SRFTQ_OK;
}

// The one decode-attention path behind both entry points: `scratch` null
// (caller's workspace) or the per-device scratch lookup of
// srftq_decode_attention_noalloc.
srftq_status decode_attention(const srftq_shape* s, int64_t t_cap, int32_t R, const uint16_t* q,
                              const srftq_cache_view* k, const srftq_cache_view* v, const int32_t* lengths,
                              float scale, float* out, void* workspace, size_t workspace_bytes,
                              srftq::ScratchFn scratch, void* stream) {
  srftq_status st = validate(s);
  if (st != SRFTQ_OK) return st;
  srftq::AttnArgs a = {};
  bool empty = false;
  if ((st = attention_args(s, t_cap, R, q, k, v, lengths, scale, out, workspace, workspace_bytes, a, empty,
                           scratch != nullptr)) != SRFTQ_OK ||
      empty)
    return st;
  a.rot = s->rot;
  if ((st = set_plus_ones(a)) != SRFTQ_OK) return st;
  if (scratch) {
    void* ws = scratch();
    if (!ws) return SRFTQ_ERR_HIP;
    AttnPlan plan;
    attn_plan(s, R, &plan);
    set_workspace(a, ws, plan);
  }
  const int di = s->d == 64 ? 0 : s->d == 96 ? 1 : s->d == 128 ? 2 : 3;
  return from_hip(kAttention[di](a, (hipStream_t)stream));
}

}  // namespace

namespace srftq {
srftq_status decode_attention_scratch(const srftq_shape* s, int64_t t_cap, int32_t R, const uint16_t* q,
                                      const srftq_cache_view* k, const srftq_cache_view* v,
                                      const int32_t* lengths, float scale, float* out, size_t scratch_bytes,
                                      ScratchFn scratch, void* stream) {
  return ::decode_attention(s, t_cap, R, q, k, v, lengths, scale, out, nullptr, scratch_bytes, scratch, stream);
}
}  // namespace srftq

extern "C" {

srftq_status srftq_validate(const srftq_shape* shape) { return validate(shape); }

size_t srftq_attention_workspace_bytes(const srftq_shape* s, int32_t q_per_kv) {
  AttnPlan p;
  return attn_plan(s, q_per_kv, &p) ? p.bytes : 0;
}

srftq_status srftq_decode_attention(const srftq_shape* s, int64_t t_cap, int32_t R, const uint16_t* q,
                                    const srftq_cache_view* k, const srftq_cache_view* v,
                                    const int32_t* lengths, float scale, float* out, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return decode_attention(s, t_cap, R, q, k, v, lengths, scale, out, workspace, workspace_bytes, nullptr, stream);
}

srftq_status srftq_decode_attention_dense(const srftq_shape* s, int64_t t_cap, int32_t R, const float* Qk,
                                          const float* Qv, int64_t q_stride, const uint16_t* q,
                                          const srftq_cache_view* k, const srftq_cache_view* v,
                                          const int32_t* lengths, float scale, float* out, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  srftq_status st = validate_dense(s, q_stride);
  if (st != SRFTQ_OK) return st;
  srftq_shape t = *s;   // rot and variant are not used
  t.rot = SRFTQ_ROT_NONE;
  t.variant = 0;
  srftq::AttnArgs a = {};
  bool empty = false;
  if ((st = attention_args(&t, t_cap, R, q, k, v, lengths, scale, out, workspace, workspace_bytes, a,
                           empty)) != SRFTQ_OK || empty)
    return st;
  if (!Qk || !Qv) return SRFTQ_ERR_NULL;
  if (!aligned16(Qk) || !aligned16(Qv)) return SRFTQ_ERR_ALIGN;
  a.dense = true;
  a.Qk = Qk;
  a.Qv = Qv;
  a.q_stride = q_stride;
  if ((st = set_plus_ones(a)) != SRFTQ_OK) return st;
  const int di = s->d == 64 ? 0 : s->d == 128 ? 2 : 3;
  return from_hip(kAttention[di](a, (hipStream_t)stream));
}

size_t srftq_codes_bytes(const srftq_shape* s) {
  if (validate(s) != SRFTQ_OK) return 0;
  return (size_t)nvec(s) * (size_t)s->d * (size_t)s->bits / 8;
}

size_t srftq_scales_count(const srftq_shape* s) {
  if (validate(s) != SRFTQ_OK) return 0;
  return (size_t)nvec(s) * (size_t)(s->d / s->group);
}

srftq_status srftq_quantize(const srftq_shape* s, const uint16_t* x, const int8_t* signs,
                            const float* lambda, uint8_t* codes, uint16_t* scales, void* stream) {
  srftq_status st = validate(s);
  if (st != SRFTQ_OK) return st;
  if (nvec(s) == 0) return SRFTQ_OK;
  return quantize_into(s, 0, nullptr, x, signs, lambda, codes, scales, stream);
}

srftq_status srftq_dequantize(const srftq_shape* s, const uint8_t* codes, const uint16_t* scales,
                              const int8_t* signs, const float* lambda, uint16_t* x_out, void* stream) {
  srftq_status st = validate(s);
  if (st != SRFTQ_OK) return st;
  if (nvec(s) == 0) return SRFTQ_OK;
  return dequantize_from(s, 0, codes, scales, signs, lambda, x_out, stream);
}

srftq_status srftq_cache_append(const srftq_shape* s, int64_t t_cap, const int32_t* pos,
                                const uint16_t* x, const int8_t* signs, const float* lambda,
                                uint8_t* codes, uint16_t* scales, void* stream) {
  srftq_status st = validate(s);
  if (st != SRFTQ_OK) return st;
  if ((st = validate_cache(s, t_cap)) != SRFTQ_OK) return st;
  if (nvec(s) == 0 || t_cap == 0) return SRFTQ_OK;
  return quantize_into(s, t_cap, pos, x, signs, lambda, codes, scales, stream);
}

srftq_status srftq_cache_read(const srftq_shape* s, int64_t t_cap, const uint8_t* codes,
                              const uint16_t* scales, const int8_t* signs, const float* lambda,
                              uint16_t* x_out, void* stream) {
  srftq_status st = validate(s);
  if (st != SRFTQ_OK) return st;
  if ((st = validate_cache(s, t_cap)) != SRFTQ_OK) return st;
  if (t_cap < s->T) return SRFTQ_ERR_SHAPE;
  if (nvec(s) == 0) return SRFTQ_OK;
  return dequantize_from(s, t_cap, codes, scales, signs, lambda, x_out, stream);
}
static srftq_status run_misc(srftq::Op op, const srftq_shape* s, const srftq::Ptrs& p, void* stream) {
  hipStream_t hs = (hipStream_t)stream;
  switch (s->d) {
    case 64: return from_hip(srftq::run_misc_d64(op, *s, p, hs));
    case 128: return from_hip(srftq::run_misc_d128(op, *s, p, hs));
    case 256: return from_hip(srftq::run_misc_d256(op, *s, p, hs));
    case 96: return from_hip(srftq::run_misc_d96(op, *s, p, hs));
    default: return SRFTQ_ERR_UNSUPPORTED;
  }
}

srftq_status srftq_rotate(const srftq_shape* s, const uint16_t* x, const int8_t* signs, float* y,
                          void* stream) {
  srftq_status st = validate(s);
  if (st != SRFTQ_OK) return st;
  if (nvec(s) == 0) return SRFTQ_OK;
  if (!x || !y) return SRFTQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(y)) return SRFTQ_ERR_ALIGN;
  if ((st = check_side(signs, nullptr)) != SRFTQ_OK) return st;
  srftq::Ptrs p = {};
  p.x = x;
  p.signs = signs ? signs : srftq::plus_ones_ptr();
  p.signs_shared = (signs == nullptr);
  if (!p.signs) return SRFTQ_ERR_HIP;
  p.y_out = y;
  return run_misc(srftq::Op::Rotate, s, p, stream);
}

srftq_status srftq_unrotate(const srftq_shape* s, const float* y, const int8_t* signs, uint16_t* x_out,
                            void* stream) {
  srftq_status st = validate(s);
  if (st != SRFTQ_OK) return st;
  if (nvec(s) == 0) return SRFTQ_OK;
  if (!y || !x_out) return SRFTQ_ERR_NULL;
  if (!aligned16(y) || !aligned16(x_out)) return SRFTQ_ERR_ALIGN;
  if ((st = check_side(signs, nullptr)) != SRFTQ_OK) return st;
  srftq::Ptrs p = {};
  p.y_in = y;
  p.signs = signs ? signs : srftq::plus_ones_ptr();
  p.signs_shared = (signs == nullptr);
  if (!p.signs) return SRFTQ_ERR_HIP;
  p.x_out = x_out;
  return run_misc(srftq::Op::Unrotate, s, p, stream);
}

srftq_status srftq_calibrate_lambda(const srftq_shape* s, const uint16_t* x, const int8_t* signs,
                                    float* lambda, void* stream) {
  srftq_status st = validate(s);
  if (st != SRFTQ_OK) return st;
  if (s->B * (int64_t)s->H == 0) return SRFTQ_OK;
  if (!lambda || (s->T > 0 && !x)) return SRFTQ_ERR_NULL;
  if ((x && !aligned16(x)) || !aligned4(lambda)) return SRFTQ_ERR_ALIGN;
  if ((st = check_side(signs, nullptr)) != SRFTQ_OK) return st;
  srftq::Ptrs p = {};
  p.x = x;
  p.signs = signs ? signs : srftq::plus_ones_ptr();
  p.signs_shared = (signs == nullptr);
  if (!p.signs) return SRFTQ_ERR_HIP;
  p.lambda_out = lambda;
  return run_misc(srftq::Op::Calibrate, s, p, stream);
}

srftq_status srftq_householder_matrix(int32_t d, int32_t k, int64_t n, const float* V, float* Q,
                                     void* stream) {
  if (d < 1 || d > 256 || k < 0 || k > 1024 || n < 0 || n > 65535) return SRFTQ_ERR_SHAPE;
  if (n == 0) return SRFTQ_OK;
  if (!Q || (k > 0 && !V)) return SRFTQ_ERR_NULL;
  if (!aligned4(Q) || (V && !aligned4(V))) return SRFTQ_ERR_ALIGN;
  return from_hip(srftq::run_householder(d, k, n, V, Q, (hipStream_t)stream));
}

srftq_status srftq_quantize_dense(const srftq_shape* s, const float* Q, int64_t q_stride, const uint16_t* x,
                                  const int8_t* signs, const float* lambda, uint8_t* codes, uint16_t* scales,
                                  void* stream) {
  srftq_status st = validate_dense(s, q_stride);
  if (st != SRFTQ_OK) return st;
  if (nvec(s) == 0) return SRFTQ_OK;
  if (!Q || !x || !codes || !scales) return SRFTQ_ERR_NULL;
  if (!aligned16(Q) || !aligned16(x) || !aligned16(codes) || !aligned16(scales)) return SRFTQ_ERR_ALIGN;
  if ((st = check_side(signs, lambda)) != SRFTQ_OK) return st;
  srftq::DenseArgs a = {};
  a.quantize = true;
  a.Q = Q;
  a.q_stride = q_stride;
  a.lambda = lambda;
  a.x = x;
  a.codes_out = codes;
  a.scales_out = scales;
  return run_dense(a, s, signs, stream);
}

srftq_status srftq_dequantize_dense(const srftq_shape* s, const float* Q, int64_t q_stride,
                                    const uint8_t* codes, const uint16_t* scales, const int8_t* signs,
                                    const float* lambda, uint16_t* x_out, void* stream) {
  srftq_status st = validate_dense(s, q_stride);
  if (st != SRFTQ_OK) return st;
  if (nvec(s) == 0) return SRFTQ_OK;
  if (!Q || !codes || !scales || !x_out) return SRFTQ_ERR_NULL;
  if (!aligned16(Q) || !aligned16(codes) || !aligned16(scales) || !aligned16(x_out)) return SRFTQ_ERR_ALIGN;
  if ((st = check_side(signs, lambda)) != SRFTQ_OK) return st;
  srftq::DenseArgs a = {};
  a.quantize = false;
  a.Q = Q;
  a.q_stride = q_stride;
  a.lambda = lambda;
  a.codes_in = codes;
  a.scales_in = scales;
  a.x_out = x_out;
  return run_dense(a, s, signs, stream);
}

const char* srftq_status_string(srftq_status status) {
  switch (status) {
    case SRFTQ_OK: return "ok";
    case SRFTQ_ERR_NULL: return "null pointer";
    case SRFTQ_ERR_SHAPE: return "invalid shape";
    case SRFTQ_ERR_UNSUPPORTED: return "unsupported (d, group, bits, rot, variant) combination";
    case SRFTQ_ERR_ALIGN: return "misaligned pointer";
    case SRFTQ_ERR_HIP: return "HIP runtime error";
    case SRFTQ_ERR_CAPACITY: return "problem needs more scratch memory than the library's fixed buffer holds";
    default: return "unknown status";
  }
}

int srftq_version(void) { return 100; }

}  // extern "C"
