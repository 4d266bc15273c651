// Host-only driver of the C ABI's validation and argument marshalling
// (csrc/api.cpp), for a build with AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_sanitizers.py).  The kernel
// dispatchers are replaced by stubs that record the launch arguments, so
// every entry point runs its checks and hands its arguments on without a GPU;
// each call's status, and what reached the stub, is checked here.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "launch.h"
#include "srftq.h"

// --- stubs of the kernel translation units and the HIP runtime -------------
namespace {
int g_launches = 0;
srftq::Ptrs g_last{};
srftq_shape g_last_shape{};
srftq::AttnArgs g_attn{};
srftq::DenseArgs g_dense{};
alignas(16) int8_t g_ones[256];
alignas(256) uint8_t g_scratch[1 << 20];
}  // namespace

#define STUB_RUN(name)                                                          \
  hipError_t srftq::name(const srftq_shape& s, const srftq::Ptrs& p, hipStream_t) { \
    ++g_launches;                                                               \
    g_last = p;                                                                 \
    g_last_shape = s;                                                           \
    return hipSuccess;                                                          \
  }
#define STUB_D(d)                                                                      \
  STUB_RUN(run_quantize_d##d##_r0) STUB_RUN(run_quantize_d##d##_r1) STUB_RUN(run_quantize_d##d##_r2) \
  STUB_RUN(run_quantize_d##d##_r3) STUB_RUN(run_dequantize_d##d##_r0) STUB_RUN(run_dequantize_d##d##_r1) \
  STUB_RUN(run_dequantize_d##d##_r2) STUB_RUN(run_dequantize_d##d##_r3)                                \
  hipError_t srftq::run_misc_d##d(srftq::Op, const srftq_shape& s, const srftq::Ptrs& p, hipStream_t) { \
    ++g_launches; g_last = p; g_last_shape = s; return hipSuccess; }                                 \
  hipError_t srftq::run_attention_d##d(const srftq::AttnArgs& a, hipStream_t) { ++g_launches; g_attn = a; return hipSuccess; }
STUB_D(64)
STUB_D(128)
STUB_D(256)
STUB_RUN(run_quantize_d96)
STUB_RUN(run_dequantize_d96)
hipError_t srftq::run_misc_d96(srftq::Op, const srftq_shape& s, const srftq::Ptrs& p, hipStream_t) {
  ++g_launches; g_last = p; g_last_shape = s; return hipSuccess;
}
hipError_t srftq::run_attention_d96(const srftq::AttnArgs& a, hipStream_t) { ++g_launches; g_attn = a; return hipSuccess; }
#define STUB_DENSE(d) \
  hipError_t srftq::run_dense_d##d(const srftq::DenseArgs& a, hipStream_t) { ++g_launches; g_dense = a; return hipSuccess; }
STUB_DENSE(64)
STUB_DENSE(128)
STUB_DENSE(256)
hipError_t srftq::run_householder(int, int, int64_t, const float*, float*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
namespace srftq {
const int8_t* plus_ones_ptr() { return g_ones; }
}  // namespace srftq
extern "C" hipError_t hipGetDevice(int* d) { *d = 0; return hipSuccess; }
extern "C" hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) { *v = 256; return hipSuccess; }
extern "C" hipError_t hipOccupancyMaxActiveBlocksPerMultiprocessor(int* n, const void*, int, size_t) {
  *n = 1;
  return hipSuccess;
}

// --- checks ------------------------------------------------------------------
static int fails = 0;
#define EXPECT(cond)                                                     \
  do {                                                                   \
    if (!(cond)) {                                                       \
      std::fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #cond);    \
      ++fails;                                                           \
    }                                                                    \
  } while (0)

static void* scratch_fn() { return g_scratch; }

int main() {
  alignas(16) static uint8_t buf[1 << 16];
  void* a = buf;
  void* mis = buf + 8;
  const srftq_shape ok = {2, 100, 3, 128, 16, 4, SRFTQ_ROT_SRFT, 0};

  // validation of every field, sizes at the int64 edges
  EXPECT(srftq_validate(nullptr) == SRFTQ_ERR_NULL);
  EXPECT(srftq_validate(&ok) == SRFTQ_OK);
  const int ds[] = {0, 1, 32, 64, 96, 100, 128, 192, 256, 512};
  const int gs[] = {-16, 0, 4, 8, 12, 16, 32, 64, 128, 256, 512};
  for (int d : ds)
    for (int g : gs)
      for (int bits = 3; bits <= 8; ++bits)
        for (int rot = -1; rot <= 3; ++rot)
          for (int var = -1; var <= 3; ++var) {
            srftq_shape s = {3, 70, 2, d, g, bits, (srftq_rot)rot, var};
            const srftq_status st = srftq_validate(&s);
            const bool want = (d == 64 || d == 96 || d == 128 || d == 256) && (bits == 4 || bits == 8) &&
                              g >= 8 && g <= d && (g & (g - 1)) == 0 && d % g == 0 && rot >= 0 && rot <= 2 &&
                              var >= 0 && var <= 2 && !(d == 96 && (rot == 1 || (rot == 0 && var == 2)));
            EXPECT((st == SRFTQ_OK) == want);
            const size_t cb = srftq_codes_bytes(&s), sc = srftq_scales_count(&s);
            EXPECT(want ? cb == (size_t)3 * 70 * 2 * d * bits / 8 : cb == 0);
            EXPECT(want ? sc == (size_t)3 * 70 * 2 * (d / g) : sc == 0);
          }
  const int64_t big[] = {INT64_MAX, INT64_MAX / 2, (int64_t)1 << 40, (int64_t)1 << 31, -1};
  for (int64_t B : big)
    for (int64_t T : big) {
      srftq_shape s = {B, T, 65535, 256, 16, 4, SRFTQ_ROT_SRFT, 0};
      (void)srftq_validate(&s);
      (void)srftq_codes_bytes(&s);
      (void)srftq_attention_workspace_bytes(&s, 16);
    }

  // quantize / dequantize: errors return before the stub, a good call reaches it
  g_launches = 0;
  EXPECT(srftq_quantize(&ok, nullptr, nullptr, nullptr, (uint8_t*)a, (uint16_t*)a, nullptr) == SRFTQ_ERR_NULL);
  EXPECT(srftq_quantize(&ok, (uint16_t*)mis, nullptr, nullptr, (uint8_t*)a, (uint16_t*)a, nullptr) == SRFTQ_ERR_ALIGN);
  EXPECT(srftq_quantize(&ok, (uint16_t*)a, (int8_t*)(buf + 1), nullptr, (uint8_t*)a, (uint16_t*)a, nullptr) ==
         SRFTQ_ERR_ALIGN);
  EXPECT(g_launches == 0);
  EXPECT(srftq_quantize(&ok, (uint16_t*)a, nullptr, (float*)a, (uint8_t*)a, (uint16_t*)a, nullptr) == SRFTQ_OK);
  EXPECT(g_launches == 1 && g_last.x == a && g_last.signs == g_ones && g_last.signs_shared && g_last.lambda == a);
  EXPECT(srftq_dequantize(&ok, (uint8_t*)a, (uint16_t*)a, (int8_t*)a, nullptr, (uint16_t*)a, nullptr) == SRFTQ_OK);
  EXPECT(g_launches == 2 && !g_last.signs_shared && g_last.codes_in == a);
  // empty problems launch nothing
  srftq_shape empty = ok;
  empty.T = 0;
  g_launches = 0;
  EXPECT(srftq_quantize(&empty, (uint16_t*)a, nullptr, nullptr, (uint8_t*)a, (uint16_t*)a, nullptr) == SRFTQ_OK);
  EXPECT(srftq_dequantize(&empty, (uint8_t*)a, (uint16_t*)a, nullptr, nullptr, (uint16_t*)a, nullptr) == SRFTQ_OK);
  EXPECT(g_launches == 0);

  // cache append / read
  g_launches = 0;
  EXPECT(srftq_cache_append(&ok, -1, nullptr, (uint16_t*)a, nullptr, nullptr, (uint8_t*)a, (uint16_t*)a, nullptr) ==
         SRFTQ_ERR_SHAPE);
  EXPECT(srftq_cache_append(&ok, 50, (int32_t*)(buf + 2), (uint16_t*)a, nullptr, nullptr, (uint8_t*)a, (uint16_t*)a,
                            nullptr) == SRFTQ_ERR_ALIGN);
  EXPECT(g_launches == 0);
  EXPECT(srftq_cache_append(&ok, 50, (int32_t*)a, (uint16_t*)a, nullptr, nullptr, (uint8_t*)a, (uint16_t*)a,
                            nullptr) == SRFTQ_OK);
  EXPECT(g_launches == 1 && g_last.pitch == 50 && g_last.pos == a);
  EXPECT(srftq_cache_read(&ok, 99, (uint8_t*)a, (uint16_t*)a, nullptr, nullptr, (uint16_t*)a, nullptr) ==
         SRFTQ_ERR_SHAPE);

  // rotate / unrotate / calibrate
  EXPECT(srftq_rotate(&ok, (uint16_t*)a, nullptr, (float*)a, nullptr) == SRFTQ_OK);
  EXPECT(srftq_unrotate(&ok, (float*)a, nullptr, (uint16_t*)a, nullptr) == SRFTQ_OK);
  EXPECT(srftq_calibrate_lambda(&ok, (uint16_t*)a, nullptr, (float*)a, nullptr) == SRFTQ_OK);
  EXPECT(srftq_rotate(&ok, nullptr, nullptr, (float*)a, nullptr) == SRFTQ_ERR_NULL);

  // decode attention, with a workspace and with the deferred scratch
  const srftq_cache_view kv = {(uint8_t*)a, (uint16_t*)a, nullptr, nullptr};
  const size_t need = srftq_attention_workspace_bytes(&ok, 6);
  EXPECT(need > 0 && need <= sizeof buf);
  g_launches = 0;
  EXPECT(srftq_decode_attention(&ok, 100, 6, (uint16_t*)a, &kv, &kv, nullptr, 0.1f, (float*)a, a, need - 1,
                                nullptr) == SRFTQ_ERR_SHAPE);
  EXPECT(srftq_decode_attention(&ok, 100, 17, (uint16_t*)a, &kv, &kv, nullptr, 0.1f, (float*)a, a, need,
                                nullptr) == SRFTQ_ERR_SHAPE);
  EXPECT(g_launches == 0);
  EXPECT(srftq_decode_attention(&ok, 100, 6, (uint16_t*)a, &kv, &kv, nullptr, 0.1f, (float*)a, a, need, nullptr) ==
         SRFTQ_OK);
  EXPECT(g_launches == 1 && (void*)g_attn.uq == a && g_attn.signs_k == g_ones && g_attn.geo.R == 6);
  EXPECT((char*)g_attn.ws_acc + 4 <= (char*)a + need);
  EXPECT(srftq::decode_attention_scratch(&ok, 100, 6, (uint16_t*)a, &kv, &kv, nullptr, 0.1f, (float*)a,
                                         sizeof g_scratch, scratch_fn, nullptr) == SRFTQ_OK);
  EXPECT(g_launches == 2 && (void*)g_attn.uq == g_scratch);
  EXPECT(srftq::decode_attention_scratch(&ok, 100, 6, (uint16_t*)a, &kv, &kv, nullptr, 0.1f, (float*)a, need - 1,
                                         scratch_fn, nullptr) == SRFTQ_ERR_CAPACITY);
  EXPECT(srftq::decode_attention_scratch(&ok, 100, 6, nullptr, &kv, &kv, nullptr, 0.1f, (float*)a,
                                         sizeof g_scratch, scratch_fn, nullptr) == SRFTQ_ERR_NULL);
  EXPECT(g_launches == 2);

  // rotations given as matrices
  srftq_shape dn = ok;
  dn.group = 16;
  EXPECT(srftq_quantize_dense(&dn, (float*)a, 0, (uint16_t*)a, nullptr, nullptr, (uint8_t*)a, (uint16_t*)a,
                              nullptr) == SRFTQ_OK);
  EXPECT(g_dense.quantize && g_dense.Q == a && g_dense.sign_stride == 0);
  EXPECT(srftq_quantize_dense(&dn, (float*)a, 7, (uint16_t*)a, nullptr, nullptr, (uint8_t*)a, (uint16_t*)a,
                              nullptr) == SRFTQ_ERR_SHAPE);
  EXPECT(srftq_dequantize_dense(&dn, nullptr, 0, (uint8_t*)a, (uint16_t*)a, nullptr, nullptr, (uint16_t*)a,
                                nullptr) == SRFTQ_ERR_NULL);
  EXPECT(srftq_householder_matrix(257, 4, 2, (float*)a, (float*)a, nullptr) != SRFTQ_OK);
  EXPECT(srftq_householder_matrix(128, 64, 2, (float*)a, (float*)a, nullptr) == SRFTQ_OK);
  EXPECT(srftq_decode_attention_dense(&dn, 100, 6, (float*)a, (float*)a, 0, (uint16_t*)a, &kv, &kv, nullptr, 0.1f,
                                      (float*)a, a, need, nullptr) == SRFTQ_OK);

  for (int st = 0; st < 8; ++st) EXPECT(srftq_status_string((srftq_status)st) != nullptr);
  if (fails) return 1;
  std::printf("abi driver: ok\n");
  return 0;
}
