/*
 * srftq.h -- C ABI of libsrftq: fused sign-randomized Fourier (SRFT) or
 * Walsh-Hadamard (SRHT) rotation + int4/int8 quantization of KV-cache
 * vectors, and the inverse, on AMD Instinct MI355X (gfx950).
 *
 * The operation is the one described in "When Quantization Is Free: an int4
 * KV cache that outruns fp16 on Apple Silicon" (gist.science technical
 * summary), section "Metodologia":
 *   1. SRFT(x) = pack(F diag(s) x): F the unitary DFT, s a fixed random +-1
 *      vector; the Hadamard variant (SRHT) replaces F by the normalized
 *      Walsh-Hadamard matrix (also the per-tile RHT = H D x of the HyperQuant
 *      summary, "Metodologia" 1).
 *   2. The fused pipeline: sign multiply; FFT; Hermitian unpack to reals;
 *      per-channel lambda rescale, per-group absmax and rounding to signed
 *      int4/int8; two int4 per byte.
 *   3. Per-channel + per-group scaling (groups of 16 in the pages).
 *
 * Conventions fixed by this library (the pages are silent on them):
 *   - F uses e^{-2 pi i jk/d} and 1/sqrt(d).  The d/2+1 Hermitian bins are
 *     packed into d orthonormal reals
 *       y = [Re X_0, sqrt2 Re X_1 .. sqrt2 Re X_{N-1}, Re X_N,
 *            sqrt2 Im X_1 .. sqrt2 Im X_{N-1}],  N = d/2.
 *     SRHT: y = H_d (s . x) / sqrt(d), H_d in Sylvester (natural) order.
 *   - z_j = lambda_j * y_j.  Per group G of `group` consecutive coordinates
 *     the definition is
 *       a = max |z_j|, sigma = fp16_rne(min(a / qmax, 65504)),
 *       q_j = 0 if sigma == 0 else clamp(rne(z_j / sigma), -qmax, qmax),
 *     qmax = 7 (bits 4) or 127 (bits 8), the codes taken against the stored
 *     fp16 sigma.  The kernels compute it in fp32: z, a and a * fp32(1/qmax)
 *     in fp32, and the quotient as the exact product z_j * r rounded half to
 *     even, r = fp32(1/sigma) correctly rounded.  r differs from 1/sigma by
 *     at most 2^-24 relative, so a code can differ from the definition's
 *     only where z_j / sigma lies within 2^-24 * |z_j / sigma| (plus the
 *     fp32 rotation error) of a half-integer, and then by +-1; sigma = 1/2^k
 *     makes r exact, so exact ties then round to even as defined.
 *   - int4 codes: two's-complement nibbles, coordinate 2i in the low nibble
 *     of byte i.  int8 codes: one two's-complement byte per coordinate.
 *   - Dequantize: yhat_j = q_j * sigma_G / lambda_j, x = s . (M^T yhat),
 *     stored as fp16 round-to-nearest-even.
 *
 * Memory layout (row-major, contiguous, element = fp16 / int8 / byte):
 *   x, x_out   fp16   [B, T, H, d]        (B tensors, e.g. layers x {K,V})
 *   signs      int8   [B, H, d]  values +1 / -1   (NULL: all +1)
 *   lambda     fp32   [B, H, d]  finite, > 0      (NULL: all 1)
 *   codes      uint8  [B, H, T, d*bits/8]   head-major quantized cache
 *   scales     fp16   [B, H, T, d/group]   head-major quantized cache
 *   y          fp32   [B, T, H, d]   (rotate / unrotate only)
 * The quantized cache is head-major: vector (b, t, h) of x is row
 * (b*H + h)*T + t of codes and scales, so each head's tokens are one
 * contiguous run (the order in which attention reads a per-head cache; the
 * pages fix no layout).
 *
 * Ownership and threading: every buffer belongs to the caller; the library
 * allocates nothing on the device, keeps no per-call state and may be called
 * from several host threads.  All data pointers are device pointers
 * (hipMalloc'ed or torch CUDA tensors).  `stream` is a hipStream_t passed as
 * void* (NULL = the default stream); calls are asynchronous on it.
 *
 * Errors: argument errors (NULL pointer, bad shape, unsupported
 * combination, misalignment) are returned before anything is launched and
 * leave every buffer untouched.  SRFTQ_ERR_HIP reports a failed launch or a
 * missing device; faults inside a kernel surface at the caller's next
 * synchronization.  lambda > 0 and finite inputs are preconditions that are
 * not checked on the device.
 */
#ifndef SRFTQ_H
#define SRFTQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SRFTQ_OK = 0,
    SRFTQ_ERR_NULL = 1,        /* a required pointer is NULL */
    SRFTQ_ERR_SHAPE = 2,       /* negative or inconsistent sizes */
    SRFTQ_ERR_UNSUPPORTED = 3, /* (rot, d, group, bits) combination not built */
    SRFTQ_ERR_ALIGN = 4,       /* a data pointer is not 16-byte aligned */
    SRFTQ_ERR_HIP = 5,         /* HIP runtime error (launch failure, no device) */
    SRFTQ_ERR_CAPACITY = 6     /* needs more scratch than the library's fixed buffer
                                  (srftq_decode_attention_noalloc only) */
} srftq_status;

typedef enum {
    SRFTQ_ROT_SRFT = 0, /* sign-randomized unitary DFT, packed to d reals */
    SRFTQ_ROT_SRHT = 1, /* sign-randomized Walsh-Hadamard (Sylvester order) */
    SRFTQ_ROT_NONE = 2  /* sign multiply only: isolates the quantizer */
} srftq_rot;

/*
 * Problem description.  Supported: d in {64, 96, 128, 256}; bits in {4, 8};
 * group a power of two with 8 <= group <= d dividing d; rot one of
 * srftq_rot; B, T >= 0, H >= 1 (B*T*H == 0 is a no-op).  `variant` selects
 * the SRFT kernel organisation: 0 = default (fastest), 1 = real-input
 * radix-2 transform, 2 = complex pairing + d/2-point complex FFT + Hermitian
 * unpack; it is ignored for SRHT and NONE.  Every variant computes the same
 * result.  d = 96 (a head size that is not a power of two: the SRFT is
 * defined for any even d, "When Quantization Is Free", Metodologia 1, unlike
 * the Walsh-Hadamard transform) takes the real-input transform with one
 * radix-3 step, for rot SRFT (variants 0 and 1) and NONE; SRHT and variant 2
 * need a power of two and return SRFTQ_ERR_UNSUPPORTED.  Decode attention
 * supports every d above, with the same rotations.
 */
typedef struct {
    int64_t B;
    int64_t T;
    int32_t H;
    int32_t d;
    int32_t group;
    int32_t bits;
    int32_t rot;
    int32_t variant;
} srftq_shape;

/* Host-only check of a shape (no device needed). */
srftq_status srftq_validate(const srftq_shape* shape);

/* Bytes of the codes tensor: B*T*H*d*bits/8.  0 for an invalid shape. */
size_t srftq_codes_bytes(const srftq_shape* shape);

/* Number of fp16 scales: B*T*H*d/group.  0 for an invalid shape. */
size_t srftq_scales_count(const srftq_shape* shape);

/*
 * Rotate-then-quantize (pipeline steps 1-5 above).
 *   x       in   fp16 [B,T,H,d], 16-B aligned
 *   signs   in   int8 [B,H,d] or NULL
 *   lambda  in   fp32 [B,H,d] or NULL
 *   codes   out  uint8 [B,H,T,d*bits/8], 16-B aligned
 *   scales  out  fp16 [B,H,T,d/group], 16-B aligned
 */
srftq_status srftq_quantize(const srftq_shape* shape, const uint16_t* x,
                            const int8_t* signs, const float* lambda,
                            uint8_t* codes, uint16_t* scales, void* stream);

/*
 * Dequantize + unrotate (the inverse read path, "rotation and de-rotation"
 * in the pages' problem statement).
 *   codes, scales  in   [B,H,T,.] as written by srftq_quantize (16-B aligned)
 *   signs, lambda  in   the same ones used to quantize (or NULL)
 *   x_out          out  fp16 [B,T,H,d], 16-B aligned
 */
srftq_status srftq_dequantize(const srftq_shape* shape, const uint8_t* codes,
                              const uint16_t* scales, const int8_t* signs,
                              const float* lambda, uint16_t* x_out, void* stream);

/*
 * The rotation alone (steps 1-3): y = M (s . x) in fp32, no lambda.
 *   x  in  fp16 [B,T,H,d];  y  out  fp32 [B,T,H,d]; both 16-B aligned.
 */
srftq_status srftq_rotate(const srftq_shape* shape, const uint16_t* x,
                          const int8_t* signs, float* y, void* stream);

/*
 * The inverse rotation alone: x_out = fp16_rne(s . (M^T y)).
 *   y  in  fp32 [B,T,H,d];  x_out  out  fp16 [B,T,H,d]; both 16-B aligned.
 */
srftq_status srftq_unrotate(const srftq_shape* shape, const float* y,
                            const int8_t* signs, uint16_t* x_out, void* stream);

/*
 * Per-channel lambda calibration (the pages' "learned or calibrated" lambda,
 * read as the inverse RMS over tokens of each rotated coordinate):
 *   lambda[b,h,j] = 1 / sqrt(mean_t y[b,t,h,j]^2), or 1 where that is 0.
 *   x  in  fp16 [B,T,H,d];  lambda  out  fp32 [B,H,d] (also used as the
 *   accumulator, so it must not alias x).  `group`, `bits` are ignored.
 */
srftq_status srftq_calibrate_lambda(const srftq_shape* shape, const uint16_t* x,
                                    const int8_t* signs, float* lambda, void* stream);

/*
 * Quantize-on-append into a preallocated cache (the pages integrate the
 * fused kernel as a growing int4 KV cache: a HuggingFace Cache subclass,
 * "When Quantization Is Free", Metodologia section 2).  The new tokens
 * x [B,T,H,d] (T tokens per tensor, e.g. T = 1 per decode step) are rotated
 * and quantized exactly as by srftq_quantize, and token t of tensor b is
 * written to row pos[b] + t of each of its heads in the caches
 *   codes   [B,H,t_cap,d*bits/8]   scales  [B,H,t_cap,d/group]
 * (the head-major layout of srftq_quantize with t_cap rows per head).
 *   pos     in  int32 [B] on the device (4-B aligned), or NULL for row t.
 *           Read on the device when the kernel runs, so a decode loop can
 *           advance it on the stream without a host round trip.
 *   Rows outside [0, t_cap) are not written (their tokens are dropped);
 *   every other row of the caches is left as it was.
 *   t_cap   >= 0 (0: nothing is written).  Other arguments, alignment and
 *           errors as for srftq_quantize.
 */
srftq_status srftq_cache_append(const srftq_shape* shape, int64_t t_cap, const int32_t* pos,
                                const uint16_t* x, const int8_t* signs, const float* lambda,
                                uint8_t* codes, uint16_t* scales, void* stream);

/*
 * Read the first T rows of every head of a cache written by
 * srftq_cache_append (t_cap rows per head, T <= t_cap, else
 * SRFTQ_ERR_SHAPE): dequantize + unrotate as srftq_dequantize, into
 * x_out fp16 [B,T,H,d].  With t_cap == T this is srftq_dequantize.
 */
srftq_status srftq_cache_read(const srftq_shape* shape, int64_t t_cap, const uint8_t* codes,
                              const uint16_t* scales, const int8_t* signs, const float* lambda,
                              uint16_t* x_out, void* stream);

/*
 * Decode attention over the quantized cache: for each tensor b and query
 * head r (query heads h*R .. h*R+R-1 share KV head h), with one new query
 * token per tensor,
 *   out[b, r] = sum_{t < len_b} softmax_t(scale * q[b, r] . k^[b, t, h]) v^[b, t, h]
 * where k^, v^ are the exact reconstructions s (.) M^T (c sigma / lambda)
 * of the cached codes (srftq_dequantize before its fp16 rounding).  The
 * pages' cache exists to be read by attention at every decode step, moving
 * a third of the fp16 bytes ("When Quantization Is Free", Resultados Clave:
 * the bandwidth saving is where the speed-up comes from); here attention
 * reads the codes directly and never materializes k^ or v^: scores are
 * taken against the rotated query M (s_k . q), the output is accumulated in
 * the rotated domain and unrotated once per query head.
 *   shape      B tensors, T = most tokens attended (<= t_cap), H KV heads,
 *              d, group (>= 16), bits, rot as the caches were written;
 *              variant is ignored.
 *   q_per_kv   R, query heads per KV head, 1..16.
 *   q          fp16 [B, H*R, d], 16-B aligned.
 *   k, v       the K and V caches: codes [B,H,t_cap,d*bits/8] and scales
 *              [B,H,t_cap,d/group] (16-B aligned), signs and lambda
 *              [B,H,d] or NULL, as written by srftq_cache_append /
 *              srftq_quantize.
 *   lengths    int32 [B] on the device (4-B aligned): tokens attended per
 *              tensor, clamped to [0, T]; NULL = T for every tensor.  A
 *              tensor with no tokens gets a zero output.
 *   scale      softmax scale (e.g. 1/sqrt(d)), finite.
 *   out        fp32 [B, H*R, d], 16-B aligned.
 *   workspace  device memory of at least srftq_attention_workspace_bytes
 *              (16-B aligned), owned by the caller; contents on entry are
 *              ignored.  Calls that share a workspace must not overlap.
 * The P.V product multiplies fp16(c_v * sigma_v) by fp16(2^14 p) (two
 * fp16 roundings per term, as attention kernels round P); every other step
 * is fp32.  Errors as for
 * srftq_quantize; a short workspace is SRFTQ_ERR_SHAPE.
 */
typedef struct {
    const uint8_t*  codes;
    const uint16_t* scales;
    const int8_t*   signs;
    const float*    lambda;
} srftq_cache_view;

size_t srftq_attention_workspace_bytes(const srftq_shape* shape, int32_t q_per_kv);

srftq_status srftq_decode_attention(const srftq_shape* shape, int64_t t_cap, int32_t q_per_kv,
                                    const uint16_t* q, const srftq_cache_view* k,
                                    const srftq_cache_view* v, const int32_t* lengths,
                                    float scale, float* out, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * srftq_decode_attention_noalloc: srftq_decode_attention for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The workspace is the library's
 * own static device array of SRFTQ_ATTENTION_SCRATCH_BYTES, one copy per
 * GPU, held until the process ends; the caller passes inputs and outputs
 * only.  Every other argument, layout and error as for
 * srftq_decode_attention; a shape whose srftq_attention_workspace_bytes
 * exceeds SRFTQ_ATTENTION_SCRATCH_BYTES is SRFTQ_ERR_CAPACITY, returned
 * before anything is launched.  The call allocates nothing (no hipMalloc,
 * no allocating library routine); on a device's first call it looks up the
 * array's address on that device (hipGetSymbolAddress).  Each call writes
 * every scratch byte it reads, so nothing needs clearing between calls; but
 * all calls on one GPU share the one array, so calls that overlap on one GPU
 * (several streams or host threads at once) race and give wrong results:
 * serialize them, or use srftq_decode_attention with a workspace each.
 */
#define SRFTQ_ATTENTION_SCRATCH_BYTES ((size_t)16 << 20)

srftq_status srftq_decode_attention_noalloc(const srftq_shape* shape, int64_t t_cap, int32_t q_per_kv,
                                            const uint16_t* q, const srftq_cache_view* k,
                                            const srftq_cache_view* v, const int32_t* lengths,
                                            float scale, float* out, void* stream);

/*
 * Rotations given as a matrix.  "When Quantization Is Free", Metodologia 3,
 * studies replacing or extending the fixed SRFT by a learned rotation R
 * (calibrated together with lambda) and by Householder rotations, k = d/2
 * reflectors at d = 256.  Either is an orthogonal d x d matrix Q, and the
 * quantizer is then the one above applied to y = Q (s . x):
 *   z_j = lambda_j y_j, per-group sigma and rounding exactly as srftq_quantize,
 *   and dequantize: x = s . (Q^T yhat), yhat_j = q_j sigma_G / lambda_j.
 * (The SRFT itself is the matrix whose columns are srftq_rotate of the unit
 * vectors; a learned R on top of it is the product R M.)
 *
 * srftq_householder_matrix: Q_m = H_1 H_2 ... H_k for m < n, with
 *   H_i = I - 2 v_i v_i^T / (v_i . v_i) (a zero v_i is the identity),
 *   computed in fp64 and rounded to fp32.
 *   d     1..256;  k  0..1024;  n  0..65535 matrices.
 *   V     in   fp32 [n, k, d] device, 4-B aligned (may be NULL when k = 0)
 *   Q     out  fp32 [n, d, d] device, 4-B aligned, row-major
 *
 * srftq_quantize_dense / srftq_dequantize_dense: as srftq_quantize /
 * srftq_dequantize (same layouts, alignment and errors) with
 *   Q         in  fp32 row-major d x d matrices, 16-B aligned; head h of
 *                 tensor b uses Q + (b*H + h) * q_stride
 *   q_stride  0 (one matrix for every head) or >= d*d, a multiple of 4
 *             (else SRFTQ_ERR_SHAPE)
 * Supported: d in {64, 128, 256}, group in {8, 16, 32}, bits in {4, 8};
 * shape.rot and shape.variant are ignored.  Q is used as given: dequantize
 * inverts quantize only when Q is orthogonal.  The product runs on the
 * matrix cores with Q split into two fp16 parts (about 22 significant bits),
 * x exact in fp16 and fp32 sums; dequantize splits yhat the same way.
 */
srftq_status srftq_householder_matrix(int32_t d, int32_t k, int64_t n, const float* V, float* Q,
                                     void* stream);

srftq_status srftq_quantize_dense(const srftq_shape* shape, const float* Q, int64_t q_stride,
                                  const uint16_t* x, const int8_t* signs, const float* lambda,
                                  uint8_t* codes, uint16_t* scales, void* stream);

srftq_status srftq_dequantize_dense(const srftq_shape* shape, const float* Q, int64_t q_stride,
                                    const uint8_t* codes, const uint16_t* scales,
                                    const int8_t* signs, const float* lambda, uint16_t* x_out,
                                    void* stream);

/*
 * srftq_decode_attention_dense: srftq_decode_attention over K and V caches
 * written by srftq_quantize_dense (a learned or Householder rotation,
 * Metodologia 3): k^ = s_k . (Qk^T yhat_k), v^ = s_v . (Qv^T yhat_v).  The
 * scores are taken against Qk (s_k . q) and the output is unrotated by Qv^T
 * once per query head; the scoring kernel is the same as for the transforms.
 *   Qk, Qv     fp32 row-major d x d matrices (16-B aligned; may be the same),
 *              head h of tensor b at Q + (b*H + h) * q_stride
 *   q_stride   as for srftq_quantize_dense
 * Every other argument, the workspace (srftq_attention_workspace_bytes of
 * the same shape) and the errors as for srftq_decode_attention; the sizes of
 * srftq_quantize_dense with group >= 16; shape.rot and shape.variant are
 * ignored.  The query rotation and the unrotation run in fp32.
 */
srftq_status srftq_decode_attention_dense(const srftq_shape* shape, int64_t t_cap, int32_t q_per_kv,
                                          const float* Qk, const float* Qv, int64_t q_stride,
                                          const uint16_t* q, const srftq_cache_view* k,
                                          const srftq_cache_view* v, const int32_t* lengths,
                                          float scale, float* out, void* workspace,
                                          size_t workspace_bytes, void* stream);

/* Static description of a status code. */
const char* srftq_status_string(srftq_status status);

/* Library version, major*10000 + minor*100 + patch. */
int srftq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SRFTQ_H */
