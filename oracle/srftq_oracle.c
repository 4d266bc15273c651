/*
 * srftq_oracle.c -- plain, slow, obviously-correct CPU oracle for the
 * sign-randomized rotate-then-quantize of KV-cache vectors.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The GPU library
 * never calls it and shares no code, header, table or constant with it.
 *
 * Source: "When Quantization Is Free: an int4 KV cache that outruns fp16 on
 * Apple Silicon" (gist.science technical summary, Spanish and French pages),
 * section "Metodologia": 1 (the SRFT definition SRFT(x) = pack(F diag(s) x),
 * F the unitary DFT, s fixed random signs) and 2 (the pipeline order: sign
 * multiply, FFT, Hermitian unpack to reals, per-channel lambda rescale,
 * per-group absmax, rounding to signed int4/int8, two int4 per byte), and
 * 3 (per-channel + per-group scaling, groups of 16).  The SRHT variant is the
 * Walsh-Hadamard alternative named in the same section 1, with the per-tile
 * form RHT(x) = H D x from the HyperQuant summary, "Metodologia" 1.
 *
 * Everything here follows the plain definitions:
 *   - the DFT is an O(d^2) direct sum in fp64 (no FFT);
 *   - the Walsh-Hadamard transform is a direct +-1 sum in fp64, Sylvester
 *     (natural) order, entry (j,k) = (-1)^popcount(j & k);
 *   - the quantizer is a scalar loop;
 *   - a rotation given as a matrix (the learned and Householder rotations
 *     of section 3) is a direct fp64 matrix-vector sum over its fp32
 *     entries, y = Q (s . x), and its transpose for the inverse.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - DFT sign e^{-2 pi i jk/d}; unitary 1/sqrt(d).
 *   - Packing of the d/2+1 Hermitian bins into d reals:
 *       y = [Re X_0, sqrt2 Re X_1 .. sqrt2 Re X_{N-1}, Re X_N,
 *            sqrt2 Im X_1 .. sqrt2 Im X_{N-1}],  N = d/2
 *     which makes the map orthonormal.
 *   - lambda multiplies the rotated coordinate (after the unpack);
 *     dequantization divides by it.
 *   - Symmetric code range [-qmax, qmax], qmax = 7 (int4) or 127 (int8).
 *   - The quantizer is the plain definition, in fp64: z = lambda * y;
 *     a = max |z| over the group; sigma = fp16 round-to-nearest-even of
 *     min(a / qmax, 65504), stored; q = 0 if sigma == 0, else
 *     clamp(rne(z / sigma), -qmax, qmax), the quotient taken against the
 *     stored fp16 sigma and rounded half to even.
 *   - int4 nibbles are two's complement, even coordinate in the low nibble.
 *   - signs == NULL means s = +1; lambda == NULL means lambda = 1.
 *
 * Layouts (all row-major, contiguous).  The quantized cache is stored
 * head-major (the pages fix no layout): vector (b, t, h) of x is row
 * (b*H + h)*T + t of codes and scales.
 *   x, x_out   fp16 bits  [B, T, H, d]
 *   y          fp64       [B, T, H, d]
 *   signs      int8 +-1   [B, H, d]
 *   lambda     fp32       [B, H, d]
 *   codes      uint8      [B, H, T, d*bits/8]
 *   scales     fp16 bits  [B, H, T, d/group]
 *   z_out      fp64       [B, H, T, d]   (rows aligned with codes)
 *   Q          fp32       row-major d x d at Q + (b*H + h) * q_stride
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_ROT_SRFT 0
#define ORACLE_ROT_SRHT 1
#define ORACLE_ROT_NONE 2

static const double ORACLE_PI = 3.14159265358979323846264338327950288;

/* ---------------------------------------------------------------------- */
/* IEEE 754 binary16 <-> binary64, written from the format definition.     */
/* ---------------------------------------------------------------------- */

double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);               /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m | 0x400), e - 25);  /* (1024+m) * 2^(e-15-10) */
    return sign ? -v : v;
}

/* Correctly rounded (round to nearest, ties to even) binary64 -> binary16. */
uint16_t oracle_f64_to_f16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v))
        return 0x7e00;
    if (a >= 65520.0)                     /* halfway to 2^16 and above -> inf */
        return sign | 0x7c00;
    if (a < ldexp(1.0, -14)) {            /* subnormal range, quantum 2^-24 */
        double r = nearbyint(ldexp(a, 24)); /* r <= 1024; 1024 = min normal */
        return sign | (uint16_t)r;
    }
    int e;
    frexp(a, &e);                         /* a = f * 2^e, f in [0.5, 1) */
    double r = nearbyint(ldexp(a, 11 - e)); /* significand in [1024, 2048] */
    int E = e - 1 + 15;
    if (r >= 2048.0) {
        r = 1024.0;
        E += 1;
    }
    if (E >= 31)
        return sign | 0x7c00;
    return sign | (uint16_t)(E << 10) | (uint16_t)((int)r - 1024);
}

/* ---------------------------------------------------------------------- */
/* The rotation of one vector, by definition.                              */
/* ---------------------------------------------------------------------- */

static int popcount_u32(uint32_t v)
{
    int c = 0;
    while (v) {
        c += (int)(v & 1u);
        v >>= 1;
    }
    return c;
}

/* cos/sin of 2*pi*m/d for m in [0, d). */
static void twiddle_table(int d, double *cs, double *sn)
{
    for (int m = 0; m < d; ++m) {
        double ang = 2.0 * ORACLE_PI * (double)m / (double)d;
        cs[m] = cos(ang);
        sn[m] = sin(ang);
    }
}

/* y = M xs  where xs = s (.) x already holds the sign-multiplied input. */
static void rotate_one(int d, int rot, const double *xs, double *y,
                       const double *cs, const double *sn)
{
    double inv = 1.0 / sqrt((double)d);
    if (rot == ORACLE_ROT_NONE) {
        for (int j = 0; j < d; ++j)
            y[j] = xs[j];
        return;
    }
    if (rot == ORACLE_ROT_SRHT) {
        for (int k = 0; k < d; ++k) {
            double acc = 0.0;
            for (int j = 0; j < d; ++j)
                acc += (popcount_u32((uint32_t)(j & k)) & 1) ? -xs[j] : xs[j];
            y[k] = inv * acc;
        }
        return;
    }
    /* SRFT: unitary DFT bins 0..N, then the orthonormal real packing. */
    int N = d / 2;
    double r2 = sqrt(2.0);
    for (int k = 0; k <= N; ++k) {
        double re = 0.0, im = 0.0;
        for (int j = 0; j < d; ++j) {
            int m = (int)(((long long)j * k) % d);
            re += xs[j] * cs[m];
            im -= xs[j] * sn[m];
        }
        re *= inv;
        im *= inv;
        if (k == 0) {
            y[0] = re;
        } else if (k == N) {
            y[N] = re;
        } else {
            y[k] = r2 * re;
            y[N + k] = r2 * im;
        }
    }
}

/* xs = M^T y: rebuild the Hermitian spectrum and take the unitary inverse DFT. */
static void unrotate_one(int d, int rot, const double *y, double *xs,
                         const double *cs, const double *sn)
{
    double inv = 1.0 / sqrt((double)d);
    if (rot == ORACLE_ROT_NONE) {
        for (int j = 0; j < d; ++j)
            xs[j] = y[j];
        return;
    }
    if (rot == ORACLE_ROT_SRHT) {
        for (int j = 0; j < d; ++j) {
            double acc = 0.0;
            for (int k = 0; k < d; ++k)
                acc += (popcount_u32((uint32_t)(j & k)) & 1) ? -y[k] : y[k];
            xs[j] = inv * acc;
        }
        return;
    }
    int N = d / 2;
    double ir2 = 1.0 / sqrt(2.0);
    double *Xr = (double *)malloc(sizeof(double) * (size_t)d);
    double *Xi = (double *)malloc(sizeof(double) * (size_t)d);
    Xr[0] = y[0];
    Xi[0] = 0.0;
    Xr[N] = y[N];
    Xi[N] = 0.0;
    for (int k = 1; k < N; ++k) {
        Xr[k] = y[k] * ir2;
        Xi[k] = y[N + k] * ir2;
        Xr[d - k] = Xr[k];
        Xi[d - k] = -Xi[k];
    }
    for (int j = 0; j < d; ++j) {
        double acc = 0.0;
        for (int k = 0; k < d; ++k) {
            int m = (int)(((long long)j * k) % d);
            /* Re( X_k e^{+i 2 pi jk/d} ) */
            acc += Xr[k] * cs[m] - Xi[k] * sn[m];
        }
        xs[j] = inv * acc;
    }
    free(Xr);
    free(Xi);
}

static int check_shape(int64_t B, int64_t T, int H, int d, int rot)
{
    if (B < 0 || T < 0 || H <= 0 || d <= 1)
        return 2;
    if (rot != ORACLE_ROT_SRFT && rot != ORACLE_ROT_SRHT && rot != ORACLE_ROT_NONE)
        return 3;
    if (rot == ORACLE_ROT_SRFT && (d % 2) != 0)
        return 3;
    if (rot == ORACLE_ROT_SRHT && (d & (d - 1)) != 0)
        return 3;
    return 0;
}

static double sign_of(const int8_t *signs, int64_t b, int H, int h, int d, int j)
{
    if (!signs)
        return 1.0;
    return signs[((size_t)b * H + h) * d + j] < 0 ? -1.0 : 1.0;
}

/* y[B,T,H,d] (fp64) = M (s (.) x) for every vector. */
int oracle_rotate(int64_t B, int64_t T, int H, int d, int rot,
                  const uint16_t *x, const int8_t *signs, double *y)
{
    int st = check_shape(B, T, H, d, rot);
    if (st)
        return st;
    int64_t nvec = B * T * H;
    double *cs = (double *)malloc(sizeof(double) * (size_t)d);
    double *sn = (double *)malloc(sizeof(double) * (size_t)d);
    twiddle_table(d, cs, sn);
#pragma omp parallel
    {
        double *xs = (double *)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(static)
        for (int64_t v = 0; v < nvec; ++v) {
            int h = (int)(v % H);
            int64_t b = v / (T * H);
            for (int j = 0; j < d; ++j)
                xs[j] = sign_of(signs, b, H, h, d, j) *
                        oracle_f16_to_f64(x[(size_t)v * d + j]);
            rotate_one(d, rot, xs, y + (size_t)v * d, cs, sn);
        }
        free(xs);
    }
    free(cs);
    free(sn);
    return 0;
}

/* x_out[B,T,H,d] (fp64) = s (.) (M^T y) for every vector. */
int oracle_unrotate(int64_t B, int64_t T, int H, int d, int rot,
                    const double *y, const int8_t *signs, double *x_out)
{
    int st = check_shape(B, T, H, d, rot);
    if (st)
        return st;
    int64_t nvec = B * T * H;
    double *cs = (double *)malloc(sizeof(double) * (size_t)d);
    double *sn = (double *)malloc(sizeof(double) * (size_t)d);
    twiddle_table(d, cs, sn);
#pragma omp parallel
    {
        double *xs = (double *)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(static)
        for (int64_t v = 0; v < nvec; ++v) {
            int h = (int)(v % H);
            int64_t b = v / (T * H);
            unrotate_one(d, rot, y + (size_t)v * d, xs, cs, sn);
            for (int j = 0; j < d; ++j)
                x_out[(size_t)v * d + j] = sign_of(signs, b, H, h, d, j) * xs[j];
        }
        free(xs);
    }
    free(cs);
    free(sn);
    return 0;
}

static int check_quant(int d, int group, int bits)
{
    if (bits != 4 && bits != 8)
        return 3;
    if (group <= 0 || group > d || (d % group) != 0)
        return 3;
    if (bits == 4 && (d % 2) != 0)
        return 3;
    return 0;
}

/* Row of vector (b, t, h) in the head-major quantized cache. */
static size_t cache_row(int64_t b, int64_t t, int h, int64_t T, int H)
{
    return ((size_t)b * (size_t)H + (size_t)h) * (size_t)T + (size_t)t;
}

/*
 * A rotation given as a matrix (the learned or Householder rotations of
 * "When Quantization Is Free", Metodologia 3): y = Q xs and its transpose
 * xs = Q^T y, plain fp64 sums over the fp32 entries of Q (row-major d x d).
 */
static void dense_apply(int d, const float *Q, const double *xs, double *y)
{
    for (int i = 0; i < d; ++i) {
        double acc = 0.0;
        for (int j = 0; j < d; ++j)
            acc += (double)Q[(size_t)i * d + j] * xs[j];
        y[i] = acc;
    }
}

static void dense_apply_t(int d, const float *Q, const double *y, double *xs)
{
    for (int j = 0; j < d; ++j) {
        double acc = 0.0;
        for (int i = 0; i < d; ++i)
            acc += (double)Q[(size_t)i * d + j] * y[i];
        xs[j] = acc;
    }
}

/*
 * Quantize every vector.  z_out (optional, fp64 [B,H,T,d]) receives the
 * values z = lambda * y the decision was taken on.  Q (optional) replaces
 * the rotation.
 */
static int quantize_impl(int64_t B, int64_t T, int H, int d, int group, int bits,
                         int rot, const float *Q, int64_t q_stride, const uint16_t *x,
                         const int8_t *signs,
                         const float *lambda, uint8_t *codes, uint16_t *scales,
                         double *z_out)
{
    int st = check_shape(B, T, H, d, rot);
    if (!st)
        st = check_quant(d, group, bits);
    if (st)
        return st;
    int64_t nvec = B * T * H;
    int qmax = (bits == 4) ? 7 : 127;
    int ng = d / group;
    size_t code_row = (size_t)d * (size_t)bits / 8;
    double *cs = (double *)malloc(sizeof(double) * (size_t)d);
    double *sn = (double *)malloc(sizeof(double) * (size_t)d);
    twiddle_table(d, cs, sn);
#pragma omp parallel
    {
        double *xs = (double *)malloc(sizeof(double) * (size_t)d);
        double *y = (double *)malloc(sizeof(double) * (size_t)d);
        double *z = (double *)malloc(sizeof(double) * (size_t)d);
        int *q = (int *)malloc(sizeof(int) * (size_t)d);
#pragma omp for schedule(static)
        for (int64_t v = 0; v < nvec; ++v) {
            int h = (int)(v % H);
            int64_t b = v / (T * H);
            size_t c = cache_row(b, (v / H) % T, h, T, H);
            for (int j = 0; j < d; ++j)
                xs[j] = sign_of(signs, b, H, h, d, j) *
                        oracle_f16_to_f64(x[(size_t)v * d + j]);
            if (Q)
                dense_apply(d, Q + ((size_t)b * H + h) * (size_t)q_stride, xs, y);
            else
                rotate_one(d, rot, xs, y, cs, sn);
            /* per-channel rescale after the rotation */
            for (int j = 0; j < d; ++j) {
                double lam = lambda ? (double)lambda[((size_t)b * H + h) * d + j] : 1.0;
                z[j] = lam * y[j];
            }
            /* per-group absmax scale, stored as fp16; codes against it */
            for (int g = 0; g < ng; ++g) {
                double a = 0.0;
                for (int j = g * group; j < (g + 1) * group; ++j) {
                    double m = fabs(z[j]);
                    if (m > a)
                        a = m;
                }
                double t = a / (double)qmax;
                if (t > 65504.0)
                    t = 65504.0;
                uint16_t sh = oracle_f64_to_f16(t);
                double sg = oracle_f16_to_f64(sh);
                scales[c * ng + g] = sh;
                for (int j = g * group; j < (g + 1) * group; ++j) {
                    if (sg == 0.0) {
                        q[j] = 0;
                    } else {
                        double n = nearbyint(z[j] / sg);   /* ties to even */
                        if (n > (double)qmax)
                            n = (double)qmax;
                        if (n < (double)-qmax)
                            n = (double)-qmax;
                        q[j] = (int)n;
                    }
                }
            }
            uint8_t *row = codes + c * code_row;
            if (bits == 8) {
                for (int j = 0; j < d; ++j)
                    row[j] = (uint8_t)(int8_t)q[j];
            } else {
                for (int i = 0; i < d / 2; ++i)
                    row[i] = (uint8_t)((q[2 * i] & 0xF) | ((q[2 * i + 1] & 0xF) << 4));
            }
            if (z_out)
                memcpy(z_out + c * d, z, sizeof(double) * (size_t)d);
        }
        free(xs);
        free(y);
        free(z);
        free(q);
    }
    free(cs);
    free(sn);
    return 0;
}

int oracle_quantize(int64_t B, int64_t T, int H, int d, int group, int bits,
                    int rot, const uint16_t *x, const int8_t *signs,
                    const float *lambda, uint8_t *codes, uint16_t *scales,
                    double *z_out)
{
    return quantize_impl(B, T, H, d, group, bits, rot, NULL, 0, x, signs, lambda, codes, scales, z_out);
}

/*
 * Quantize with the rotation y = Q_bh (s . x): Q_bh = Q + (b*H + h) * q_stride,
 * row-major d x d fp32 (q_stride 0: one matrix for every head).
 */
int oracle_quantize_dense(int64_t B, int64_t T, int H, int d, int group, int bits,
                          const float *Q, int64_t q_stride, const uint16_t *x, const int8_t *signs,
                          const float *lambda, uint8_t *codes, uint16_t *scales,
                          double *z_out)
{
    if (!Q)
        return 1;
    if (q_stride < 0)
        return 2;
    return quantize_impl(B, T, H, d, group, bits, ORACLE_ROT_NONE, Q, q_stride, x, signs, lambda,
                         codes, scales, z_out);
}

/*
 * Dequantize every vector: yhat_j = q_j * sigma_G / lambda_j (fp64), then
 * x = s (.) M^T yhat (M^T = Q^T when Q is given).  x_out receives fp16 (RNE
 * from fp64); x64_out (optional) receives the fp64 values before that
 * rounding.
 */
static int dequantize_impl(int64_t B, int64_t T, int H, int d, int group, int bits,
                           int rot, const float *Q, int64_t q_stride, const uint8_t *codes,
                           const uint16_t *scales,
                           const int8_t *signs, const float *lambda,
                           uint16_t *x_out, double *x64_out)
{
    int st = check_shape(B, T, H, d, rot);
    if (!st)
        st = check_quant(d, group, bits);
    if (st)
        return st;
    int64_t nvec = B * T * H;
    int ng = d / group;
    size_t code_row = (size_t)d * (size_t)bits / 8;
    double *cs = (double *)malloc(sizeof(double) * (size_t)d);
    double *sn = (double *)malloc(sizeof(double) * (size_t)d);
    twiddle_table(d, cs, sn);
#pragma omp parallel
    {
        double *yh = (double *)malloc(sizeof(double) * (size_t)d);
        double *xs = (double *)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(static)
        for (int64_t v = 0; v < nvec; ++v) {
            int h = (int)(v % H);
            int64_t b = v / (T * H);
            size_t c = cache_row(b, (v / H) % T, h, T, H);
            const uint8_t *row = codes + c * code_row;
            for (int j = 0; j < d; ++j) {
                int qj;
                if (bits == 8) {
                    qj = (int)(int8_t)row[j];
                } else {
                    int nib = (row[j / 2] >> (4 * (j % 2))) & 0xF;
                    qj = nib >= 8 ? nib - 16 : nib;    /* sign-extend */
                }
                double sg = oracle_f16_to_f64(scales[c * ng + j / group]);
                double lam = lambda ? (double)lambda[((size_t)b * H + h) * d + j] : 1.0;
                yh[j] = (double)qj * sg / lam;
            }
            if (Q)
                dense_apply_t(d, Q + ((size_t)b * H + h) * (size_t)q_stride, yh, xs);
            else
                unrotate_one(d, rot, yh, xs, cs, sn);
            for (int j = 0; j < d; ++j) {
                double val = sign_of(signs, b, H, h, d, j) * xs[j];
                if (x64_out)
                    x64_out[(size_t)v * d + j] = val;
                if (x_out)
                    x_out[(size_t)v * d + j] = oracle_f64_to_f16(val);
            }
        }
        free(yh);
        free(xs);
    }
    free(cs);
    free(sn);
    return 0;
}

int oracle_dequantize(int64_t B, int64_t T, int H, int d, int group, int bits,
                      int rot, const uint8_t *codes, const uint16_t *scales,
                      const int8_t *signs, const float *lambda,
                      uint16_t *x_out, double *x64_out)
{
    return dequantize_impl(B, T, H, d, group, bits, rot, NULL, 0, codes, scales, signs, lambda, x_out,
                           x64_out);
}

/* Dequantize with the rotation x = s (.) Q_bh^T yhat (Q_bh as above). */
int oracle_dequantize_dense(int64_t B, int64_t T, int H, int d, int group, int bits,
                            const float *Q, int64_t q_stride, const uint8_t *codes,
                            const uint16_t *scales,
                            const int8_t *signs, const float *lambda,
                            uint16_t *x_out, double *x64_out)
{
    if (!Q)
        return 1;
    if (q_stride < 0)
        return 2;
    return dequantize_impl(B, T, H, d, group, bits, ORACLE_ROT_NONE, Q, q_stride, codes, scales, signs,
                           lambda, x_out, x64_out);
}

/*
 * Per-channel lambda calibration ("learned or calibrated" in the pages'
 * stage 4), read as lambda_{b,h,j} = 1 / RMS_t( y_{b,t,h,j} ) over the
 * rotated coordinates of that tensor; 1 where the RMS is 0.  Stored fp32.
 */
int oracle_calibrate_lambda(int64_t B, int64_t T, int H, int d, int rot,
                            const uint16_t *x, const int8_t *signs, float *lambda)
{
    int st = check_shape(B, T, H, d, rot);
    if (st)
        return st;
    double *cs = (double *)malloc(sizeof(double) * (size_t)d);
    double *sn = (double *)malloc(sizeof(double) * (size_t)d);
    twiddle_table(d, cs, sn);
    int64_t nhead = B * H;
#pragma omp parallel
    {
        double *xs = (double *)malloc(sizeof(double) * (size_t)d);
        double *y = (double *)malloc(sizeof(double) * (size_t)d);
        double *acc = (double *)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(static)
        for (int64_t bh = 0; bh < nhead; ++bh) {
            int64_t b = bh / H;
            int h = (int)(bh % H);
            for (int j = 0; j < d; ++j)
                acc[j] = 0.0;
            for (int64_t t = 0; t < T; ++t) {
                size_t v = (size_t)((b * T + t) * H + h);
                for (int j = 0; j < d; ++j)
                    xs[j] = sign_of(signs, b, H, h, d, j) * oracle_f16_to_f64(x[v * d + j]);
                rotate_one(d, rot, xs, y, cs, sn);
                for (int j = 0; j < d; ++j)
                    acc[j] += y[j] * y[j];
            }
            for (int j = 0; j < d; ++j) {
                double ms = T > 0 ? acc[j] / (double)T : 0.0;
                lambda[(size_t)bh * d + j] = ms > 0.0 ? (float)(1.0 / sqrt(ms)) : 1.0f;
            }
        }
        free(xs);
        free(y);
        free(acc);
    }
    free(cs);
    free(sn);
    return 0;
}

/* Elementwise helpers for the tests. */
void oracle_f16_array_to_f64(const uint16_t *h, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f16_to_f64(h[i]);
}

void oracle_f64_array_to_f16(const double *v, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f64_to_f16(v[i]);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads the parallel loops use from now on (timing on one core). */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}
