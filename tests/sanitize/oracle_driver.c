/*
 * Drives every oracle entry point on small inputs, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitizers.py):
 * all head sizes, rotations, groups and code widths, NULL signs and lambda,
 * empty inputs, and the rotation-matrix entry points.  Exits 0 when every
 * call returns its expected status; the sanitizers report anything else.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_rotate(int64_t, int64_t, int, int, int, const uint16_t *, const int8_t *, double *);
int oracle_unrotate(int64_t, int64_t, int, int, int, const double *, const int8_t *, double *);
int oracle_quantize(int64_t, int64_t, int, int, int, int, int, const uint16_t *, const int8_t *,
                    const float *, uint8_t *, uint16_t *, double *);
int oracle_dequantize(int64_t, int64_t, int, int, int, int, int, const uint8_t *, const uint16_t *,
                      const int8_t *, const float *, uint16_t *, double *);
int oracle_quantize_dense(int64_t, int64_t, int, int, int, int, const float *, int64_t, const uint16_t *,
                          const int8_t *, const float *, uint8_t *, uint16_t *, double *);
int oracle_dequantize_dense(int64_t, int64_t, int, int, int, int, const float *, int64_t, const uint8_t *,
                            const uint16_t *, const int8_t *, const float *, uint16_t *, double *);
int oracle_calibrate_lambda(int64_t, int64_t, int, int, int, const uint16_t *, const int8_t *, float *);
uint16_t oracle_f64_to_f16(double);

static uint32_t rng = 12345u;
static uint32_t next(void) { rng = rng * 1664525u + 1013904223u; return rng >> 8; }

static int fails = 0;
#define EXPECT(call, want)                                                          \
    do {                                                                            \
        int st_ = (call);                                                           \
        if (st_ != (want)) {                                                        \
            fprintf(stderr, "%s:%d: status %d, expected %d\n", __FILE__, __LINE__, st_, want); \
            ++fails;                                                                \
        }                                                                           \
    } while (0)

int main(void)
{
    const int ds[] = {8, 64, 96, 128, 256};
    for (unsigned di = 0; di < sizeof ds / sizeof ds[0]; ++di) {
        int d = ds[di];
        int64_t B = 2, T = 5;
        int H = 3;
        size_t n = (size_t)(B * T * H * d);
        uint16_t *x = malloc(n * 2), *xo = malloc(n * 2);
        double *y = malloc(n * 8), *x64 = malloc(n * 8), *z = malloc(n * 8);
        int8_t *s = malloc((size_t)(B * H * d));
        float *lam = malloc((size_t)(B * H * d) * 4), *Q = malloc((size_t)d * d * 4);
        uint8_t *codes = malloc(n);
        uint16_t *scales = malloc(n * 2);
        for (size_t i = 0; i < n; ++i)
            x[i] = oracle_f64_to_f16(((double)(next() % 2001) - 1000.0) / 250.0);
        for (int i = 0; i < B * H * d; ++i) {
            s[i] = (next() & 1) ? 1 : -1;
            lam[i] = 0.5f + (float)(next() % 100) / 50.0f;
        }
        for (int i = 0; i < d * d; ++i)
            Q[i] = (i % (d + 1) == 0) ? 1.0f : 0.0f;
        for (int rot = 0; rot < 3; ++rot) {
            int ok = (rot == 1 && (d & (d - 1))) ? 3 : 0;   /* Hadamard needs a power of two */
            EXPECT(oracle_rotate(B, T, H, d, rot, x, s, y), ok);
            EXPECT(oracle_unrotate(B, T, H, d, rot, y, s, x64), ok);
            EXPECT(oracle_calibrate_lambda(B, T, H, d, rot, x, NULL, lam), ok);
            for (int g = 8; g <= d; g *= 2) {
                if (d % g)
                    continue;
                for (int bits = 4; bits <= 8; bits += 4) {
                    EXPECT(oracle_quantize(B, T, H, d, g, bits, rot, x, s, lam, codes, scales, z), ok);
                    EXPECT(oracle_dequantize(B, T, H, d, g, bits, rot, codes, scales, s, lam, xo, x64), ok);
                    EXPECT(oracle_quantize(B, T, H, d, g, bits, rot, x, NULL, NULL, codes, scales, NULL), ok);
                    EXPECT(oracle_dequantize(B, T, H, d, g, bits, rot, codes, scales, NULL, NULL, xo, NULL), ok);
                    EXPECT(oracle_quantize(B, 0, H, d, g, bits, rot, x, s, lam, codes, scales, z), ok);
                }
            }
        }
        EXPECT(oracle_quantize_dense(B, T, H, d, 8, 4, Q, 0, x, s, lam, codes, scales, z), 0);
        EXPECT(oracle_dequantize_dense(B, T, H, d, 8, 4, Q, 0, codes, scales, s, lam, xo, x64), 0);
        EXPECT(oracle_quantize_dense(B, T, H, d, 8, 4, NULL, 0, x, s, lam, codes, scales, z), 1);
        EXPECT(oracle_quantize(B, T, H, d, 5, 4, 0, x, s, lam, codes, scales, z), 3);
        EXPECT(oracle_quantize(B, T, H, d, 8, 5, 0, x, s, lam, codes, scales, z), 3);
        EXPECT(oracle_quantize(-1, T, H, d, 8, 4, 0, x, s, lam, codes, scales, z), 2);
        free(x); free(xo); free(y); free(x64); free(z); free(s); free(lam); free(Q); free(codes); free(scales);
    }
    if (fails)
        return 1;
    printf("oracle driver: ok\n");
    return 0;
}
