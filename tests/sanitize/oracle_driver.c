/*
 * Sanitizer driver for the CPU oracle (oracle/kq_oracle.c): built with
 * AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitizers.py
 * and run on the CPU.  It calls every oracle entry point on small seeded
 * inputs of many shapes (one block, ragged widths, empty matrices, special
 * values: zeros, -0, subnormals, NaN, Inf) with buffers sized exactly, and
 * checks the status codes.  Any out-of-bounds access, leak or undefined
 * operation aborts the run with a sanitizer report.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_kq_transform(const uint16_t *, int64_t, int64_t, const float *, int64_t, double *, double *);
int oracle_kq_quantize(const uint16_t *, int64_t, int64_t, const float *, int64_t, uint8_t *, uint8_t *, float *);
int oracle_kq_transform_lu(const uint16_t *, int64_t, int64_t, const float *, int64_t, double *, double *);
int oracle_kq_quantize_lu(const uint16_t *, int64_t, int64_t, const float *, int64_t, uint8_t *, uint8_t *, float *);
int oracle_fwht_transform(const uint16_t *, int64_t, int64_t, double *, double *);
int oracle_fwht_quantize(const uint16_t *, int64_t, int64_t, uint8_t *, uint8_t *, float *);
int oracle_sq_quantize(const uint16_t *, int64_t, int64_t, const float *, uint8_t *, uint8_t *, float *);
int oracle_mx_quantize_f32(const float *, int64_t, int64_t, uint8_t *, uint8_t *);
int oracle_mx_dequant(const uint8_t *, const uint8_t *, int64_t, int64_t, double *);
int oracle_mx_gemm(const uint8_t *, const uint8_t *, int64_t, const uint8_t *, const uint8_t *, int64_t, int64_t,
                   double *, double *);
int oracle_adaln(const uint16_t *, int64_t, int64_t, const float *, const float *, int64_t, float, double *,
                 uint16_t *, uint8_t *);
int oracle_kq_transform16(const uint16_t *, int64_t, int64_t, const float *, int64_t, double *, double *);
int oracle_kq_quantize16(const uint16_t *, int64_t, int64_t, const float *, int64_t, uint8_t *, uint8_t *, float *);
int oracle_kron_block_inverse(const float *, double *);
uint16_t oracle_double_to_bf16(double);
int oracle_e8m0_exponent(float);
int oracle_fp4_code(float, int);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t next32(void)
{
    /* xorshift64*: test input bits only */
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    return (uint32_t)((state * 0x2545F4914F6CDD1Dull) >> 32);
}

static uint16_t rand_bf16(int special)
{
    uint32_t r = next32();
    if (special) {
        switch (r % 8) {
        case 0: return 0x0000;                           /* +0 */
        case 1: return 0x8000;                           /* -0 */
        case 2: return (uint16_t)(0x0001 + (r >> 8) % 0x7F); /* subnormal */
        case 3: return 0x7F80;                           /* +Inf */
        case 4: return 0x7FC1;                           /* NaN */
        default: break;
        }
    }
    /* finite, exponent in a moderate range, random sign and fraction */
    uint16_t e = (uint16_t)(100 + (r >> 3) % 50);
    return (uint16_t)(((r & 1) << 15) | (e << 7) | ((r >> 16) & 0x7F));
}

static void *xmalloc(size_t n)
{
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

#define CHECK(expr, want)                                                                                          \
    do {                                                                                                           \
        int got_ = (expr);                                                                                         \
        if (got_ != (want)) {                                                                                      \
            fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #expr, got_, (want));   \
            exit(1);                                                                                               \
        }                                                                                                          \
    } while (0)

static void factors(float *f, int64_t n, int lu)
{
    for (int64_t i = 0; i < n; ++i) {
        if (lu) /* (a, b, c) with a bounded away from 0 */
            f[i] = (i % 3 == 0) ? 0.5f + (float)(next32() % 1000) / 1000.0f : (float)((int)(next32() % 2001) - 1000) / 1000.0f;
        else
            f[i] = ((i % 4 == 0) || (i % 4 == 3) ? 1.0f : 0.0f) + (float)((int)(next32() % 601) - 300) / 1000.0f;
    }
}

static void one_shape(int64_t M, int64_t d, int special)
{
    const int64_t n = M * d, nB = d / 32, nT = nB;
    uint16_t *x = xmalloc((size_t)n * 2);
    for (int64_t i = 0; i < n; ++i)
        x[i] = rand_bf16(special);
    float *f = xmalloc((size_t)nT * 20 * 4), *lu = xmalloc((size_t)nT * 15 * 4), *sc = xmalloc((size_t)d * 4);
    factors(f, nT * 20, 0);
    factors(lu, nT * 15, 1);
    for (int64_t c = 0; c < d; ++c)
        sc[c] = 0.25f + (float)(next32() % 1000) / 100.0f;
    double *y = xmalloc((size_t)n * 8), *z = xmalloc((size_t)n * 8);
    float *y32 = xmalloc((size_t)n * 4);
    uint8_t *q = xmalloc((size_t)n / 2), *s = xmalloc((size_t)(M * nB));
    for (int shared = 0; shared < 2; ++shared) {
        const int64_t t = shared ? 1 : nT;
        CHECK(oracle_kq_transform(x, M, d, f, t, y, z), 0);
        CHECK(oracle_kq_quantize(x, M, d, f, t, q, s, y32), 0);
        CHECK(oracle_kq_quantize(x, M, d, f, t, q, s, NULL), 0);
        CHECK(oracle_kq_transform_lu(x, M, d, lu, t, y, z), 0);
        CHECK(oracle_kq_quantize_lu(x, M, d, lu, t, q, s, y32), 0);
    }
    CHECK(oracle_fwht_transform(x, M, d, y, z), 0);
    CHECK(oracle_fwht_quantize(x, M, d, q, s, y32), 0);
    CHECK(oracle_sq_quantize(x, M, d, sc, q, s, y32), 0);
    for (int64_t i = 0; i < n; ++i)
        y32[i] = (float)((int)(next32() % 20001) - 10000) / 777.0f;
    CHECK(oracle_mx_quantize_f32(y32, M, d, q, s), 0);
    /* dequantize and multiply the codes just written with themselves */
    double *dq = xmalloc((size_t)n * 8), *out = xmalloc((size_t)(M * M) * 8), *mag = xmalloc((size_t)(M * M) * 8);
    CHECK(oracle_mx_dequant(q, s, M, d, dq), 0);
    CHECK(oracle_mx_gemm(q, s, M, q, s, M, d, out, mag), 0);
    /* AdaLN front-end with two samples */
    const int64_t T = M > 1 ? (M + 1) / 2 : 1, S = (M + T - 1) / T;
    float *sh = xmalloc((size_t)(S * d) * 4), *sl = xmalloc((size_t)(S * d) * 4);
    for (int64_t i = 0; i < S * d; ++i) {
        sh[i] = (float)((int)(next32() % 201) - 100) / 100.0f;
        sl[i] = (float)((int)(next32() % 201) - 100) / 100.0f;
    }
    uint16_t *xb = xmalloc((size_t)n * 2);
    uint8_t *xfl = xmalloc((size_t)n);
    CHECK(oracle_adaln(x, M, d, sh, sl, T, 1e-6f, y, xb, xfl), 0);
    /* 16-element blocks */
    const int64_t nT16 = d / 16;
    float *f16 = xmalloc((size_t)nT16 * 16 * 4);
    factors(f16, nT16 * 16, 0);
    uint8_t *s16 = xmalloc((size_t)(M * nT16));
    CHECK(oracle_kq_transform16(x, M, d, f16, nT16, y, z), 0);
    CHECK(oracle_kq_quantize16(x, M, d, f16, 1, q, s16, y32), 0);
    free(x); free(f); free(lu); free(sc); free(y); free(z); free(y32); free(q); free(s); free(dq); free(out);
    free(mag); free(sh); free(sl); free(xb); free(xfl); free(f16); free(s16);
}

int main(void)
{
    static const int64_t shapes[][2] = {{1, 32}, {3, 64}, {2, 96}, {5, 160}, {1, 1152}, {7, 544}, {4, 2240}};
    for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i)
        for (int special = 0; special < 2; ++special)
            one_shape(shapes[i][0], shapes[i][1], special);
    /* shape and argument errors are reported, not acted on */
    uint16_t x[64] = {0};
    float f[40] = {0};
    uint8_t q[32], s[2];
    CHECK(oracle_kq_quantize(x, 1, 48, f, 1, q, s, NULL), 2);
    CHECK(oracle_kq_quantize(x, 1, 64, f, 3, q, s, NULL), 2);
    CHECK(oracle_kq_quantize(NULL, 1, 64, f, 1, q, s, NULL), 1);
    CHECK(oracle_kq_quantize(x, 0, 64, f, 1, q, s, NULL), 0);
    double inv[1024];
    float sing[20] = {1, 1, 1, 1, 1, 0, 0, 1, 1, 0, 0, 1, 1, 0, 0, 1, 1, 0, 0, 1};
    CHECK(oracle_kron_block_inverse(sing, inv), 4);
    /* scalar helpers over edge values */
    const double dv[] = {0.0, -0.0, 1e-45, 3.4e38, 1e300, -1e-300, INFINITY, -INFINITY, NAN, 0.5, 1.00390625};
    for (size_t i = 0; i < sizeof dv / sizeof dv[0]; ++i)
        (void)oracle_double_to_bf16(dv[i]);
    const float fv[] = {0.0f, 1e-45f, 1.17549435e-38f, 6.0f, 7.99f, 3.4e38f, INFINITY};
    for (size_t i = 0; i < sizeof fv / sizeof fv[0]; ++i) {
        int E = oracle_e8m0_exponent(fv[i]);
        (void)oracle_fp4_code(fv[i], E < -127 ? -127 : (E > 127 ? 127 : E));
    }
    puts("oracle driver ok");
    return 0;
}
