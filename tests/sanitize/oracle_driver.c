/* Runs every oracle function on small inputs, edge cases included (empty
 * shapes, all-zero rows, threshold 0 and +inf, ties, subnormal E4M3 values,
 * non-finite input, an int32 overflow), for builds under AddressSanitizer and
 * UndefinedBehaviorSanitizer.  Exits non-zero on an unexpected status; the
 * sanitizers abort on any finding.  Test infrastructure only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_widen(const uint16_t*, int, int64_t, float*);
int oracle_e4m3_encode(const float*, int64_t, uint8_t*);
int oracle_e4m3_decode(const uint8_t*, int64_t, double*);
int oracle_quantize_tensor(const uint16_t*, int, int64_t, int64_t, int8_t*, float*);
int oracle_quantize_weight(const uint16_t*, int, int64_t, int64_t, int8_t*, float*);
int oracle_quantize_weight_fp8(const uint16_t*, int, int64_t, int64_t, uint8_t*, float*);
int oracle_quantize_act(const uint16_t*, int, int64_t, int64_t, float, int8_t*, float*, int32_t*,
                        int32_t*, uint16_t*);
int oracle_quantize_act_fp8(const uint16_t*, int, int64_t, int64_t, float, uint8_t*, float*,
                            int32_t*, int32_t*, uint16_t*);
int oracle_int8_rows(const int8_t*, const int8_t*, int64_t, int64_t, int64_t, const int64_t*,
                     int64_t, int32_t*);
int oracle_recover_weight(const int8_t*, const float*, int64_t, int64_t, double*);
int oracle_output_rows(const int32_t*, const float*, const float*, const uint16_t*, int,
                       const int32_t*, int32_t, const int8_t*, const uint16_t*, int64_t, int64_t,
                       int64_t, const int64_t*, int64_t, double*);
int oracle_fp8_rows(const uint8_t*, const uint8_t*, int64_t, int64_t, int64_t, const int64_t*,
                    int64_t, double*);
int oracle_output_rows_fp8(const double*, const float*, const float*, const uint16_t*, int,
                           const int32_t*, int32_t, const uint8_t*, const uint16_t*, int64_t,
                           int64_t, int64_t, const int64_t*, int64_t, double*);

static int failures = 0;
#define EXPECT(cond)                                                   \
    do {                                                               \
        if (!(cond)) {                                                 \
            fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                \
        }                                                              \
    } while (0)

static uint32_t rng = 12345u;
static uint32_t next_u32(void) {
    rng ^= rng << 13;
    rng ^= rng >> 17;
    rng ^= rng << 5;
    return rng;
}
/* a finite fp16 (dtype 0) or bf16 (dtype 1) bit pattern of moderate size */
static uint16_t rand16(int dtype) {
    const float v = ((float)(next_u32() % 20001) - 10000.0f) / 1000.0f; /* [-10, 10] */
    uint32_t b;
    memcpy(&b, &v, 4);
    if (dtype == 1) return (uint16_t)(b >> 16);
    /* fp16 from the float: exponent rebias, mantissa truncated */
    const uint32_t s = (b >> 16) & 0x8000u;
    const int e = (int)((b >> 23) & 0xff) - 127 + 15;
    if (e <= 0) return (uint16_t)s;
    return (uint16_t)(s | ((uint32_t)e << 10) | ((b >> 13) & 0x3ffu));
}

static void run_shape(int dtype, int64_t M, int64_t N, int64_t K, float t, int fp8) {
    const int64_t MK = M * K, NK = N * K;
    uint16_t* X = calloc((size_t)(MK + 1), 2);
    uint16_t* W = calloc((size_t)(NK + 1), 2);
    uint16_t* bias = calloc((size_t)(N + 1), 2);
    for (int64_t i = 0; i < MK; ++i) X[i] = rand16(dtype);
    for (int64_t i = 0; i < NK; ++i) W[i] = rand16(dtype);
    for (int64_t i = 0; i < N; ++i) bias[i] = rand16(dtype);
    if (M > 1)
        for (int64_t k = 0; k < K; ++k) X[1 * K + k] = 0; /* an all-zero row */
    if (N > 1)
        for (int64_t k = 0; k < K; ++k) W[1 * K + k] = 0; /* an all-zero weight row */
    int8_t* CA = calloc((size_t)(MK + 1), 1);
    int8_t* CB = calloc((size_t)(NK + 1), 1);
    float* SCA = calloc((size_t)(M + 1), 4);
    float* SCB = calloc((size_t)(N + 1), 4);
    int32_t* idx = calloc((size_t)(K + 1), 4);
    uint16_t* XO = calloc((size_t)(MK + 1), 2);
    int32_t n_out = -1;
    int64_t* rows = calloc((size_t)(M + 1), 8);
    for (int64_t r = 0; r < M; ++r) rows[r] = r;
    float* wide = calloc((size_t)(MK + 1), 4);
    EXPECT(oracle_widen(X, dtype, MK, wide) == 0);
    if (!fp8) {
        EXPECT(oracle_quantize_weight(W, dtype, N, K, CB, SCB) == 0);
        EXPECT(oracle_quantize_act(X, dtype, M, K, t, CA, SCA, idx, &n_out, XO) == 0);
        EXPECT(n_out >= 0 && n_out <= K);
        int32_t* C = calloc((size_t)(M * N + 1), 4);
        double* Y = calloc((size_t)(M * N + 1), 8);
        double* Wdq = calloc((size_t)(NK + 1), 8);
        EXPECT(oracle_int8_rows(CA, CB, M, N, K, rows, M, C) == 0);
        EXPECT(oracle_output_rows(C, SCA, SCB, X, dtype, idx, n_out, CB, bias, M, N, K, rows, M, Y) == 0);
        EXPECT(oracle_output_rows(C, SCA, SCB, X, dtype, idx, n_out, CB, NULL, M, N, K, rows, M, Y) == 0);
        EXPECT(oracle_recover_weight(CB, SCB, N, K, Wdq) == 0);
        int8_t* Q = calloc((size_t)(MK + 1), 1);
        EXPECT(oracle_quantize_tensor(X, dtype, M, K, Q, SCA) == 0);
        free(Q);
        free(C);
        free(Y);
        free(Wdq);
    } else {
        uint8_t* CA8 = (uint8_t*)CA;
        uint8_t* CB8 = (uint8_t*)CB;
        EXPECT(oracle_quantize_weight_fp8(W, dtype, N, K, CB8, SCB) == 0);
        EXPECT(oracle_quantize_act_fp8(X, dtype, M, K, t, CA8, SCA, idx, &n_out, XO) == 0);
        double* C = calloc((size_t)(M * N + 1), 8);
        double* Y = calloc((size_t)(M * N + 1), 8);
        EXPECT(oracle_fp8_rows(CA8, CB8, M, N, K, rows, M, C) == 0);
        EXPECT(oracle_output_rows_fp8(C, SCA, SCB, X, dtype, idx, n_out, CB8, bias, M, N, K, rows, M, Y) == 0);
        free(C);
        free(Y);
    }
    free(X); free(W); free(bias); free(CA); free(CB); free(SCA); free(SCB);
    free(idx); free(XO); free(rows); free(wide);
}

int main(void) {
    const float inf = INFINITY;
    for (int dtype = 0; dtype < 2; ++dtype)
        for (int fp8 = 0; fp8 < 2; ++fp8) {
            run_shape(dtype, 0, 5, 64, 6.0f, fp8);    /* no rows */
            run_shape(dtype, 3, 0, 64, 6.0f, fp8);    /* no outputs */
            run_shape(dtype, 5, 7, 128, 6.0f, fp8);
            run_shape(dtype, 4, 3, 192, 0.0f, fp8);   /* every column an outlier */
            run_shape(dtype, 4, 3, 192, inf, fp8);    /* none */
            run_shape(dtype, 9, 11, 320, 2.5f, fp8);
        }
    /* E4M3 round trip over every code, and ties, subnormals, saturation */
    {
        uint8_t codes[256];
        double vals[256];
        float f[256];
        for (int i = 0; i < 256; ++i) codes[i] = (uint8_t)i;
        EXPECT(oracle_e4m3_decode(codes, 256, vals) == 0);
        for (int i = 0; i < 256; ++i) f[i] = isnan(vals[i]) ? 0.0f : (float)vals[i];
        EXPECT(oracle_e4m3_encode(f, 256, codes) == 0);
        const float edge[] = {0.0f, -0.0f, 0.0009765625f, 0.0029296875f, 1.0625f, 448.0f, 447.9f, 0.001f};
        uint8_t out[8];
        EXPECT(oracle_e4m3_encode(edge, 8, out) == 0);
    }
    /* non-finite input is refused */
    {
        uint16_t x[64] = {0};
        int8_t q[64];
        float s[1];
        int32_t id[64], n;
        uint16_t xo[64];
        x[3] = 0x7c00; /* fp16 +inf */
        EXPECT(oracle_quantize_act(x, 0, 1, 64, 6.0f, q, s, id, &n, xo) != 0);
        EXPECT(oracle_quantize_weight(x, 0, 1, 64, q, s) != 0);
    }
    /* an int32 overflow of the int8 product is reported */
    {
        const int64_t K = 140000;
        int8_t* a = malloc((size_t)K);
        int8_t* b = malloc((size_t)K);
        memset(a, 127, (size_t)K);
        memset(b, 127, (size_t)K);
        const int64_t r0 = 0;
        int32_t c;
        EXPECT(oracle_int8_rows(a, b, 1, 1, K, &r0, 1, &c) != 0);
        free(a);
        free(b);
    }
    /* invalid arguments */
    {
        float dst[1];
        uint16_t src[1] = {0};
        EXPECT(oracle_widen(src, 2, 1, dst) != 0);
        EXPECT(oracle_widen(src, 0, -1, dst) != 0);
        const int64_t bad_row = 5;
        int32_t c;
        int8_t a[64] = {0};
        EXPECT(oracle_int8_rows(a, a, 1, 1, 64, &bad_row, 1, &c) != 0);
    }
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("oracle driver: ok\n");
    return 0;
}
