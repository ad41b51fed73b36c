/*
 * CPU oracle for the LLM.int8() mixed-precision decomposition matmul.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product (the HIP
 * library) never calls it, links it or shares code with it.
 *
 * Plain, slow, single-threaded C.  Each step is the plain definition written
 * out, in the order the pages give it.  Page titles used in the citations:
 *   [GENTLE] "A Gentle Introduction to 8-bit Matrix Multiplication for
 *            transformers at scale" (Chinese translation).
 *   [HF-INT8] "Hugging Face 将 LLM.int8() 8 位矩阵乘法集成到 Transformers 和
 *            Accelerate 中".
 *   [ABSTRACT] "LLM.int8() : Multiplication matricielle a 8 bits pour les
 *            Transformers a grande echelle".
 *   [ZHICHAI] the zhichai.top summary of LLM.int8() (its outlook section,
 *            "未来展望", lists the method's limitations).
 *
 * Readings taken where the pages leave a step open:
 *   - outlier test is |x| >= threshold, column-wise over every row of the call
 *     ([GENTLE] "inside the MatMul": magnitude 6 or greater; "LLM.int8()
 *     summary": outliers are extracted by column from the hidden states);
 *   - the activation row scale SCA covers only the non-outlier columns, and
 *     outlier entries of CA are 0;
 *   - scale = 127.0f / absmax as one IEEE fp32 division, q = round-half-even
 *     of (x * scale) as one fp32 multiply, clamped to [-127, 127]
 *     ([GENTLE] "absmax quantization" worked example);
 *   - an all-zero vector (absmax 0) quantizes to zeros with scale 0;
 *   - weights are scaled per output channel (row n of W [N,K]); the recovered
 *     weight is CB[n,k] * SCB[n] / 127 ([GENTLE] "Usage" printouts);
 *   - the int8 product is dequantized by SCA[m] * SCB[n] / 127^2 (outer
 *     product of the two absmax vectors, [GENTLE] "absmax quantization");
 *   - the outlier product uses the recovered weights; Y = int8 part +
 *     outlier part + bias.  Y is evaluated in double precision.
 *   - FP8 variant ([ZHICHAI] "未来展望": an 8-bit floating-point type is named
 *     as future work for the method, no format given): the same decomposition
 *     with OCP FP8 E4M3 codes in place of int8 -- sign, 4 exponent bits (bias
 *     7), 3 mantissa bits, subnormals, no infinities, NaN = S.1111.111,
 *     largest finite 448.  scale = 448.0f / absmax (one fp32 division), code =
 *     e4m3(x * scale) (one fp32 multiply, then round to nearest with ties to
 *     the even code; a result that rounds to zero keeps its sign; magnitudes
 *     from 464 up have no finite code and give NaN).  A zero vector keeps
 *     scale 0 and the codes of its signed zeros.  Outlier entries of CA are
 *     code 0x00.  The product is sum_k value(CA)value(CB) (exact in double:
 *     every E4M3 value is a multiple of 2^-9 below 2^9, so K <= 2^13 products
 *     need at most 49 significant bits), dequantized by SCA*SCB/448^2; the
 *     recovered weight is value(CB) * SCB / 448.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off -fno-fast-math
 * (SSE arithmetic on x86-64, so every float operation is one IEEE binary32
 * operation, round-to-nearest-even).

 */
#include <fenv.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OK 0
#define ERR_ARG 1
#define ERR_NONFINITE 2
#define ERR_OVERFLOW 3

/* ---- 16-bit -> fp32 widening, exact, by bit manipulation ---------------- */

static float f16_to_f32(uint16_t h) {
    uint32_t sign = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    float mag;
    if (e == 0)
        mag = ldexpf((float)m, -24);                 /* subnormal: m * 2^-24 */
    else if (e == 31)
        mag = m ? NAN : INFINITY;
    else
        mag = ldexpf((float)(m | 0x400), (int)e - 25); /* (1024+m) * 2^(e-25) */
    return sign ? -mag : mag;
}

static float bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static float widen(uint16_t v, int dtype) { return dtype == 0 ? f16_to_f32(v) : bf16_to_f32(v); }

int oracle_widen(const uint16_t* src, int dtype, int64_t n, float* dst) {
    if ((dtype != 0 && dtype != 1) || n < 0) return ERR_ARG;
    for (int64_t i = 0; i < n; ++i) dst[i] = widen(src[i], dtype);
    return OK;
}

/* ---- absmax quantization of one value ([GENTLE] "absmax quantization") -- */

static float absmax_scale(float absmax) {
    return 127.0f / absmax; /* one IEEE fp32 division */
}

static int8_t quantize_value(float x, float scale) {
    float product = x * scale; /* one fp32 multiply */
    float r = nearbyintf(product); /* round half to even (default mode) */
    if (r > 127.0f) r = 127.0f;
    if (r < -127.0f) r = -127.0f;
    return (int8_t)r;
}

/* ---- FP8 E4M3 encoding and values ([ZHICHAI] "未来展望"; format above) ---- */

/* value of a code: (-1)^s 2^(e-7) (1 + m/8) for e > 0, (-1)^s 2^-6 (m/8) for */
/* e = 0; S.1111.111 is NaN                                                   */
static double e4m3_value(uint8_t c) {
    const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double v = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

/* nearest code, ties to the even code (even mantissa field) */
static uint8_t e4m3_encode(float x) {
    const uint8_t sign = signbit(x) ? 0x80 : 0x00;
    if (isnan(x)) return (uint8_t)(sign | 0x7f);
    const double a = fabs((double)x);
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: multiples of 2^-9; q = 8 is the code of 2^-6 */
        const double q = nearbyint(a * 512.0);
        return (uint8_t)(sign | (uint8_t)q);
    }
    int e2;
    frexp(a, &e2);
    int E = e2 - 1;                       /* 2^E <= a < 2^(E+1) */
    const double sig = ldexp(a, 3 - E);   /* in [8, 16): 3 fraction bits above the point */
    double q = nearbyint(sig); /* ties to even (default rounding mode) */
    if (q == 16.0) {
        q = 8.0;
        E += 1;
    }
    if (E > 8 || (E == 8 && q == 15.0)) return (uint8_t)(sign | 0x7f); /* no finite code */
    return (uint8_t)(sign | (uint8_t)((E + 7) << 3) | (uint8_t)(q - 8.0));
}

static float e4m3_scale(float absmax) {
    return 448.0f / absmax; /* one IEEE fp32 division */
}

static uint8_t e4m3_quantize_value(float x, float scale) {
    float product = x * scale; /* one fp32 multiply */
    return e4m3_encode(product);
}

int oracle_e4m3_encode(const float* x, int64_t n, uint8_t* out) {
    if (n < 0) return ERR_ARG;
    if (fegetround() != FE_TONEAREST) return ERR_ARG;
    for (int64_t i = 0; i < n; ++i) out[i] = e4m3_encode(x[i]);
    return OK;
}

int oracle_e4m3_decode(const uint8_t* c, int64_t n, double* out) {
    if (n < 0) return ERR_ARG;
    for (int64_t i = 0; i < n; ++i) out[i] = e4m3_value(c[i]);
    return OK;
}

/* ---- per-tensor absmax quantization (the baseline) ------------------------ */
/* One scale for the whole tensor: amax = max over every element of |A|;       */
/* Q = q(A, 127/amax); scale[r] = amax for every row r (so the pair can stand  */
/* in for a vector-wise (codes, scales) pair).  [GENTLE] "absmax quantization" */
/* (the scale of a whole vector/tensor), the scheme that the vector-wise and   */
/* decomposed schemes are measured against.                                    */

int oracle_quantize_tensor(const uint16_t* A, int dtype, int64_t rows, int64_t cols,
                           int8_t* Q, float* scale) {
    if ((dtype != 0 && dtype != 1) || rows < 0 || cols < 0) return ERR_ARG;
    if (fegetround() != FE_TONEAREST) return ERR_ARG;
    const int64_t n = rows * cols;
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = widen(A[i], dtype);
        if (!isfinite(a)) return ERR_NONFINITE;
        a = fabsf(a);
        if (a > amax) amax = a;
    }
    for (int64_t r = 0; r < rows; ++r) scale[r] = amax;
    if (amax == 0.0f) {
        memset(Q, 0, (size_t)n);
        return OK;
    }
    float s = absmax_scale(amax);
    for (int64_t i = 0; i < n; ++i) Q[i] = quantize_value(widen(A[i], dtype), s);
    return OK;
}

/* ---- weight quantization: per output row n ------------------------------ */
/* SCB[n] = max_k |W[n,k]|; CB[n,k] = q(W[n,k], 127/SCB[n]).                   */
/* [GENTLE] "absmax quantization" (vector-wise: absmax per column of B = W^T,  */
/* i.e. per row of W) and "Usage" (weight.CB int8 [out,in], weight.SCB).       */

/* fp8 = 0: int8 codes; fp8 = 1: E4M3 codes (SCB as above, code =            */
/* e4m3(W[n,k] * 448/SCB[n]), scale 0 for a zero row).                          */
static int quantize_weight_codes(const uint16_t* W, int dtype, int64_t N, int64_t K, int fp8,
                                 void* codes, float* SCB) {
    if ((dtype != 0 && dtype != 1) || N < 0 || K < 0) return ERR_ARG;
    if (fegetround() != FE_TONEAREST) return ERR_ARG;
    int8_t* CB = (int8_t*)codes;
    uint8_t* CB8 = (uint8_t*)codes;
    for (int64_t n = 0; n < N; ++n) {
        const uint16_t* row = W + n * K;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float w = widen(row[k], dtype);
            if (!isfinite(w)) return ERR_NONFINITE;
            float a = fabsf(w);
            if (a > amax) amax = a;
        }
        SCB[n] = amax;
        if (fp8) {
            float s = amax == 0.0f ? 0.0f : e4m3_scale(amax);
            for (int64_t k = 0; k < K; ++k) CB8[n * K + k] = e4m3_quantize_value(widen(row[k], dtype), s);
            continue;
        }
        if (amax == 0.0f) {
            memset(CB + n * K, 0, (size_t)K);
            continue;
        }
        float s = absmax_scale(amax);
        for (int64_t k = 0; k < K; ++k) CB[n * K + k] = quantize_value(widen(row[k], dtype), s);
    }
    return OK;
}

int oracle_quantize_weight(const uint16_t* W, int dtype, int64_t N, int64_t K, int8_t* CB,
                           float* SCB) {
    return quantize_weight_codes(W, dtype, N, K, 0, CB, SCB);
}

int oracle_quantize_weight_fp8(const uint16_t* W, int dtype, int64_t N, int64_t K, uint8_t* CB,
                               float* SCB) {
    return quantize_weight_codes(W, dtype, N, K, 1, CB, SCB);
}

/* ---- activation quantization -------------------------------------------- */
/* 1. outlier columns: O = { k : max_m |X[m,k]| >= t }, ascending              */
/*    ([GENTLE] "LLM.int8() summary" step 1; "inside the MatMul": 6 or more). */
/* 2. SCA[m] = max over k not in O of |X[m,k]|; CA[m,k] = q(X[m,k],127/SCA[m]) */
/*    for k not in O, 0 for k in O (row-wise quantization of the hidden       */
/*    states, [GENTLE] "inside the MatMul"; [HF-INT8] core idea).             */
/* 3. XO[m,j] = X[m, idx[j]] (the 16-bit outlier part, kept as bit patterns). */
/* XO has room for M * K values and holds [M, n_out] row-major.               */

/* fp8 = 1: E4M3 codes, e4m3(X[m,k] * 448/SCA[m]) (scale 0 for SCA[m] = 0),   */
/* 0x00 in the outlier columns.                                                */
static int quantize_act_codes(const uint16_t* X, int dtype, int64_t M, int64_t K, float t, int fp8,
                              void* codes, float* SCA, int32_t* idx, int32_t* n_out,
                              uint16_t* XO) {
    if ((dtype != 0 && dtype != 1) || M < 0 || K < 0 || isnan(t) || t < 0.0f) return ERR_ARG;
    int8_t* CA = (int8_t*)codes;
    uint8_t* CA8 = (uint8_t*)codes;
    if (fegetround() != FE_TONEAREST) return ERR_ARG;
    for (int64_t i = 0; i < M * K; ++i)
        if (!isfinite(widen(X[i], dtype))) return ERR_NONFINITE;

    unsigned char* is_out = (unsigned char*)calloc((size_t)(K > 0 ? K : 1), 1);
    if (!is_out) return ERR_ARG;
    int32_t count = 0;
    for (int64_t k = 0; k < K; ++k) {
        float colmax = 0.0f;
        for (int64_t m = 0; m < M; ++m) {
            float a = fabsf(widen(X[m * K + k], dtype));
            if (a > colmax) colmax = a;
        }
        int outlier = M > 0 && colmax >= t;
        is_out[k] = (unsigned char)outlier;
        if (outlier) idx[count++] = (int32_t)k;
    }
    *n_out = count;

    for (int64_t m = 0; m < M; ++m) {
        const uint16_t* row = X + m * K;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            if (is_out[k]) continue;
            float a = fabsf(widen(row[k], dtype));
            if (a > amax) amax = a;
        }
        SCA[m] = amax;
        if (fp8) {
            float s = amax == 0.0f ? 0.0f : e4m3_scale(amax);
            for (int64_t k = 0; k < K; ++k) {
                int zero = is_out[k];
                CA8[m * K + k] = zero ? 0x00 : e4m3_quantize_value(widen(row[k], dtype), s);
            }
        } else {
            float s = amax == 0.0f ? 0.0f : absmax_scale(amax);
            for (int64_t k = 0; k < K; ++k) {
                int zero = is_out[k] || amax == 0.0f;
                CA[m * K + k] = zero ? 0 : quantize_value(widen(row[k], dtype), s);
            }
        }
        for (int32_t j = 0; j < count; ++j) XO[m * (int64_t)count + j] = row[idx[j]];
    }
    free(is_out);
    return OK;
}

int oracle_quantize_act(const uint16_t* X, int dtype, int64_t M, int64_t K, float t, int8_t* CA,
                        float* SCA, int32_t* idx, int32_t* n_out, uint16_t* XO) {
    return quantize_act_codes(X, dtype, M, K, t, 0, CA, SCA, idx, n_out, XO);
}

int oracle_quantize_act_fp8(const uint16_t* X, int dtype, int64_t M, int64_t K, float t,
                            uint8_t* CA, float* SCA, int32_t* idx, int32_t* n_out, uint16_t* XO) {
    return quantize_act_codes(X, dtype, M, K, t, 1, CA, SCA, idx, n_out, XO);
}

/* ---- int8 product of selected rows --------------------------------------- */
/* C[r,n] = sum_k CA[rows[r],k] * CB[n,k], exact in int64, must fit int32.     */
/* ([GENTLE] "LLM.int8() summary" step 2, non-outliers multiplied in int8.)   */

int oracle_int8_rows(const int8_t* CA, const int8_t* CB, int64_t M, int64_t N, int64_t K,
                     const int64_t* rows, int64_t n_rows, int32_t* C) {
    if (M < 0 || N < 0 || K < 0 || n_rows < 0) return ERR_ARG;
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t m = rows[r];
        if (m < 0 || m >= M) return ERR_ARG;
        const int8_t* a = CA + m * K;
        for (int64_t n = 0; n < N; ++n) {
            const int8_t* b = CB + n * K;
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k) acc += (int64_t)a[k] * (int64_t)b[k];
            if (acc > INT32_MAX || acc < INT32_MIN) return ERR_OVERFLOW;
            C[r * N + n] = (int32_t)acc;
        }
    }
    return OK;
}

/* ---- recovered weights: CB[n,k] * SCB[n] / 127 ([GENTLE] "Usage") -------- */

static double recovered_weight(const int8_t* CB, const float* SCB, int64_t K, int64_t n, int64_t k) {
    return (double)CB[n * K + k] * (double)SCB[n] / 127.0;
}

int oracle_recover_weight(const int8_t* CB, const float* SCB, int64_t N, int64_t K, double* Wdq) {
    if (N < 0 || K < 0) return ERR_ARG;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) Wdq[n * K + k] = recovered_weight(CB, SCB, K, n, k);
    return OK;
}

/* ---- the output rows ------------------------------------------------------ */
/* Y[m,n] = C[m,n] * SCA[m] * SCB[n] / 127^2                (dequantize)       */
/*        + sum_{j < n_out} X[m, idx[j]] * CB[n,idx[j]] * SCB[n] / 127          */
/*        + bias[n]                                                            */
/* ([GENTLE] "LLM.int8() summary" step 3: dequantize the int8 result, add the  */
/* 16-bit outlier result.)  Evaluated in double; C is the int8 product of the  */
/* same rows (from oracle_int8_rows).  bias may be NULL.                       */

int oracle_output_rows(const int32_t* C, const float* SCA, const float* SCB,
                       const uint16_t* X, int dtype, const int32_t* idx, int32_t n_out,
                       const int8_t* CB, const uint16_t* bias,
                       int64_t M, int64_t N, int64_t K,
                       const int64_t* rows, int64_t n_rows, double* Y) {
    if ((dtype != 0 && dtype != 1) || M < 0 || N < 0 || K < 0 || n_rows < 0 || n_out < 0)
        return ERR_ARG;
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t m = rows[r];
        if (m < 0 || m >= M) return ERR_ARG;
        for (int64_t n = 0; n < N; ++n) {
            double y_int8 = (double)C[r * N + n] * (double)SCA[m] * (double)SCB[n] / 16129.0;
            double y_out = 0.0;
            for (int32_t j = 0; j < n_out; ++j) {
                int64_t k = idx[j];
                y_out += (double)widen(X[m * K + k], dtype) * recovered_weight(CB, SCB, K, n, k);
            }
            double b = bias ? (double)widen(bias[n], dtype) : 0.0;
            Y[r * N + n] = y_int8 + y_out + b;
        }
    }
    return OK;
}

/* ---- FP8 variant: product and output rows ([ZHICHAI] "未来展望"; readings  */
/* in the header) ----------------------------------------------------------- */
/* C[r,n] = sum_k value(CA[rows[r],k]) * value(CB[n,k]), exact in double.       */

int oracle_fp8_rows(const uint8_t* CA, const uint8_t* CB, int64_t M, int64_t N, int64_t K,
                    const int64_t* rows, int64_t n_rows, double* C) {
    if (M < 0 || N < 0 || K < 0 || n_rows < 0 || K > 8192) return ERR_ARG;
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t m = rows[r];
        if (m < 0 || m >= M) return ERR_ARG;
        const uint8_t* a = CA + m * K;
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t* b = CB + n * K;
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double va = e4m3_value(a[k]), vb = e4m3_value(b[k]);
                if (isnan(va) || isnan(vb)) return ERR_NONFINITE;
                acc += va * vb;
            }
            C[r * N + n] = acc;
        }
    }
    return OK;
}

/* Y[m,n] = C[m,n] * SCA[m] * SCB[n] / 448^2                                  */
/*        + sum_{j < n_out} X[m, idx[j]] * value(CB[n,idx[j]]) * SCB[n] / 448   */
/*        + bias[n]            (in double; bias may be NULL)                    */

int oracle_output_rows_fp8(const double* C, const float* SCA, const float* SCB,
                           const uint16_t* X, int dtype, const int32_t* idx, int32_t n_out,
                           const uint8_t* CB, const uint16_t* bias, int64_t M, int64_t N,
                           int64_t K, const int64_t* rows, int64_t n_rows, double* Y) {
    if ((dtype != 0 && dtype != 1) || M < 0 || N < 0 || K < 0 || n_rows < 0 || n_out < 0)
        return ERR_ARG;
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t m = rows[r];
        if (m < 0 || m >= M) return ERR_ARG;
        for (int64_t n = 0; n < N; ++n) {
            double y8 = C[r * N + n] * (double)SCA[m] * (double)SCB[n] / 200704.0;
            double y_out = 0.0;
            for (int32_t j = 0; j < n_out; ++j) {
                int64_t k = idx[j];
                y_out += (double)widen(X[m * K + k], dtype) * e4m3_value(CB[n * K + k]) *
                         (double)SCB[n] / 448.0;
            }
            double b = bias ? (double)widen(bias[n], dtype) : 0.0;
            Y[r * N + n] = y8 + y_out + b;
        }
    }
    return OK;
}
