"""Planted mistakes for the oracle, as text patches of oracle/llmint8_oracle.c.

Each entry: a description and the (original, replacement) pairs that turn a
copy of the oracle source into a wrong oracle.  Every original text occurs
exactly once in the source.  tests/test_oracle_mutants.py builds each copy on
the CPU and checks that at least one pin fails.  The oracle itself holds none
of them.
"""

MUTANTS = {
    1: ('strict > instead of >= at the threshold', [
        ('        int outlier = M > 0 && colmax >= t;',
         '        int outlier = M > 0 && colmax > t; /* mistake: strict comparison */'),
    ]),
    2: ('row scale also covers outlier columns', [
        ('            if (is_out[k]) continue;',
         '            /* mistake: the row scale also covers the outlier columns */'),
    ]),
    3: ('weight scale per input column', [
        ('    for (int64_t n = 0; n < N; ++n) {\n        const uint16_t* row = W + n * K;',
         '    if (fp8) return ERR_ARG; /* this planted mistake concerns the int8 codes */\n    /* mistake: one scale per input column instead of per output row */\n    for (int64_t k = 0; k < K; ++k) {\n        float amax = 0.0f;\n        for (int64_t n = 0; n < N; ++n) {\n            float a = fabsf(widen(W[n * K + k], dtype));\n            if (a > amax) amax = a;\n        }\n        for (int64_t n = 0; n < N; ++n)\n            CB[n * K + k] = amax == 0.0f ? 0 : quantize_value(widen(W[n * K + k], dtype), absmax_scale(amax));\n    }\n    for (int64_t n = 0; n < N; ++n) {\n        float amax = 0.0f;\n        for (int64_t k = 0; k < K; ++k) {\n            float a = fabsf(widen(W[n * K + k], dtype));\n            if (a > amax) amax = a;\n        }\n        SCB[n] = amax;\n    }\n    return OK;\n    for (int64_t n = 0; n < N; ++n) {\n        const uint16_t* row = W + n * K;'),
    ]),
    4: ('round half away from zero', [
        ('    float r = nearbyintf(product); /* round half to even (default mode) */',
         '    float r = (product < 0) ? -floorf(-product + 0.5f) : floorf(product + 0.5f); /* half away */'),
    ]),
    5: ('dequantize by 127 instead of 127^2', [
        ('            double y_int8 = (double)C[r * N + n] * (double)SCA[m] * (double)SCB[n] / 16129.0;',
         '            double y_int8 = (double)C[r * N + n] * (double)SCA[m] * (double)SCB[n] / 127.0;'),
    ]),
    6: ('recovered weight missing SCB/127', [
        ('    return (double)CB[n * K + k] * (double)SCB[n] / 127.0;',
         '    (void)SCB;\n    return (double)CB[n * K + k]; /* mistake: scale not applied */'),
    ]),
    7: ('bias dropped', [
        ('            double b = bias ? (double)widen(bias[n], dtype) : 0.0;\n            Y[r * N + n] = y_int8 + y_out + b;',
         '            (void)bias;\n            double b = 0.0; /* mistake: bias dropped */\n            Y[r * N + n] = y_int8 + y_out + b;'),
    ]),
    8: ('outlier entries left in CA', [
        ('                int zero = is_out[k];',
         '                int zero = 0; /* mistake: outlier entries not removed */'),
        ('                int zero = is_out[k] || amax == 0.0f;',
         '                int zero = amax == 0.0f; /* mistake: outlier entries not removed */'),
    ]),
    9: ('outlier part subtracted', [
        ('            Y[r * N + n] = y_int8 + y_out + b;',
         '            Y[r * N + n] = y_int8 - y_out + b; /* mistake: wrong sign */'),
    ]),
    10: ('outlier gather ignores the index list', [
        ('        for (int32_t j = 0; j < count; ++j) XO[m * (int64_t)count + j] = row[idx[j]];',
         '        for (int32_t j = 0; j < count; ++j) XO[m * (int64_t)count + j] = row[j]; /* mistake: index */'),
    ]),
    11: ('int8 product drops a term', [
        ('            for (int64_t k = 0; k < K; ++k) acc += (int64_t)a[k] * (int64_t)b[k];',
         '            for (int64_t k = 0; k + 1 < K; ++k) acc += (int64_t)a[k] * (int64_t)b[k]; /* mistake: drops a term */'),
    ]),
    12: ('per-tensor scale taken per row', [
        ('    for (int64_t r = 0; r < rows; ++r) scale[r] = amax;',
         '    /* mistake: the scale taken per row, not over the whole tensor */\n    for (int64_t r = 0; r < rows; ++r) {\n        float ra = 0.0f;\n        for (int64_t c = 0; c < cols; ++c) {\n            float a = fabsf(widen(A[r * cols + c], dtype));\n            if (a > ra) ra = a;\n        }\n        scale[r] = ra;\n        for (int64_t c = 0; c < cols; ++c)\n            Q[r * cols + c] = ra == 0.0f ? 0 : quantize_value(widen(A[r * cols + c], dtype), absmax_scale(ra));\n    }\n    (void)amax;\n    return OK;\n    for (int64_t r = 0; r < rows; ++r) scale[r] = amax;'),
    ]),
    13: ('E4M3 ties rounded away from zero', [
        ('    double q = nearbyint(sig); /* ties to even (default rounding mode) */',
         '    double q = floor(sig + 0.5); /* mistake: ties away from zero */'),
    ]),
    14: ('FP8 product dequantized by 448 instead of 448^2', [
        ('            double y8 = C[r * N + n] * (double)SCA[m] * (double)SCB[n] / 200704.0;',
         '            double y8 = C[r * N + n] * (double)SCA[m] * (double)SCB[n] / 448.0; /* mistake */'),
    ]),
    15: ('E4M3 subnormals flushed to zero', [
        ('        const double q = nearbyint(a * 512.0);\n        return (uint8_t)(sign | (uint8_t)q);',
         '        return sign; /* mistake: subnormals flushed to zero */'),
    ]),
    16: ('FP8 scale uses the int8 range 127', [
        ('    return 448.0f / absmax; /* one IEEE fp32 division */',
         '    return 127.0f / absmax; /* mistake: the int8 range */'),
    ]),
}
