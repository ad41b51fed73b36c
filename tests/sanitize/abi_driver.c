/* Calls every entry point of the C ABI with arguments its validation must
 * refuse (negative or unsupported sizes, a bad dtype, NULL or misaligned
 * pointers, a NaN or negative threshold, a short workspace), and the size
 * queries over ordinary and extreme shapes, for a host build under
 * AddressSanitizer and UndefinedBehaviorSanitizer.  Every refused call returns
 * before any HIP call, so no GPU is needed.  Exits non-zero on an unexpected
 * status; the sanitizers abort on any finding.  Test infrastructure only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "llmint8.h"

static int failures = 0;
#define EXPECT(cond)                                                        \
    do {                                                                    \
        if (!(cond)) {                                                      \
            fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                     \
        }                                                                   \
    } while (0)
#define REFUSED(call) EXPECT((call) == LLMINT8_ERR_INVALID_ARGUMENT || (call) == LLMINT8_ERR_UNSUPPORTED)

/* host buffers stand in for device pointers: validation never dereferences */
static _Alignas(16) unsigned char buf[1 << 16];

int main(void) {
    void* p = buf;
    void* odd = buf + 8; /* 8-byte aligned only */
    const int64_t big = INT64_MAX, sizes[] = {-1, 0, 1, 16, 17, 64, 4096, 133120, 133184, 1LL << 31, big};
    const int nsz = (int)(sizeof(sizes) / sizeof(sizes[0]));
    /* size queries: any shape, no overflow */
    for (int a = 0; a < nsz; ++a)
        for (int b = 0; b < nsz; ++b)
            for (int c = 0; c < nsz; ++c) {
                (void)llmint8_matmul_workspace_size(sizes[a], sizes[b], sizes[c]);
                (void)llmint8_linear_workspace_size(sizes[a], sizes[b], sizes[c]);
                (void)llmint8_linear_fp8_workspace_size(sizes[a], sizes[b], sizes[c]);
            }
    for (int a = 0; a < nsz; ++a)
        for (int b = 0; b < nsz; ++b) {
            (void)llmint8_quantize_act_workspace_size(sizes[a], sizes[b]);
            (void)llmint8_quantize_tensor_workspace_size(sizes[a], sizes[b]);
        }
    EXPECT(llmint8_matmul_workspace_size(-1, 64, 64) == 0);
    EXPECT(llmint8_quantize_act_workspace_size(64, 100) == 0);

    /* weight quantization */
    REFUSED(llmint8_quantize_weight(p, 2, 4, 64, p, p, NULL));          /* dtype */
    REFUSED(llmint8_quantize_weight(p, 0, -1, 64, p, p, NULL));         /* N < 0 */
    REFUSED(llmint8_quantize_weight(p, 0, 4, 100, p, p, NULL));         /* K % 64 */
    REFUSED(llmint8_quantize_weight(p, 0, 4, 133184, p, p, NULL));      /* K > max */
    REFUSED(llmint8_quantize_weight(NULL, 0, 4, 64, p, p, NULL));       /* W NULL */
    REFUSED(llmint8_quantize_weight(p, 0, 4, 64, odd, p, NULL));        /* CB misaligned */
    REFUSED(llmint8_quantize_weight_fp8(p, 0, 4, 64, NULL, p, NULL));
    REFUSED(llmint8_quantize_weight_fp8(p, 1, big, 64, p, p, NULL));

    /* per-tensor quantization */
    REFUSED(llmint8_quantize_tensor(p, 0, 4, 96, p, p, p, sizeof buf, NULL));
    REFUSED(llmint8_quantize_tensor(NULL, 0, 4, 64, p, p, p, sizeof buf, NULL));
    REFUSED(llmint8_quantize_tensor(p, 0, -4, 64, p, p, p, sizeof buf, NULL));

    /* activation quantization */
    REFUSED(llmint8_quantize_act(p, 0, 4, 64, NAN, p, p, p, p, p, p, sizeof buf, NULL));
    REFUSED(llmint8_quantize_act(p, 0, 4, 64, -1.0f, p, p, p, p, p, p, sizeof buf, NULL));
    REFUSED(llmint8_quantize_act(p, 0, 4, 64, 6.0f, p, p, p, NULL, p, p, sizeof buf, NULL));
    REFUSED(llmint8_quantize_act(p, 0, 4, 64, 6.0f, p, p, odd, p, p, p, sizeof buf, NULL));
    REFUSED(llmint8_quantize_act(p, 3, 4, 64, 6.0f, p, p, p, p, p, p, sizeof buf, NULL));
    REFUSED(llmint8_quantize_act(p, 0, 2048, 4096, 6.0f, p, p, p, p, p, p, 16, NULL)); /* workspace */
    REFUSED(llmint8_quantize_act_fp8(p, 0, 4, 64, NAN, p, p, p, p, p, p, sizeof buf, NULL));
    REFUSED(llmint8_quantize_act_fp8(p, 0, 4, 65, 6.0f, p, p, p, p, p, p, sizeof buf, NULL));

    /* the product */
    REFUSED(llmint8_matmul(0, 4, 4, 96, p, p, p, p, p, p, p, NULL, p, NULL, NULL, 0, NULL));
    REFUSED(llmint8_matmul(0, -4, 4, 64, p, p, p, p, p, p, p, NULL, p, NULL, NULL, 0, NULL));
    REFUSED(llmint8_matmul(0, 4, 4, 64, NULL, p, p, p, p, p, p, NULL, p, NULL, NULL, 0, NULL));
    REFUSED(llmint8_matmul(0, 4, 4, 64, p, p, p, p, p, p, p, odd, p, NULL, NULL, 0, NULL));
    REFUSED(llmint8_matmul(0, 4, 4, 64, p, p, p, p, p, p, p, NULL, p, odd, NULL, 0, NULL));
    REFUSED(llmint8_matmul(0, 4, 4, 64, p, p, p, p, p, p, p, NULL, p, NULL, odd, 64, NULL));
    REFUSED(llmint8_matmul(5, 4, 4, 64, p, p, p, p, p, p, p, NULL, p, NULL, NULL, 0, NULL));
    REFUSED(llmint8_matmul_profiled(0, 4, 4, 100, p, p, p, p, p, p, p, NULL, p, NULL, NULL, 0, NULL,
                                    NULL, NULL));
    REFUSED(llmint8_matmul_fp8(0, 4, 4, 64, p, p, p, p, p, NULL, p, NULL, p, NULL, NULL, 0, NULL));
    REFUSED(llmint8_matmul_fp8_profiled(0, big, 4, 64, p, p, p, p, p, p, p, NULL, p, NULL, NULL, 0,
                                        NULL, NULL, NULL));

    /* the one-call forward */
    REFUSED(llmint8_linear(p, 0, 4, 4, 64, NAN, p, p, NULL, p, p, p, p, p, p, NULL, p, sizeof buf, NULL));
    REFUSED(llmint8_linear(p, 0, 4, 4, 64, 6.0f, NULL, p, NULL, p, p, p, p, p, p, NULL, p, sizeof buf,
                           NULL));
    REFUSED(llmint8_linear(p, 0, 2048, 4096, 4096, 6.0f, p, p, NULL, p, p, p, p, p, p, NULL, p, 64,
                           NULL)); /* workspace too small */
    REFUSED(llmint8_linear(p, 0, 4, 4, 64, 6.0f, p, p, NULL, p, p, p, p, p, p, NULL, odd, sizeof buf,
                           NULL));
    REFUSED(llmint8_linear_profiled(p, 0, 4, 4, 100, 6.0f, p, p, NULL, p, p, p, p, p, p, NULL, p,
                                    sizeof buf, NULL, NULL, NULL));
    REFUSED(llmint8_linear_noalloc(p, 0, 4, 4, 64, -2.0f, p, p, NULL, p, p, p, p, p, p, NULL, NULL));
    REFUSED(llmint8_linear_noalloc(p, 0, 512, 14336, 57344, 6.0f, p, p, NULL, p, p, p, p, p, p, NULL,
                                   NULL)); /* scratch too small */
    REFUSED(llmint8_linear_fp8(p, 1, 4, 4, 64, 6.0f, p, p, NULL, NULL, p, p, p, p, p, NULL, p,
                               sizeof buf, NULL));
    REFUSED(llmint8_linear_fp8_profiled(p, 1, 4, 4, 128, 6.0f, p, p, NULL, p, p, p, p, p, p, NULL,
                                        odd, sizeof buf, NULL, NULL, NULL));

    /* the diagnostic */
    REFUSED(llmint8_peak_mfma(0, NULL, 262144, p, 1024, 1, 1, NULL));
    REFUSED(llmint8_peak_mfma(0, p, 16, p, 1024, 1, 1, NULL));
    REFUSED(llmint8_peak_mfma(0, p, 262144, p, 1024, 0, 1, NULL));

    /* status text for every code and for codes outside the enum */
    for (int s = -2; s < 8; ++s) EXPECT(llmint8_status_string((llmint8_status)s) != NULL);
    EXPECT(llmint8_last_hip_error() == 0);

    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("abi driver: ok\n");
    return 0;
}
