/*
 * llmint8 -- the LLM.int8() mixed-precision decomposition matmul on AMD
 * Instinct MI355X (gfx950), as a C-ABI shared library (libllmint8.so).
 *
 * Computes Y = X . W^T for a transformer linear layer (X [M,K] tokens x
 * features, W [N,K] output channels x features) in three parts, following
 * "A Gentle Introduction to 8-bit Matrix Multiplication for transformers at
 * scale" (sections "LLM.int8() summary" and "inside the MatMul"):
 *   1. feature columns of X holding any |x| >= threshold are outliers;
 *   2. everything else is absmax-quantized to int8 per row of X (SCA) and per
 *      output channel of W (CB, SCB), multiplied with int32 accumulation and
 *      dequantized by SCA[m] * SCB[n] / 127^2;
 *   3. the outlier columns of X are multiplied in 16-bit against the matching
 *      recovered weights CB[n,k] * SCB[n] / 127 ("Usage" section) and added in,
 *      with the optional bias, into a 16-bit Y.
 *
 * Conventions for every entry point
 *   - Every pointer is caller-owned DEVICE memory on the current HIP device,
 *     16-byte aligned.  Nothing is retained after return.  All matrices are
 *     row-major and densely packed (row stride = number of columns).
 *   - Work is enqueued asynchronously on `stream` (NULL = the null stream).
 *     The library never synchronizes and never copies to the host; the
 *     outlier count stays in device memory.  Keep buffers alive until the
 *     stream has passed the call.
 *   - Arguments are validated before any HIP call.  On an error nothing is
 *     enqueued.  No C++ exception crosses this interface.
 *   - Calls are reentrant; calls that share output buffers or a workspace
 *     must not overlap.
 *   - dtype is LLMINT8_F16 or LLMINT8_BF16; X, W, bias, X_outlier and Y share it.
 *     (The pages require fp16 inputs; bf16 follows the same rules with a bf16
 *     outlier product and a bf16 output.)
 *   - K must be a positive multiple of 64 and at most LLMINT8_K_MAX, which
 *     keeps |int32 accumulator| <= K * 127^2 < 2^31.  M and N may be any
 *     value in [0, 2^31); M == 0 or N == 0 is a valid empty call.
 */
#ifndef LLMINT8_H
#define LLMINT8_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum llmint8_status {
    LLMINT8_OK = 0,
    LLMINT8_ERR_INVALID_ARGUMENT = 1, /* NULL/misaligned pointer, negative size, bad dtype,
                                         NaN or negative threshold, workspace too small */
    LLMINT8_ERR_UNSUPPORTED = 2,      /* K not a positive multiple of 64, K > LLMINT8_K_MAX,
                                         size >= 2^31, device is not gfx950 */
    LLMINT8_ERR_HIP = 3               /* a HIP call or launch failed; see llmint8_last_hip_error */
} llmint8_status;

typedef enum llmint8_dtype { LLMINT8_F16 = 0, LLMINT8_BF16 = 1 } llmint8_dtype;

#define LLMINT8_K_ALIGN 64
#define LLMINT8_K_MAX 133120 /* largest multiple of 64 with K * 127^2 < 2^31 */

/*
 * Weight quantization, once per weight ("Usage": quantization happens when the
 * layer is moved to the GPU; vector-wise absmax per output channel, "absmax
 * quantization").
 *   W   [N,K] 16-bit, read only.
 *   CB  [N,K] int8 out: CB[n,k] = rne(W[n,k] * (127 / SCB[n])) in [-127,127]
 *       (fp32 divide, fp32 multiply, round half to even); 0 when SCB[n] == 0.
 *   SCB [N] fp32 out: SCB[n] = max_k |W[n,k]|.
 * The recovered weight is CB[n,k] * SCB[n] / 127.
 */
llmint8_status llmint8_quantize_weight(const void* W, int dtype, int64_t N, int64_t K,
                                       int8_t* CB, float* SCB, hipStream_t stream);

/* Bytes of device workspace llmint8_quantize_tensor needs (0 for invalid sizes). */
size_t llmint8_quantize_tensor_workspace_size(int64_t rows, int64_t cols);

/*
 * Per-tensor absmax quantization, the baseline scheme ("absmax quantization":
 * scale by 127 / absmax, with one absmax for the whole tensor), for comparing
 * schemes.  No outlier extraction.
 *   A      [rows, cols] 16-bit, read only, finite; cols a positive multiple of 64.
 *   Q      [rows, cols] int8 out: rne(A * (127 / amax)), amax = max |A| over the
 *          whole tensor; all 0 when amax == 0.
 *   scale  [rows] fp32 out: amax in every entry, so (Q, scale) can be passed to
 *          llmint8_matmul as (CA, SCA) or as (CB, SCB) -- with n_outliers = 0 the
 *          product is dequantized by amax_X * amax_W / 127^2.
 *   workspace  llmint8_quantize_tensor_workspace_size bytes, no initialization.
 * rows == 0 is a no-op.  Errors: as llmint8_quantize_act.
 */
llmint8_status llmint8_quantize_tensor(const void* A, int dtype, int64_t rows, int64_t cols,
                                       int8_t* Q, float* scale, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace llmint8_quantize_act needs for M x K (may be 0). */
size_t llmint8_quantize_act_workspace_size(int64_t M, int64_t K);

/*
 * Activation quantization with outlier extraction ("LLM.int8() summary" step 1,
 * "inside the MatMul": columns holding a magnitude of threshold or more; row-wise
 * absmax quantization of the hidden states).  The outlier set is taken over all M
 * rows of this call.
 *   X           [M,K] 16-bit, read only.  Finite values only.
 *   threshold   fp32, >= 0; +inf gives no outliers, 0 makes every column one.
 *   CA          [M,K] int8 out: rne(X[m,k] * (127 / SCA[m])) for non-outlier k,
 *               0 for outlier k and for rows with SCA[m] == 0.
 *   SCA         [M] fp32 out: max over non-outlier k of |X[m,k]| (0 if none).
 *   outlier_idx [K] int32 out: the first n_out entries are the outlier columns in
 *               ascending order; later entries are unspecified.
 *   n_outliers  [1] int32 out: n_out.
 *   X_outlier   capacity M*K 16-bit out: holds XO [M, n_pad] row-major with
 *               n_pad = round_up(n_out, 32) <= K, XO[m,j] = X[m, idx[j]] for
 *               j < n_out and 0 for n_out <= j < n_pad.
 *   workspace   device scratch of llmint8_quantize_act_workspace_size(M,K) bytes
 *               (may be NULL when that is 0); contents need no initialization.
 */
llmint8_status llmint8_quantize_act(const void* X, int dtype, int64_t M, int64_t K,
                                    float threshold, int8_t* CA, float* SCA,
                                    int32_t* outlier_idx, int32_t* n_outliers, void* X_outlier,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of optional device workspace llmint8_matmul can use for M x N x K
 * (0 for the weight-streaming product and for invalid sizes: M <= 16, or
 * M <= 64 with M * N * K <= 6e9 or with a streaming grid of one round:
 * for M <= 32 at most 512 workgroups, ceil(N/64) when N >= 16384, else
 * ceil(N/16); for M > 32, N >= 16384 and ceil(N/64) <= 256).  Otherwise
 * the product works on
 * tiles of 256 rows by W columns, W = 256 or 224: for each W, T(W) =
 * ceil(M/256) * ceil(N/W) tiles, S(W) workgroups per tile (below), and the
 * W with the fewer MFMA cycles per CU, ceil(T*S/256) * W * ceil(ceil(K/128)/S),
 * is taken, 256 on a tie (224 at 512 x 57344 x 14336 and 512 x 14336 x 57344;
 * the environment variable LLMINT8_TILE_COLS, "256" or "224", forces one,
 * for tests).  The workspace is the sum of:
 *   - split K, when the T tiles fill at most half of the 256 CUs (T <= 128):
 *     S = min(floor(256/T), floor(K/1024), 8) workgroups per tile (if S >= 2),
 *     needing 4T bytes of counters rounded up to 256, then S * T * 256 * W * 4
 *     bytes of partial tiles;
 *   - N * min(K, 1024) bytes: the weight codes at up to 1024 outlier
 *     columns. */
size_t llmint8_matmul_workspace_size(int64_t M, int64_t N, int64_t K);

/*
 * The decomposed product ("LLM.int8() summary" steps 2-3):
 *   Y[m,n] = (C[m,n] * SCA[m] / 127 + sum_{j<n_out} XO[m,j] * CB[n, idx[j]]) * SCB[n] / 127
 *            + bias[n],
 *   C[m,n] = sum_k CA[m,k] * CB[n,k]  (exact int32),
 * which equals C * SCA * SCB / 127^2 + XO . (recovered W[:, idx])^T + bias.
 * Inputs are the outputs of llmint8_quantize_act (CA, SCA, outlier_idx,
 * n_outliers, X_outlier) and llmint8_quantize_weight (CB, SCB); in particular
 * the first n_outliers entries of outlier_idx are distinct columns below K in
 * ascending order (the product relies on it and does not check it).
 *   bias   [N] 16-bit or NULL.
 *   Y      [M,N] 16-bit out (round to nearest even from fp32).
 *   C_i32  [M,N] int32 out or NULL: when given, the same kernels also store the
 *          exact int8 accumulators (for parity checks).
 *   workspace  optional scratch, 16-byte aligned; NULL / 0 bytes is always
 *          valid.  Past the weight-streaming shapes it is used in this order:
 *          - the split-K region (sizes at llmint8_matmul_workspace_size),
 *            when the shape splits and the workspace holds it: the product
 *            then spreads K over several workgroups per tile;
 *          - the rest, R bytes, for the weight codes at the outlier columns,
 *            gathered once per call (by the activation kernel in
 *            llmint8_linear, else by a small kernel ahead of the GEMM) into N
 *            rows of C bytes, C a multiple of 64: C = 64 * floor(R / (64 N)),
 *            at most K (1024 at the default size, every column with N * K
 *            bytes); at most 16 columns go in rows of 16 bytes instead.  The
 *            product's tiles read their rows' codes there rather than from CB
 *            (a 128-byte line per row and column, for every tile row), and
 *            with more than 16 columns the outlier part runs as a second
 *            pipelined K loop over them.  With more outlier columns than C (n_outliers is read
 *            on the device) the product gathers each tile's codes itself,
 *            several times slower, unless the outlier columns are exactly
 *            0 .. n_outliers-1 (every column at threshold 0), whose codes it
 *            reads from CB directly.
 *          The contents need no initialization and are not kept.  Calls
 *          that share a workspace must not overlap.
 */
llmint8_status llmint8_matmul(int dtype, int64_t M, int64_t N, int64_t K,
                              const int8_t* CA, const float* SCA, const int32_t* outlier_idx,
                              const int32_t* n_outliers, const void* X_outlier,
                              const int8_t* CB, const float* SCB, const void* bias,
                              void* Y, int32_t* C_i32,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Same as llmint8_matmul, for measurement: the HIP events `start` and `stop`
 * (either may be NULL) are bound to the dispatch of the main int8 GEMM kernel
 * through hipExtLaunchKernel, so hipEventElapsedTime(start, stop) is that
 * kernel's own device time.
 */
llmint8_status llmint8_matmul_profiled(int dtype, int64_t M, int64_t N, int64_t K,
                                       const int8_t* CA, const float* SCA,
                                       const int32_t* outlier_idx, const int32_t* n_outliers,
                                       const void* X_outlier, const int8_t* CB, const float* SCB,
                                       const void* bias, void* Y, int32_t* C_i32,
                                       void* workspace, size_t workspace_bytes,
                                       hipStream_t stream, hipEvent_t start, hipEvent_t stop);

/* Bytes of device workspace llmint8_linear needs for M x N x K (may be 0). */
size_t llmint8_linear_workspace_size(int64_t M, int64_t N, int64_t K);

/*
 * The whole forward of an LLM.int8() linear layer in one call: the results of
 * llmint8_quantize_act followed by llmint8_matmul (the layer's forward in the
 * "Usage" section: int8 weights placed once, 16-bit activations in, 16-bit
 * output).  Arguments have the meanings given above; CA, SCA, outlier_idx,
 * n_outliers and X_outlier are filled exactly as llmint8_quantize_act fills
 * them.  C_i32 may be NULL.  For M <= 16 with K <= 4096, or M <= 8 with
 * K <= 8192, the forward is one fused kernel (each workgroup re-derives the
 * tiny activation quantization while its weight slab streams in); otherwise it
 * is the quantize_act launches followed by the matmul kernel.
 * workspace: at least llmint8_linear_workspace_size bytes, 16-byte aligned:
 * llmint8_quantize_act's workspace rounded up to 256 bytes, then the rest
 * used as llmint8_matmul's (more bytes hold more outlier columns).
 */
llmint8_status llmint8_linear(const void* X, int dtype, int64_t M, int64_t N, int64_t K,
                              float threshold, const int8_t* CB, const float* SCB,
                              const void* bias, void* Y, int8_t* CA, float* SCA,
                              int32_t* outlier_idx, int32_t* n_outliers, void* X_outlier,
                              int32_t* C_i32, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* llmint8_linear with `start`/`stop` bound to the dispatch of its int8 GEMM
 * kernel (the fused kernel when M is small), as in llmint8_matmul_profiled. */
llmint8_status llmint8_linear_profiled(const void* X, int dtype, int64_t M, int64_t N, int64_t K,
                                       float threshold, const int8_t* CB, const float* SCB,
                                       const void* bias, void* Y, int8_t* CA, float* SCA,
                                       int32_t* outlier_idx, int32_t* n_outliers, void* X_outlier,
                                       int32_t* C_i32, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream, hipEvent_t start, hipEvent_t stop);

/*
 * For callers that cannot allocate device memory: code being captured into a
 * HIP graph, serving loops and harnesses that forbid hipMalloc.  The same
 * forward as llmint8_linear, with the same arguments and results, minus the
 * workspace: the scratch memory it needs (the activation kernel's partial
 * column masks, split-K partial tiles and arrival counters, the weight codes at
 * the outlier columns) lives in a static device array of
 * LLMINT8_SCRATCH_BYTES bytes that the library holds on each device it runs on
 * until the process ends.  Nothing is allocated or freed, by the library or
 * by any library routine it calls.
 *   - Shapes whose llmint8_linear_workspace_size exceeds LLMINT8_SCRATCH_BYTES
 *     are refused with LLMINT8_ERR_UNSUPPORTED before any HIP call.  Decode
 *     batches need none, 2048 x 16384 x 4096 needs 16 MiB, 4096 x 28672 x 8192
 *     28 MiB and 512 x 57344 x 14336 56 MiB; 512 x 14336 x 57344 (70 MiB with
 *     its split-K partial tiles) is refused.
 *   - Every call on a device uses that device's one array: calls on the same
 *     device that overlap in time (on different streams, or from threads that
 *     enqueue concurrently) race on it and give undefined results.  Calls
 *     ordered on one stream are safe; each call clears what it needs cleared.
 *   - The first call on a device looks up the array's device address
 *     (hipGetSymbolAddress) with that device current.
 */
#define LLMINT8_SCRATCH_BYTES (64u << 20)
llmint8_status llmint8_linear_noalloc(const void* X, int dtype, int64_t M, int64_t N, int64_t K,
                                      float threshold, const int8_t* CB, const float* SCB,
                                      const void* bias, void* Y, int8_t* CA, float* SCA,
                                      int32_t* outlier_idx, int32_t* n_outliers, void* X_outlier,
                                      int32_t* C_i32, hipStream_t stream);

/*
 * ---- FP8 (E4M3) variant of the decomposition -------------------------------
 * The zhichai.top summary of LLM.int8() (outlook section, its list of the
 * method's limitations) names an 8-bit floating-point type as future work.
 * These entry points run the same decomposition -- the same outlier columns,
 * row and channel absmax scales and 16-bit outlier product -- with OCP FP8
 * E4M3 codes in place of int8, on gfx950's fp8 matrix instructions:
 *   code  = e4m3(x * (448 / absmax)): fp32 divide, fp32 multiply, then the
 *           nearest E4M3 value (ties to the even code, subnormals kept, a
 *           result that rounds to zero keeps its sign).  E4M3: sign, 4
 *           exponent bits (bias 7), 3 mantissa bits, largest finite 448, no
 *           infinities; codes 0x7F/0xFF (NaN) are never produced.
 *   value(code) is that E4M3 number; the recovered weight is
 *           value(CB[n,k]) * SCB[n] / 448.
 *   C[m,n] = sum_k value(CA[m,k]) * value(CB[n,k]), accumulated in fp32 by the
 *           matrix cores (every product is exact; the sum's rounding order is
 *           the hardware's), and
 *   Y[m,n] = (C[m,n] * SCA[m] / 448 + sum_{j<n_out} XO[m,j] * value(CB[n,idx[j]]))
 *            * SCB[n] / 448 + bias[n].
 * Codes travel as uint8 bytes.  Sizes, dtypes, pointers, streams and errors
 * follow the conventions at the top of this file.  A vector whose absmax is 0
 * gets scale 0 and the codes of its signed zeros (0x00 / 0x80).
 */

/* E4M3 weight codes, as llmint8_quantize_weight with 448 for 127:
 *   CB [N,K] uint8 out: e4m3(W[n,k] * (448 / SCB[n]));  SCB [N] fp32 out: row absmax. */
llmint8_status llmint8_quantize_weight_fp8(const void* W, int dtype, int64_t N, int64_t K,
                                           uint8_t* CB, float* SCB, hipStream_t stream);

/* E4M3 activation codes with outlier extraction, as llmint8_quantize_act (same
 * outlier_idx, n_outliers, X_outlier, SCA and workspace) except
 *   CA [M,K] uint8 out: e4m3(X[m,k] * (448 / SCA[m])) for non-outlier k, 0x00 for
 *      outlier k. */
llmint8_status llmint8_quantize_act_fp8(const void* X, int dtype, int64_t M, int64_t K,
                                        float threshold, uint8_t* CA, float* SCA,
                                        int32_t* outlier_idx, int32_t* n_outliers,
                                        void* X_outlier, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream);

/* The FP8 product Y (formula above) from llmint8_quantize_act_fp8 and
 * llmint8_quantize_weight_fp8 outputs.  C_f32 [M,N] fp32 out or NULL: the
 * accumulated C before scaling.  workspace: as llmint8_matmul. */
llmint8_status llmint8_matmul_fp8(int dtype, int64_t M, int64_t N, int64_t K,
                                  const uint8_t* CA, const float* SCA,
                                  const int32_t* outlier_idx, const int32_t* n_outliers,
                                  const void* X_outlier, const uint8_t* CB, const float* SCB,
                                  const void* bias, void* Y, float* C_f32, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/* llmint8_matmul_fp8 with `start`/`stop` bound to the dispatch of its GEMM kernel. */
llmint8_status llmint8_matmul_fp8_profiled(int dtype, int64_t M, int64_t N, int64_t K,
                                           const uint8_t* CA, const float* SCA,
                                           const int32_t* outlier_idx,
                                           const int32_t* n_outliers, const void* X_outlier,
                                           const uint8_t* CB, const float* SCB, const void* bias,
                                           void* Y, float* C_f32, void* workspace,
                                           size_t workspace_bytes, hipStream_t stream,
                                           hipEvent_t start, hipEvent_t stop);

/* Bytes of device workspace llmint8_linear_fp8 needs for M x N x K (may be 0). */
size_t llmint8_linear_fp8_workspace_size(int64_t M, int64_t N, int64_t K);

/* The whole FP8 forward: llmint8_quantize_act_fp8 then llmint8_matmul_fp8 (two or
 * four launches), filling CA, SCA, outlier_idx, n_outliers, X_outlier as the
 * former does and C_f32 (may be NULL) as the latter.
 * workspace: llmint8_linear_fp8_workspace_size bytes. */
llmint8_status llmint8_linear_fp8(const void* X, int dtype, int64_t M, int64_t N, int64_t K,
                                  float threshold, const uint8_t* CB, const float* SCB,
                                  const void* bias, void* Y, uint8_t* CA, float* SCA,
                                  int32_t* outlier_idx, int32_t* n_outliers, void* X_outlier,
                                  float* C_f32, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/* llmint8_linear_fp8 with `start`/`stop` bound to the dispatch of its GEMM kernel. */
llmint8_status llmint8_linear_fp8_profiled(const void* X, int dtype, int64_t M, int64_t N,
                                           int64_t K, float threshold, const uint8_t* CB,
                                           const float* SCB, const void* bias, void* Y,
                                           uint8_t* CA, float* SCA, int32_t* outlier_idx,
                                           int32_t* n_outliers, void* X_outlier, float* C_f32,
                                           void* workspace, size_t workspace_bytes,
                                           hipStream_t stream, hipEvent_t start,
                                           hipEvent_t stop);

/* Diagnostic for the roofline report, not a step of the method: the device's
 * sustained matrix-core rate, the measured ceiling reported beside the
 * published peak.  Launches `blocks` workgroups of 256 threads; every wave
 * runs 4 * iters back-to-back MFMAs on four independent accumulators --
 * fp8 = 0: v_mfma_i32_32x32x32_i8 (65536 operations each); fp8 = 1:
 * v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3 codes (131072 each) -- so the
 * launch performs blocks * 16 * iters * (65536 or 131072) operations.
 * operands: device, at least 262144 bytes of codes read once per wave (the
 * power drawn, and so the clock, depends on them: pass random codes, finite
 * ones for E4M3).  sink: device, at least blocks * 1024 bytes, one word per
 * thread (written so that nothing is optimised away).  Time the launch with
 * events on `stream`.  Errors: LLMINT8_ERR_INVALID_ARGUMENT for NULL or
 * misaligned pointers, buffers too small, blocks or iters below 1;
 * LLMINT8_ERR_UNSUPPORTED when the device is not gfx950. */
llmint8_status llmint8_peak_mfma(int fp8, const int8_t* operands, size_t operand_bytes,
                                 int32_t* sink, size_t sink_bytes, int blocks, int iters,
                                 hipStream_t stream);

/* Static English text for a status code. */
const char* llmint8_status_string(llmint8_status s);

/* The hipError_t behind the calling thread's last LLMINT8_ERR_HIP (0 if none). */
int llmint8_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LLMINT8_H */
