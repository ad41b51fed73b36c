// C-ABI of libllmint8: argument validation, device check and dispatch.
// The operations and their page citations are documented in include/llmint8.h.
#include <mutex>
#include <string.h>

#include "../../include/llmint8.h"
#include "common.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxDim = 0x7fffffff;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool bad_ptr(const void* p) { return p == nullptr || !aligned16(p); }

llmint8_status check_dtype(int dtype) {
    return (dtype == LLMINT8_F16 || dtype == LLMINT8_BF16) ? LLMINT8_OK
                                                             : LLMINT8_ERR_INVALID_ARGUMENT;
}

// Sizes: negative -> invalid; K must be a positive multiple of 64 <= K_MAX.
llmint8_status check_sizes(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0) return LLMINT8_ERR_INVALID_ARGUMENT;
    if (M > kMaxDim || N > kMaxDim) return LLMINT8_ERR_UNSUPPORTED;
    if (K == 0 || K % LLMINT8_K_ALIGN != 0 || K > LLMINT8_K_MAX) return LLMINT8_ERR_UNSUPPORTED;
    return LLMINT8_OK;
}

llmint8_status hip_fail(hipError_t e) {
    g_last_hip_error = (int)e;
    return LLMINT8_ERR_HIP;
}

// The current device must be gfx950.  Cached per device id.
std::mutex g_dev_mu;
signed char g_dev_ok[64];  // 0 unknown, 1 ok, -1 not gfx950

llmint8_status check_device() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= 64) return LLMINT8_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_dev_ok[dev] == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return hip_fail(e);
        g_dev_ok[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    }
    return g_dev_ok[dev] == 1 ? LLMINT8_OK : LLMINT8_ERR_UNSUPPORTED;
}

// fp8: CA / CB hold E4M3 code bytes and the product goes to C_f32 (C_i32 unused)
llmint8_status matmul_impl(int dtype, bool fp8, int64_t M, int64_t N, int64_t K,
                           const int8_t* CA, const float* SCA, const int32_t* outlier_idx,
                           const int32_t* n_outliers, const void* X_outlier, const int8_t* CB,
                           const float* SCB, const void* bias, void* Y, int32_t* C_i32,
                           float* C_f32, void* workspace, size_t workspace_bytes,
                           hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop) {
    llmint8_status s = check_dtype(dtype);
    if (s != LLMINT8_OK) return s;
    if ((s = check_sizes(M, N, K)) != LLMINT8_OK) return s;
    if (M == 0 || N == 0) return LLMINT8_OK;
    if (bad_ptr(CA) || bad_ptr(SCA) || bad_ptr(outlier_idx) || bad_ptr(n_outliers) ||
        bad_ptr(X_outlier) || bad_ptr(CB) || bad_ptr(SCB) || bad_ptr(Y))
        return LLMINT8_ERR_INVALID_ARGUMENT;
    if ((bias && !aligned16(bias)) || (C_i32 && !aligned16(C_i32)) ||
        (C_f32 && !aligned16(C_f32)) || (workspace && !aligned16(workspace)))
        return LLMINT8_ERR_INVALID_ARGUMENT;
    if ((s = check_device()) != LLMINT8_OK) return s;
    llmint8::MatmulArgs a;
    a.bf16 = dtype == LLMINT8_BF16;
    a.fp8 = fp8;
    a.C_f32 = fp8 ? C_f32 : nullptr;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.CA = CA;
    a.SCA = SCA;
    a.idx = outlier_idx;
    a.n_out = n_outliers;
    a.XO = static_cast<const uint16_t*>(X_outlier);
    a.CB = CB;
    a.SCB = SCB;
    a.bias = static_cast<const uint16_t*>(bias);
    a.Y = static_cast<uint16_t*>(Y);
    a.C_i32 = fp8 ? nullptr : C_i32;
    a.ws = workspace;
    a.ws_bytes = workspace ? workspace_bytes : 0;
    hipError_t e = llmint8::launch_matmul(a, stream, ev_start, ev_stop);
    return e == hipSuccess ? LLMINT8_OK : hip_fail(e);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The FP8 forward has the fused decode kernel (M <= 8) but not the other
// fused small-M kernel.
size_t linear_workspace(int64_t M, int64_t N, int64_t K, bool fp8) {
    if (M == 0 || N == 0) return llmint8::quantize_act_workspace(M, K);
    if (llmint8::linear_decode_supported((int)M, (int)K)) return 0;
    if (!fp8 && llmint8::linear_small_m_supported((int)M, (int)K)) return 0;
    const size_t act = llmint8::quantize_act_workspace(M, K);
    const size_t mm = llmint8::matmul_workspace(M, N, K);
    return mm == 0 ? act : align256(act) + mm;
}

// ---- device scratch for the entry point that allocates nothing -------------
// One array per device (each device's code object holds its own copy), kept
// until the process ends.  Host code never passes the array's name to a
// kernel: its device address comes from hipGetSymbolAddress, taken once per
// device with that device current, and kept in g_scratch.
static __device__ __align__(256) unsigned char scratch[LLMINT8_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch[64];

// The current device's scratch address (device ids are checked by
// check_device first).
llmint8_status scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= 64) return LLMINT8_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e);
        if (p == nullptr) return hip_fail(hipErrorInvalidSymbol);
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return LLMINT8_OK;
}

// use_scratch: the workspace is the device's static scratch array (the
// workspace arguments are ignored); shapes that need more than it holds are
// refused before any HIP call.
llmint8_status linear_impl(const void* X, int dtype, bool fp8, int64_t M, int64_t N, int64_t K,
                           float threshold, const int8_t* CB, const float* SCB, const void* bias,
                           void* Y, int8_t* CA, float* SCA, int32_t* outlier_idx,
                           int32_t* n_outliers, void* X_outlier, int32_t* C_i32, float* C_f32,
                           void* workspace, size_t workspace_bytes, hipStream_t stream,
                           hipEvent_t ev_start, hipEvent_t ev_stop, bool use_scratch = false) {
    llmint8_status s = check_dtype(dtype);
    if (s != LLMINT8_OK) return s;
    if ((s = check_sizes(M, N, K)) != LLMINT8_OK) return s;
    if (threshold != threshold || threshold < 0.0f) return LLMINT8_ERR_INVALID_ARGUMENT;
    if (bad_ptr(n_outliers)) return LLMINT8_ERR_INVALID_ARGUMENT;
    if (M > 0 && (bad_ptr(X) || bad_ptr(CA) || bad_ptr(SCA) || bad_ptr(outlier_idx) ||
                  bad_ptr(X_outlier)))
        return LLMINT8_ERR_INVALID_ARGUMENT;
    if (M > 0 && N > 0 && (bad_ptr(CB) || bad_ptr(SCB) || bad_ptr(Y)))
        return LLMINT8_ERR_INVALID_ARGUMENT;
    if ((bias && !aligned16(bias)) || (C_i32 && !aligned16(C_i32)) ||
        (C_f32 && !aligned16(C_f32)) || (workspace && !aligned16(workspace)))
        return LLMINT8_ERR_INVALID_ARGUMENT;
    const size_t need = linear_workspace(M, N, K, fp8);
    if (use_scratch) {
        if (need > (size_t)LLMINT8_SCRATCH_BYTES) return LLMINT8_ERR_UNSUPPORTED;
    } else if (need > 0 && (workspace == nullptr || workspace_bytes < need)) {
        return LLMINT8_ERR_INVALID_ARGUMENT;
    }
    if ((s = check_device()) != LLMINT8_OK) return s;
    if (use_scratch) {
        workspace = nullptr;
        workspace_bytes = 0;
        if (need > 0) {
            if ((s = scratch_address(&workspace)) != LLMINT8_OK) return s;
            workspace_bytes = need;
        }
    }
    const bool bf16 = dtype == LLMINT8_BF16;
    hipError_t e;
    if (M > 0 && N > 0 && llmint8::linear_decode_supported((int)M, (int)K)) {
        e = llmint8::launch_linear_decode(X, bf16, fp8, (int)M, (int)N, (int)K, threshold, CB, SCB,
                                          bias, Y, CA, SCA, outlier_idx, n_outliers, X_outlier,
                                          fp8 ? nullptr : C_i32, fp8 ? C_f32 : nullptr, stream,
                                          ev_start, ev_stop);
        return e == hipSuccess ? LLMINT8_OK : hip_fail(e);
    }
    if (!fp8 && M > 0 && N > 0 && llmint8::linear_small_m_supported((int)M, (int)K)) {
        e = llmint8::launch_linear_small_m(X, bf16, (int)M, (int)N, (int)K, threshold, CB, SCB,
                                           bias, Y, CA, SCA, outlier_idx, n_outliers, X_outlier,
                                           C_i32, stream, ev_start, ev_stop);
        return e == hipSuccess ? LLMINT8_OK : hip_fail(e);
    }
    // the product's share of the workspace follows the activation kernels'
    const size_t act_ws = align256(llmint8::quantize_act_workspace(M, K));
    void* mm_ws = workspace && workspace_bytes > act_ws ? static_cast<char*>(workspace) + act_ws : nullptr;
    const size_t mm_bytes = mm_ws ? workspace_bytes - act_ws : 0;
    // For the tiled product, the activation kernel also gathers the weight
    // codes at the outlier columns when the workspace holds no more columns
    // than it can list (it knows the columns first); no extra launch.
    llmint8::CodeGather gather;
    if (!llmint8::small_m_product(M, N, K) && N > 0 && mm_ws) {
        const llmint8::TiledLayout L = llmint8::tiled_layout((int)M, (int)N, (int)K, mm_ws, mm_bytes);
        if (L.codes != nullptr && L.cap <= llmint8::kActGatherCols) {
            gather.CB = CB;
            gather.N = (int)N;
            gather.cap = L.cap;
            gather.min_cols = L.min_cols;
            gather.out = L.codes;
        }
    }
    e = llmint8::launch_quantize_act(X, bf16, fp8, (int)M, (int)K, threshold, CA, SCA, outlier_idx,
                                     n_outliers, X_outlier, workspace, stream, &gather);
    if (e != hipSuccess) return hip_fail(e);
    if (M == 0 || N == 0) return LLMINT8_OK;
    llmint8::MatmulArgs a;
    a.bf16 = bf16;
    a.fp8 = fp8;
    a.C_f32 = fp8 ? C_f32 : nullptr;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.CA = CA;
    a.SCA = SCA;
    a.idx = outlier_idx;
    a.n_out = n_outliers;
    a.XO = static_cast<const uint16_t*>(X_outlier);
    a.CB = CB;
    a.SCB = SCB;
    a.bias = static_cast<const uint16_t*>(bias);
    a.Y = static_cast<uint16_t*>(Y);
    a.C_i32 = fp8 ? nullptr : C_i32;
    a.ws = mm_ws;
    a.ws_bytes = mm_bytes;
    a.codes_gathered = gather.out != nullptr;
    e = llmint8::launch_matmul(a, stream, ev_start, ev_stop);
    return e == hipSuccess ? LLMINT8_OK : hip_fail(e);
}

}  // namespace

namespace llmint8 {

size_t matmul_workspace(int64_t M, int64_t N, int64_t K) {
    return small_m_product(M, N, K) ? 0 : gemm_tiled_workspace(M, N, K);
}

hipError_t launch_matmul(const MatmulArgs& a, hipStream_t stream, hipEvent_t ev_start,
                         hipEvent_t ev_stop) {
    if (small_m_product(a.M, a.N, a.K)) return launch_gemm_small_m(a, stream, ev_start, ev_stop);
    return launch_gemm_tiled(a, stream, ev_start, ev_stop);
}

}  // namespace llmint8

namespace {

llmint8_status quantize_weight_impl(const void* W, int dtype, bool fp8, int64_t N, int64_t K,
                                   int8_t* CB, float* SCB, hipStream_t stream) {
    llmint8_status s = check_dtype(dtype);
    if (s != LLMINT8_OK) return s;
    if ((s = check_sizes(0, N, K)) != LLMINT8_OK) return s;
    if (N == 0) return LLMINT8_OK;
    if (bad_ptr(W) || bad_ptr(CB) || bad_ptr(SCB)) return LLMINT8_ERR_INVALID_ARGUMENT;
    if ((s = check_device()) != LLMINT8_OK) return s;
    hipError_t e = llmint8::launch_quantize_weight(W, dtype == LLMINT8_BF16, fp8, (int)N, (int)K,
                                                   CB, SCB, stream);
    return e == hipSuccess ? LLMINT8_OK : hip_fail(e);
}

llmint8_status quantize_act_impl(const void* X, int dtype, bool fp8, int64_t M, int64_t K,
                                 float threshold, int8_t* CA, float* SCA, int32_t* outlier_idx,
                                 int32_t* n_outliers, void* X_outlier, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
    llmint8_status s = check_dtype(dtype);
    if (s != LLMINT8_OK) return s;
    if ((s = check_sizes(M, 0, K)) != LLMINT8_OK) return s;
    if (threshold != threshold || threshold < 0.0f) return LLMINT8_ERR_INVALID_ARGUMENT;
    if (bad_ptr(n_outliers)) return LLMINT8_ERR_INVALID_ARGUMENT;
    if (M > 0) {
        if (bad_ptr(X) || bad_ptr(CA) || bad_ptr(SCA) || bad_ptr(outlier_idx) || bad_ptr(X_outlier))
            return LLMINT8_ERR_INVALID_ARGUMENT;
        const size_t need = llmint8::quantize_act_workspace(M, K);
        if (need > 0 && (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need))
            return LLMINT8_ERR_INVALID_ARGUMENT;
    }
    if ((s = check_device()) != LLMINT8_OK) return s;
    hipError_t e = llmint8::launch_quantize_act(X, dtype == LLMINT8_BF16, fp8, (int)M, (int)K,
                                                threshold, CA, SCA, outlier_idx, n_outliers,
                                                X_outlier, workspace, stream);
    return e == hipSuccess ? LLMINT8_OK : hip_fail(e);
}

}  // namespace

namespace llmint8 {
// peak_probe.hip
hipError_t launch_mfma_peak(bool fp8, const int8_t* operands, int iters, int32_t* sink, int blocks,
                            hipStream_t stream);
}  // namespace llmint8

extern "C" {

llmint8_status llmint8_quantize_weight(const void* W, int dtype, int64_t N, int64_t K, int8_t* CB,
                                       float* SCB, hipStream_t stream) {
    return quantize_weight_impl(W, dtype, false, N, K, CB, SCB, stream);
}

llmint8_status llmint8_quantize_weight_fp8(const void* W, int dtype, int64_t N, int64_t K,
                                           uint8_t* CB, float* SCB, hipStream_t stream) {
    return quantize_weight_impl(W, dtype, true, N, K, reinterpret_cast<int8_t*>(CB), SCB, stream);
}

size_t llmint8_quantize_tensor_workspace_size(int64_t rows, int64_t cols) {
    if (check_sizes(rows, 0, cols) != LLMINT8_OK) return 0;
    return llmint8::quantize_tensor_workspace();
}

llmint8_status llmint8_quantize_tensor(const void* A, int dtype, int64_t rows, int64_t cols,
                                       int8_t* Q, float* scale, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
    llmint8_status s = check_dtype(dtype);
    if (s != LLMINT8_OK) return s;
    if ((s = check_sizes(rows, 0, cols)) != LLMINT8_OK) return s;
    if (rows == 0) return LLMINT8_OK;
    if (bad_ptr(A) || bad_ptr(Q) || bad_ptr(scale) || bad_ptr(workspace) ||
        workspace_bytes < llmint8::quantize_tensor_workspace())
        return LLMINT8_ERR_INVALID_ARGUMENT;
    if ((s = check_device()) != LLMINT8_OK) return s;
    hipError_t e = llmint8::launch_quantize_tensor(A, dtype == LLMINT8_BF16, rows, cols, Q, scale,
                                                   workspace, stream);
    return e == hipSuccess ? LLMINT8_OK : hip_fail(e);
}

size_t llmint8_quantize_act_workspace_size(int64_t M, int64_t K) {
    if (check_sizes(M, 0, K) != LLMINT8_OK) return 0;
    return llmint8::quantize_act_workspace(M, K);
}

llmint8_status llmint8_quantize_act(const void* X, int dtype, int64_t M, int64_t K,
                                    float threshold, int8_t* CA, float* SCA,
                                    int32_t* outlier_idx, int32_t* n_outliers, void* X_outlier,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return quantize_act_impl(X, dtype, false, M, K, threshold, CA, SCA, outlier_idx, n_outliers,
                             X_outlier, workspace, workspace_bytes, stream);
}

llmint8_status llmint8_quantize_act_fp8(const void* X, int dtype, int64_t M, int64_t K,
                                        float threshold, uint8_t* CA, float* SCA,
                                        int32_t* outlier_idx, int32_t* n_outliers,
                                        void* X_outlier, void* workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
    return quantize_act_impl(X, dtype, true, M, K, threshold, reinterpret_cast<int8_t*>(CA), SCA,
                             outlier_idx, n_outliers, X_outlier, workspace, workspace_bytes,
                             stream);
}

size_t llmint8_matmul_workspace_size(int64_t M, int64_t N, int64_t K) {
    if (check_sizes(M, N, K) != LLMINT8_OK) return 0;
    return llmint8::matmul_workspace(M, N, K);
}

llmint8_status llmint8_matmul(int dtype, int64_t M, int64_t N, int64_t K, const int8_t* CA,
                              const float* SCA, const int32_t* outlier_idx,
                              const int32_t* n_outliers, const void* X_outlier, const int8_t* CB,
                              const float* SCB, const void* bias, void* Y, int32_t* C_i32,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return matmul_impl(dtype, false, M, N, K, CA, SCA, outlier_idx, n_outliers, X_outlier, CB, SCB,
                       bias, Y, C_i32, nullptr, workspace, workspace_bytes, stream, nullptr,
                       nullptr);
}

llmint8_status llmint8_matmul_profiled(int dtype, int64_t M, int64_t N, int64_t K,
                                       const int8_t* CA, const float* SCA,
                                       const int32_t* outlier_idx, const int32_t* n_outliers,
                                       const void* X_outlier, const int8_t* CB, const float* SCB,
                                       const void* bias, void* Y, int32_t* C_i32,
                                       void* workspace, size_t workspace_bytes,
                                       hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    return matmul_impl(dtype, false, M, N, K, CA, SCA, outlier_idx, n_outliers, X_outlier, CB, SCB,
                       bias, Y, C_i32, nullptr, workspace, workspace_bytes, stream, start, stop);
}

size_t llmint8_linear_workspace_size(int64_t M, int64_t N, int64_t K) {
    if (check_sizes(M, N, K) != LLMINT8_OK) return 0;
    return linear_workspace(M, N, K, false);
}

llmint8_status llmint8_linear(const void* X, int dtype, int64_t M, int64_t N, int64_t K,
                              float threshold, const int8_t* CB, const float* SCB,
                              const void* bias, void* Y, int8_t* CA, float* SCA,
                              int32_t* outlier_idx, int32_t* n_outliers, void* X_outlier,
                              int32_t* C_i32, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
    return linear_impl(X, dtype, false, M, N, K, threshold, CB, SCB, bias, Y, CA, SCA, outlier_idx,
                       n_outliers, X_outlier, C_i32, nullptr, workspace, workspace_bytes, stream,
                       nullptr, nullptr);
}

llmint8_status llmint8_linear_profiled(const void* X, int dtype, int64_t M, int64_t N, int64_t K,
                                       float threshold, const int8_t* CB, const float* SCB,
                                       const void* bias, void* Y, int8_t* CA, float* SCA,
                                       int32_t* outlier_idx, int32_t* n_outliers, void* X_outlier,
                                       int32_t* C_i32, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    return linear_impl(X, dtype, false, M, N, K, threshold, CB, SCB, bias, Y, CA, SCA, outlier_idx,
                       n_outliers, X_outlier, C_i32, nullptr, workspace, workspace_bytes, stream,
                       start, stop);
}

llmint8_status llmint8_linear_noalloc(const void* X, int dtype, int64_t M, int64_t N, int64_t K,
                                      float threshold, const int8_t* CB, const float* SCB,
                                      const void* bias, void* Y, int8_t* CA, float* SCA,
                                      int32_t* outlier_idx, int32_t* n_outliers, void* X_outlier,
                                      int32_t* C_i32, hipStream_t stream) {
    return linear_impl(X, dtype, false, M, N, K, threshold, CB, SCB, bias, Y, CA, SCA, outlier_idx,
                       n_outliers, X_outlier, C_i32, nullptr, nullptr, 0, stream, nullptr, nullptr,
                       true);
}

llmint8_status llmint8_matmul_fp8(int dtype, int64_t M, int64_t N, int64_t K, const uint8_t* CA,
                                  const float* SCA, const int32_t* outlier_idx,
                                  const int32_t* n_outliers, const void* X_outlier,
                                  const uint8_t* CB, const float* SCB, const void* bias, void* Y,
                                  float* C_f32, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
    return matmul_impl(dtype, true, M, N, K, reinterpret_cast<const int8_t*>(CA), SCA, outlier_idx,
                       n_outliers, X_outlier, reinterpret_cast<const int8_t*>(CB), SCB, bias, Y,
                       nullptr, C_f32, workspace, workspace_bytes, stream, nullptr, nullptr);
}

llmint8_status llmint8_matmul_fp8_profiled(int dtype, int64_t M, int64_t N, int64_t K,
                                           const uint8_t* CA, const float* SCA,
                                           const int32_t* outlier_idx,
                                           const int32_t* n_outliers, const void* X_outlier,
                                           const uint8_t* CB, const float* SCB, const void* bias,
                                           void* Y, float* C_f32, void* workspace,
                                           size_t workspace_bytes, hipStream_t stream,
                                           hipEvent_t start, hipEvent_t stop) {
    return matmul_impl(dtype, true, M, N, K, reinterpret_cast<const int8_t*>(CA), SCA, outlier_idx,
                       n_outliers, X_outlier, reinterpret_cast<const int8_t*>(CB), SCB, bias, Y,
                       nullptr, C_f32, workspace, workspace_bytes, stream, start, stop);
}

size_t llmint8_linear_fp8_workspace_size(int64_t M, int64_t N, int64_t K) {
    if (check_sizes(M, N, K) != LLMINT8_OK) return 0;
    return linear_workspace(M, N, K, true);
}

llmint8_status llmint8_linear_fp8(const void* X, int dtype, int64_t M, int64_t N, int64_t K,
                                  float threshold, const uint8_t* CB, const float* SCB,
                                  const void* bias, void* Y, uint8_t* CA, float* SCA,
                                  int32_t* outlier_idx, int32_t* n_outliers, void* X_outlier,
                                  float* C_f32, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
    return linear_impl(X, dtype, true, M, N, K, threshold, reinterpret_cast<const int8_t*>(CB), SCB,
                       bias, Y, reinterpret_cast<int8_t*>(CA), SCA, outlier_idx, n_outliers,
                       X_outlier, nullptr, C_f32, workspace, workspace_bytes, stream, nullptr,
                       nullptr);
}

llmint8_status llmint8_linear_fp8_profiled(const void* X, int dtype, int64_t M, int64_t N,
                                           int64_t K, float threshold, const uint8_t* CB,
                                           const float* SCB, const void* bias, void* Y,
                                           uint8_t* CA, float* SCA, int32_t* outlier_idx,
                                           int32_t* n_outliers, void* X_outlier, float* C_f32,
                                           void* workspace, size_t workspace_bytes,
                                           hipStream_t stream, hipEvent_t start,
                                           hipEvent_t stop) {
    return linear_impl(X, dtype, true, M, N, K, threshold, reinterpret_cast<const int8_t*>(CB), SCB,
                       bias, Y, reinterpret_cast<int8_t*>(CA), SCA, outlier_idx, n_outliers,
                       X_outlier, nullptr, C_f32, workspace, workspace_bytes, stream, start, stop);
}

llmint8_status llmint8_peak_mfma(int fp8, const int8_t* operands, size_t operand_bytes,
                                 int32_t* sink, size_t sink_bytes, int blocks, int iters,
                                 hipStream_t stream) {
    if ((fp8 != 0 && fp8 != 1) || bad_ptr(operands) || bad_ptr(sink) || blocks < 1 || iters < 1)
        return LLMINT8_ERR_INVALID_ARGUMENT;
    if (operand_bytes < 262144 || sink_bytes / 1024 < (size_t)blocks) return LLMINT8_ERR_INVALID_ARGUMENT;
    llmint8_status s = check_device();
    if (s != LLMINT8_OK) return s;
    hipError_t e = llmint8::launch_mfma_peak(fp8 == 1, operands, iters, sink, blocks, stream);
    return e == hipSuccess ? LLMINT8_OK : hip_fail(e);
}

const char* llmint8_status_string(llmint8_status s) {
    // A C caller may pass any int; its bytes are read as one (loading a value
    // outside the enumerators as the enum type would be undefined in C++).
    static_assert(sizeof(llmint8_status) == sizeof(int), "status is int-sized");
    int code;
    memcpy(&code, &s, sizeof code);
    switch (code) {
        case LLMINT8_OK: return "ok";
        case LLMINT8_ERR_INVALID_ARGUMENT: return "invalid argument";
        case LLMINT8_ERR_UNSUPPORTED: return "unsupported shape or device";
        case LLMINT8_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

int llmint8_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
