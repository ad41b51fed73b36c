// Sustained matrix-core rate of the device, the measured ceiling beside the
// published peak in the roofline report.  Every wave runs back-to-back MFMAs
// on four independent accumulators with operands read once from a buffer of
// random codes (the power drawn, and so the clock reached, depends on the
// operand bits), then folds its accumulators into one word so that nothing
// is optimised away.  int8: v_mfma_i32_32x32x32_i8 (65536 operations each);
// E4M3: v_mfma_scale_f32_32x32x64_f8f6f4 (131072 operations each).
#include "common.h"

namespace llmint8 {

namespace {

constexpr int kPeakThreads = 256;

template <bool FP8>
__global__ __launch_bounds__(kPeakThreads) void mfma_peak_kernel(const int8_t* __restrict__ operands,
                                                                 int iters, int32_t* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    // 64 distinct operand sets of 64 lanes x 64 bytes (256 KiB in all)
    const int w = (blockIdx.x * (kPeakThreads / 64) + (threadIdx.x >> 6)) & 63;
    const int8_t* p = operands + (size_t)(w * 64 + lane) * 64;
    const v8i a = *reinterpret_cast<const v8i*>(p);
    const v8i b = *reinterpret_cast<const v8i*>(p + 32);
    int32_t x = 0;
    if constexpr (FP8) {
        v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
        for (int i = 0; i < iters; ++i) {
            c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 0, 0, 0, 127, 0, 127);
            c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c1, 0, 0, 0, 127, 0, 127);
            c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c2, 0, 0, 0, 127, 0, 127);
            c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, b, c3, 0, 0, 0, 127, 0, 127);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float f0 = c0[v], f1 = c1[v], f2 = c2[v], f3 = c3[v];  // by value
            x ^= __builtin_bit_cast(int32_t, f0) ^ __builtin_bit_cast(int32_t, f1) ^
                 __builtin_bit_cast(int32_t, f2) ^ __builtin_bit_cast(int32_t, f3);
        }
    } else {
        const v4i alo = __builtin_shufflevector(a, a, 0, 1, 2, 3), ahi = __builtin_shufflevector(a, a, 4, 5, 6, 7);
        const v4i blo = __builtin_shufflevector(b, b, 0, 1, 2, 3), bhi = __builtin_shufflevector(b, b, 4, 5, 6, 7);
        v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
        for (int i = 0; i < iters; ++i) {
            c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(alo, blo, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(ahi, bhi, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(alo, bhi, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(ahi, blo, c3, 0, 0, 0);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int32_t i0 = c0[v], i1 = c1[v], i2 = c2[v], i3 = c3[v];
            x ^= i0 ^ i1 ^ i2 ^ i3;
        }
    }
    sink[(size_t)blockIdx.x * kPeakThreads + threadIdx.x] = x;
}

}  // namespace

int peak_probe_threads() { return kPeakThreads; }

hipError_t launch_mfma_peak(bool fp8, const int8_t* operands, int iters, int32_t* sink, int blocks,
                            hipStream_t stream) {
    if (fp8)
        mfma_peak_kernel<true><<<blocks, kPeakThreads, 0, stream>>>(operands, iters, sink);
    else
        mfma_peak_kernel<false><<<blocks, kPeakThreads, 0, stream>>>(operands, iters, sink);
    return hipGetLastError();
}

}  // namespace llmint8
