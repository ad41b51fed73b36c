// Shared device helpers and kernel launchers of libllmint8 (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

namespace llmint8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned short v8u16 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// ---- 16-bit <-> fp32 ------------------------------------------------------
template <bool BF16>
__device__ __forceinline__ float widen16(uint16_t bits) {
    if constexpr (BF16) {
        return __builtin_bit_cast(float, (uint32_t)bits << 16);
    } else {
        return (float)__builtin_bit_cast(_Float16, bits);
    }
}

// fp32 -> 16-bit, round to nearest even (finite inputs).
template <bool BF16>
__device__ __forceinline__ uint16_t narrow16(float f) {
    if constexpr (BF16) {
        uint32_t u = __builtin_bit_cast(uint32_t, f);
        u += 0x7FFFu + ((u >> 16) & 1u);
        return (uint16_t)(u >> 16);
    } else {
        return __builtin_bit_cast(uint16_t, (_Float16)f);
    }
}

// ---- absmax quantization of one value ------------------------------------
// scale = 127.0f / absmax is computed once per vector with the correctly
// rounded fp32 divide; q = rne(x * scale) with one fp32 multiply and
// v_rndne_f32, clamped to [-127, 127].
__device__ __forceinline__ int quantize_value(float x, float scale) {
    float p = x * scale;
    float r = __builtin_rintf(p);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// ---- launchers (each returns hipGetLastError() after its launches) --------
hipError_t launch_quantize_weight(const void* W, bool bf16, int N, int K, int8_t* CB, float* SCB,
                                  hipStream_t stream);

size_t quantize_act_workspace(int64_t M, int64_t K);
hipError_t launch_quantize_act(const void* X, bool bf16, int M, int K, float threshold,
                               int8_t* CA, float* SCA, int32_t* idx, int32_t* n_out, void* XO,
                               void* ws, hipStream_t stream);

struct MatmulArgs {
    bool bf16;
    int M, N, K;
    const int8_t* CA;
    const float* SCA;
    const int32_t* idx;
    const int32_t* n_out;
    const uint16_t* XO;
    const int8_t* CB;
    const float* SCB;
    const uint16_t* bias;
    uint16_t* Y;
    int32_t* C_i32;
    void* ws;
    size_t ws_bytes;
};

size_t matmul_workspace(int64_t M, int64_t N, int64_t K);
hipError_t launch_matmul(const MatmulArgs& a, hipStream_t stream, hipEvent_t ev_start,
                         hipEvent_t ev_stop);

// Kernel families used by launch_matmul.
constexpr int kSmallM = 16;  // M <= kSmallM takes the streaming kernel
hipError_t launch_gemm_small_m(const MatmulArgs& a, hipStream_t stream, hipEvent_t ev_start,
                               hipEvent_t ev_stop);
hipError_t launch_gemm_tiled(const MatmulArgs& a, hipStream_t stream, hipEvent_t ev_start,
                             hipEvent_t ev_stop);

}  // namespace llmint8
