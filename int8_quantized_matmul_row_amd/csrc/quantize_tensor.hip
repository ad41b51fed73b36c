// Per-tensor absmax quantization: one scale for the whole tensor.
//
// "A Gentle Introduction to 8-bit Matrix Multiplication for transformers at
// scale", section "absmax quantization": scale by 127 / absmax, here with the
// absmax of the whole tensor -- the baseline that the vector-wise scales and
// the outlier decomposition improve on.  The absmax is written to every row's
// scale, so (Q, scale) can stand in for a vector-wise (codes, scales) pair in
// the int8 product, whose dequantization SCA[m] * SCB[n] / 127^2 then applies
// the two tensor scales.
//
// Two launches, no atomics: 16-byte loads, packed 16-bit magnitude maxima
// (which order like the values) per block into the workspace; then every block
// reduces those partials itself and quantizes its share of the tensor.
#include "common.h"

namespace llmint8 {

namespace {

constexpr int kQtThreads = 256;
constexpr int kQtMaxPartials = 1024;
constexpr int kQtMaxBlocks = 4096;

__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* lds) {
    const uint32_t w = wave_max_u32(v);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) lds[wave] = w;
    __syncthreads();
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < kQtThreads / 64; ++i) m = max(m, lds[i]);
    return m;
}

// partial[b] = max |A| over the 8-element chunks b * 256 + t + stride * i
__global__ __launch_bounds__(kQtThreads) void tensor_absmax_partial(const uint16_t* __restrict__ A,
                                                                    int64_t n8,
                                                                    uint32_t* __restrict__ partial) {
    __shared__ uint32_t lds[kQtThreads / 64];
    uint32_t m = 0;
    for (int64_t i = (int64_t)blockIdx.x * kQtThreads + threadIdx.x; i < n8;
         i += (int64_t)gridDim.x * kQtThreads) {
        const v4i w = *reinterpret_cast<const v4i*>(A + i * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) m = max_u16x2(m, abs2((uint32_t)w[e]));
    }
    const uint32_t b = block_max_u32(max(m & 0xffffu, m >> 16), lds);
    if (threadIdx.x == 0) partial[blockIdx.x] = b;
}

template <bool BF16>
__global__ __launch_bounds__(kQtThreads) void tensor_quantize(
    const uint16_t* __restrict__ A, int64_t rows, int64_t n8, const uint32_t* __restrict__ partial,
    int nparts, int8_t* __restrict__ Q, float* __restrict__ scale) {
    __shared__ uint32_t lds[kQtThreads / 64];
    uint32_t m = 0;
    for (int i = threadIdx.x; i < nparts; i += kQtThreads) m = max(m, partial[i]);
    const float amax = widen16<BF16>((uint16_t)block_max_u32(m, lds));
    // |x| <= amax, so |x * s| <= 127 and the low byte of rne(x * s) + 1.5 * 2^23
    // is the code; s = 0 (an all-zero tensor) gives 0 everywhere
    const float s = amax == 0.0f ? 0.0f : 127.0f / amax;
    for (int64_t i = (int64_t)blockIdx.x * kQtThreads + threadIdx.x; i < n8;
         i += (int64_t)gridDim.x * kQtThreads) {
        const v8u16 v = *reinterpret_cast<const v8u16*>(A + i * 8);
        uint32_t q[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = quantize_low_byte(widen16<BF16>(v[e]), s);
        const uint32_t lo = __builtin_amdgcn_perm(__builtin_amdgcn_perm(q[3], q[2], 0x0c0c0400u),
                                                  __builtin_amdgcn_perm(q[1], q[0], 0x0c0c0400u),
                                                  0x05040100u);
        const uint32_t hi = __builtin_amdgcn_perm(__builtin_amdgcn_perm(q[7], q[6], 0x0c0c0400u),
                                                  __builtin_amdgcn_perm(q[5], q[4], 0x0c0c0400u),
                                                  0x05040100u);
        *reinterpret_cast<uint2*>(Q + i * 8) = make_uint2(lo, hi);
    }
    if (blockIdx.x == 0)
        for (int64_t r = threadIdx.x; r < rows; r += kQtThreads) scale[r] = amax;
}

}  // namespace

size_t quantize_tensor_workspace() { return kQtMaxPartials * sizeof(uint32_t); }

hipError_t launch_quantize_tensor(const void* A, bool bf16, int64_t rows, int64_t cols, int8_t* Q,
                                  float* scale, void* ws, hipStream_t stream) {
    const int64_t n8 = rows * cols / 8;
    const int nparts = (int)std::min<int64_t>(kQtMaxPartials, (n8 + kQtThreads - 1) / kQtThreads);
    const int nblocks = (int)std::min<int64_t>(kQtMaxBlocks, (n8 + kQtThreads - 1) / kQtThreads);
    const uint16_t* a = static_cast<const uint16_t*>(A);
    uint32_t* partial = static_cast<uint32_t*>(ws);
    tensor_absmax_partial<<<nparts, kQtThreads, 0, stream>>>(a, n8, partial);
    if (bf16)
        tensor_quantize<true><<<nblocks, kQtThreads, 0, stream>>>(a, rows, n8, partial, nparts, Q,
                                                                  scale);
    else
        tensor_quantize<false><<<nblocks, kQtThreads, 0, stream>>>(a, rows, n8, partial, nparts, Q,
                                                                   scale);
    return hipGetLastError();
}

}  // namespace llmint8
