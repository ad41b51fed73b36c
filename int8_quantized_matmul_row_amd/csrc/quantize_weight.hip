// Weight quantization: per output channel absmax -> CB int8, SCB fp32.
//
// "A Gentle Introduction to 8-bit Matrix Multiplication for transformers at
// scale", section "absmax quantization" (scale by 127/absmax and round) and
// section "Usage" (the layer's weight becomes int8 CB of the same [out, in]
// shape plus one absmax SCB per output row, once, when the layer is placed on
// the GPU).  Vector-wise: one absmax per column of B = W^T, i.e. per row of W.
//
// One 64-lane wave owns one row of W.  Each lane reads 16-byte pieces (8
// values) at a 1 KiB stride so one wave instruction covers 1 KiB of the row;
// pass 1 finds the row absmax with a butterfly reduction, pass 2 re-reads the
// row (an L2 hit) and writes 8 int8 codes per lane.  The kernel is HBM-bound:
// 2NK bytes read once from HBM, NK + 4N written.
//
// FP8 = true writes E4M3 codes instead (scale 448/absmax, the 8-bit
// floating-point variant that the zhichai.top summary of LLM.int8() lists as
// future work; format and rounding in common.h).  A zero row has scale 0 and
// the codes of its signed zeros.
#include "common.h"

namespace llmint8 {

template <bool BF16, bool FP8>
__global__ __launch_bounds__(256) void quantize_weight_kernel(const uint16_t* __restrict__ W,
                                                              int N, int K,
                                                              int8_t* __restrict__ CB,
                                                              float* __restrict__ SCB) {
    const int lane = threadIdx.x & 63;
    const int nchunk = K >> 3;  // 8 values per 16-byte piece; K % 64 == 0
    for (int row = blockIdx.x * 4 + (threadIdx.x >> 6); row < N; row += gridDim.x * 4) {
        const uint16_t* w = W + (size_t)row * K;
        float amax = 0.0f;
#pragma unroll 4
        for (int c = lane; c < nchunk; c += kWave) {
            v8u16 v = *reinterpret_cast<const v8u16*>(w + (size_t)c * 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(widen16<BF16>(v[e])));
        }
        amax = wave_max(amax);
        if (lane == 0) SCB[row] = amax;
        const float scale = amax == 0.0f ? 0.0f : code_max<FP8>() / amax;
        int8_t* cb = CB + (size_t)row * K;
#pragma unroll 4
        for (int c = lane; c < nchunk; c += kWave) {
            v8u16 v = *reinterpret_cast<const v8u16*>(w + (size_t)c * 8);
            uint32_t lo = 0, hi = 0;
            if constexpr (FP8) {
                lo = e4m3_pack4(widen16<BF16>(v[0]), widen16<BF16>(v[1]), widen16<BF16>(v[2]),
                                widen16<BF16>(v[3]), scale);
                hi = e4m3_pack4(widen16<BF16>(v[4]), widen16<BF16>(v[5]), widen16<BF16>(v[6]),
                                widen16<BF16>(v[7]), scale);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    lo |= (uint32_t)(quantize_value(widen16<BF16>(v[e]), scale) & 0xff) << (8 * e);
                    hi |= (uint32_t)(quantize_value(widen16<BF16>(v[e + 4]), scale) & 0xff) << (8 * e);
                }
            }
            *reinterpret_cast<uint2*>(cb + (size_t)c * 8) = make_uint2(lo, hi);
        }
    }
}

hipError_t launch_quantize_weight(const void* W, bool bf16, bool fp8, int N, int K, int8_t* CB,
                                  float* SCB, hipStream_t stream) {
    const int rows_per_block = 4;
    long blocks = (N + rows_per_block - 1) / rows_per_block;
    if (blocks > 65536) blocks = 65536;  // grid-stride beyond this
    void (*fn)(const uint16_t*, int, int, int8_t*, float*) =
        bf16 ? (fp8 ? quantize_weight_kernel<true, true> : quantize_weight_kernel<true, false>)
             : (fp8 ? quantize_weight_kernel<false, true> : quantize_weight_kernel<false, false>);
    fn<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(static_cast<const uint16_t*>(W), N, K, CB,
                                                         SCB);
    return hipGetLastError();
}

}  // namespace llmint8
