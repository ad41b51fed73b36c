// Small-M LLM.int8() product (decode: a handful of tokens), HBM-bound.
//
// "A Gentle Introduction to 8-bit Matrix Multiplication for transformers at
// scale", section "LLM.int8() summary": non-outliers multiplied in int8, the
// int8 result dequantized and added to the 16-bit outlier result; section
// "absmax quantization": denormalize by the outer product of the row and
// column absmax vectors.
//
// At M <= 16 the int8 weight CB (N*K bytes) is almost all of the traffic, so
// the kernel is a weight stream: workgroup b owns output channels
// [16b, 16b+16); its waves split K into 64-wide steps (step s goes to wave
// s % WAVES).  For step s, lane l loads 16 bytes of CB row n0 + l%16 at column
// 64s + 16*(l/16) and the matching 16 bytes of CA row l%16, and one
// v_mfma_i32_16x16x64_i8 accumulates the 16x16 int32 tile (the k order inside
// an instruction is the same for both operands, so any placement of the 64
// columns over lanes gives the exact dot product).  Loads are issued BATCH
// steps ahead of the MFMAs that consume them.  The per-wave partial tiles are
// summed through LDS, then 256 threads each finish one (m, n):
//   Y = (C * SCA[m]/127 + sum_j XO[m,j] * CB[n, idx[j]]) * SCB[n]/127 + bias[n]
// With more than 32 outlier columns the outlier sum runs as 16-bit MFMAs over
// blocks of 32 outlier ranks (XO rows against the gathered weight codes).
//
// FP8 (the E4M3 variant; format in common.h): each 16-byte step feeds two
// v_mfma_f32_16x16x32_fp8_fp8, one per 8-byte half (again the same split for
// both operands), into fp32 accumulators; the per-wave tiles are summed in a
// fixed order, and 127 becomes 448 in the epilogue, with CB's outlier codes
// decoded to their E4M3 values.
#include "common.h"

namespace llmint8 {

namespace {

constexpr int kBatch = 8;
constexpr int kDenseOut = 32;  // more outlier columns than this: the outlier product as MFMAs

template <int WAVES>
__device__ __forceinline__ void load_steps(const int8_t* __restrict__ pa, const int8_t* __restrict__ pb,
                                           bool a_ok, bool b_ok, int s0, int nsteps, v4i* a, v4i* b) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
        const int s = s0 + i * WAVES;
        const bool in = s < nsteps;
        b[i] = (in && b_ok) ? *reinterpret_cast<const v4i*>(pb + (size_t)s * 64) : v4i{0, 0, 0, 0};
        a[i] = (in && a_ok) ? *reinterpret_cast<const v4i*>(pa + (size_t)s * 64) : v4i{0, 0, 0, 0};
    }
}

__device__ __forceinline__ v4i mfma_steps(const v4i* a, const v4i* b, v4i acc) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], b[i], acc, 0, 0, 0);
    return acc;
}

__device__ __forceinline__ v4f mfma_steps(const v4i* a, const v4i* b, v4f acc) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
        const v2l a2 = __builtin_bit_cast(v2l, a[i]), b2 = __builtin_bit_cast(v2l, b[i]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a2[0], b2[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a2[1], b2[1], acc, 0, 0, 0);
    }
    return acc;
}

template <bool FP8>
struct SmallAcc {
    typedef v4i vec;
    typedef int elem;
};
template <>
struct SmallAcc<true> {
    typedef v4f vec;
    typedef float elem;
};

template <bool BF16, bool FP8, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void gemm_small_m_kernel(
    int M, int N, int K, const int8_t* __restrict__ CA, const float* __restrict__ SCA,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ n_out_ptr,
    const uint16_t* __restrict__ XO, const int8_t* __restrict__ CB, const float* __restrict__ SCB,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y, int32_t* __restrict__ C_i32,
    float* __restrict__ C_f32) {
    typedef typename SmallAcc<FP8>::vec acc_t;
    typedef typename SmallAcc<FP8>::elem elem_t;
    __shared__ elem_t red[WAVES][4][64];
    __shared__ float red_o[WAVES][4][64];  // the 16-bit outlier product's partial tiles (many columns)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = blockIdx.x * 16;
    const int r16 = lane & 15, kg = lane >> 4;
    const int nsteps = K >> 6;
    const bool a_ok = r16 < M;
    const bool b_ok = n0 + r16 < N;
    const int8_t* pa = CA + (size_t)(a_ok ? r16 : 0) * K + kg * 16;
    const int8_t* pb = CB + (size_t)(b_ok ? n0 + r16 : 0) * K + kg * 16;

    acc_t acc = {0, 0, 0, 0};
    v4i a0[kBatch], b0[kBatch], a1[kBatch], b1[kBatch];
    load_steps<WAVES>(pa, pb, a_ok, b_ok, wave, nsteps, a0, b0);
    for (int s = wave; s < nsteps; s += 2 * kBatch * WAVES) {
        load_steps<WAVES>(pa, pb, a_ok, b_ok, s + kBatch * WAVES, nsteps, a1, b1);
        acc = mfma_steps(a0, b0, acc);
        load_steps<WAVES>(pa, pb, a_ok, b_ok, s + 2 * kBatch * WAVES, nsteps, a0, b0);
        acc = mfma_steps(a1, b1, acc);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][v][lane] = acc[v];
    // Many outlier columns: the 16-bit outlier product as v_mfma_f32_16x16x32
    // over blocks of 32 outlier ranks (block q to wave q % WAVES): A = XO rows
    // (lane: token r16, ranks 32q + 8kg .. +8, contiguous; XO is 0 past
    // n_out), B = the weight codes at those ranks' columns as 16-bit values
    // (exact; ranks past n_out read the last outlier column, against XO's 0).
    // A loop over the columns per output would take one dependent load each.
    const int n_out = *n_out_ptr;
    const bool dense_out = n_out > kDenseOut;
    if (dense_out) {
        const int n_pad = (n_out + 31) & ~31;
        const uint16_t* xo = XO + (size_t)min(r16, M - 1) * n_pad + kg * 8;
        const int8_t* cbr = CB + (size_t)min(n0 + r16, N - 1) * K;
        v4f acc_o = {0, 0, 0, 0};
        for (int q = wave; q * 32 < n_out; q += WAVES) {
            const int j0 = q * 32 + kg * 8;
            const v8u16 a = *reinterpret_cast<const v8u16*>(xo + q * 32);
            const v4i i0 = *reinterpret_cast<const v4i*>(idx + j0);
            const v4i i1 = *reinterpret_cast<const v4i*>(idx + j0 + 4);
            const int last = idx[n_out - 1];
            v8u16 b;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int col = j0 + e < n_out ? (e < 4 ? i0[e] : i1[e - 4]) : last;
                b[e] = narrow16<BF16>(code_value<FP8>(cbr[col]));
            }
            if constexpr (BF16)
                acc_o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b),
                                                                acc_o, 0, 0, 0);
            else
                acc_o = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b),
                                                               acc_o, 0, 0, 0);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float f = acc_o[v];  // by value: bit_cast of a vector element reads element 0
            red_o[wave][v][lane] = f;
        }
    }
    __syncthreads();
    if (tid >= 256) return;

    // element tid: accumulator register v of lane l -> row 4*(l/16) + v, column l%16
    const int v = tid >> 6, l = tid & 63;
    elem_t c = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) c += red[w][v][l];
    const int m = 4 * (l >> 4) + v;
    const int n = n0 + (l & 15);
    if (m >= M || n >= N) return;
    if constexpr (FP8) {
        if (C_f32) C_f32[(size_t)m * N + n] = c;
    } else {
        if (C_i32) C_i32[(size_t)m * N + n] = c;
    }

    float y = (float)c * (SCA[m] / code_max<FP8>());
    if (dense_out) {
        float o = 0.0f;  // the waves' partial sums, in a fixed order
#pragma unroll
        for (int w = 0; w < WAVES; ++w) o += red_o[w][v][l];
        y += o;
    } else if (n_out > 0) {
        const int n_pad = (n_out + 31) & ~31;
        const uint16_t* xo = XO + (size_t)m * n_pad;
        const int8_t* cb = CB + (size_t)n * K;
#pragma unroll 4
        for (int j = 0; j < n_out; ++j) y += widen16<BF16>(xo[j]) * code_value<FP8>(cb[idx[j]]);
    }
    y *= SCB[n] / code_max<FP8>();
    if (bias) y += widen16<BF16>(bias[n]);
    Y[(size_t)m * N + n] = narrow16<BF16>(y);
}

}  // namespace

hipError_t launch_gemm_small_m(const MatmulArgs& a, hipStream_t stream, hipEvent_t ev_start,
                               hipEvent_t ev_stop) {
    constexpr int W = 8;
    dim3 grid((a.N + 15) / 16), block(W * 64);
    void (*fn)(int, int, int, const int8_t*, const float*, const int32_t*, const int32_t*,
               const uint16_t*, const int8_t*, const float*, const uint16_t*, uint16_t*, int32_t*,
               float*) =
        a.bf16 ? (a.fp8 ? gemm_small_m_kernel<true, true, W> : gemm_small_m_kernel<true, false, W>)
               : (a.fp8 ? gemm_small_m_kernel<false, true, W> : gemm_small_m_kernel<false, false, W>);
    if (ev_start || ev_stop) {
        hipExtLaunchKernelGGL(fn, grid, block, 0, stream, ev_start, ev_stop, 0, a.M, a.N, a.K, a.CA,
                              a.SCA, a.idx, a.n_out, a.XO, a.CB, a.SCB, a.bias, a.Y, a.C_i32,
                              a.C_f32);
    } else {
        fn<<<grid, block, 0, stream>>>(a.M, a.N, a.K, a.CA, a.SCA, a.idx, a.n_out, a.XO, a.CB,
                                       a.SCB, a.bias, a.Y, a.C_i32, a.C_f32);
    }
    return hipGetLastError();
}

}  // namespace llmint8
