// Small-M LLM.int8() product (decode: a handful of tokens), HBM-bound.
//
// "A Gentle Introduction to 8-bit Matrix Multiplication for transformers at
// scale", section "LLM.int8() summary": non-outliers multiplied in int8, the
// int8 result dequantized and added to the 16-bit outlier result; section
// "absmax quantization": denormalize by the outer product of the row and
// column absmax vectors.
//
// At M <= 64 the int8 weight CB (N*K bytes) is most of the traffic, so the
// kernel is a weight stream: workgroup b owns output channels [16b, 16b+16);
// its waves split K into 64-wide steps (step s goes to wave s % WAVES).  For
// step s, lane l loads 16 bytes of CB row n0 + l%16 at column 64s + 16*(l/16)
// and the matching 16 bytes of CA row 16t + l%16 for each group t of 16 token
// rows (MT groups: 1, 2 or 4), and one v_mfma_i32_16x16x64_i8 per group
// accumulates its 16x16 int32 tile (the k order inside an instruction is the
// same for both operands, so any placement of the 64 columns over lanes gives
// the exact dot product): every weight byte is loaded once for all the
// tokens.  Loads are issued BATCH steps ahead of the MFMAs that consume them
// (fewer steps for more groups, so that the registers in flight stay the
// same).  The per-wave partial tiles are summed through LDS, then each thread
// finishes (m, n) elements:
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

constexpr int kDenseOut = 32;  // more outlier columns than this: the outlier product as MFMAs

// steps s0 + i*WAVES (i < KB) of the weight rows of every channel group and
// of the activation rows of every token group (steps past K, rows past M or
// N load zeros)
template <int WAVES, int MT, int NC, int KB>
__device__ __forceinline__ void load_steps(const int8_t* const (&pa)[MT], const int8_t* const (&pb)[NC],
                                           const bool (&a_ok)[MT], const bool (&b_ok)[NC], int s0, int nsteps,
                                           v4i (&a)[MT][KB], v4i (&b)[NC][KB]) {
#pragma unroll
    for (int i = 0; i < KB; ++i) {
        const int s = s0 + i * WAVES;
        const bool in = s < nsteps;
#pragma unroll
        for (int c = 0; c < NC; ++c)
            b[c][i] = (in && b_ok[c]) ? *reinterpret_cast<const v4i*>(pb[c] + (size_t)s * 64) : v4i{0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < MT; ++t)
            a[t][i] = (in && a_ok[t]) ? *reinterpret_cast<const v4i*>(pa[t] + (size_t)s * 64) : v4i{0, 0, 0, 0};
    }
}

template <int MT, int NC, int KB>
__device__ __forceinline__ void mfma_steps(const v4i (&a)[MT][KB], const v4i (&b)[NC][KB], v4i (&acc)[NC][MT]) {
#pragma unroll
    for (int i = 0; i < KB; ++i)
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int t = 0; t < MT; ++t)
                acc[c][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[t][i], b[c][i], acc[c][t], 0, 0, 0);
}

template <int MT, int NC, int KB>
__device__ __forceinline__ void mfma_steps(const v4i (&a)[MT][KB], const v4i (&b)[NC][KB], v4f (&acc)[NC][MT]) {
#pragma unroll
    for (int i = 0; i < KB; ++i)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const v2l b2 = __builtin_bit_cast(v2l, b[c][i]);
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const v2l a2 = __builtin_bit_cast(v2l, a[t][i]);
                acc[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a2[0], b2[0], acc[c][t], 0, 0, 0);
                acc[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a2[1], b2[1], acc[c][t], 0, 0, 0);
            }
        }
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

template <bool BF16, bool FP8, int WAVES, int MT, int NC, int KB>
__global__ __launch_bounds__(WAVES * 64) void gemm_small_m_kernel(
    int M, int N, int K, const int8_t* __restrict__ CA, const float* __restrict__ SCA,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ n_out_ptr,
    const uint16_t* __restrict__ XO, const int8_t* __restrict__ CB, const float* __restrict__ SCB,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y, int32_t* __restrict__ C_i32,
    float* __restrict__ C_f32) {
    typedef typename SmallAcc<FP8>::vec acc_t;
    typedef typename SmallAcc<FP8>::elem elem_t;
    constexpr int kB = KB;  // K steps in flight per wave
    __shared__ elem_t red[WAVES][MT][4][64];
    __shared__ float red_o[WAVES][MT][4][64];  // the 16-bit outlier product's partial tiles (many columns)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = blockIdx.x * 16 * NC;
    const int r16 = lane & 15, kg = lane >> 4;
    const int nsteps = K >> 6;
    bool a_ok[MT], b_ok[NC];
    const int8_t* pa[MT];
    const int8_t* pb[NC];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const int r = 16 * t + r16;
        a_ok[t] = r < M;
        pa[t] = CA + (size_t)(a_ok[t] ? r : 0) * K + kg * 16;
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int n = n0 + 16 * c + r16;
        b_ok[c] = n < N;
        pb[c] = CB + (size_t)(b_ok[c] ? n : 0) * K + kg * 16;
    }

    acc_t acc[NC][MT];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[c][t] = acc_t{0, 0, 0, 0};
    v4i a0[MT][kB], b0[NC][kB], a1[MT][kB], b1[NC][kB];
    load_steps<WAVES, MT, NC, kB>(pa, pb, a_ok, b_ok, wave, nsteps, a0, b0);
    for (int s = wave; s < nsteps; s += 2 * kB * WAVES) {
        load_steps<WAVES, MT, NC, kB>(pa, pb, a_ok, b_ok, s + kB * WAVES, nsteps, a1, b1);
        mfma_steps<MT, NC, kB>(a0, b0, acc);
        load_steps<WAVES, MT, NC, kB>(pa, pb, a_ok, b_ok, s + 2 * kB * WAVES, nsteps, a0, b0);
        mfma_steps<MT, NC, kB>(a1, b1, acc);
    }
    // Many outlier columns: the 16-bit outlier product as v_mfma_f32_16x16x32
    // over blocks of 32 outlier ranks (block q to wave q % WAVES): A = XO rows
    // (lane: token 16t + r16, ranks 32q + 8kg .. +8, contiguous; XO is 0 past
    // n_out), B = the weight codes at those ranks' columns as 16-bit values
    // (exact; ranks past n_out read the last outlier column, against XO's 0).
    // A loop over the columns per output would take one dependent load each.
    const int n_out = *n_out_ptr;
    const bool dense_out = n_out > kDenseOut;
    v4f acc_o[NC][MT];
    if (dense_out) {
        const int n_pad = (n_out + 31) & ~31;
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int t = 0; t < MT; ++t) acc_o[c][t] = v4f{0, 0, 0, 0};
        for (int q = wave; q * 32 < n_out; q += WAVES) {
            const int j0 = q * 32 + kg * 8;
            const v4i i0 = *reinterpret_cast<const v4i*>(idx + j0);
            const v4i i1 = *reinterpret_cast<const v4i*>(idx + j0 + 4);
            const int last = idx[n_out - 1];
            int col[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) col[e] = j0 + e < n_out ? (e < 4 ? i0[e] : i1[e - 4]) : last;
            v8u16 a[MT];
#pragma unroll
            for (int t = 0; t < MT; ++t)
                a[t] = *reinterpret_cast<const v8u16*>(XO + (size_t)min(16 * t + r16, M - 1) * n_pad + kg * 8 + q * 32);
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int8_t* cbr = CB + (size_t)min(n0 + 16 * c + r16, N - 1) * K;
                v8u16 b;
#pragma unroll
                for (int e = 0; e < 8; ++e) b[e] = narrow16<BF16>(code_value<FP8>(cbr[col[e]]));
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    if constexpr (BF16)
                        acc_o[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(v8bf, a[t]), __builtin_bit_cast(v8bf, b), acc_o[c][t], 0, 0, 0);
                    else
                        acc_o[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            __builtin_bit_cast(v8h, a[t]), __builtin_bit_cast(v8h, b), acc_o[c][t], 0, 0, 0);
                }
            }
        }
    }

    // one channel group at a time through LDS: element e is accumulator
    // register v of lane l of token group t -> row 16t + 4*(l/16) + v, column
    // n0 + 16c + l%16
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        if (c > 0) __syncthreads();  // the previous group's partial tiles are read out
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) red[wave][t][v][lane] = acc[c][t][v];
        if (dense_out) {
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float f = acc_o[c][t][v];  // by value: bit_cast of a vector element reads element 0
                    red_o[wave][t][v][lane] = f;
                }
        }
        __syncthreads();
        for (int e = tid; e < MT * 256; e += WAVES * 64) {
            const int t = e >> 8, v = (e >> 6) & 3, l = e & 63;
            elem_t cs = 0;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) cs += red[w][t][v][l];
            const int m = 16 * t + 4 * (l >> 4) + v;
            const int n = n0 + 16 * c + (l & 15);
            if (m >= M || n >= N) continue;
            if constexpr (FP8) {
                if (C_f32) C_f32[(size_t)m * N + n] = cs;
            } else {
                if (C_i32) C_i32[(size_t)m * N + n] = cs;
            }

            float y = (float)cs * (SCA[m] / code_max<FP8>());
            if (dense_out) {
                float o = 0.0f;  // the waves' partial sums, in a fixed order
#pragma unroll
                for (int w = 0; w < WAVES; ++w) o += red_o[w][t][v][l];
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
    }
}

constexpr int kWaves = 8;
typedef void (*small_m_kernel_t)(int, int, int, const int8_t*, const float*, const int32_t*, const int32_t*,
                                 const uint16_t*, const int8_t*, const float*, const uint16_t*, uint16_t*,
                                 int32_t*, float*);

template <int MT, int NC, int KB>
small_m_kernel_t small_m_variant(bool bf16, bool fp8) {
    if (bf16)
        return fp8 ? gemm_small_m_kernel<true, true, kWaves, MT, NC, KB>
                   : gemm_small_m_kernel<true, false, kWaves, MT, NC, KB>;
    return fp8 ? gemm_small_m_kernel<false, true, kWaves, MT, NC, KB>
               : gemm_small_m_kernel<false, false, kWaves, MT, NC, KB>;
}

}  // namespace

hipError_t launch_gemm_small_m(const MatmulArgs& a, hipStream_t stream, hipEvent_t ev_start,
                               hipEvent_t ev_stop) {
    constexpr int W = kWaves;
    dim3 grid((a.N + 15) / 16), block(W * 64);
    // Token groups of 16 (1, 2, 4) by M; more than 8 rows and at least a
    // round of 64-channel workgroups: four channel groups per workgroup, each
    // wave reading its CA rows once for 64 weight rows. K steps in flight per
    // wave: the deepest batch within 128 VGPRs (two workgroups per CU, which
    // measured faster than deeper batches in one), except four groups of 16
    // rows in 64 channels (238 VGPRs at any depth) and up to 8 rows, which
    // stream faster with 8 steps in flight in one workgroup per CU (151
    // VGPRs; 2 x 28672 x 16384: 113 against 120 us).
    const bool wide = small_m_wide(a.M, a.N);
    small_m_kernel_t fn;
    if (wide) {
        fn = a.M <= 16   ? small_m_variant<1, 4, 2>(a.bf16, a.fp8)
             : a.M <= 32 ? small_m_variant<2, 4, 1>(a.bf16, a.fp8)
                         : small_m_variant<4, 4, 2>(a.bf16, a.fp8);
        grid = dim3((a.N + 63) / 64);
    } else {
        fn = a.M <= 8    ? small_m_variant<1, 1, 8>(a.bf16, a.fp8)
             : a.M <= 16 ? small_m_variant<1, 1, 4>(a.bf16, a.fp8)
             : a.M <= 32 ? small_m_variant<2, 1, 4>(a.bf16, a.fp8)
                         : small_m_variant<4, 1, 2>(a.bf16, a.fp8);
    }
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
