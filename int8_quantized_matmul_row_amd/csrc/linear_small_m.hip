// Fused LLM.int8() linear layer for a handful of tokens (decode), one launch.
//
// "A Gentle Introduction to 8-bit Matrix Multiplication for transformers at
// scale": section "LLM.int8() summary" (1. extract the outlier columns of the
// hidden states, 2. multiply outliers in 16-bit and the rest in int8, 3.
// dequantize the int8 result and add the outlier result), section "inside the
// MatMul" (magnitude 6 or more; row-wise scales for the hidden states,
// per-output-channel scales for the weight), section "absmax quantization"
// (scale by 127/absmax; denormalize by the outer product of the two absmax
// vectors), section "Usage" (recovered weight CB * SCB / 127).
//
// At M <= 16 the int8 weight (N*K bytes) is nearly all of the traffic.  Every
// workgroup owns 16 output channels.  Vector loads retire in issue order, so
// the workgroup first issues its share of X (M x K 16-bit, L2 resident after
// the first workgroups) and its epilogue operands, then its whole CB slab
// (16 rows x K, 16-byte loads, 64-wide K steps spread over the 8 waves).  While
// the weight streams from HBM it quantizes the activations itself, exactly as
// llmint8_quantize_act does: column maxima over all M rows and the outlier
// mask, the row absmax over non-outlier columns, int8 codes into LDS, the
// ascending outlier list.  Then v_mfma_i32_16x16x64_i8 combines the LDS
// activations with the weight registers; the weight bytes of the outlier
// columns are picked out of those same registers.  Wave partials are summed in
// LDS and 256 threads finish one (m, n) each:
//   Y = (C * SCA[m]/127 + sum_j XO[m,j] * CB[n, idx[j]]) * SCB[n]/127 + bias[n].
// Workgroup 0 also writes the activation outputs (CA, SCA, idx, n_out, XO) so
// the call has the same results as llmint8_quantize_act + llmint8_matmul.
#include "common.h"

namespace llmint8 {

constexpr int kLinThreads = 512;
constexpr int kLinWaves = 8;
constexpr int kLinPad = 16;          // LDS row padding: 16 rows hit distinct banks
constexpr int kLinMaxCA = 16 * (4096 + kLinPad);  // int8 activations in LDS
constexpr int kLinMaxChunks = 1024;  // K / 8 (K <= 8192)
constexpr int kLinOutCap = 64;       // outliers staged in LDS (more: read from memory)

bool linear_small_m_supported(int M, int K) {
    return M >= 1 && ((M <= 16 && K <= 4096) || (M <= 8 && K <= 8192));
}

__device__ __forceinline__ uint32_t pack_q4(int a, int b, int c, int d) {
    return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
           ((uint32_t)(d & 0xff) << 24);
}

// MR: activation rows held (8 or 16, >= M); CPT: 8-column chunks per thread
// (K <= 4096 -> 1, K <= 8192 -> 2 with MR = 8); STEPS: 64-wide K steps per wave
// (>= K/64/8).  All loads are unconditional from clamped, in-bounds addresses:
// a conditional load would end in a join that waits for it, serializing the
// stream.  Rows, chunks and steps beyond the real shape are masked where used.
template <bool BF16, int MR, int CPT, int STEPS>
__global__ __launch_bounds__(kLinThreads) void linear_small_m_kernel(
    const uint16_t* __restrict__ X, int M, int N, int K, float t,
    const int8_t* __restrict__ CB, const float* __restrict__ SCB,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y,
    int8_t* __restrict__ CA_out, float* __restrict__ SCA_out, int32_t* __restrict__ idx_out,
    int32_t* __restrict__ n_out_out, uint16_t* __restrict__ XO_out,
    int32_t* __restrict__ C_i32) {
    __shared__ __attribute__((aligned(16))) int8_t ca[kLinMaxCA];
    __shared__ uint8_t mask[kLinMaxChunks];
    __shared__ int chunk_rank[kLinMaxChunks + 1];  // outliers before each 8-column chunk
    __shared__ uint16_t xo_lds[16][kLinOutCap];
    __shared__ float cbo[16][kLinOutCap];  // CB[n0 + i, idx[j]]
    __shared__ unsigned rowmax_bits[16];  // 16-bit magnitude pattern of each row max
    __shared__ float sca[16];
    __shared__ float scl[16];  // 127 / SCA (0 for an all-zero row)
    __shared__ int scan_lds[kLinWaves];
    __shared__ int red[kLinWaves][4][64];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = blockIdx.x * 16;
    const int nchunk = K >> 3;
    const int nsteps = K >> 6;

    // ---- 1a. activation pieces: chunks c = tid + 512 j, rows r < MR, in
    // xr[j * MR + r]; out-of-range chunks and rows load chunk 0 / row 0.
    v8u16 xr[CPT * MR];
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int c = tid + kLinThreads * j;
        const int cc = c < nchunk ? c : 0;
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            const int rr = r < M ? r : 0;
            xr[j * MR + r] = *reinterpret_cast<const v8u16*>(X + (size_t)rr * K + (size_t)cc * 8);
        }
    }
    // ---- 1b. epilogue operands that do not depend on the activations --------
    const int e_n = tid & 15, e_m = tid >> 4;  // output (e_m, n0 + e_n) for tid < 256
    const int n_e = n0 + e_n;
    const bool e_ok = tid < 256 && e_m < M && n_e < N;
    // raw values only: using them here would make the stream wait for them
    const int n_c = min(n_e, N - 1);
    const float scb_raw = SCB[n_c];
    const uint16_t bias_raw = *(bias ? bias + n_c : reinterpret_cast<const uint16_t*>(SCB + n_c));
    // ---- 1c. this workgroup's CB slab: wave w takes K steps w, w+8, ... -------
    const int r16 = lane & 15, kg = lane >> 4;
    const int8_t* pb = CB + (size_t)min(n0 + r16, N - 1) * K + kg * 16;
    v4i breg[STEPS];
#pragma unroll
    for (int i = 0; i < STEPS; ++i) {
        const int s = min(wave + i * kLinWaves, nsteps - 1);
        breg[i] = *reinterpret_cast<const v4i*>(pb + (size_t)s * 64);
    }
    if (tid < 16) rowmax_bits[tid] = 0u;

    // ---- 2. outlier mask: column max over the M rows, one byte per 8 columns --
    // Magnitudes are compared as 16-bit patterns (packed pairs); for finite
    // values this orders exactly like the fp32 values.
    const uint32_t tb = threshold_bits<BF16>(t);
    uint32_t mbits[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int c = tid + kLinThreads * j;
        uint32_t cm[4] = {0, 0, 0, 0};
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            if (r < M) {
                const v4i w = __builtin_bit_cast(v4i, xr[j * MR + r]);
#pragma unroll
                for (int i = 0; i < 4; ++i) cm[i] = max_u16x2(cm[i], abs2((uint32_t)w[i]));
            }
        }
        uint32_t bits = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            bits |= ((cm[i] & 0xffffu) >= tb ? 1u : 0u) << (2 * i);
            bits |= ((cm[i] >> 16) >= tb ? 1u : 0u) << (2 * i + 1);
        }
        mbits[j] = c < nchunk ? bits : 0u;
        if (c < nchunk) mask[c] = (uint8_t)bits;
    }
    __syncthreads();

    // ---- 3. row absmax over non-outlier columns; rank of every chunk ----------
    // keep16: 0x7fff in the 16-bit halves of non-outlier columns, 0 otherwise
    uint32_t keep16[CPT][4];
#pragma unroll
    for (int j = 0; j < CPT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            keep16[j][i] = (((mbits[j] >> (2 * i)) & 1u) ? 0u : 0x7fffu) |
                           (((mbits[j] >> (2 * i + 1)) & 1u) ? 0u : 0x7fff0000u);
    // per-thread maxima of rows r and r+1 packed in one word, reduced across
    // 16-lane rows with DPP, then one LDS atomic per 16 lanes and row
#pragma unroll
    for (int r = 0; r < MR; r += 2) {
        if (r < M) {
            uint32_t m2[2] = {0, 0};
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int j = 0; j < CPT; ++j) {
                    if (tid + kLinThreads * j < nchunk) {
                        const v4i w = __builtin_bit_cast(v4i, xr[j * MR + r + h]);
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            m2[h] = max_u16x2(m2[h], (uint32_t)w[i] & keep16[j][i]);
                    }
                }
            }
            const uint32_t a = max(m2[0] & 0xffffu, m2[0] >> 16);
            const uint32_t b = max(m2[1] & 0xffffu, m2[1] >> 16);
            const uint32_t pr = row16_max_u16x2(a | (b << 16));
            if ((lane & 15) == 0) {
                atomicMax(&rowmax_bits[r], pr & 0xffffu);
                if (r + 1 < M) atomicMax(&rowmax_bits[r + 1], pr >> 16);
            }
        }
    }
    {
        // thread t owns chunks 2t and 2t + 1 for the exclusive scan (K/8 <= 1024)
        const int c0 = 2 * tid;
        const int a0 = c0 < nchunk ? __popc((uint32_t)mask[c0]) : 0;
        const int a1 = c0 + 1 < nchunk ? __popc((uint32_t)mask[c0 + 1]) : 0;
        const int cnt = a0 + a1;
        const int incl = wave_incl_scan(cnt);
        if (lane == 63) scan_lds[wave] = incl;
        __syncthreads();
        int base = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kLinWaves; ++w) {
            if (w < wave) base += scan_lds[w];
            total += scan_lds[w];
        }
        const int ex = base + incl - cnt;
        if (c0 < nchunk) chunk_rank[c0] = ex;
        if (c0 + 1 < nchunk) chunk_rank[c0 + 1] = ex + a0;
        if (tid == 0) chunk_rank[nchunk] = total;
    }
    __syncthreads();
    const int n_out = chunk_rank[nchunk];
    const int n_pad = (n_out + 31) & ~31;
    if (tid < 16) {
        const float amax = widen16<BF16>((uint16_t)rowmax_bits[tid]);
        sca[tid] = amax;
        scl[tid] = amax == 0.0f ? 0.0f : 127.0f / amax;
    }
    __syncthreads();

    // ---- 4. int8 activations into LDS; outlier list and values ----------------
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int c = tid + kLinThreads * j;
        if (c < nchunk) {
            const uint32_t bits = mbits[j];
            const int rank0 = bits ? chunk_rank[c] : 0;
            uint32_t keep_lo = 0, keep_hi = 0;  // 0xff per non-outlier byte
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                keep_lo |= ((bits >> e) & 1u) ? 0u : (0xffu << (8 * e));
                keep_hi |= ((bits >> (e + 4)) & 1u) ? 0u : (0xffu << (8 * e));
            }
            if (bits && blockIdx.x == 0) {
                int rk = rank0;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if ((bits >> e) & 1u) idx_out[rk++] = c * 8 + e;
            }
#pragma unroll
            for (int r = 0; r < MR; ++r) {
                if (r < M) {
                    const v8u16 v = xr[j * MR + r];
                    const float scale = scl[r];
                    // non-outlier |x| <= SCA, so |x * scale| <= 127 and the low
                    // byte is the code; outlier columns are masked to 0
                    uint32_t q[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) q[e] = quantize_low_byte(widen16<BF16>(v[e]), scale);
                    const uint2 packed = make_uint2(
                        ((q[0] & 0xffu) | ((q[1] & 0xffu) << 8) | ((q[2] & 0xffu) << 16) | (q[3] << 24)) & keep_lo,
                        ((q[4] & 0xffu) | ((q[5] & 0xffu) << 8) | ((q[6] & 0xffu) << 16) | (q[7] << 24)) & keep_hi);
                    *reinterpret_cast<uint2*>(ca + r * (K + kLinPad) + c * 8) = packed;
                    if (blockIdx.x == 0)
                        *reinterpret_cast<uint2*>(CA_out + (size_t)r * K + c * 8) = packed;
                    if (bits) {
                        int rk = rank0;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            if ((bits >> e) & 1u) {
                                if (rk < kLinOutCap) xo_lds[r][rk] = v[e];
                                if (blockIdx.x == 0) XO_out[(size_t)r * n_pad + rk] = v[e];
                                ++rk;
                            }
                        }
                    }
                }
            }
        }
    }
    if (blockIdx.x == 0) {
        if (tid == 0) *n_out_out = n_out;
        if (tid < M) SCA_out[tid] = sca[tid];
        const int padw = n_pad - n_out;
        for (int i = tid; i < M * padw; i += kLinThreads) {
            const int r = i / padw;
            XO_out[(size_t)r * n_pad + n_out + (i - r * padw)] = 0;
        }
    }
    __syncthreads();

    // ---- 5. int8 MFMA over this wave's K steps; outlier weight bytes ----------
    const bool a_ok = r16 < M;
    const int8_t* pa = ca + r16 * (K + kLinPad) + kg * 16;
    v4i acc = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < STEPS; ++i) {
        const int s = wave + i * kLinWaves;
        if (s < nsteps) {
            const v4i a = a_ok ? *reinterpret_cast<const v4i*>(pa + s * 64) : v4i{0, 0, 0, 0};
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, breg[i], acc, 0, 0, 0);
            // this lane holds CB[n0 + r16, 64 s + 16 kg + b], b < 16: chunks
            // 8 s + 2 kg and 8 s + 2 kg + 1
            if (n_out > 0) {
                const int c = 8 * s + 2 * kg;
                const uint32_t bits = (uint32_t)mask[c] | ((uint32_t)mask[c + 1] << 8);
                if (bits) {
                    int rk = chunk_rank[c];
#pragma unroll
                    for (int b = 0; b < 16; ++b) {
                        if ((bits >> b) & 1u) {
                            if (rk < kLinOutCap)
                                cbo[r16][rk] = (float)(int8_t)((breg[i][b >> 2] >> (8 * (b & 3))) & 0xff);
                            ++rk;
                        }
                    }
                }
            }
        }
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][v][lane] = acc[v];
    __syncthreads();

    // ---- 6. epilogue: one output per thread ------------------------------------
    if (!e_ok) return;
    // accumulator register v of lane l holds row 4*(l/16) + v, column l%16
    const int l = (e_m >> 2) * 16 + e_n, v = e_m & 3;
    int c32 = 0;
#pragma unroll
    for (int w = 0; w < kLinWaves; ++w) c32 += red[w][v][l];
    if (C_i32) C_i32[(size_t)e_m * N + n_e] = c32;
    float y = (float)c32 * (sca[e_m] / 127.0f);
    const int staged = min(n_out, kLinOutCap);
    for (int j = 0; j < staged; ++j) y += widen16<BF16>(xo_lds[e_m][j]) * cbo[e_n][j];
    if (n_out > kLinOutCap) {
        // more outliers than staged: walk the mask for the rest (slow path)
        int j = 0;
        for (int c = 0; c < nchunk; ++c) {
            uint32_t bits = mask[c];
            while (bits) {
                const int k = c * 8 + __builtin_ctz(bits);
                bits &= bits - 1;
                if (j >= kLinOutCap)
                    y += widen16<BF16>(X[(size_t)e_m * K + k]) * (float)CB[(size_t)n_e * K + k];
                ++j;
            }
        }
    }
    const float bv = bias ? widen16<BF16>(bias_raw) : 0.0f;
    Y[(size_t)e_m * N + n_e] = narrow16<BF16>(y * (scb_raw / 127.0f) + bv);
}

template <bool BF16, int MR, int CPT, int STEPS>
void launch_variant(dim3 grid, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop,
                    const uint16_t* x, int M, int N, int K, float t, const int8_t* CB,
                    const float* SCB, const uint16_t* b, uint16_t* y, int8_t* CA, float* SCA,
                    int32_t* idx, int32_t* n_out, uint16_t* xo, int32_t* C_i32) {
    auto fn = linear_small_m_kernel<BF16, MR, CPT, STEPS>;
    if (ev_start || ev_stop)
        hipExtLaunchKernelGGL(fn, grid, dim3(kLinThreads), 0, stream, ev_start, ev_stop, 0, x, M,
                              N, K, t, CB, SCB, b, y, CA, SCA, idx, n_out, xo, C_i32);
    else
        fn<<<grid, kLinThreads, 0, stream>>>(x, M, N, K, t, CB, SCB, b, y, CA, SCA, idx, n_out,
                                             xo, C_i32);
}

template <bool BF16>
void launch_dtype(dim3 grid, hipStream_t stream, hipEvent_t e0, hipEvent_t e1, const uint16_t* x,
                  int M, int N, int K, float t, const int8_t* CB, const float* SCB,
                  const uint16_t* b, uint16_t* y, int8_t* CA, float* SCA, int32_t* idx,
                  int32_t* n_out, uint16_t* xo, int32_t* C_i32) {
    const int steps = (K / 64 + kLinWaves - 1) / kLinWaves;  // per wave
#define LIN_ARGS grid, stream, e0, e1, x, M, N, K, t, CB, SCB, b, y, CA, SCA, idx, n_out, xo, C_i32
    if (K > 4096) {
        launch_variant<BF16, 8, 2, 16>(LIN_ARGS);
    } else if (M > 8) {
        if (steps <= 2) launch_variant<BF16, 16, 1, 2>(LIN_ARGS);
        else if (steps <= 4) launch_variant<BF16, 16, 1, 4>(LIN_ARGS);
        else launch_variant<BF16, 16, 1, 8>(LIN_ARGS);
    } else {
        if (steps <= 2) launch_variant<BF16, 8, 1, 2>(LIN_ARGS);
        else if (steps <= 4) launch_variant<BF16, 8, 1, 4>(LIN_ARGS);
        else launch_variant<BF16, 8, 1, 8>(LIN_ARGS);
    }
#undef LIN_ARGS
}

hipError_t launch_linear_small_m(const void* X, bool bf16, int M, int N, int K, float t,
                                 const int8_t* CB, const float* SCB, const void* bias, void* Y,
                                 int8_t* CA, float* SCA, int32_t* idx, int32_t* n_out, void* XO,
                                 int32_t* C_i32, hipStream_t stream, hipEvent_t ev_start,
                                 hipEvent_t ev_stop) {
    dim3 grid((N + 15) / 16);
    const uint16_t* x = static_cast<const uint16_t*>(X);
    const uint16_t* b = static_cast<const uint16_t*>(bias);
    uint16_t* y = static_cast<uint16_t*>(Y);
    uint16_t* xo = static_cast<uint16_t*>(XO);
    if (bf16)
        launch_dtype<true>(grid, stream, ev_start, ev_stop, x, M, N, K, t, CB, SCB, b, y, CA, SCA,
                           idx, n_out, xo, C_i32);
    else
        launch_dtype<false>(grid, stream, ev_start, ev_stop, x, M, N, K, t, CB, SCB, b, y, CA, SCA,
                            idx, n_out, xo, C_i32);
    return hipGetLastError();
}

}  // namespace llmint8
