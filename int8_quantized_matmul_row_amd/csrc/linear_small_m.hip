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
// At M <= 16 the int8 weight (N*K bytes) is nearly all of the traffic.  Each
// workgroup owns NB output channels (32, or 16 when K > 4096) and the whole K
// range, so it needs no other workgroup's results:
//  * it issues its share of X (M x K 16-bit), its epilogue operands and its
//    NB x K weight block (16-byte loads in the MFMA operand layout, contiguous
//    K steps per wave) up front; vector loads retire in issue order, so X is
//    usable while the weight is still streaming in;
//  * it quantizes the activations itself, exactly as llmint8_quantize_act
//    does: column maxima over all M rows and the outlier mask, the row absmax
//    over non-outlier columns (packed 16-bit maxima, DPP reductions), the int8
//    codes into LDS, the ascending outlier ranks;
//  * v_mfma_i32_16x16x64_i8 combines the LDS activations with the weight
//    registers; the weight bytes of the outlier columns are picked out of those
//    same registers into LDS;
//  * one thread per (token, channel) adds the K-group partial sums and writes
//      Y = (C * SCA[m]/127 + sum_j XO[m,j] * CB[n, idx[j]]) * SCB[n]/127 + bias[n];
//    with more than 64 outlier columns (up to every column at threshold 0) the
//    outlier sum runs as 16-bit MFMAs over all of K against X masked to its
//    outlier columns and the weight registers.
// The activation outputs (CA, SCA, the outlier list and count, XO) are written
// too, so the call has the results of llmint8_quantize_act followed by
// llmint8_matmul: CA spread over the workgroups, the rest by workgroup 0.
#include "common.h"

namespace llmint8 {

namespace {

constexpr int kLinThreads = 512;
constexpr int kLinWaves = 8;
constexpr int kLinMaxChunks = 1024;                  // K / 8 (K <= 8192)
constexpr int kLinCaBytes = 16 * (4096 + 16);        // >= rows * (K + 16) for every variant
constexpr int kLinOutCap = 64;                       // outliers staged in LDS (more: the product as MFMAs)

// MR: activation rows held (8 or 16, >= M); CPT: 8-column chunks per thread
// (K <= 4096 -> 1, K <= 8192 -> 2 with MR = 8); NB: output channels per
// workgroup (16 or 32); SPW: 64-wide K steps per wave.  Waves split as
// NB/16 channel tiles x (8 / (NB/16)) K groups; wave w takes tile w % T and
// the contiguous K steps [g * SPW, g * SPW + SPW) of group g = w / T.
// All loads are unconditional from clamped, in-bounds addresses: a conditional
// load would end in a join that waits for it and serialize the stream.  Rows,
// chunks and steps beyond the real shape are masked where used.
template <bool BF16, int MR, int CPT, int NB, int SPW>
__global__ __launch_bounds__(kLinThreads) void linear_small_m_kernel(
    const uint16_t* __restrict__ X, int M, int N, int K, float t,
    const int8_t* __restrict__ CB, const float* __restrict__ SCB,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y,
    int8_t* __restrict__ CA_out, float* __restrict__ SCA_out, int32_t* __restrict__ idx_out,
    int32_t* __restrict__ n_out_out, uint16_t* __restrict__ XO_out,
    int32_t* __restrict__ C_i32) {
    constexpr int T = NB / 16;          // channel tiles
    constexpr int G = kLinWaves / T;    // K groups per tile
    __shared__ __attribute__((aligned(16))) int8_t ca[kLinCaBytes];
    __shared__ uint8_t mask[kLinMaxChunks];
    __shared__ int chunk_rank[kLinMaxChunks + 1];  // outliers before each 8-column chunk
    __shared__ float xo_s[16][kLinOutCap];          // XO[m, j], j < kLinOutCap
    __shared__ float cbo[NB][kLinOutCap];           // CB[n0 + i, idx[j]], j < kLinOutCap
    __shared__ uint32_t rmax_w[kLinWaves][16];      // per-wave row maxima (16-bit patterns)
    __shared__ float sca[16];
    __shared__ float scl[16];                       // 127 / SCA (0 for an all-zero row)
    __shared__ int scan_lds[kLinWaves];
    __shared__ int red[kLinWaves][4][64];
    __shared__ float red_o[kLinWaves][4][64];     // the outlier product's partial tiles (many columns)

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = blockIdx.x * NB;
    const int nchunk = K >> 3, nsteps = K >> 6;
    const int ca_stride = K + 16;  // 16 rows at one offset hit distinct banks

    // ---- 1a. activation pieces: chunks c = tid + 512 j, rows r < MR ----------
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
    // ---- 1b. epilogue operands: thread -> (token e_m, channel n0 + e_n) -------
    const int e_n = tid % NB, e_m = tid / NB;
    const int n_e = n0 + e_n;
    const bool e_ok = e_m < M && n_e < N;
    const int n_c = min(n_e, N - 1);
    // raw values only: using them here would make the stream wait for them
    const float scb_raw = SCB[n_c];
    const uint16_t bias_raw = *(bias ? bias + n_c : reinterpret_cast<const uint16_t*>(SCB + n_c));
    // ---- 1c. the weight block: lane (row r16, 16-byte group kg) holds
    // CB[n0 + 16 tt + r16, 64 s + 16 kg ...] for this wave's steps s ----------
    const int tt = wave % T, grp = wave / T, r16 = lane & 15, kg = lane >> 4;
    const int8_t* pb = CB + (size_t)min(n0 + tt * 16 + r16, N - 1) * K + kg * 16;
    v4i breg[SPW];
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int s = min(grp * SPW + i, nsteps - 1);
        breg[i] = *reinterpret_cast<const v4i*>(pb + (size_t)s * 64);
    }

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
            // rows beyond M hold row 0 again, which changes no maximum
            const v4i w = __builtin_bit_cast(v4i, xr[j * MR + r]);
#pragma unroll
            for (int i = 0; i < 4; ++i) cm[i] = max_u16x2(cm[i], abs2((uint32_t)w[i]));
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

    // ---- 3. row absmax over non-outlier columns (a thread's own mask bits
    // suffice); per-wave maxima through DPP, one LDS word per wave and row -----
    {
        uint32_t keep16[CPT][4];  // 0x7fff in the 16-bit halves of non-outlier columns
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const bool ok = tid + kLinThreads * j < nchunk;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                keep16[j][i] = !ok ? 0u
                                   : ((((mbits[j] >> (2 * i)) & 1u) ? 0u : 0x7fffu) |
                                      (((mbits[j] >> (2 * i + 1)) & 1u) ? 0u : 0x7fff0000u));
        }
#pragma unroll
        for (int r = 0; r < MR; r += 2) {
            uint32_t h2[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t m2 = 0;
#pragma unroll
                for (int j = 0; j < CPT; ++j) {
                    const v4i w = __builtin_bit_cast(v4i, xr[j * MR + r + h]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) m2 = max_u16x2(m2, (uint32_t)w[i] & keep16[j][i]);
                }
                h2[h] = max(m2 & 0xffffu, m2 >> 16);
            }
            const uint32_t pr = row16_max_u16x2(h2[0] | (h2[1] << 16));
            const uint32_t q0 = (uint32_t)__builtin_amdgcn_readlane((int)pr, 0);
            const uint32_t q1 = (uint32_t)__builtin_amdgcn_readlane((int)pr, 16);
            const uint32_t q2 = (uint32_t)__builtin_amdgcn_readlane((int)pr, 32);
            const uint32_t q3 = (uint32_t)__builtin_amdgcn_readlane((int)pr, 48);
            const uint32_t wm = max_u16x2(max_u16x2(q0, q1), max_u16x2(q2, q3));
            if (lane == 0) {
                rmax_w[wave][r] = r < M ? (wm & 0xffffu) : 0u;
                rmax_w[wave][r + 1] = r + 1 < M ? (wm >> 16) : 0u;
            }
        }
    }
    __syncthreads();  // mask and per-wave row maxima complete

    // ---- 4. ranks: exclusive scan of the chunks' outlier counts; row scales ---
    {
        // thread t owns chunks 2t and 2t + 1 (K/8 <= 1024)
        const int c0 = 2 * tid;
        const int a0 = c0 < nchunk ? __popc((uint32_t)mask[c0]) : 0;
        const int a1 = c0 + 1 < nchunk ? __popc((uint32_t)mask[c0 + 1]) : 0;
        const int cnt = a0 + a1;
        const int incl = wave_incl_scan(cnt);
        if (lane == 63) scan_lds[wave] = incl;
        if (tid < 16) {
            uint32_t m = 0;
#pragma unroll
            for (int w = 0; w < kLinWaves; ++w) m = max(m, rmax_w[w][tid]);
            const float amax = widen16<BF16>((uint16_t)m);
            sca[tid] = amax;
            scl[tid] = amax == 0.0f ? 0.0f : 127.0f / amax;
        }
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

    // ---- 5. int8 activations into LDS; staged outlier activations -------------
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int c = tid + kLinThreads * j;
        if (c < nchunk) {
            const uint32_t bits = mbits[j];
            uint32_t keep_lo = 0, keep_hi = 0;  // 0xff per non-outlier byte
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                keep_lo |= ((bits >> e) & 1u) ? 0u : (0xffu << (8 * e));
                keep_hi |= ((bits >> (e + 4)) & 1u) ? 0u : (0xffu << (8 * e));
            }
            // this workgroup's share of the CA output: chunks c = blockIdx.x mod grid
            const bool export_ca = c % gridDim.x == blockIdx.x;
            const int rank0 = bits ? chunk_rank[c] : 0;
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
                    const uint32_t lo = __builtin_amdgcn_perm(
                        __builtin_amdgcn_perm(q[3], q[2], 0x0c0c0400u),
                        __builtin_amdgcn_perm(q[1], q[0], 0x0c0c0400u), 0x05040100u);
                    const uint32_t hi = __builtin_amdgcn_perm(
                        __builtin_amdgcn_perm(q[7], q[6], 0x0c0c0400u),
                        __builtin_amdgcn_perm(q[5], q[4], 0x0c0c0400u), 0x05040100u);
                    const uint2 packed = make_uint2(lo & keep_lo, hi & keep_hi);
                    *reinterpret_cast<uint2*>(ca + r * ca_stride + c * 8) = packed;
                    if (export_ca) *reinterpret_cast<uint2*>(CA_out + (size_t)r * K + c * 8) = packed;
                    if (bits) {
                        int rk = rank0;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            if ((bits >> e) & 1u) {
                                if (rk < kLinOutCap) xo_s[r][rk] = widen16<BF16>(v[e]);
                                ++rk;
                            }
                        }
                    }
                }
            }
        }
    }
    // workgroup 0 writes the outlier list, its count, XO and SCA
    if (blockIdx.x == 0) {
        const int n_pad = (n_out + 31) & ~31;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int c = tid + kLinThreads * j;
            const uint32_t bits = mbits[j];
            if (bits) {
                const int rank0 = chunk_rank[c];
                int rk = rank0;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if ((bits >> e) & 1u) idx_out[rk++] = c * 8 + e;
#pragma unroll
                for (int r = 0; r < MR; ++r) {
                    if (r < M) {
                        const v8u16 v = xr[j * MR + r];
                        rk = rank0;
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if ((bits >> e) & 1u) XO_out[(size_t)r * n_pad + rk++] = v[e];
                    }
                }
            }
        }
        if (tid == 0) *n_out_out = n_out;
        if (tid < M) SCA_out[tid] = sca[tid];
        const int padw = n_pad - n_out;
        for (int i = tid; i < M * padw; i += kLinThreads) {
            const int r = i / padw;
            XO_out[(size_t)r * n_pad + n_out + (i - r * padw)] = 0;
        }
    }
    __syncthreads();

    // ---- 6. int8 MFMA over this wave's K steps; outlier weight bytes ----------
    // A = CA rows (lane row r16 = token), B = CB rows (channel): accumulator
    // register v of lane l holds token 4*(l/16) + v, channel n0 + 16 tt + l%16.
    {
        const bool a_ok = r16 < M;
        const int8_t* pa = ca + r16 * ca_stride + kg * 16;
        v4i acc = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int s = grp * SPW + i;
            if (s < nsteps) {
                const v4i a = a_ok ? *reinterpret_cast<const v4i*>(pa + s * 64) : v4i{0, 0, 0, 0};
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, breg[i], acc, 0, 0, 0);
            }
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) red[wave][v][lane] = acc[v];
    }
    // More outlier columns than kLinOutCap: the 16-bit outlier product as two
    // v_mfma_f32_16x16x32 per step over this wave's steps: A = X (read again,
    // from L2) masked to its outlier columns (lane: token r16, the same 16
    // columns as its weight bytes; token rows past M read row M-1, unused),
    // B = the weight codes as 16-bit values (exact).  A loop over the columns
    // per output would take one dependent load each.
    const bool dense_out = n_out > kLinOutCap;
    if (dense_out) {
        const uint16_t* px = X + (size_t)min(r16, M - 1) * K + kg * 16;
        v4f acc_o = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int s = grp * SPW + i;
            if (s < nsteps) {
                const int c = 8 * s + 2 * kg;
                const uint32_t bits = (uint32_t)mask[c] | ((uint32_t)mask[c + 1] << 8);
                v8u16 x0 = *reinterpret_cast<const v8u16*>(px + (size_t)s * 64);
                v8u16 x1 = *reinterpret_cast<const v8u16*>(px + (size_t)s * 64 + 8);
                v8u16 b0, b1;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    x0[e] = (bits >> e) & 1u ? x0[e] : (unsigned short)0;
                    x1[e] = (bits >> (8 + e)) & 1u ? x1[e] : (unsigned short)0;
                    b0[e] = narrow16<BF16>((float)(int8_t)((uint32_t)breg[i][e >> 2] >> (8 * (e & 3))));
                    b1[e] = narrow16<BF16>((float)(int8_t)((uint32_t)breg[i][2 + (e >> 2)] >> (8 * (e & 3))));
                }
                if constexpr (BF16) {
                    acc_o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, x0),
                                                                    __builtin_bit_cast(v8bf, b0), acc_o, 0, 0, 0);
                    acc_o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, x1),
                                                                    __builtin_bit_cast(v8bf, b1), acc_o, 0, 0, 0);
                } else {
                    acc_o = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, x0),
                                                                   __builtin_bit_cast(v8h, b0), acc_o, 0, 0, 0);
                    acc_o = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, x1),
                                                                   __builtin_bit_cast(v8h, b1), acc_o, 0, 0, 0);
                }
            }
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float f = acc_o[v];  // by value: bit_cast of a vector element reads element 0
            red_o[wave][v][lane] = f;
        }
    } else if (n_out > 0) {
        // lane (r16, kg) holds the weight bytes of chunks 8 s + 2 kg and 8 s + 2 kg + 1
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int s = grp * SPW + i;
            if (s < nsteps) {
                const int c = 8 * s + 2 * kg;
                uint32_t bits = (uint32_t)mask[c] | ((uint32_t)mask[c + 1] << 8);
                if (bits) {
                    int rk = chunk_rank[c];
                    while (bits) {
                        const int b = __builtin_ctz(bits);
                        bits &= bits - 1;
                        if (rk < kLinOutCap)
                            cbo[tt * 16 + r16][rk] =
                                (float)(int8_t)((breg[i][b >> 2] >> (8 * (b & 3))) & 0xff);
                        ++rk;
                    }
                }
            }
        }
    }
    __syncthreads();

    // ---- 7. epilogue: one output per thread ------------------------------------
    if (!e_ok) return;
    const int et = e_n >> 4, l = (e_n & 15) + 16 * (e_m >> 2), v = e_m & 3;
    int c32 = 0;
#pragma unroll
    for (int g = 0; g < G; ++g) c32 += red[et + T * g][v][l];
    if (C_i32) C_i32[(size_t)e_m * N + n_e] = c32;
    float y = (float)c32 * (sca[e_m] / 127.0f);
    if (dense_out) {
        float o = 0.0f;  // the groups' partial sums, in a fixed order
#pragma unroll
        for (int g = 0; g < G; ++g) o += red_o[et + T * g][v][l];
        y += o;
    } else {
        for (int j = 0; j < n_out; ++j) y += xo_s[e_m][j] * cbo[e_n][j];
    }
    const float bv = bias ? widen16<BF16>(bias_raw) : 0.0f;
    Y[(size_t)e_m * N + n_e] = narrow16<BF16>(y * (scb_raw / 127.0f) + bv);
}

template <bool BF16, int MR, int CPT, int NB, int SPW>
void launch_variant(hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop,
                    const uint16_t* x, int M, int N, int K, float t, const int8_t* CB,
                    const float* SCB, const uint16_t* b, uint16_t* y, int8_t* CA, float* SCA,
                    int32_t* idx, int32_t* n_out, uint16_t* xo, int32_t* C_i32) {
    auto fn = linear_small_m_kernel<BF16, MR, CPT, NB, SPW>;
    const dim3 grid((N + NB - 1) / NB);
    if (ev_start || ev_stop)
        hipExtLaunchKernelGGL(fn, grid, dim3(kLinThreads), 0, stream, ev_start, ev_stop, 0, x, M,
                              N, K, t, CB, SCB, b, y, CA, SCA, idx, n_out, xo, C_i32);
    else
        fn<<<grid, kLinThreads, 0, stream>>>(x, M, N, K, t, CB, SCB, b, y, CA, SCA, idx, n_out,
                                             xo, C_i32);
}

#define LIN_ARGS stream, e0, e1, x, M, N, K, t, CB, SCB, b, y, CA, SCA, idx, n_out, xo, C_i32

// steps per wave: K / 64 over the 8 / (NB/16) K groups, rounded up to a power of two
template <bool BF16, int MR, int CPT, int NB>
void launch_steps(hipStream_t stream, hipEvent_t e0, hipEvent_t e1, const uint16_t* x, int M,
                  int N, int K, float t, const int8_t* CB, const float* SCB, const uint16_t* b,
                  uint16_t* y, int8_t* CA, float* SCA, int32_t* idx, int32_t* n_out,
                  uint16_t* xo, int32_t* C_i32) {
    constexpr int G = kLinWaves / (NB / 16);
    const int spw = (K / 64 + G - 1) / G;
    if (spw <= 1) launch_variant<BF16, MR, CPT, NB, 1>(LIN_ARGS);
    else if (spw <= 2) launch_variant<BF16, MR, CPT, NB, 2>(LIN_ARGS);
    else if (spw <= 4) launch_variant<BF16, MR, CPT, NB, 4>(LIN_ARGS);
    else if (spw <= 8) launch_variant<BF16, MR, CPT, NB, 8>(LIN_ARGS);
    else launch_variant<BF16, MR, CPT, NB, 16>(LIN_ARGS);
}

template <bool BF16>
void launch_dtype(hipStream_t stream, hipEvent_t e0, hipEvent_t e1, const uint16_t* x, int M,
                  int N, int K, float t, const int8_t* CB, const float* SCB, const uint16_t* b,
                  uint16_t* y, int8_t* CA, float* SCA, int32_t* idx, int32_t* n_out,
                  uint16_t* xo, int32_t* C_i32) {
    if (K > 4096) launch_steps<BF16, 8, 2, 16>(LIN_ARGS);
    else if (M > 8) launch_steps<BF16, 16, 1, 32>(LIN_ARGS);
    else launch_steps<BF16, 8, 1, 32>(LIN_ARGS);
}

#undef LIN_ARGS

}  // namespace

bool linear_small_m_supported(int M, int K) {
    return M >= 1 && ((M <= 16 && K <= 4096) || (M <= 8 && K <= 8192));
}

hipError_t launch_linear_small_m(const void* X, bool bf16, int M, int N, int K, float t,
                                 const int8_t* CB, const float* SCB, const void* bias, void* Y,
                                 int8_t* CA, float* SCA, int32_t* idx, int32_t* n_out, void* XO,
                                 int32_t* C_i32, hipStream_t stream, hipEvent_t e0,
                                 hipEvent_t e1) {
    const uint16_t* x = static_cast<const uint16_t*>(X);
    const uint16_t* b = static_cast<const uint16_t*>(bias);
    uint16_t* y = static_cast<uint16_t*>(Y);
    uint16_t* xo = static_cast<uint16_t*>(XO);
    if (bf16)
        launch_dtype<true>(stream, e0, e1, x, M, N, K, t, CB, SCB, b, y, CA, SCA, idx, n_out, xo,
                           C_i32);
    else
        launch_dtype<false>(stream, e0, e1, x, M, N, K, t, CB, SCB, b, y, CA, SCA, idx, n_out, xo,
                            C_i32);
    return hipGetLastError();
}

}  // namespace llmint8
