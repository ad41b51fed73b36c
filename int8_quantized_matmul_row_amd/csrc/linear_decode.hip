// Fused LLM.int8() linear layer for decode batches (M <= 8, M*K <= 32768), one
// launch, written for a short instruction stream.
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
// Every workgroup (16 output channels, 8 waves) must derive the whole
// activation quantization itself, so its latency chain sets the kernel time.
// Measured per workgroup with in-kernel timestamps, the chain is: X arrives,
// the activation passes run, then the MFMAs and the epilogue; the weight block
// only has to land before the MFMAs.  Hence:
//  * X (at most 64 KiB) goes to LDS with global_load_lds_dwordx4, 1 KiB per
//    instruction; the weight block (16 x K bytes) is issued into registers in
//    the MFMA operand layout only once X has landed, because X's misses would
//    otherwise queue behind the whole chip's weight requests;
//  * each thread then reads its 8-column chunks of every row from LDS once,
//    and the column maxima, the mask, the row maxima (two rows per packed
//    word: four independent wave reductions), the ranks and the codes all
//    work from those registers;
//  * the outlier columns' weight bytes each output needs are fetched with a
//    few byte loads as soon as the outlier list is known (they land with or
//    after the weight block), and the outlier activations are read from LDS.
// Per workgroup: column maxima and the outlier mask, row absmax over
// non-outlier columns (packed 16-bit maxima, DPP wave reductions), ascending
// outlier ranks, int8 codes into LDS, v_mfma_i32_16x16x64_i8 over K, and one
// thread per (token, channel) for
//   Y = (C * SCA[m]/127 + sum_j XO[m,j] * CB[n, idx[j]]) * SCB[n]/127 + bias[n].
// The activation outputs (CA spread over the workgroups; SCA, the outlier list
// and count, XO from workgroup 0) are written too, so the call has the results
// of llmint8_quantize_act followed by llmint8_matmul.
#include "common.h"

namespace llmint8 {

namespace {

constexpr int kDecThreads = 512;
constexpr int kDecWaves = 8;
constexpr int kDecMaxRows = 8;
constexpr int kDecXBytes = 65536;                  // M * K * 2
constexpr int kDecCaBytes = 32896;                 // >= M * (K + 16) for M * K <= 32768
constexpr int kDecMaxK = 8192;
constexpr int kDecGather = 8;                      // outlier weight bytes fetched early

// FP8: E4M3 codes (the 8-bit floating-point variant; format in common.h)
// instead of int8.  CPT: 8-column chunks per thread (K <= 4096 -> 1, else 2);
// NB: output channels per workgroup; SPW: 64-wide K steps per wave; FULL: M == 8.  Waves split as NB/16
// channel tiles x 8/(NB/16) K groups: wave w takes tile w % T and the
// contiguous steps [g * SPW, g * SPW + SPW) of group g = w / T.
template <bool BF16, bool FP8, int CPT, int NB, int SPW, bool FULL>
__global__ __launch_bounds__(kDecThreads) void linear_decode_kernel(
    const uint16_t* __restrict__ X, int M, int N, int K, float t,
    const int8_t* __restrict__ CB, const float* __restrict__ SCB,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y,
    int8_t* __restrict__ CA_out, float* __restrict__ SCA_out, int32_t* __restrict__ idx_out,
    int32_t* __restrict__ n_out_out, uint16_t* __restrict__ XO_out,
    int32_t* __restrict__ C_i32, float* __restrict__ C_f32) {
    constexpr int T = NB / 16;
    constexpr int G = kDecWaves / T;
    __shared__ __attribute__((aligned(16))) uint16_t xl[(kDecXBytes + 1024) / 2];
    __shared__ __attribute__((aligned(16))) int8_t ca[kDecCaBytes];
    __shared__ uint16_t idx_s[kDecMaxK];           // ascending outlier columns
    __shared__ uint32_t mask_w[kDecMaxK / 32];     // outlier bits, chunk c in byte c
    __shared__ uint32_t rmax_w[kDecWaves][kDecMaxRows / 2];  // rows 2p, 2p+1 packed
    __shared__ float sca[kDecMaxRows];
    __shared__ int s_nout;
    __shared__ uint16_t xo_s[kDecMaxRows][kDecGather];  // XO of the first kDecGather outlier columns (0 past n_out)
    __shared__ int red[kDecWaves][4][64];          // int32 partial tiles, or fp32 bit patterns
    __shared__ float red_o[kDecWaves][4][64];      // the 16-bit outlier product's partial tiles (many columns)

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar arithmetic
    const int n0 = blockIdx.x * NB;
    const int nchunk = K >> 3, nsteps = K >> 6;
    const int ca_stride = K + 16;  // 16 rows at one offset hit distinct banks
    const int xbytes = M * K * 2;

    // ---- 1a. X into LDS: instruction q (1 KiB) issued by wave q % 8 ----------
    {
        const int nq = (xbytes + 1023) >> 10;
        const uint32_t base = lds_address(reinterpret_cast<const int8_t*>(xl));
        const int8_t* xg = reinterpret_cast<const int8_t*>(X);
        const int w0 = __builtin_amdgcn_readfirstlane(wave);
        for (int q = w0; q < nq; q += kDecWaves)  // the tail lanes re-read the last 16 bytes
            dma16(xg + min(q * 1024 + lane * 16, xbytes - 16),
                  __builtin_amdgcn_readfirstlane(base + q * 1024));
    }
    // every wave's X requests are issued before anything waits for them
    stage_barrier();
    // ---- 1b. epilogue operands: thread -> (token e_m, channel n0 + e_n) -------
    const int e_n = tid % NB, e_m = tid / NB;
    const int n_e = n0 + e_n;
    const bool e_ok = e_m < M && n_e < N;
    const int n_c = min(n_e, N - 1);
    // raw values only: using them here would make the stream wait for them
    const float scb_raw = SCB[n_c];
    const uint16_t bias_raw = *(bias ? bias + n_c : reinterpret_cast<const uint16_t*>(SCB + n_c));
    // X has landed once at most the two younger loads are outstanding.  The
    // weight block is issued only now: issued earlier, its requests queue
    // ahead of X's misses everywhere in the memory system (X then lands in
    // ~4.8k cycles instead of ~1.8k), and it still arrives before the
    // activation passes below are done.
    wait_vmcnt<2>();
    __syncthreads();
    // ---- 1c. the weight block: lane (row r16, 16-byte group kg) holds
    // CB[n0 + 16 tt + r16, 64 s + 16 kg ...] for this wave's steps s.  It is
    // issued in four slots spread over the register passes below: a wave that
    // issues all of it at once stalls on the address path (~1k cycles) ahead
    // of its own arithmetic, and the next barrier waits for the slowest wave.
    const int tt = wave % T, grp = wave / T, r16 = lane & 15, kg = lane >> 4;
    const int8_t* pb = CB + (size_t)min(n0 + tt * 16 + r16, N - 1) * K + kg * 16;
    v4i breg[SPW];
    auto issue_weights = [&](int slot) {
#pragma unroll
        for (int i = slot * SPW / 4; i < (slot + 1) * SPW / 4; ++i) {
            const int s = min(grp * SPW + i, nsteps - 1);
            breg[i] = *reinterpret_cast<const v4i*>(pb + (size_t)s * 64);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- 2. this thread's 8-column chunks of every row, LDS -> registers ------
    // (all reads issued together; rows >= M read as 0, which changes no maximum)
    v4i xr[CPT][kDecMaxRows];
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int c = tid + kDecThreads * j;
        const uint32_t off = (uint32_t)(c < nchunk ? c : 0) * 16;
#pragma unroll
        for (int r = 0; r < kDecMaxRows; ++r)
            xr[j][r] = FULL || r < M ? lds_load<v4i>(xl, (uint32_t)(r * K * 2) + off) : v4i{0, 0, 0, 0};
    }
    issue_weights(0);

    // ---- 3. outlier mask: column max over the M rows, 8 bits per chunk --------
    // Magnitudes are compared as 16-bit patterns (packed pairs); for finite
    // values this orders exactly like the fp32 values.
    // keep16: 0xffff in the 16-bit halves of non-outlier columns.  Both
    // magnitude patterns are at most 0x7fff, so cm - tb as a signed 16-bit
    // difference is negative exactly when the column stays (cm < tb).
    const uint32_t tb = threshold_bits<BF16>(t);
    const uint32_t tb2 = tb | (tb << 16);
    uint32_t mbits[CPT];
    uint32_t keep16[CPT][4];
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        uint32_t cm[4] = {0, 0, 0, 0};
#pragma unroll
        for (int r = 0; r < kDecMaxRows; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) cm[i] = max_u16x2(cm[i], abs2((uint32_t)xr[j][r][i]));
        uint32_t w = 0;  // outlier flag of column 2i in bit 2i, of column 2i+1 in bit 16+2i
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            keep16[j][i] = ashr16x2(sub_i16x2(cm[i], tb2), 15);
            w |= (~keep16[j][i] & 0x00010001u) << (2 * i);
        }
        const uint32_t bits = (w & 0x55u) | ((w >> 15) & 0xaau);
        mbits[j] = tid + kDecThreads * j < nchunk ? bits : 0u;
    }
    issue_weights(1);

    // ---- 4. row absmax over non-outlier columns: rows 2p and 2p+1 share one
    // packed word, so four independent wave maxima cover eight rows -----------
    {
        uint32_t rm[kDecMaxRows / 2] = {0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            // a chunk past K holds chunk 0 again, which changes no maximum
            uint32_t keep[4];  // 0x7fff in the 16-bit halves of non-outlier columns
#pragma unroll
            for (int i = 0; i < 4; ++i) keep[i] = keep16[j][i] & 0x7fff7fffu;
#pragma unroll
            for (int r = 0; r < kDecMaxRows; ++r) {
                uint32_t m2 = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) m2 = max_u16x2(m2, (uint32_t)xr[j][r][i] & keep[i]);
                const uint32_t h = max(m2 & 0xffffu, m2 >> 16);
                rm[r >> 1] = max_u16x2(rm[r >> 1], (r & 1) ? h << 16 : h);
            }
        }
        issue_weights(2);
#pragma unroll
        for (int p = 0; p < kDecMaxRows / 2; ++p) {
            const uint32_t v = row16_max_u16x2(rm[p]);
            const uint32_t a = __builtin_amdgcn_readlane((int)v, 0), b = __builtin_amdgcn_readlane((int)v, 16);
            const uint32_t c = __builtin_amdgcn_readlane((int)v, 32), d = __builtin_amdgcn_readlane((int)v, 48);
            rm[p] = max_u16x2(max_u16x2(a, b), max_u16x2(c, d));
        }
        issue_weights(3);
        if (lane == 0) {
#pragma unroll
            for (int p = 0; p < kDecMaxRows / 2; ++p) rmax_w[wave][p] = rm[p];
        }
    }

    // ---- the mask bytes and the row scales ----------------------------------
    // Each thread's outlier bits (one byte per chunk) go to LDS for the list.
    // After the barrier every wave derives the row scales itself (lane r of
    // each group of 8 reduces row r's per-wave maxima), so they are uniform
    // values and need no second barrier.
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int c = tid + kDecThreads * j;
        if (c < nchunk) reinterpret_cast<uint8_t*>(mask_w)[c] = (uint8_t)mbits[j];
    }
    __syncthreads();  // per-wave row maxima and the mask complete
    float scl_r[kDecMaxRows];  // 127 / SCA (0 for an all-zero row)
    {
        const int r = lane & (kDecMaxRows - 1);
        uint32_t m = 0;
#pragma unroll
        for (int w = 0; w < kDecWaves; ++w) m = max(m, (rmax_w[w][r >> 1] >> (16 * (r & 1))) & 0xffffu);
        const float amax = widen16<BF16>((uint16_t)m);
        const float sc = amax == 0.0f ? 0.0f : code_max<FP8>() / amax;
        if (wave == 0 && lane < M) sca[lane] = amax;
#pragma unroll
        for (int q = 0; q < kDecMaxRows; ++q)
            scl_r[q] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc), q));
    }
    // wave 0: the ascending outlier list (lane l takes the contiguous words
    // kWpl l .. kWpl l + kWpl - 1, so its columns are contiguous in the list),
    // the count, and the outlier values of the first kDecGather columns for
    // the epilogue; published by the barrier before the MFMAs
    if (wave == 0) {
        constexpr int kWpl = kDecMaxK / 32 / 64;
        const int nwords = K >> 5;
        uint32_t w[kWpl];
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < kWpl; ++i) {
            const int wi = lane * kWpl + i;
            w[i] = wi < nwords ? mask_w[wi] : 0u;
            cnt += __popc(w[i]);
        }
        const int incl = wave_incl_scan(cnt);
        int r = incl - cnt;
#pragma unroll
        for (int i = 0; i < kWpl; ++i) {
            uint32_t bits = w[i];
            while (bits) {
                idx_s[r++] = (uint16_t)((lane * kWpl + i) * 32 + __builtin_ctz(bits));
                bits &= bits - 1;
            }
        }
        const int total = __builtin_amdgcn_readlane(incl, 63);
        if (lane == 0) s_nout = total;
        // (this wave's own list writes precede these reads in its LDS queue)
        const int gm = lane / kDecGather, gj = lane % kDecGather;
        if (gm < kDecMaxRows)
            xo_s[gm][gj] = gj < total && gm < M ? xl[gm * K + idx_s[gj]] : (uint16_t)0;
    }

    // ---- 5. int8 activations into LDS, from the registers ----------------------
    // With all eight rows present (FULL) the rows need no test, so the compiler
    // can interleave their independent chains; the codes stay in registers for
    // the workgroup's share of the CA output, written after the loop.
    {
        uint32_t keep_lo[CPT], keep_hi[CPT];  // 0xff per non-outlier byte
        bool export_ca[CPT];                  // this workgroup's share of the CA output
        // workgroup b exports the chunks [b * per, b * per + per)
        const int per = (nchunk + (int)gridDim.x - 1) / (int)gridDim.x;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            // byte e of keep_lo: a byte of column e's 16-bit keep mask (columns
            // 2i and 2i+1 are the halves of keep16 word i)
            keep_lo[j] = __builtin_amdgcn_perm(keep16[j][1], keep16[j][0], 0x06040200u);
            keep_hi[j] = __builtin_amdgcn_perm(keep16[j][3], keep16[j][2], 0x06040200u);
            const int c = tid + kDecThreads * j;
            export_ca[j] = c < nchunk && (unsigned)(c - (int)blockIdx.x * per) < (unsigned)per;
        }
        const float nz = opaque_neg_zero();
        v2u codes[CPT][kDecMaxRows];
#pragma unroll
        for (int r = 0; r < kDecMaxRows; ++r) {
            if (FULL || r < M) {
                const float scale = scl_r[r];
#pragma unroll
                for (int j = 0; j < CPT; ++j) {
                    const int c = tid + kDecThreads * j;
                    const v8u16 v = __builtin_bit_cast(v8u16, xr[j][r]);
                    uint32_t lo, hi;
                    if constexpr (FP8 && !BF16) {
                        _Float16 h[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) h[e] = __builtin_bit_cast(_Float16, (uint16_t)v[e]);
                        lo = e4m3_pack4_f16(h[0], h[1], h[2], h[3], scale, nz);
                        hi = e4m3_pack4_f16(h[4], h[5], h[6], h[7], scale, nz);
                    } else if constexpr (FP8) {
                        lo = e4m3_pack4(widen16<BF16>(v[0]), widen16<BF16>(v[1]), widen16<BF16>(v[2]),
                                        widen16<BF16>(v[3]), scale);
                        hi = e4m3_pack4(widen16<BF16>(v[4]), widen16<BF16>(v[5]), widen16<BF16>(v[6]),
                                        widen16<BF16>(v[7]), scale);
                    } else {
                        // non-outlier |x| <= SCA, so |x * scale| <= 127 and the low
                        // byte is the code
                        uint32_t q[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            if constexpr (BF16) q[e] = quantize_low_byte(widen16<true>(v[e]), scale);
                            else q[e] = quantize_low_byte_f16(__builtin_bit_cast(_Float16, (uint16_t)v[e]), scale);
                        }
                        lo = __builtin_amdgcn_perm(__builtin_amdgcn_perm(q[3], q[2], 0x0c0c0400u),
                                                   __builtin_amdgcn_perm(q[1], q[0], 0x0c0c0400u), 0x05040100u);
                        hi = __builtin_amdgcn_perm(__builtin_amdgcn_perm(q[7], q[6], 0x0c0c0400u),
                                                   __builtin_amdgcn_perm(q[5], q[4], 0x0c0c0400u), 0x05040100u);
                    }
                    // outlier columns are masked to code 0
                    codes[j][r] = v2u{lo & keep_lo[j], hi & keep_hi[j]};
                    // a chunk past K (its registers hold chunk 0) parks its bytes in
                    // the row's 16-byte pad, which no MFMA reads
                    const uint32_t col = c < nchunk ? (uint32_t)c * 8 : (uint32_t)K;
                    lds_store<v2u>(ca, (uint32_t)(r * ca_stride) + col, codes[j][r]);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            if (export_ca[j]) {
                const int c = tid + kDecThreads * j;
#pragma unroll
                for (int r = 0; r < kDecMaxRows; ++r)
                    if (FULL || r < M)  // M * K <= 32768: 32-bit offsets
                        *reinterpret_cast<v2u*>(CA_out + (uint32_t)(r * K + c * 8)) = codes[j][r];
            }
        }
    }
    __syncthreads();  // the codes, the outlier list and its count complete
    const int n_out = s_nout;
    // With more than kDecGather outlier columns the 16-bit product runs as
    // MFMAs over the whole of K against X masked to its outlier columns (a
    // column-by-column loop in the epilogue would take one dependent load per
    // column: 233 us at t = 0 on 8x4096x4096).
    const bool dense_out = n_out > kDecGather;
    // this output's weight bytes in the first outlier columns; their latency
    // hides under the MFMAs (unconditional: a load under a branch would be
    // awaited where the branch rejoins; unused when dense_out)
    int cbg[kDecGather];
    {
        const int8_t* cbrow = CB + (size_t)n_c * K;
#pragma unroll
        for (int j = 0; j < kDecGather; ++j)  // the column is the same in every lane
            cbg[j] = cbrow[__builtin_amdgcn_readfirstlane(j < n_out ? (int)idx_s[j] : 0)];
    }
    // the outlier list, XO, the count and SCA, spread over the workgroups
    {
        const int n_pad = (n_out + 31) & ~31;
        const int stride = (int)gridDim.x * kDecThreads;
        for (int j = (int)blockIdx.x * kDecThreads + tid; j < n_out; j += stride) idx_out[j] = idx_s[j];
        for (int e = (int)blockIdx.x * kDecThreads + tid; e < M * n_pad; e += stride) {
            const int r = e / n_pad, j = e - r * n_pad;
            XO_out[e] = j < n_out ? xl[r * K + idx_s[j]] : (uint16_t)0;
        }
        if (blockIdx.x == 0) {
            if (tid == 0) *n_out_out = n_out;
            if (tid < M) SCA_out[tid] = sca[tid];
        }
    }

    // ---- 6. MFMA over this wave's K steps ---------------------------------------
    // A = CA rows (lane row r16 = token), B = CB rows (channel): accumulator
    // register v of lane l holds token 4*(l/16) + v, channel n0 + 16 tt + l%16.
    // int8: one v_mfma_i32_16x16x64_i8 per step; FP8: two
    // v_mfma_f32_16x16x32_fp8_fp8 on the 8-byte halves (the same split for
    // both operands, so the sum covers the step's 64 columns once).
    // All A operands are read first, unconditionally: token rows past M read
    // row M-1 (their accumulator rows are never used) and steps past K read
    // the last step (their MFMAs are skipped by a uniform test).
    {
        const int8_t* pa = ca + min(r16, M - 1) * ca_stride + kg * 16;
        v4i areg[SPW];
#pragma unroll
        for (int i = 0; i < SPW; ++i)
            areg[i] = *reinterpret_cast<const v4i*>(pa + min(grp * SPW + i, nsteps - 1) * 64);
        if constexpr (FP8) {
            v4f acc = {0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < SPW; ++i) {
                if (grp * SPW + i < nsteps) {
                    const v2l a2 = __builtin_bit_cast(v2l, areg[i]), b2 = __builtin_bit_cast(v2l, breg[i]);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a2[0], b2[0], acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a2[1], b2[1], acc, 0, 0, 0);
                }
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float f = acc[v];  // by value: bit_cast of a vector element reads element 0
                red[wave][v][lane] = __builtin_bit_cast(int, f);
            }
        } else {
            // two independent chains (even and odd steps); integer sums are exact
            v4i acc[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
#pragma unroll
            for (int i = 0; i < SPW; ++i)
                if (grp * SPW + i < nsteps)
                    acc[i & 1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(areg[i], breg[i], acc[i & 1], 0, 0, 0);
#pragma unroll
            for (int v = 0; v < 4; ++v) red[wave][v][lane] = acc[0][v] + acc[1][v];
        }
        if (dense_out) {
            // the 16-bit outlier product over this wave's steps: A = X masked
            // to its outlier columns (lane: token r16, the same 16 columns as
            // its weight bytes; mask bits from LDS, each bit widened to a
            // 16-bit lane mask), B = the weight codes as 16-bit values
            // (exact), two v_mfma_f32_16x16x32 per step on the 8-column halves
            const uint16_t* px = xl + min(r16, M - 1) * K + kg * 16;
            v4f acc_o = {0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < SPW; ++i) {
                const int s = grp * SPW + i;
                if (s < nsteps) {
                    const int col = s * 64 + kg * 16;
                    const uint32_t bits = (mask_w[col >> 5] >> (col & 31)) & 0xffffu;
                    v8u16 x0 = *reinterpret_cast<const v8u16*>(px + s * 64);
                    v8u16 x1 = *reinterpret_cast<const v8u16*>(px + s * 64 + 8);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        x0[e] = (bits >> e) & 1u ? x0[e] : (unsigned short)0;
                        x1[e] = (bits >> (8 + e)) & 1u ? x1[e] : (unsigned short)0;
                    }
                    v8u16 b0, b1;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        b0[e] = narrow16<BF16>(code_value<FP8>((int8_t)((uint32_t)breg[i][e >> 2] >> (8 * (e & 3)))));
                        b1[e] = narrow16<BF16>(code_value<FP8>((int8_t)((uint32_t)breg[i][2 + (e >> 2)] >> (8 * (e & 3)))));
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
                const float f = acc_o[v];  // by value (see the FP8 partials above)
                red_o[wave][v][lane] = f;
            }
        }
    }
    __syncthreads();

    // ---- 7. epilogue: one output per thread ------------------------------------
    if (!e_ok) return;
    const int et = e_n >> 4, l = (e_n & 15) + 16 * (e_m >> 2), v = e_m & 3;
    float y;
    if constexpr (FP8) {
        float c = 0.0f;  // the groups' partial sums, in a fixed order
#pragma unroll
        for (int g = 0; g < G; ++g) c += __builtin_bit_cast(float, red[et + T * g][v][l]);
        if (C_f32) C_f32[(size_t)e_m * N + n_e] = c;
        y = c * (sca[e_m] / code_max<FP8>());
    } else {
        int c32 = 0;
#pragma unroll
        for (int g = 0; g < G; ++g) c32 += red[et + T * g][v][l];
        if (C_i32) C_i32[(size_t)e_m * N + n_e] = c32;
        y = (float)c32 * (sca[e_m] / code_max<FP8>());
    }
    if (dense_out) {
        float o = 0.0f;  // the groups' partial sums, in a fixed order
#pragma unroll
        for (int g = 0; g < G; ++g) o += red_o[et + T * g][v][l];
        y += o;
    } else {
#pragma unroll
        for (int j = 0; j < kDecGather; ++j)
            if (j < n_out) y += widen16<BF16>(xo_s[e_m][j]) * code_value<FP8>((int8_t)cbg[j]);
    }
    const float bv = bias ? widen16<BF16>(bias_raw) : 0.0f;
    Y[(size_t)e_m * N + n_e] = narrow16<BF16>(y * (scb_raw / code_max<FP8>()) + bv);
}

template <bool BF16, bool FP8, int CPT, int NB, int SPW, bool FULL>
void launch_variant(hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop,
                    const uint16_t* x, int M, int N, int K, float t, const int8_t* CB,
                    const float* SCB, const uint16_t* b, uint16_t* y, int8_t* CA, float* SCA,
                    int32_t* idx, int32_t* n_out, uint16_t* xo, int32_t* C_i32, float* C_f32) {
    auto fn = linear_decode_kernel<BF16, FP8, CPT, NB, SPW, FULL>;
    const dim3 grid((N + NB - 1) / NB);
    if (ev_start || ev_stop)
        hipExtLaunchKernelGGL(fn, grid, dim3(kDecThreads), 0, stream, ev_start, ev_stop, 0, x, M,
                              N, K, t, CB, SCB, b, y, CA, SCA, idx, n_out, xo, C_i32, C_f32);
    else
        fn<<<grid, kDecThreads, 0, stream>>>(x, M, N, K, t, CB, SCB, b, y, CA, SCA, idx, n_out,
                                             xo, C_i32, C_f32);
}

#define DEC_ARGS stream, e0, e1, x, M, N, K, t, CB, SCB, b, y, CA, SCA, idx, n_out, xo, C_i32, C_f32
#define DEC_PARAMS                                                                              \
    hipStream_t stream, hipEvent_t e0, hipEvent_t e1, const uint16_t *x, int M, int N, int K,   \
        float t, const int8_t *CB, const float *SCB, const uint16_t *b, uint16_t *y,           \
        int8_t *CA, float *SCA, int32_t *idx, int32_t *n_out, uint16_t *xo, int32_t *C_i32,     \
        float *C_f32

// steps per wave: K / 64 over the K groups, rounded up to a power of two
template <bool BF16, bool FP8, int CPT, int NB, bool FULL>
void launch_steps(DEC_PARAMS) {
    constexpr int G = kDecWaves / (NB / 16);
    const int spw = (K / 64 + G - 1) / G;
    if (spw <= 1) launch_variant<BF16, FP8, CPT, NB, 1, FULL>(DEC_ARGS);
    else if (spw <= 2) launch_variant<BF16, FP8, CPT, NB, 2, FULL>(DEC_ARGS);
    else if (spw <= 4) launch_variant<BF16, FP8, CPT, NB, 4, FULL>(DEC_ARGS);
    else if (spw <= 8) launch_variant<BF16, FP8, CPT, NB, 8, FULL>(DEC_ARGS);
    else launch_variant<BF16, FP8, CPT, NB, 16, FULL>(DEC_ARGS);
}

template <bool BF16, bool FP8>
void launch_dtype(DEC_PARAMS) {
    // K > 4096 implies M <= 4 (M * K <= 32768), so FULL needs CPT = 1
    if (K > 4096) launch_steps<BF16, FP8, 2, 16, false>(DEC_ARGS);
    else if (M == kDecMaxRows) launch_steps<BF16, FP8, 1, 16, true>(DEC_ARGS);
    else launch_steps<BF16, FP8, 1, 16, false>(DEC_ARGS);
}

#undef DEC_ARGS
#undef DEC_PARAMS

}  // namespace

bool linear_decode_supported(int M, int K) {
    return M >= 1 && M <= kDecMaxRows && K <= kDecMaxK && (int64_t)M * K <= kDecXBytes / 2;
}

hipError_t launch_linear_decode(const void* X, bool bf16, bool fp8, int M, int N, int K, float t,
                                const int8_t* CB, const float* SCB, const void* bias, void* Y,
                                int8_t* CA, float* SCA, int32_t* idx, int32_t* n_out, void* XO,
                                int32_t* C_i32, float* C_f32, hipStream_t stream, hipEvent_t e0,
                                hipEvent_t e1) {
    const uint16_t* x = static_cast<const uint16_t*>(X);
    const uint16_t* b = static_cast<const uint16_t*>(bias);
    uint16_t* y = static_cast<uint16_t*>(Y);
    uint16_t* xo = static_cast<uint16_t*>(XO);
    if (bf16) {
        if (fp8) launch_dtype<true, true>(stream, e0, e1, x, M, N, K, t, CB, SCB, b, y, CA, SCA, idx, n_out, xo, C_i32, C_f32);
        else launch_dtype<true, false>(stream, e0, e1, x, M, N, K, t, CB, SCB, b, y, CA, SCA, idx, n_out, xo, C_i32, C_f32);
    } else {
        if (fp8) launch_dtype<false, true>(stream, e0, e1, x, M, N, K, t, CB, SCB, b, y, CA, SCA, idx, n_out, xo, C_i32, C_f32);
        else launch_dtype<false, false>(stream, e0, e1, x, M, N, K, t, CB, SCB, b, y, CA, SCA, idx, n_out, xo, C_i32, C_f32);
    }
    return hipGetLastError();
}

}  // namespace llmint8
