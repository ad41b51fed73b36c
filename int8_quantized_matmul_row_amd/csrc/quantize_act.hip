// Activation quantization with outlier-column extraction.
//
// "A Gentle Introduction to 8-bit Matrix Multiplication for transformers at
// scale": section "LLM.int8() summary" (step 1: extract the outliers of the
// input hidden states by column), section "inside the MatMul" (outliers are
// the entries of magnitude 6 or more; the hidden states are quantized
// row-wise), section "absmax quantization" (scale by 127/absmax and round).
// The whole feature column goes to the 16-bit part when any of the M rows of
// the call reaches the threshold, so every row depends on every other row
// through the outlier set.
//
// Outputs: CA [M,K] int8 (outlier columns 0), SCA [M] fp32 (absmax over the
// non-outlier columns), idx [n_out] ascending, n_out, XO [M, n_pad] 16-bit
// (n_pad = round_up(n_out, 32), zero padded).  With FP8 the codes of CA are
// E4M3 bytes (scale 448/absmax, format in common.h; outlier columns 0x00).
//
// Two paths:
//  * small M (M <= 16 and M*K <= 128K): one launch of M workgroups.  Each
//    workgroup reads all of X (tiny, L2 resident) to build the outlier mask in
//    LDS, ranks the outliers with a block scan, then quantizes its own row.
//  * otherwise two launches, both reading X with 16-byte coalesced loads:
//      A  per (row group, 256-column slab): column maxima of the magnitudes,
//         thresholded -> one outlier mask per row group (a bit per column);
//      C  every workgroup ORs the G group masks and ranks the outliers
//         (popcount prefixes per 32 columns); then one wave per row: absmax
//         over non-outlier columns, quantize, write CA; scatter the row's
//         outlier values into XO by rank; workgroup 0 also writes idx and
//         n_out.
//    X is read twice in all (A, then C), CA written once.
#include "common.h"

namespace llmint8 {

namespace {

constexpr int kThreads = 256;
constexpr int kMaskBytesMax = 133120 / 8;  // K <= 133120
constexpr int kMaskWordsMax = 133120 / 32;
constexpr int kSlabChunks = 8;             // 8-column chunks per slab of kernel A (K % 64 == 0)
constexpr int kRowLanes = kThreads / kSlabChunks;
constexpr int kSmallMaxM = 16;
constexpr int kSmallMaxElems = 1 << 17;

__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
    return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
           ((uint32_t)(d & 0xff) << 24);
}

// Quantize 8 values with a mask byte (set bit = outlier -> code 0).
template <bool BF16, bool FP8>
__device__ __forceinline__ uint2 quantize8(v8u16 v, uint32_t bits, float scale) {
    if constexpr (FP8) {
        uint32_t keep = 0;  // 0xff in the byte of every non-outlier value
#pragma unroll
        for (int e = 0; e < 4; ++e) keep |= ((bits >> e) & 1u) ? 0u : 0xffu << (8 * e);
        const uint32_t keep_hi = ((bits & 0x10u) ? 0u : 0xffu) | ((bits & 0x20u) ? 0u : 0xff00u) |
                                 ((bits & 0x40u) ? 0u : 0xff0000u) | ((bits & 0x80u) ? 0u : 0xff000000u);
        const uint32_t lo = e4m3_pack4(widen16<BF16>(v[0]), widen16<BF16>(v[1]), widen16<BF16>(v[2]),
                                       widen16<BF16>(v[3]), scale);
        const uint32_t hi = e4m3_pack4(widen16<BF16>(v[4]), widen16<BF16>(v[5]), widen16<BF16>(v[6]),
                                       widen16<BF16>(v[7]), scale);
        return make_uint2(lo & keep, hi & keep_hi);
    } else {
        int q[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            q[e] = ((bits >> e) & 1u) ? 0 : quantize_value(widen16<BF16>(v[e]), scale);
        return make_uint2(pack4(q[0], q[1], q[2], q[3]), pack4(q[4], q[5], q[6], q[7]));
    }
}

// Exclusive scan of one int per thread over a 256-thread block.
__device__ __forceinline__ int block_exclusive_scan(int v, int* lds /*[4]*/, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int incl = wave_incl_scan(v);
    if (lane == 63) lds[wave] = incl;
    __syncthreads();
    int wave_off = 0, sum = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        if (w < wave) wave_off += lds[w];
        sum += lds[w];
    }
    __syncthreads();
    *total = sum;
    return wave_off + incl - v;
}

__device__ __forceinline__ float block_max(float v, float* lds /*[4]*/) {
    v = wave_max(v);
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = fmaxf(fmaxf(lds[0], lds[1]), fmaxf(lds[2], lds[3]));
    __syncthreads();
    return r;
}

// ---------------------------------------------------------------------------
// Small-M path: one workgroup per row, everything in one launch.
template <bool BF16, bool FP8>
__global__ __launch_bounds__(kThreads) void act_quant_small(
    const uint16_t* __restrict__ X, int M, int K, float t, int8_t* __restrict__ CA,
    float* __restrict__ SCA, int32_t* __restrict__ idx, int32_t* __restrict__ n_out,
    uint16_t* __restrict__ XO) {
    __shared__ uint8_t mask[kMaskBytesMax];
    __shared__ int scan_lds[4];
    __shared__ float red_lds[4];
    const int tid = threadIdx.x;
    const int m = blockIdx.x;
    const int nchunk = K >> 3;

    // 1. column max over all M rows -> one mask byte per 8 columns
    for (int c = tid; c < nchunk; c += kThreads) {
        float cm[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int r = 0; r < M; ++r) {
            v8u16 v = *reinterpret_cast<const v8u16*>(X + (size_t)r * K + (size_t)c * 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) cm[e] = fmaxf(cm[e], fabsf(widen16<BF16>(v[e])));
        }
        uint32_t bits = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) bits |= (cm[e] >= t ? 1u : 0u) << e;
        mask[c] = (uint8_t)bits;
    }
    __syncthreads();

    // 2. rank the outliers: thread t owns a contiguous run of mask bytes
    const int per = (nchunk + kThreads - 1) / kThreads;
    const int c0 = min(tid * per, nchunk), c1 = min(c0 + per, nchunk);
    int cnt = 0;
    for (int c = c0; c < c1; ++c) cnt += __popc((uint32_t)mask[c]);
    int total;
    int rank = block_exclusive_scan(cnt, scan_lds, &total);
    const int n_pad = (total + 31) & ~31;
    const uint16_t* xrow = X + (size_t)m * K;
    uint16_t* xo = XO + (size_t)m * n_pad;
    for (int c = c0; c < c1; ++c) {
        uint32_t bits = mask[c];
        while (bits) {
            const int e = __builtin_ctz(bits);
            bits &= bits - 1;
            const int k = c * 8 + e;
            if (m == 0) idx[rank] = k;
            xo[rank] = xrow[k];
            ++rank;
        }
    }
    for (int j = total + tid; j < n_pad; j += kThreads) xo[j] = 0;
    if (m == 0 && tid == 0) *n_out = total;

    // 3. row absmax over the non-outlier columns
    float amax = 0.0f;
    for (int c = tid; c < nchunk; c += kThreads) {
        v8u16 v = *reinterpret_cast<const v8u16*>(xrow + (size_t)c * 8);
        const uint32_t bits = mask[c];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (!((bits >> e) & 1u)) amax = fmaxf(amax, fabsf(widen16<BF16>(v[e])));
    }
    amax = block_max(amax, red_lds);
    if (tid == 0) SCA[m] = amax;
    const float scale = amax == 0.0f ? 0.0f : code_max<FP8>() / amax;

    // 4. quantize the row
    int8_t* carow = CA + (size_t)m * K;
    for (int c = tid; c < nchunk; c += kThreads) {
        v8u16 v = *reinterpret_cast<const v8u16*>(xrow + (size_t)c * 8);
        *reinterpret_cast<uint2*>(carow + (size_t)c * 8) = quantize8<BF16, FP8>(v, mask[c], scale);
    }
}

// ---------------------------------------------------------------------------
// Large-M path, kernel A: for one group of rows and one 64-column slab, the
// column maxima of the magnitudes (as 16-bit patterns, which order like the
// values), thresholded: bit e of byte c of the group's mask is set when column
// 8c+e reaches t in one of the group's rows.  grid = (slabs, groups); thread
// (row lane rl = tid/8, chunk lane cl = tid%8) reads rows r0+rl, r0+rl+32, ...
// of its 8-column chunk with 16-byte loads, 8 of them in flight (a wave
// instruction reads 8 rows x 128 bytes).  Narrow slabs keep the number of
// row groups, which kernel C combines, small.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void act_colmask_partial(const uint16_t* __restrict__ X, int M,
                                                                int K, int rows_per_group, float t,
                                                                uint32_t* __restrict__ mask_g) {
    __shared__ uint32_t red[kRowLanes][kSlabChunks][4];
    __shared__ __attribute__((aligned(4))) uint8_t mbytes[kSlabChunks];
    const int tid = threadIdx.x, cl = tid % kSlabChunks, rl = tid / kSlabChunks;
    const int nwords = K >> 5;
    const int c = blockIdx.x * kSlabChunks + cl;  // < K/8: K % 64 == 0
    const int r0 = blockIdx.y * rows_per_group, r1 = min(r0 + rows_per_group, M);
    uint32_t cm[4] = {0, 0, 0, 0};
    const uint16_t* p = X + (size_t)c * 8;
#pragma unroll 8
    for (int r = r0 + rl; r < r1; r += kRowLanes) {
        const v4i v = *reinterpret_cast<const v4i*>(p + (size_t)r * K);
#pragma unroll
        for (int i = 0; i < 4; ++i) cm[i] = max_u16x2(cm[i], abs2((uint32_t)v[i]));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) red[rl][cl][i] = cm[i];
    __syncthreads();
    if (tid < kSlabChunks) {
#pragma unroll
        for (int q = 1; q < kRowLanes; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) cm[i] = max_u16x2(cm[i], red[q][cl][i]);
        const uint32_t tb = threshold_bits<BF16>(t);
        uint32_t bits = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            bits |= ((cm[i] & 0xffffu) >= tb ? 1u : 0u) << (2 * i);
            bits |= ((cm[i] >> 16) >= tb ? 1u : 0u) << (2 * i + 1);
        }
        mbytes[cl] = (uint8_t)bits;
    }
    __syncthreads();
    if (tid < kSlabChunks / 4) {
        const int w = blockIdx.x * (kSlabChunks / 4) + tid;  // < nwords: K % 64 == 0
        mask_g[(size_t)blockIdx.y * nwords + w] = reinterpret_cast<const uint32_t*>(mbytes)[tid];
    }
}

// 0xffff in the 16-bit halves of word i (columns 2i, 2i+1 of a chunk) whose
// mask bit is clear.
__device__ __forceinline__ uint32_t keep_halves(uint32_t bits, int i) {
    return (((bits >> (2 * i)) & 1u) ? 0u : 0xffffu) | (((bits >> (2 * i + 1)) & 1u) ? 0u : 0xffff0000u);
}

// Codes of 8 values none of which is an outlier (|x| <= absmax, so
// |x * scale| <= 127 (448) up to rounding).  int8: the fp32 product plus
// 1.5 * 2^23 holds rint(product) in its low byte; E4M3: v_cvt_pk_fp8_f32.
// From fp16 the product is one v_fma_mix_f32 (see common.h).
template <bool BF16, bool FP8>
__device__ __forceinline__ uint2 codes8(v4i x, float scale, float nz) {
    const v8u16 v = __builtin_bit_cast(v8u16, x);
    uint32_t lo, hi;
    if constexpr (FP8 && !BF16) {
        _Float16 h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = __builtin_bit_cast(_Float16, (uint16_t)v[e]);
        lo = e4m3_pack4_f16(h[0], h[1], h[2], h[3], scale, nz);
        hi = e4m3_pack4_f16(h[4], h[5], h[6], h[7], scale, nz);
    } else if constexpr (FP8) {
        lo = e4m3_pack4(widen16<true>(v[0]), widen16<true>(v[1]), widen16<true>(v[2]), widen16<true>(v[3]), scale);
        hi = e4m3_pack4(widen16<true>(v[4]), widen16<true>(v[5]), widen16<true>(v[6]), widen16<true>(v[7]), scale);
    } else {
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
    return make_uint2(lo, hi);
}

// Kernel C: the mask is the OR of the G group masks (one word = 32 columns);
// exclusive popcount prefixes per word rank the outliers.  Then wpr waves per
// row (1, or 2 or 4 for rows longer than 4096 columns): the row is read in batches
// of 8 chunks per lane (4096 columns), all loads of a batch in flight, each
// of the row's waves taking a contiguous run of batches; absmax over the
// non-outlier columns (combined across the row's waves in LDS), codes, and
// the outlier values scattered into XO by rank.  A wave's run of one batch
// is read once (it stays in registers); longer runs are read again for the
// codes.
template <bool BF16, bool FP8>
__global__ __launch_bounds__(kThreads) void act_quant_rows(
    const uint16_t* __restrict__ X, int M, int K, const uint32_t* __restrict__ mask_g, int G,
    int8_t* __restrict__ CA, float* __restrict__ SCA, int32_t* __restrict__ idx,
    int32_t* __restrict__ n_out, uint16_t* __restrict__ XO, int wpr, CodeGather gather) {
    __shared__ uint32_t mw[kMaskWordsMax];
    __shared__ int wpre[kMaskWordsMax];
    __shared__ int scan_lds[4];
    __shared__ uint32_t s_am[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nchunk = K >> 3, nwords = K >> 5;
    constexpr int B = 8;  // chunks per lane per batch
    const int nbatch = (nchunk + B * kWave - 1) / (B * kWave);
    // wpr (1, 2 or 4) waves per row: rows_wg rows per workgroup and pass;
    // this wave takes batches [b_begin, b_end) of row g rows_wg + wave / wpr
    // of row group g
    const int rows_wg = 4 / wpr, part = wave & (wpr - 1);
    const int nb_part = (nbatch + wpr - 1) / wpr;
    const int b_begin = min(part * nb_part, nbatch), b_end = min(b_begin + nb_part, nbatch);
    const int row_groups = (M + rows_wg - 1) / rows_wg;
    v4i xv[B];
    auto load_batch = [&](const uint16_t* xrow, int b) {
#pragma unroll
        for (int j = 0; j < B; ++j) {
            // from a clamped address (no branch, so no wait here); chunks past
            // K count as all-outlier below and are never stored
            const int c = (b * B + j) * kWave + lane;
            xv[j] = *reinterpret_cast<const v4i*>(xrow + (size_t)min(c, nchunk - 1) * 8);
        }
    };
    // the first row's first batch is requested before the mask, so that the
    // two latencies overlap
    const int m_first = blockIdx.x * rows_wg + wave / wpr;
    if (m_first < M && b_begin < b_end) load_batch(X + (size_t)m_first * K, b_begin);
    // the mask and the exclusive prefix of its popcounts; thread t owns a
    // contiguous run of words
    const int per = (nwords + kThreads - 1) / kThreads;
    const int w0 = min(tid * per, nwords), w1 = min(w0 + per, nwords);
    int s = 0;
    for (int w = w0; w < w1; ++w) {
        uint32_t v = 0;
#pragma unroll 8
        for (int g = 0; g < G; ++g) v |= mask_g[(size_t)g * nwords + w];
        mw[w] = v;
        s += __popc(v);
    }
    int total;
    int off = block_exclusive_scan(s, scan_lds, &total);
    for (int w = w0; w < w1; ++w) {
        wpre[w] = off;
        off += __popc(mw[w]);
    }
    __syncthreads();
    const int n_pad = (total + 31) & ~31;

    if (blockIdx.x == 0) {
        if (tid == 0) *n_out = total;
        for (int w = tid; w < nwords; w += kThreads) {
            uint32_t b = mw[w];
            int r = wpre[w];
            while (b) {
                idx[r++] = w * 32 + __builtin_ctz(b);
                b &= b - 1;
            }
        }
    }

    // row groups: uniform over the workgroup (the row's waves meet at barriers)
    for (int grp = blockIdx.x; grp < row_groups; grp += gridDim.x) {
        const int m = grp * rows_wg + wave / wpr;
        const bool row_ok = m < M;
        const uint16_t* xrow = X + (size_t)min(m, M - 1) * K;
        auto chunk_bits = [&](int c) -> uint32_t {
            return c < nchunk ? (mw[c >> 2] >> (8 * (c & 3))) & 0xffu : 0xffu;
        };
        // Outlier columns (and chunks past K) are zeroed in the registers, in
        // the rare chunks that have any, so the maxima and the codes need no
        // further mask: a zero gives code 0 (+0 in E4M3).
        auto mask_batch = [&](int b) {
#pragma unroll
            for (int j = 0; j < B; ++j) {
                const uint32_t bits = chunk_bits((b * B + j) * kWave + lane);
                if (bits) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) xv[j][i] = (int)((uint32_t)xv[j][i] & keep_halves(bits, i));
                }
            }
        };
        uint32_t am2 = 0;  // packed magnitude maxima
        if (row_ok) {
            for (int b = b_begin; b < b_end; ++b) {
                if (b > b_begin || grp != (int)blockIdx.x) load_batch(xrow, b);
                mask_batch(b);
#pragma unroll
                for (int j = 0; j < B; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) am2 = max_u16x2(am2, abs2((uint32_t)xv[j][i]));
            }
        }
        uint32_t am = wave_max_u32(max(am2 & 0xffffu, am2 >> 16));
        if (wpr > 1) {  // the row's waves combine their maxima
            if (lane == 0) s_am[wave] = am;
            __syncthreads();
            for (int t = 0; t < wpr; ++t) am = max(am, s_am[(wave & ~(wpr - 1)) + t]);
            __syncthreads();  // s_am is written again for the next row group
        }
        if (!row_ok) continue;  // no barrier below in this pass
        const float amax = widen16<BF16>((uint16_t)am);
        if (lane == 0 && part == 0) SCA[m] = amax;
        const float scale = amax == 0.0f ? 0.0f : code_max<FP8>() / amax;
        const float nz = opaque_neg_zero();
        int8_t* carow = CA + (size_t)m * K;
        uint16_t* xo = XO + (size_t)m * n_pad;
        for (int b = b_begin; b < b_end; ++b) {
            if (b_end - b_begin > 1) {  // a single batch is still in registers
                load_batch(xrow, b);
                mask_batch(b);
            }
#pragma unroll
            for (int j = 0; j < B; ++j) {
                const int c = (b * B + j) * kWave + lane;
                if (c < nchunk) {
                    *reinterpret_cast<uint2*>(carow + (size_t)c * 8) = codes8<BF16, FP8>(xv[j], scale, nz);
                    uint32_t bits = chunk_bits(c);
                    if (bits) {  // the outlier values, read again (their registers were zeroed)
                        const uint32_t word = mw[c >> 2];
                        int r = wpre[c >> 2] + __popc(word & ((1u << (8 * (c & 3))) - 1u));
                        while (bits) {
                            const int e = __builtin_ctz(bits);
                            bits &= bits - 1;
                            xo[r++] = xrow[c * 8 + e];
                        }
                    }
                }
            }
        }
        if (part == 0)
            for (int j = total + lane; j < n_pad; j += kWave) xo[j] = 0;
    }

    // the weight codes at the outlier columns for the product that follows
    // (when asked for, and when the product reads them from the gather: more
    // than min_cols columns, not simply 0 .. total-1): this workgroup's share
    // of the work items
    if (gather.out != nullptr && total > gather.min_cols && total <= gather.cap) {
        __shared__ int s_cols[kActGatherCols];
        for (int w = tid; w < nwords; w += kThreads) {
            uint32_t b = mw[w];
            int r = wpre[w];
            while (b) {
                s_cols[r++] = w * 32 + __builtin_ctz(b);
                b &= b - 1;
            }
        }
        __syncthreads();  // s_cols complete (every wave reads it); mw read for the last time
        // mw, no longer read, holds the gather's segment buffers
        static_assert(sizeof(mw) >= (kThreads / 16) * kGatherSeg, "gather buffers");
        auto col = [&](int c) { return s_cols[c]; };
        if (s_cols[total - 1] == total - 1) {
            // columns 0 .. total-1: the product reads CB itself
        } else if (total <= kOutLds) {
            gather_first_codes(gather.N, K, total, col, gather.CB, gather.out, (int64_t)blockIdx.x * kThreads + tid,
                               (int64_t)gridDim.x * kThreads);
        } else if (gather_all_sparse(K, total)) {
            gather_codes<kThreads>(
                gather.N, K, gather.cap, total, col, (total + kGatherRun - 1) / kGatherRun,
                [&](int i) { return GatherChunk{kGatherRun * i, min(kGatherRun * (i + 1), total), -1}; },
                gather.CB, gather.out, reinterpret_cast<int8_t*>(mw), tid, blockIdx.x, gridDim.x);
        } else {
            // the chunk list, from the word prefixes (32 columns per word)
            __shared__ GatherChunks s_chunks;
            if (tid == 0)
                build_gather_chunks(
                    K, total,
                    [&](int sg) { return sg * (kGatherSeg / 32) < nwords ? wpre[sg * (kGatherSeg / 32)] : total; },
                    s_chunks);
            __syncthreads();
            gather_codes<kThreads>(
                gather.N, K, gather.cap, total, col, s_chunks.n,
                [&](int i) { return GatherChunk{s_chunks.lo[i], s_chunks.lo[i + 1], s_chunks.seg[i]}; },
                gather.CB, gather.out, reinterpret_cast<int8_t*>(mw), tid, blockIdx.x, gridDim.x);
        }
    }
}

__global__ void write_zero_count(int32_t* n_out) { *n_out = 0; }

// workgroups of the row kernel below which it leaves the weight codes'
// gather to the product
constexpr int kActGatherMinBlocks = 64;

struct ActPlan {
    bool small;
    int slabs;            // K/64: 64-column slabs of kernel A
    int groups;           // G row groups of kernel A, each writing a mask of K/8 bytes
    int rows_per_group;
    size_t bytes;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

ActPlan plan_act(int64_t M, int64_t K) {
    ActPlan p{};
    p.small = M <= kSmallMaxM && M * K <= kSmallMaxElems;
    const int64_t nchunk = K / 8;
    p.slabs = (int)(nchunk / kSlabChunks);  // K % 64 == 0
    // about 512 workgroups for kernel A; few row groups (kernel C combines
    // their masks: 8 or fewer for K >= 4096), each of at least 32 rows
    int64_t g = (512 + p.slabs - 1) / p.slabs;
    const int64_t gmax = (M + 31) / 32;
    if (g > gmax) g = gmax;
    if (g > 64) g = 64;
    if (g < 1) g = 1;
    p.rows_per_group = (int)((M + g - 1) / g);
    p.groups = (int)((M + p.rows_per_group - 1) / p.rows_per_group);
    p.bytes = p.small ? 0 : align256((size_t)p.groups * (size_t)(K / 8));
    return p;
}

}  // namespace

size_t quantize_act_workspace(int64_t M, int64_t K) {
    if (M <= 0 || K <= 0) return 0;
    return plan_act(M, K).bytes;
}

hipError_t launch_quantize_act(const void* Xv, bool bf16, bool fp8, int M, int K, float t,
                               int8_t* CA, float* SCA, int32_t* idx, int32_t* n_out, void* XOv,
                               void* ws, hipStream_t stream, CodeGather* gather) {
    const uint16_t* X = static_cast<const uint16_t*>(Xv);
    uint16_t* XO = static_cast<uint16_t*>(XOv);
    CodeGather g;
    if (gather != nullptr) {
        g = *gather;
        if (g.cap > kActGatherCols) g.out = nullptr;
        gather->out = nullptr;  // set again below when act_quant_rows gathers
    }
    if (M == 0) {
        write_zero_count<<<1, 1, 0, stream>>>(n_out);
        return hipGetLastError();
    }
    const ActPlan p = plan_act(M, K);
    if (p.small) {
        void (*fn)(const uint16_t*, int, int, float, int8_t*, float*, int32_t*, int32_t*, uint16_t*) =
            bf16 ? (fp8 ? act_quant_small<true, true> : act_quant_small<true, false>)
                 : (fp8 ? act_quant_small<false, true> : act_quant_small<false, false>);
        fn<<<M, kThreads, 0, stream>>>(X, M, K, t, CA, SCA, idx, n_out, XO);
        return hipGetLastError();
    }
    uint32_t* mask_g = static_cast<uint32_t*>(ws);
    dim3 ga(p.slabs, p.groups);
    if (bf16)
        act_colmask_partial<true><<<ga, kThreads, 0, stream>>>(X, M, K, p.rows_per_group, t, mask_g);
    else
        act_colmask_partial<false><<<ga, kThreads, 0, stream>>>(X, M, K, p.rows_per_group, t, mask_g);
    // waves per row: a row longer than one batch (4096 columns) is shared by
    // 2 or 4 waves, so that fewer waves read their run twice and short M
    // still fills the CUs
    const int nbatch = (K / 8 + 511) / 512;
    const int wpr = nbatch >= 4 ? 4 : nbatch >= 2 ? 2 : 1;
    const int rows_wg = 4 / wpr;
    // at most 4 workgroups per CU (256 CUs): each combines the row groups'
    // masks and scans them once, then loops over its row groups (at
    // 4096 x 8192, 2048 workgroups of two rows each took 36.0 us, 1024 took
    // 33.6 and 512 took 34.9)
    int blocks = (M + rows_wg - 1) / rows_wg;
    if (blocks > 1024) blocks = 1024;
    // the weight codes' gather (N rows of work) only with enough workgroups:
    // a grid sized for a few token rows would take it in many dependent
    // passes, and the product's own gather kernel does it instead
    if (blocks < kActGatherMinBlocks) g.out = nullptr;
    void (*fn)(const uint16_t*, int, int, const uint32_t*, int, int8_t*, float*, int32_t*, int32_t*,
               uint16_t*, int, CodeGather) =
        bf16 ? (fp8 ? act_quant_rows<true, true> : act_quant_rows<true, false>)
             : (fp8 ? act_quant_rows<false, true> : act_quant_rows<false, false>);
    fn<<<blocks, kThreads, 0, stream>>>(X, M, K, mask_g, p.groups, CA, SCA, idx, n_out, XO, wpr, g);
    if (gather != nullptr) gather->out = g.out;
    return hipGetLastError();
}

}  // namespace llmint8
