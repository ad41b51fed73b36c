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
//  * otherwise three launches, all reading X with 16-byte coalesced loads:
//      A  column max of each (row group, 512-column slab) -> partial [G, K]
//      B  max over the G partials, compare with the threshold -> one mask
//         byte per 8 columns, its rank inside a 256-column group, group counts
//      C  one wave per row: absmax over non-outlier columns, quantize, write
//         CA; scatter the row's outlier values into XO by rank; workgroup 0
//         also writes idx and n_out.
#include "common.h"

namespace llmint8 {

namespace {

constexpr int kThreads = 256;
constexpr int kMaskBytesMax = 133120 / 8;  // K <= 133120
constexpr int kRankGroup = 32;             // mask bytes (256 columns) per rank group
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
// Large-M path, kernel A: partial column max over a group of rows.
// grid = (ceil(K/512), G); wave w of the block takes rows row0+w, row0+w+4, ...
template <bool BF16>
__global__ __launch_bounds__(kThreads) void act_colmax_partial(const uint16_t* __restrict__ X,
                                                               int M, int K, int rows_per_group,
                                                               float* __restrict__ partial) {
    __shared__ float red[3][kWave][8];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = blockIdx.x * kWave + lane;  // 8-column piece
    const int nchunk = K >> 3;
    const int r0 = blockIdx.y * rows_per_group;
    const int r1 = min(r0 + rows_per_group, M);
    float cm[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (c < nchunk) {
#pragma unroll 4
        for (int r = r0 + wave; r < r1; r += 4) {
            v8u16 v = *reinterpret_cast<const v8u16*>(X + (size_t)r * K + (size_t)c * 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) cm[e] = fmaxf(cm[e], fabsf(widen16<BF16>(v[e])));
        }
    }
    if (wave > 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) red[wave - 1][lane][e] = cm[e];
    }
    __syncthreads();
    if (wave == 0 && c < nchunk) {
#pragma unroll
        for (int w = 0; w < 3; ++w)
#pragma unroll
            for (int e = 0; e < 8; ++e) cm[e] = fmaxf(cm[e], red[w][lane][e]);
        float* dst = partial + (size_t)blockIdx.y * K + (size_t)c * 8;
        *reinterpret_cast<v4f*>(dst) = v4f{cm[0], cm[1], cm[2], cm[3]};
        *reinterpret_cast<v4f*>(dst + 4) = v4f{cm[4], cm[5], cm[6], cm[7]};
    }
}

// Kernel B: threshold the column max; one mask byte per 8 columns, ranked
// inside groups of kRankGroup bytes.  256 threads = 32 mask bytes x 8 lanes,
// the 8 lanes of a byte split the G partial rows.
__global__ __launch_bounds__(kThreads) void act_outlier_mask(const float* __restrict__ partial,
                                                             int G, int K, float t,
                                                             uint8_t* __restrict__ mask,
                                                             int32_t* __restrict__ rank8,
                                                             int32_t* __restrict__ group_count) {
    __shared__ int cnt_lds[kRankGroup];
    const int sub = threadIdx.x & 7;
    const int local = threadIdx.x >> 3;  // 0..31
    const int c = blockIdx.x * kRankGroup + local;
    const int nchunk = K >> 3;
    float cm[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (c < nchunk) {
        for (int g = sub; g < G; g += 8) {
            const float* src = partial + (size_t)g * K + (size_t)c * 8;
            v4f a = *reinterpret_cast<const v4f*>(src);
            v4f b = *reinterpret_cast<const v4f*>(src + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                cm[e] = fmaxf(cm[e], a[e]);
                cm[e + 4] = fmaxf(cm[e + 4], b[e]);
            }
        }
    }
    // max over the 8 lanes of each mask byte: xor 1, xor 2 (quad_perm), then
    // the half-row mirror (lane i <-> 7 - i within 8 lanes)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float v = cm[e];
        v = fmaxf(v, __builtin_bit_cast(float, dpp_i<0xB1>(0, __builtin_bit_cast(int, v))));
        v = fmaxf(v, __builtin_bit_cast(float, dpp_i<0x4E>(0, __builtin_bit_cast(int, v))));
        v = fmaxf(v, __builtin_bit_cast(float, dpp_i<0x141>(0, __builtin_bit_cast(int, v))));
        cm[e] = v;
    }
    uint32_t bits = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) bits |= (cm[e] >= t ? 1u : 0u) << e;
    if (c >= nchunk) bits = 0;
    if (sub == 0) {
        cnt_lds[local] = __popc(bits);
        if (c < nchunk) mask[c] = (uint8_t)bits;
    }
    __syncthreads();
    if (sub == 0 && c < nchunk) {
        int before = 0;
        for (int q = 0; q < local; ++q) before += cnt_lds[q];
        rank8[c] = before;
    }
    if (threadIdx.x == 0) {
        int s = 0;
        for (int q = 0; q < kRankGroup; ++q) s += cnt_lds[q];
        group_count[blockIdx.x] = s;
    }
}

// Kernel C: one wave per row.  Group offsets are rebuilt per workgroup from
// the group counts (at most K/256 of them).
template <bool BF16, bool FP8>
__global__ __launch_bounds__(kThreads) void act_quant_rows(
    const uint16_t* __restrict__ X, int M, int K, const uint8_t* __restrict__ mask_g,
    const int32_t* __restrict__ rank8, const int32_t* __restrict__ group_count, int n_groups,
    int8_t* __restrict__ CA, float* __restrict__ SCA, int32_t* __restrict__ idx,
    int32_t* __restrict__ n_out, uint16_t* __restrict__ XO) {
    __shared__ uint8_t mask[kMaskBytesMax];
    __shared__ int goff[kMaskBytesMax / kRankGroup + 1];
    __shared__ int scan_lds[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nchunk = K >> 3;
    for (int c = tid; c < nchunk; c += kThreads) mask[c] = mask_g[c];
    // group offsets: exclusive scan of group_count, in runs of `per` groups per thread
    const int per = (n_groups + kThreads - 1) / kThreads;
    const int g0 = min(tid * per, n_groups), g1 = min(g0 + per, n_groups);
    int s = 0;
    for (int g = g0; g < g1; ++g) s += group_count[g];
    int total;
    int off = block_exclusive_scan(s, scan_lds, &total);
    for (int g = g0; g < g1; ++g) {
        goff[g] = off;
        off += group_count[g];
    }
    __syncthreads();
    const int n_pad = (total + 31) & ~31;

    if (blockIdx.x == 0) {
        if (tid == 0) *n_out = total;
        for (int c = tid; c < nchunk; c += kThreads) {
            uint32_t bits = mask[c];
            int r = goff[c / kRankGroup] + (bits ? rank8[c] : 0);
            while (bits) {
                const int e = __builtin_ctz(bits);
                bits &= bits - 1;
                idx[r++] = c * 8 + e;
            }
        }
    }

    for (int m = blockIdx.x * 4 + wave; m < M; m += gridDim.x * 4) {
        const uint16_t* xrow = X + (size_t)m * K;
        float amax = 0.0f;
#pragma unroll 4
        for (int c = lane; c < nchunk; c += kWave) {
            v8u16 v = *reinterpret_cast<const v8u16*>(xrow + (size_t)c * 8);
            const uint32_t bits = mask[c];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (!((bits >> e) & 1u)) amax = fmaxf(amax, fabsf(widen16<BF16>(v[e])));
        }
        amax = wave_max(amax);
        if (lane == 0) SCA[m] = amax;
        const float scale = amax == 0.0f ? 0.0f : code_max<FP8>() / amax;
        int8_t* carow = CA + (size_t)m * K;
        uint16_t* xo = XO + (size_t)m * n_pad;
#pragma unroll 4
        for (int c = lane; c < nchunk; c += kWave) {
            v8u16 v = *reinterpret_cast<const v8u16*>(xrow + (size_t)c * 8);
            uint32_t bits = mask[c];
            *reinterpret_cast<uint2*>(carow + (size_t)c * 8) = quantize8<BF16, FP8>(v, bits, scale);
            if (bits) {
                int r = goff[c / kRankGroup] + rank8[c];
                while (bits) {
                    const int e = __builtin_ctz(bits);
                    bits &= bits - 1;
                    xo[r++] = v[e];
                }
            }
        }
        for (int j = total + lane; j < n_pad; j += kWave) xo[j] = 0;
    }
}

__global__ void write_zero_count(int32_t* n_out) { *n_out = 0; }

struct ActPlan {
    bool small;
    int slabs;            // ceil(K / 512)
    int groups;           // G row groups for the partial column max
    int rows_per_group;
    int n_rank_groups;    // ceil(K/8 / 32)
    size_t off_mask, off_rank, off_count, bytes;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

ActPlan plan_act(int64_t M, int64_t K) {
    ActPlan p{};
    p.small = M <= kSmallMaxM && M * K <= kSmallMaxElems;
    const int64_t nchunk = K / 8;
    p.slabs = (int)((nchunk + kWave - 1) / kWave);
    // about 1024 workgroups for kernel A, at least 8 rows per group
    int64_t g = (1024 + p.slabs - 1) / p.slabs;
    int64_t gmax = (M + 7) / 8;
    if (g > gmax) g = gmax;
    if (g < 1) g = 1;
    if (g > 64) g = 64;
    p.rows_per_group = (int)((M + g - 1) / g);
    p.groups = (int)((M + p.rows_per_group - 1) / p.rows_per_group);
    p.n_rank_groups = (int)((nchunk + kRankGroup - 1) / kRankGroup);
    p.off_mask = align256((size_t)p.groups * K * sizeof(float));
    p.off_rank = p.off_mask + align256((size_t)nchunk);
    p.off_count = p.off_rank + align256((size_t)nchunk * sizeof(int32_t));
    p.bytes = p.off_count + align256((size_t)p.n_rank_groups * sizeof(int32_t));
    if (p.small) p.bytes = 0;
    return p;
}

}  // namespace

size_t quantize_act_workspace(int64_t M, int64_t K) {
    if (M <= 0 || K <= 0) return 0;
    return plan_act(M, K).bytes;
}

hipError_t launch_quantize_act(const void* Xv, bool bf16, bool fp8, int M, int K, float t,
                               int8_t* CA, float* SCA, int32_t* idx, int32_t* n_out, void* XOv,
                               void* ws, hipStream_t stream) {
    const uint16_t* X = static_cast<const uint16_t*>(Xv);
    uint16_t* XO = static_cast<uint16_t*>(XOv);
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
    char* base = static_cast<char*>(ws);
    float* partial = reinterpret_cast<float*>(base);
    uint8_t* mask = reinterpret_cast<uint8_t*>(base + p.off_mask);
    int32_t* rank8 = reinterpret_cast<int32_t*>(base + p.off_rank);
    int32_t* gcount = reinterpret_cast<int32_t*>(base + p.off_count);
    dim3 ga(p.slabs, p.groups);
    if (bf16)
        act_colmax_partial<true><<<ga, kThreads, 0, stream>>>(X, M, K, p.rows_per_group, partial);
    else
        act_colmax_partial<false><<<ga, kThreads, 0, stream>>>(X, M, K, p.rows_per_group, partial);
    act_outlier_mask<<<p.n_rank_groups, kThreads, 0, stream>>>(partial, p.groups, K, t, mask,
                                                               rank8, gcount);
    int blocks = (M + 3) / 4;
    if (blocks > 65536) blocks = 65536;
    void (*fn)(const uint16_t*, int, int, const uint8_t*, const int32_t*, const int32_t*, int,
               int8_t*, float*, int32_t*, int32_t*, uint16_t*) =
        bf16 ? (fp8 ? act_quant_rows<true, true> : act_quant_rows<true, false>)
             : (fp8 ? act_quant_rows<false, true> : act_quant_rows<false, false>);
    fn<<<blocks, kThreads, 0, stream>>>(X, M, K, mask, rank8, gcount, p.n_rank_groups, CA, SCA, idx,
                                        n_out, XO);
    return hipGetLastError();
}

}  // namespace llmint8
