// Tiled LLM.int8() product for prefill shapes, bound by MFMA throughput.
//
// "A Gentle Introduction to 8-bit Matrix Multiplication for transformers at
// scale": section "LLM.int8() summary" (non-outliers in int8, outliers in
// 16-bit, dequantize and add), section "inside the MatMul" (row-wise scales
// for the hidden states, per-output-channel scales for the weight), section
// "absmax quantization" (denormalize by the outer product of the two absmax
// vectors), section "Usage" (recovered weight CB * SCB / 127).
//
// Design (gfx950: 256 CUs in 8 XCDs, 160 KiB LDS per CU, 64 LDS banks):
//  * Workgroup tile 256 x 256; 4 waves in a 2 x 2 grid, each wave owns a
//    128 x 128 sub-tile = 4 x 4 blocks of 32 x 32 (256 accumulators per lane,
//    in AGPRs).  One workgroup per CU.  The wave layout is a compile-time
//    choice: 8 waves of 128 x 64 (two per SIMD) measure within 1% of this
//    on most shapes and 12% slower with K split.
//  * K advances in 64-byte stages through a 4-deep ring of LDS buffers
//    (A 256 x 64 + B 256 x 64 bytes each, 128 KiB in all).  Stages are filled
//    by global_load_lds_dwordx4: each wave instruction moves 16 rows x 64 bytes
//    straight from memory into LDS, no registers involved, three stages ahead
//    of the MFMAs.  One barrier per stage.
//  * LDS rows are 64 bytes; 16-byte chunk c of row r sits in slot c ^ ((r>>2)&3),
//    so a 16-lane phase of 16-byte fragment reads (16 consecutive rows, one
//    chunk) touches all 64 banks once.
//  * A lane's operand for a block and stage is 32 bytes: chunks l/32 and
//    2 + l/32 of its row, the same for both operands.  int8: two
//    v_mfma_i32_32x32x32_i8 (the low halves are the stage's first 32 columns,
//    the high halves the second 32).  FP8 (the E4M3 variant; format in
//    common.h): one v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 operands, unit
//    scales), which sees one permutation of the 64 columns on both sides.
//  * The A blocks are refilled with the next stage right after their last use
//    in the current one; the B blocks (used by every MFMA of a stage) have a
//    second register set filled early in the stage.  Loads, reads and MFMAs
//    are interleaved in a fixed order (sched_barrier), and the loop has no
//    branches: stages run in groups of four with constant ring slots, and
//    loads past K are clamped.
//  * Tile order: blocks are dispatched round-robin over the 8 XCDs; block b is
//    remapped so that each XCD walks a contiguous range of a grouped raster
//    (8 tile rows per group) and its tiles share CA/CB panels in its own L2.
//  * Epilogue, fused: accumulators -> fp32 times SCA[m]/127 (FP8: /448); the
//    outlier columns (n_out read from device memory, no host sync) run as
//    v_mfma_f32_32x32x16_{f16,bf16} of XO against the codes of the weights
//    at idx (int8 values and E4M3 values are exact in 16-bit), into the same
//    accumulators; then times SCB[n]/127 (/448), plus bias, rounded to
//    16-bit, staged in LDS and written with full 16-byte row-contiguous
//    stores.  The tile's scales, bias and the weight codes of its first 16
//    outlier columns are loaded once, with the prologue's stage loads, and
//    kept in LDS.
//  * Few tiles (at most half the CUs, e.g. M = 512 against a 57344-long K):
//    given a workspace, K is split over up to 8 workgroups per tile.  Each
//    stores its int32 (FP8: fp32) accumulators there and counts itself in
//    with an atomic; the last to arrive adds the partial sums in split order
//    (the same result whichever arrives last; exact for int8) and runs the
//    epilogue.  The counters are zeroed by a kernel ahead of the GEMM.
//  * More than 16 outlier columns: given a workspace, a gather kernel first
//    writes the weight codes at the outlier columns, as 16-bit values, in
//    1 KiB blocks of 32 rows x 16 columns, so that the epilogue reads each
//    MFMA operand with one 16-byte load per lane instead of eight byte
//    gathers from rows K bytes apart.  Without one (or past its capacity)
//    the epilogue gathers the bytes itself.
#include "common.h"

namespace llmint8 {

namespace {

constexpr int BM = 256, BN = 256;
constexpr int BKS = 128;  // K bytes per stage: one whole 128-byte line of every row
constexpr int kStages = 2;
constexpr int kStageBytes = (BM + BN) * BKS;  // 64 KiB
constexpr int kWavesN = 2;                  // waves along N (2 along M)
constexpr int kWaves = 2 * kWavesN;
constexpr int kThreads = 64 * kWaves;
constexpr int JB = 8 / kWavesN;             // 32-column blocks per wave
constexpr int kWaveN = 32 * JB;             // columns per wave
constexpr int kDmaInst = BM / kWaves / 8;   // stage-load instructions (8 rows each) per operand and wave
constexpr int kGroupM = 4;
constexpr int kOutLds = 16;  // outlier columns whose weight codes are staged in LDS
constexpr int kGatherThreads = 256;
constexpr int kCUs = 256;             // compute units of the device (gfx950)
constexpr int kMaxSplit = 8;          // workgroups per tile when K is split
constexpr int kMinSplitStages = 8;    // K stages (128 bytes) per split, at least
static_assert(kOutLds == kGatherFirst, "the gathered codes start where the LDS ones end");
constexpr int kYStride = BN * 2 + 16;  // bytes per staged Y row (padding shifts banks)
constexpr int kSmemBytes =
    kStages * kStageBytes > BM * kYStride ? kStages * kStageBytes : BM * kYStride;

__device__ __forceinline__ void map_tile(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int total = tiles_m * tiles_n;
    int L = bid;
    if ((total & 7) == 0) L = (bid & 7) * (total >> 3) + (bid >> 3);
    const int per_group = kGroupM * tiles_n;
    const int group = L / per_group;
    const int first_m = group * kGroupM;
    const int gsz = min(tiles_m - first_m, kGroupM);
    const int in_group = L - group * per_group;
    tm = first_m + in_group % gsz;
    tn = in_group / gsz;
}

template <bool BF16>
struct Vec16;
template <>
struct Vec16<false> {
    typedef v8h type;
};
template <>
struct Vec16<true> {
    typedef v8bf type;
};

template <bool BF16>
__device__ __forceinline__ v16f mfma16(typename Vec16<BF16>::type a, typename Vec16<BF16>::type b,
                                       v16f c) {
    if constexpr (BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

template <bool FP8>
struct TileAcc {
    typedef v16i type;
};
template <>
struct TileAcc<true> {
    typedef v16f type;
};
template <bool FP8>
struct Part4 {
    typedef v4i type;
};
template <>
struct Part4<true> {
    typedef v4f type;
};

// Two fp32 values -> packed 16-bit pair (a in the low half), each rounded to
// nearest even: one v_cvt_pk_{f16,bf16}_f32.
template <bool BF16>
__device__ __forceinline__ uint32_t pack16x2(float a, float b) {
    if constexpr (BF16) {
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        const bf16x2_t v = {(__bf16)a, (__bf16)b};
        return __builtin_bit_cast(uint32_t, v);
    } else {
        typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
        const f16x2_t v = {(_Float16)a, (_Float16)b};
        return __builtin_bit_cast(uint32_t, v);
    }
}

__device__ __forceinline__ v8i cat8(v4i lo, v4i hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

}  // namespace

// Ahead of the GEMM: workgroup 0 zeroes the split-K arrival counters (if
// any), and the weight codes at outlier columns kOutLds and on are gathered
// for the epilogue (layout with gathered_block) when the activation kernel
// has not written them (wo_all != nullptr).
template <bool BF16, bool FP8>
__global__ __launch_bounds__(kGatherThreads) void gemm_prep(
    int N, int K, int cap, const int32_t* __restrict__ idx, const int32_t* __restrict__ n_out_ptr,
    const int8_t* __restrict__ CB, uint16_t* __restrict__ wo_all, uint32_t* __restrict__ counters,
    int n_counters) {
    if (blockIdx.x == 0)
        for (int t = threadIdx.x; t < n_counters; t += kGatherThreads) counters[t] = 0;
    if (wo_all == nullptr) return;
    const int n_out = *n_out_ptr;
    if (n_out <= kOutLds || n_out > cap) return;  // the epilogue does not read it
    gather_code_blocks<BF16, FP8>(N, K, cap, n_out, [&](int c) { return idx[c]; }, CB, wo_all,
                                  blockIdx.x, gridDim.x);
}

template <bool BF16, bool FP8, bool SPLIT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void gemm_tiled_kernel(int M, int N, int K, int tiles_m, int tiles_n,
                       const int8_t* __restrict__ CA, const float* __restrict__ SCA,
                       const int32_t* __restrict__ idx, const int32_t* __restrict__ n_out_ptr,
                       const uint16_t* __restrict__ XO, const int8_t* __restrict__ CB,
                       const float* __restrict__ SCB, const uint16_t* __restrict__ bias,
                       uint16_t* __restrict__ Y, int32_t* __restrict__ C_i32,
                       float* __restrict__ C_f32, const uint16_t* __restrict__ wo_all,
                       int wo_cap, int split, uint32_t* __restrict__ counters,
                       int32_t* __restrict__ part) {
    __shared__ __attribute__((aligned(16))) int8_t smem[kSmemBytes];
    __shared__ float s_sa[BM], s_sb[BN], s_bias[BN];
    // weight codes of the tile's rows at the first kOutLds outlier columns, as
    // 16-bit values (0 past n_out): row r, column e at s_wo[r * kOutLds + e]
    __shared__ __attribute__((aligned(16))) uint16_t s_wo[BN * kOutLds];
    // the tile's rows of XO at the first kOutLds outlier columns: row r at
    // s_xo[r * kOutLds] (0 past n_out: XO's padding)
    __shared__ __attribute__((aligned(16))) uint16_t s_xo[BM * kOutLds];

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / kWavesN, wn = wave % kWavesN;
    // SPLIT: workgroup b takes split ks = b % split of tile b / split, K
    // stages [ks nk / split, (ks + 1) nk / split); otherwise split is 1
    if constexpr (!SPLIT) split = 1;
    const int tile = blockIdx.x / split, ks = blockIdx.x - tile * split;
    int tm, tn;
    map_tile(tile, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    // K runs in 128-byte stages; a K that is an odd multiple of 64 ends in a
    // half stage, of which only the first 64-byte unit is computed.
    const int nk_all = (K + BKS - 1) / BKS;
    const int kt_begin = ks * nk_all / split, nk = (ks + 1) * nk_all / split - kt_begin;
    const bool half_last = (K % BKS) != 0 && ks == split - 1;

    // ---- stage loads: buffer_load_dwordx4 ... lds, one instruction = 8 rows x
    // 128 bytes, whole lines.  Wave w fills rows [64w, 64w + 64) of A and of
    // B, instruction i rows 64w + 8i + lane/8; lane p lands in slot p%8 of its
    // row and so fetches the logical 16-byte chunk (p%8) ^ ((row/2) % 8).  Each
    // operand is addressed through a descriptor based at the tile's first row
    // and holding exactly its valid rows: rows past M (N) re-read the last
    // valid row (their results are never stored), and the unused half of a
    // half stage reads 0 past the last row instead of leaving the matrix.
    const int rows_a = min(BM, M - m0), rows_b = min(BN, N - n0);
    const v4i rsrc_a = buffer_rsrc(CA + (size_t)m0 * K, (uint32_t)rows_a * (uint32_t)K);
    const v4i rsrc_b = buffer_rsrc(CB + (size_t)n0 * K, (uint32_t)rows_b * (uint32_t)K);
    uint32_t voff_a[kDmaInst], voff_b[kDmaInst];
#pragma unroll
    for (int i = 0; i < kDmaInst; ++i) {
        const int r = 8 * kDmaInst * wave + 8 * i + (lane >> 3);
        const int ch = ((lane & 7) ^ ((4 * i + (lane >> 4)) & 7)) * 16;
        voff_a[i] = (uint32_t)min(r, rows_a - 1) * (uint32_t)K + (uint32_t)kt_begin * BKS + ch;
        voff_b[i] = (uint32_t)min(r, rows_b - 1) * (uint32_t)K + (uint32_t)kt_begin * BKS + ch;
    }
    const uint32_t lds_base =
        __builtin_amdgcn_readfirstlane(lds_address(smem) + 8 * kDmaInst * wave * BKS);  // this wave's rows
    // stage-load instruction d (A rows for d < kDmaInst, then B rows) of stage
    // kt (relative to kt_begin) into ring buffer u
    auto dma = [&](int d, int kt, int u) {
        const uint32_t kd = (uint32_t)kt * BKS;
        if (d < kDmaInst)
            dma_line(rsrc_a, voff_a[d] + kd, lds_base + u * kStageBytes + 8 * d * BKS);
        else
            dma_line(rsrc_b, voff_b[d - kDmaInst] + kd,
                     lds_base + u * kStageBytes + BM * BKS + 8 * (d - kDmaInst) * BKS);
    };
    auto issue = [&](int kt, int u) {
#pragma unroll
        for (int d = 0; d < 2 * kDmaInst; ++d) dma(d, kt, u);
    };

    // ---- fragments: lane l reads row (l & 31) of each 32-row block.  In
    // 64-byte unit h of a stage, its 32 bytes are the logical chunks
    // 4h + l/32 and 4h + 2 + l/32 (the same for A and B), at LDS slot
    // chunk ^ ((row/2) % 8): each 16-lane phase of a read (16 rows, one chunk)
    // touches all 64 banks once.  Fragment f < 4 is A block f, f >= 4 is B
    // block f - 4.
    const int rr = lane & 31;
    const int a_off = wm * 128 * BKS, b_off = BM * BKS + wn * kWaveN * BKS;
    auto read_frag = [&](int u, int h, int e, int f) -> v4i {
        const int slot = ((4 * h + 2 * e + (lane >> 5)) ^ ((rr >> 1) & 7)) * 16;
        const int off = u * kStageBytes + slot + (f < 4 ? a_off + 32 * f * BKS : b_off + 32 * (f - 4) * BKS);
        return lds_load<v4i>(smem, (uint32_t)(rr * BKS + off));
    };

    typedef typename TileAcc<FP8>::type acc_t;
    acc_t acc[4][JB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < JB; ++j) acc[i][j] = acc_t{};

    // epilogue operands, fetched now so their latency hides under the K loop
    const int n_out = *n_out_ptr;
    // The row and column scales, bias and outlier weight codes go to LDS
    // after the prologue's wait: their loads are issued with its stage loads,
    // so their latency hides under them.  Every load is unconditional, from a
    // clamped address (a load under a branch is awaited where the branch
    // rejoins).  Outlier gather: lane column e = tid % 16, rows tid/16 + 16 q;
    // lanes past n_out read column 0 (discarded).
    const int t8 = kThreads > 256 ? (tid & 255) : tid;  // threads 256 and on repeat 0..255
    float sa_raw = SCA[min(m0 + t8, M - 1)];
    const int n_sb = min(n0 + t8, N - 1);
    float sb_raw = SCB[n_sb];
    uint16_t bias_raw = *(bias ? bias + n_sb : XO);  // XO: any readable element
    const int e_out = tid & (kOutLds - 1);
    const bool e_valid = e_out < n_out;
    int e_col = 0;
#pragma unroll
    for (int u = 0; u < kOutLds; ++u) {  // uniform reads; idx holds K >= 64 entries
        int c = idx[u];
        asm volatile("" : "+s"(c));  // all sixteen read, then selected without branches
        e_col = u == e_out ? c : e_col;
    }
    if (!e_valid) e_col = 0;

    // The prologue loads stages 0 and 1; from then on, stage kt loads stage
    // kt + 2 into the buffer it has just finished with, clamped to the last
    // stage (past K they re-read it into a buffer no wave reads again), so
    // every stage runs the same branch-free code.  All loads are awaited
    // before the epilogue reuses the ring.
    issue(0, 0);
    constexpr int kWoPasses = BN * kOutLds / kThreads;  // rows tid/16 + (kThreads/16) q
    int32_t wo_raw[kWoPasses];
#pragma unroll
    for (int q = 0; q < kWoPasses; ++q)
        wo_raw[q] = CB[(size_t)min(n0 + (tid >> 4) + (kThreads / 16) * q, N - 1) * K + e_col];
    // XO's first kOutLds columns of tile row t8 (in bounds for n_pad = 0 too:
    // XO holds M * K >= 64 elements)
    const int n_pad0 = (n_out + 31) & ~31;
    const v4i* xo_src = reinterpret_cast<const v4i*>(XO + (size_t)min(m0 + t8, M - 1) * n_pad0);
    v4i xo_raw0 = xo_src[0], xo_raw1 = xo_src[1];
    issue(min(1, nk - 1), 1);
    wait_vmcnt<2 * kDmaInst>();  // stage 0 and everything issued before stage 1
    stage_barrier();

    // Fragment f of a unit is 32 bytes per lane.  FP8: one
    // v_mfma_scale_f32_32x32x64_f8f6f4 per block and unit (the instruction
    // sees one permutation of the 64 columns on both sides).  int8: two
    // v_mfma_i32_32x32x32_i8, on the low halves (the unit's chunks 0, 1) and
    // on the high halves (chunks 2, 3).
    auto mma = [&](const v8i& b, const v8i& a, acc_t c) -> acc_t {
        if constexpr (FP8) {
            return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, 0, 0, 0, 127, 0, 127);
        } else {
            c = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_shufflevector(b, b, 0, 1, 2, 3),
                                                       __builtin_shufflevector(a, a, 0, 1, 2, 3), c, 0, 0, 0);
            return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_shufflevector(b, b, 4, 5, 6, 7),
                                                          __builtin_shufflevector(a, a, 4, 5, 6, 7), c, 0, 0, 0);
        }
    };
    auto read_frag8 = [&](int u, int h, int f) -> v8i {
        return cat8(read_frag(u, h, 0, f), read_frag(u, h, 1, f));
    };
    // Unit pipeline: MFMA q of a unit is block (i, j) = (q/JB, q%JB).  A block
    // i is refilled with the next unit in place right after its last use (MFMA
    // JB i + JB-1); the B blocks, used until the unit's last MFMAs, have a
    // second register set (gb1 holds unit 1 of every stage, gb0 unit 0).
    v8i ga[4], gb0[JB], gb1[JB];
#pragma unroll
    for (int f = 0; f < 4; ++f) ga[f] = read_frag8(0, 0, f);
#pragma unroll
    for (int f = 0; f < JB; ++f) gb0[f] = read_frag8(0, 0, 4 + f);
    // Stage kt in ring buffer u (a compile-time constant: stages run in pairs).
    // Unit 0 reads unit 1 of the same buffer.  Two MFMA blocks into unit 1,
    // every wave waits for its loads of stage kt+1 and for its reads of this
    // buffer, and meets the others at the barrier: stage kt+1 has landed in
    // buffer 1-u, and no wave reads buffer u again.  The rest of unit 1 reads
    // unit 0 of stage kt+1 and spreads the loads of stage kt+2 into buffer u
    // over its MFMAs, so each load has a whole stage to land.
    constexpr int kBarrierAt = 2;
    auto stage = [&](int kt, int u) {
#pragma unroll
        for (int q = 0; q < 4 * JB; ++q) {
            const int i = q / JB, j = q % JB;
            acc[i][j] = mma(gb0[j], ga[i], acc[i][j]);
            if (q < JB) gb1[q] = read_frag8(u, 1, 4 + q);
            if (j == JB - 1) ga[i] = read_frag8(u, 1, i);
            __builtin_amdgcn_sched_barrier(0);
        }
        const int kn = min(kt + 2, nk - 1);
#pragma unroll
        for (int q = 0; q < 4 * JB; ++q) {
            const int i = q / JB, j = q % JB;
            acc[i][j] = mma(gb1[j], ga[i], acc[i][j]);
            if (q == kBarrierAt - 1) {
                __builtin_amdgcn_s_waitcnt(0);  // vmcnt, expcnt and lgkmcnt all zero
                stage_barrier();
            }
            if (q >= kBarrierAt) {
                // (at the last stage these read a stale buffer; unused)
                if (q - kBarrierAt < JB) gb0[q - kBarrierAt] = read_frag8(1 - u, 0, 4 + q - kBarrierAt);
                if (j == JB - 1) ga[i] = read_frag8(1 - u, 0, i);
                // loads d0 .. d1-1 of the 2 kDmaInst go out with MFMA q
                constexpr int kSlots = 4 * JB - kBarrierAt;
                const int d0 = (q - kBarrierAt) * 2 * kDmaInst / kSlots;
                const int d1 = (q - kBarrierAt + 1) * 2 * kDmaInst / kSlots;
#pragma unroll
                for (int d = d0; d < d1; ++d) dma(d, kn, u);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // The last stage of a K that is an odd multiple of 64: unit 0 only, in a
    // buffer known at run time.
    auto half_stage = [&]() {
#pragma unroll
        for (int q = 0; q < 4 * JB; ++q) {
            const int i = q / JB, j = q % JB;
            acc[i][j] = mma(gb0[j], ga[i], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    const int nfull = half_last ? nk - 1 : nk;
    int kt = 0;
    for (; kt + 2 <= nfull; kt += 2) {
        stage(kt, 0);
        stage(kt + 1, 1);
    }
    if (kt < nfull) {
        stage(kt, 0);
        ++kt;
    }
    if (half_last) half_stage();
    wait_vmcnt<0>();  // the clamped loads past K have landed too

    // The epilogue operands loaded in the prologue go to LDS only now: a use
    // there would make the compiler wait for every load in flight, the second
    // stage's included (it cannot see the stage loads).  The values are pinned
    // until here so that their conversions are not hoisted either.
    asm volatile("" : "+v"(sa_raw), "+v"(sb_raw), "+v"(bias_raw), "+v"(xo_raw0), "+v"(xo_raw1));
#pragma unroll
    for (int q = 0; q < kWoPasses; ++q) asm volatile("" : "+v"(wo_raw[q]));
    if (kThreads == 256 || tid < 256) {
        s_sa[tid] = sa_raw;
        s_sb[tid] = sb_raw / code_max<FP8>();
        s_bias[tid] = bias ? widen16<BF16>(bias_raw) : 0.0f;
        *reinterpret_cast<v4i*>(s_xo + tid * kOutLds) = xo_raw0;
        *reinterpret_cast<v4i*>(s_xo + tid * kOutLds + 8) = xo_raw1;
    }
    {
        const uint32_t e_mask = e_valid ? 0xFFFFu : 0u;  // a mask, not a select: no branches
#pragma unroll
        for (int q = 0; q < kWoPasses; ++q)
            s_wo[((tid >> 4) + (kThreads / 16) * q) * kOutLds + e_out] =
                (uint16_t)(narrow16<BF16>(code_value<FP8>((int8_t)wo_raw[q])) & e_mask);
    }

    // ---- split K: the partial sums meet in the workspace ---------------------
    // Stored in register order: 16 bytes (registers 4c..4c+3 of a block) per
    // lane, a wave's 64 lanes contiguous, so every access is a full 1 KiB.
    if constexpr (SPLIT) {
        __shared__ int s_last;
        constexpr int kWaveWords = 4 * JB * 16 * 64;  // blocks x 16 registers x 64 lanes
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < JB; ++j)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    // whole vectors through bit casts (a bit cast of one vector
                    // element reads element 0)
                    const v16i bits = __builtin_bit_cast(v16i, acc[i][j]);
                    const v4i w = {bits[4 * c], bits[4 * c + 1], bits[4 * c + 2], bits[4 * c + 3]};
                    *reinterpret_cast<v4i*>(part + (((size_t)tile * split + ks) * kWaves + wave) * kWaveWords +
                                            ((i * JB + j) * 4 + c) * 256 + lane * 4) = w;
                }
        __threadfence();  // the stores are visible device-wide before the count
        __syncthreads();
        if (tid == 0) s_last = atomicAdd(counters + tile, 1u) == (unsigned)(split - 1);
        __syncthreads();
        if (!s_last) return;  // another workgroup finishes this tile
        __threadfence();
        // sum in split order, this workgroup's own part read back too (the
        // same result whichever workgroup arrives last)
        const int32_t* p0 = part + (size_t)tile * split * (kWaves * kWaveWords) + wave * kWaveWords + lane * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < JB; ++j) {
                acc_t t;
#pragma unroll
                for (int sp = 0; sp < kMaxSplit; ++sp) {
                    if (sp < split) {
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const auto x = __builtin_bit_cast(typename Part4<FP8>::type,
                                                              *reinterpret_cast<const v4i*>(
                                                                  p0 + (size_t)sp * (kWaves * kWaveWords) +
                                                                  ((i * JB + j) * 4 + c) * 256));
#pragma unroll
                            for (int e = 0; e < 4; ++e) t[4 * c + e] = sp == 0 ? x[e] : t[4 * c + e] + x[e];
                        }
                    }
                }
                acc[i][j] = t;
            }
    }

    // ---- epilogue ----------------------------------------------------------
    // Block (i, j) is held transposed: register v of lane l is row
    // m = 32 i + l%32 and column n = 32 j + 8 (v/4) + 4 (l/32) + v%4 of the
    // wave's sub-tile, so four consecutive registers are four consecutive
    // columns of one output row.  One 32-row block at a time: dequantize, add
    // the outlier product, scale, bias, round, and stage 8-byte pieces in LDS.
    __syncthreads();  // every wave is done reading the stage buffers
    // the lane index again, from v_mbcnt (opaque, so that it is not kept in a
    // register across the K loop)
    int lane_e;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane_e));
    const int kh = lane_e >> 5, rr_e = lane_e & 31, tid_e = wave * 64 + lane_e;
    const int m_lane = wm * 128 + rr_e;              // + 32 i
    const int n_lane = wn * kWaveN + 4 * kh;       // + 32 j + 8 (v/4) + v%4
    uint16_t* ys = reinterpret_cast<uint16_t*>(smem);
    typedef typename Vec16<BF16>::type vec_t;
    const int n_pad = (n_out + 31) & ~31;
    // this lane's row of block column 0 in the gathered codes, per j (rows of
    // blocks past N clamp to the last block: their results are not stored)
    const bool gathered = wo_all != nullptr && n_out <= wo_cap;
    const uint16_t* wo_blocks[JB] = {};
    if (gathered) {
        const int row_blocks = (N + 31) / 32;
#pragma unroll
        for (int j = 0; j < JB; ++j)
            wo_blocks[j] = wo_all + gathered_block(min((n0 + wn * kWaveN + 32 * j) / 32, row_blocks - 1), 0, wo_cap) +
                           rr_e * 16 + 8 * kh;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + m_lane + 32 * i;
        if (FP8 ? C_f32 != nullptr : C_i32 != nullptr) {
#pragma unroll
            for (int j = 0; j < JB; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int n = n0 + n_lane + 32 * j + 8 * (v >> 2) + (v & 3);
                    if (m < M && n < N) {
                        if constexpr (FP8) C_f32[(size_t)m * N + n] = acc[i][j][v];
                        else C_i32[(size_t)m * N + n] = acc[i][j][v];
                    }
                }
        }
        // outlier k-block 0: the row's XO values, staged in LDS
        const bool have_out = n_out > 0;
        const v8u16 xraw = *reinterpret_cast<const v8u16*>(s_xo + (m_lane + 32 * i) * kOutLds + 8 * kh);
        const float sa = s_sa[m_lane + 32 * i] / code_max<FP8>();
        v16f f[JB];
#pragma unroll
        for (int j = 0; j < JB; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) f[j][v] = (float)acc[i][j][v] * sa;

        if (have_out) {
            // XO rows as the B operand (transposed product); int8 codes and
            // E4M3 values are exact in fp16 and bf16
            const vec_t xa = __builtin_bit_cast(vec_t, xraw);
#pragma unroll
            for (int j = 0; j < JB; ++j) {
                const v8u16 raw = *reinterpret_cast<const v8u16*>(
                    s_wo + (wn * kWaveN + 32 * j + rr_e) * kOutLds + 8 * kh);
                f[j] = mfma16<BF16>(__builtin_bit_cast(vec_t, raw), xa, f[j]);
            }
        }
        // further outlier k-blocks (more than 16 outlier columns)
        if (gathered) {
            // the codes gathered beforehand: block (row block, j0 / 16), row l % 32,
            // columns 8 kh .. 8 kh + 7.  Four k-blocks per round, all their
            // loads issued first (one wave per SIMD: the latency of one round
            // of loads is not hidden by anything else); blocks past n_out
            // re-read the last one and skip their MFMAs.
            const int j_last = (n_out - 1) & ~15;
            const uint16_t* xo_row = XO + (size_t)min(m, M - 1) * n_pad + 8 * kh;
            for (int j0 = kOutLds; j0 < n_out; j0 += 64) {
                v8u16 xraw4[4], raw[4][JB];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int jb = min(j0 + 16 * u, j_last);
                    xraw4[u] = *reinterpret_cast<const v8u16*>(xo_row + jb);
#pragma unroll
                    for (int j = 0; j < JB; ++j)
                        raw[u][j] = *reinterpret_cast<const v8u16*>(wo_blocks[j] + 32 * jb);
                }
                // every load is issued before the first wait (the compiler
                // would otherwise sink each one into the branch that uses it)
                if constexpr (JB == 4)
                    asm volatile(""
                                 : "+v"(xraw4[0]), "+v"(xraw4[1]), "+v"(xraw4[2]), "+v"(xraw4[3]),
                                   "+v"(raw[0][0]), "+v"(raw[0][1]), "+v"(raw[0][2]), "+v"(raw[0][3]),
                                   "+v"(raw[1][0]), "+v"(raw[1][1]), "+v"(raw[1][2]), "+v"(raw[1][3]),
                                   "+v"(raw[2][0]), "+v"(raw[2][1]), "+v"(raw[2][2]), "+v"(raw[2][3]),
                                   "+v"(raw[3][0]), "+v"(raw[3][1]), "+v"(raw[3][2]), "+v"(raw[3][3]));
                else
                    asm volatile(""
                                 : "+v"(xraw4[0]), "+v"(xraw4[1]), "+v"(xraw4[2]), "+v"(xraw4[3]),
                                   "+v"(raw[0][0]), "+v"(raw[0][1]), "+v"(raw[1][0]), "+v"(raw[1][1]),
                                   "+v"(raw[2][0]), "+v"(raw[2][1]), "+v"(raw[3][0]), "+v"(raw[3][1]));
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (j0 + 16 * u < n_out) {
                        const vec_t xa = __builtin_bit_cast(vec_t, xraw4[u]);
#pragma unroll
                        for (int j = 0; j < JB; ++j)
                            f[j] = mfma16<BF16>(__builtin_bit_cast(vec_t, raw[u][j]), xa, f[j]);
                    }
                }
            }
        } else {
            for (int j0 = kOutLds; j0 < n_out; j0 += 16) {
                const vec_t xa = __builtin_bit_cast(
                    vec_t, *reinterpret_cast<const v8u16*>(XO + (size_t)min(m, M - 1) * n_pad + j0 + 8 * kh));
                // The block's 16 columns are read as uniform (scalar) values;
                // lanes with kh = 1 take the second 8.  Adjacent columns from a
                // multiple of 8 on (every block when t = 0 makes every column
                // an outlier) are one 8-byte load per row; otherwise one byte
                // load each, columns past n_out reading the last outlier
                // column (no branch around a load) and masked to 0.
                const int first = idx[j0], last = idx[min(j0 + 15, n_out - 1)];
                int b[JB][8];
                uint32_t keep = 0xffu;
                if (j0 + 16 <= n_out && last - first == 15 && (first & 7) == 0) {
#pragma unroll
                    for (int j = 0; j < JB; ++j) {
                        const int8_t* cb = CB + (size_t)min(n0 + wn * kWaveN + 32 * j + rr_e, N - 1) * K;
                        const uint2 w8 = *reinterpret_cast<const uint2*>(cb + first + 8 * kh);
#pragma unroll
                        for (int e = 0; e < 8; ++e) b[j][e] = (int)((e < 4 ? w8.x : w8.y) >> (8 * (e & 3)));
                    }
                } else {
                    int kcol[8];
                    keep = 0;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        int c0 = idx[min(j0 + e, n_out - 1)], c1 = idx[min(j0 + 8 + e, n_out - 1)];
                        asm volatile("" : "+s"(c0), "+s"(c1));
                        kcol[e] = kh ? c1 : c0;
                        keep |= (j0 + 8 * kh + e < n_out ? 1u : 0u) << e;
                    }
#pragma unroll
                    for (int j = 0; j < JB; ++j) {
                        const int8_t* cb = CB + (size_t)min(n0 + wn * kWaveN + 32 * j + rr_e, N - 1) * K;
#pragma unroll
                        for (int e = 0; e < 8; ++e) b[j][e] = cb[kcol[e]];
                    }
                    // all 32 byte loads in flight before the first wait
#pragma unroll
                    for (int j = 0; j < JB; j += 2)
                        asm volatile(""
                                     : "+v"(b[j][0]), "+v"(b[j][1]), "+v"(b[j][2]), "+v"(b[j][3]),
                                       "+v"(b[j][4]), "+v"(b[j][5]), "+v"(b[j][6]), "+v"(b[j][7]),
                                       "+v"(b[j + 1][0]), "+v"(b[j + 1][1]), "+v"(b[j + 1][2]),
                                       "+v"(b[j + 1][3]), "+v"(b[j + 1][4]), "+v"(b[j + 1][5]),
                                       "+v"(b[j + 1][6]), "+v"(b[j + 1][7]));
                }
#pragma unroll
                for (int j = 0; j < JB; ++j) {
                    v8u16 raw;
#pragma unroll
                    for (int e = 0; e < 8; ++e)  // exact in fp16 and bf16
                        raw[e] = (uint16_t)(narrow16<BF16>(code_value<FP8>((int8_t)b[j][e])) &
                                            (0u - ((keep >> e) & 1u)));
                    f[j] = mfma16<BF16>(__builtin_bit_cast(vec_t, raw), xa, f[j]);
                }
            }
        }

#pragma unroll
        for (int j = 0; j < JB; ++j)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int nl = n_lane + 32 * j + 8 * a4;
                float y[4];
#pragma unroll
                for (int b = 0; b < 4; ++b) y[b] = f[j][4 * a4 + b] * s_sb[nl + b] + s_bias[nl + b];
                *reinterpret_cast<uint2*>(ys + (m_lane + 32 * i) * (kYStride / 2) + nl) =
                    make_uint2(pack16x2<BF16>(y[0], y[1]), pack16x2<BF16>(y[2], y[3]));
            }
    }
    __syncthreads();
    const int rows = min(BM, M - m0), cols = min(BN, N - n0);
    if ((N & 7) == 0) {
        // 32 lanes per 512-byte row, 8 rows per pass of the workgroup
        const int c8 = (tid_e & 31) * 8;
        for (int r = tid_e >> 5; r < rows; r += kThreads / 32) {
            if (c8 < cols)
                *reinterpret_cast<v4i*>(Y + (size_t)(m0 + r) * N + n0 + c8) =
                    *reinterpret_cast<const v4i*>(smem + r * kYStride + c8 * 2);
        }
    } else {
        for (int e = tid_e; e < rows * BN; e += kThreads) {
            const int r = e / BN, c = e - r * BN;
            if (c < cols) Y[(size_t)(m0 + r) * N + n0 + c] = ys[r * (kYStride / 2) + c];
        }
    }
}

// Bytes of gathered outlier codes for an N x K weight holding `cap` outlier
// columns (a multiple of 32).
static size_t gathered_codes_bytes(int64_t N, int64_t cap) { return (size_t)((N + 31) / 32) * 64 * cap; }

// Workgroups per tile: split K when the tiles fill at most half the CUs, into
// as many parts as keep one workgroup per CU, each at least kMinSplitStages
// stages long.
static int split_of(int64_t M, int64_t N, int64_t K) {
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    if (tiles * 2 > kCUs) return 1;
    int64_t s = kCUs / tiles;
    if (s > K / BKS / kMinSplitStages) s = K / BKS / kMinSplitStages;
    if (s > kMaxSplit) s = kMaxSplit;
    return s < 1 ? 1 : (int)s;
}

// arrival counters (padded to 256 bytes), then split x tiles partial tiles
static size_t split_bytes(int64_t M, int64_t N, int64_t K) {
    const int split = split_of(M, N, K);
    if (split <= 1) return 0;
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    return (((size_t)tiles * 4 + 255) & ~(size_t)255) + (size_t)split * tiles * BM * BN * 4;
}

size_t gemm_tiled_workspace(int64_t M, int64_t N, int64_t K) {
    size_t b = split_bytes(M, N, K);
    if (N > 0 && K > kOutLds) {
        const int64_t k32 = (K + 31) & ~(int64_t)31;
        b += gathered_codes_bytes(N, k32 < kActGatherCols ? k32 : kActGatherCols);
    }
    return b;
}

// The split region first, when the workspace holds it; the gathered codes
// take the rest: as many multiples of 32 columns as fit, at most K rounded up.
TiledLayout tiled_layout(int M, int N, int K, void* ws, size_t ws_bytes) {
    TiledLayout L;
    if (ws == nullptr || M <= 0 || N <= 0) return L;
    char* p = static_cast<char*>(ws);
    const size_t sb = split_bytes(M, N, K);
    if (sb > 0 && ws_bytes >= sb) {
        const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
        L.split = split_of(M, N, K);
        L.counters = reinterpret_cast<uint32_t*>(p);
        L.n_counters = tiles;
        L.part = reinterpret_cast<int32_t*>(p + (((size_t)tiles * 4 + 255) & ~(size_t)255));
        p += sb;
        ws_bytes -= sb;
    }
    if (K > kOutLds) {
        const size_t fit = ws_bytes / gathered_codes_bytes(N, 32), k_blocks = (size_t)((K + 31) & ~31) / 32;
        L.cap = (int)(fit < k_blocks ? fit : k_blocks) * 32;
        if (L.cap > 0) L.codes = reinterpret_cast<uint16_t*>(p);
    }
    return L;
}

hipError_t launch_gemm_tiled(const MatmulArgs& a, hipStream_t stream, hipEvent_t ev_start,
                             hipEvent_t ev_stop) {
    const int tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
    const TiledLayout L = tiled_layout(a.M, a.N, a.K, a.ws, a.ws_bytes);
    uint16_t* gather_to = a.codes_gathered ? nullptr : L.codes;
    if (gather_to != nullptr || L.split > 1) {
        void (*g)(int, int, int, const int32_t*, const int32_t*, const int8_t*, uint16_t*, uint32_t*, int) =
            a.bf16 ? (a.fp8 ? gemm_prep<true, true> : gemm_prep<true, false>)
                   : (a.fp8 ? gemm_prep<false, true> : gemm_prep<false, false>);
        const int row_blocks = (a.N + 31) / 32;
        const int blocks = gather_to == nullptr ? 1 : row_blocks < 512 ? row_blocks : 512;
        g<<<blocks, kGatherThreads, 0, stream>>>(a.N, a.K, L.cap, a.idx, a.n_out, a.CB, gather_to,
                                                 L.counters, L.split > 1 ? L.n_counters : 0);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    dim3 grid(tiles_m * tiles_n * L.split), block(kThreads);
    typedef void (*kernel_t)(int, int, int, int, int, const int8_t*, const float*, const int32_t*,
                             const int32_t*, const uint16_t*, const int8_t*, const float*,
                             const uint16_t*, uint16_t*, int32_t*, float*, const uint16_t*, int, int,
                             uint32_t*, int32_t*);
    const kernel_t fn =
        L.split > 1
            ? (a.bf16 ? (a.fp8 ? gemm_tiled_kernel<true, true, true> : gemm_tiled_kernel<true, false, true>)
                      : (a.fp8 ? gemm_tiled_kernel<false, true, true> : gemm_tiled_kernel<false, false, true>))
            : (a.bf16 ? (a.fp8 ? gemm_tiled_kernel<true, true, false> : gemm_tiled_kernel<true, false, false>)
                      : (a.fp8 ? gemm_tiled_kernel<false, true, false> : gemm_tiled_kernel<false, false, false>));
    if (ev_start || ev_stop) {
        hipExtLaunchKernelGGL(fn, grid, block, 0, stream, ev_start, ev_stop, 0, a.M, a.N, a.K,
                              tiles_m, tiles_n, a.CA, a.SCA, a.idx, a.n_out, a.XO, a.CB, a.SCB,
                              a.bias, a.Y, a.C_i32, a.C_f32, L.codes, L.cap, L.split, L.counters,
                              L.part);
    } else {
        fn<<<grid, block, 0, stream>>>(a.M, a.N, a.K, tiles_m, tiles_n, a.CA, a.SCA, a.idx, a.n_out,
                                       a.XO, a.CB, a.SCB, a.bias, a.Y, a.C_i32, a.C_f32, L.codes,
                                       L.cap, L.split, L.counters, L.part);
    }
    return hipGetLastError();
}

}  // namespace llmint8
