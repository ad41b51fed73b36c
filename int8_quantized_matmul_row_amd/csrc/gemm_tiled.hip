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
//    in AGPRs).  One workgroup per CU.  Where it fills the CUs better (N with
//    a factor 7, such as 57344 and 14336 at M = 512), the tile is 256 x 224:
//    4 waves in a 4 x 1 grid, each 64 x 224 = 2 x 7 blocks (224 accumulators);
//    the host picks the width from the shape (rounds of workgroups times the
//    work of one).
//  * K advances in 128-byte stages (one whole line of every row) through a
//    2-deep ring of LDS buffers (A 256 x 128 + B 256 x 128 bytes, 64 KiB
//    each).  Stages are filled by buffer_load_dwordx4 ... lds: each wave
//    instruction moves 8 rows x 128 bytes straight from memory into LDS, no
//    registers involved.  One barrier per stage, one MFMA block into the
//    stage's second 64-byte unit; after it the next stage's first unit is read
//    and the stage after that is loaded into the buffer just finished, so
//    every load has a whole stage to land.
//  * LDS rows are 128 bytes; 16-byte chunk c of row r sits in slot
//    c ^ ((r/2) % 8), so a 16-lane phase of 16-byte fragment reads (16
//    consecutive rows, one chunk) touches all 64 banks once.
//  * A lane's operand for a block and 64-byte unit is 32 bytes: chunks
//    4h + l/32 and 4h + 2 + l/32 of its row (unit h), the same for both
//    operands.  int8: two v_mfma_i32_32x32x32_i8 (low halves: the unit's
//    first 32 columns).  FP8 (the E4M3 variant; format in common.h): one
//    v_mfma_scale_f32_32x32x64_f8f6f4, which sees one permutation of the 64
//    columns on both sides.
//  * The A blocks are refilled with the next unit right after their last use;
//    the B blocks (used by every MFMA of a unit) have a second register set.
//    Loads, reads and MFMAs are interleaved in a fixed order (sched_barrier),
//    the stages run in pairs with constant ring slots, and loads past K are
//    clamped.  Operands are read through per-tile buffer descriptors that hold
//    exactly the tile's valid rows: a K that is an odd multiple of 64 ends in
//    a half stage whose unused half reads 0 past the last row.
//  * Tile order: blocks are dispatched round-robin over the 8 XCDs; block b is
//    remapped so that each XCD walks a contiguous range of a grouped raster
//    (4 tile rows per group) and its tiles share CA/CB panels in its own L2.
//  * Few tiles (at most half the CUs, e.g. M = 512 against a 57344-long K):
//    given a workspace, K is split over up to 8 workgroups per tile.  Each
//    stores its int32 (FP8: fp32) accumulators there with device-coherent
//    stores (no fence writes back the XCD's L2) and counts itself in with an
//    atomic; the last to arrive reads every part back coherently, adds them in
//    split order (the same result whichever arrives last; exact for int8) and
//    runs the epilogue.  The counters are zeroed by a kernel ahead of the GEMM.
//  * Epilogue: accumulators -> fp32 times SCA[m]/127 (FP8: /448), plus the
//    16-bit outlier product as v_mfma_f32_32x32x16_{f16,bf16} of the weight
//    codes at the outlier columns (int8 values and E4M3 values are exact in
//    16-bit) against XO, then times SCB[n]/127 (/448), plus bias, rounded to
//    16-bit, staged in LDS and written with full 16-byte row-contiguous
//    stores.  The kernel reads n_out (device memory, no host sync) and takes
//    one of two paths, which share no registers (a single kernel with two
//    separate bodies costs one dispatch):
//      - plain_body: at most 16 outlier columns, from operands staged in LDS
//        with the prologue's loads (the 224-column tile whose K is not split
//        takes their weight codes from the B stages during the K loop
//        instead); or, when the other path cannot take the call (more
//        columns than the gathered codes hold and not simply columns
//        0 .. n_out-1, or C exported), per-32-row-block gathers.
//      - outlier_body: more than 16 outlier columns.  After the int8 loop
//        (skipped when every column is an outlier: CA is then all zero), the
//        accumulators are dequantized in place and a second K loop of the
//        same two-buffer pipeline runs over 64-column stages of XO and of the
//        weight codes: CB's own first columns when the outlier columns are
//        0 .. n_out-1 (every column at threshold 0), else the codes gathered
//        once per call (gemm_prep, or the activation kernel) into the
//        workspace.
#include <cstdlib>
#include <cstring>

#include "common.h"

namespace llmint8 {

namespace {

constexpr int BM = 256;   // tile rows
constexpr int kRowsB = 256;  // weight rows per stage in LDS (the widest tile; rows past a narrower tile's are clamped re-reads)
constexpr int BKS = 128;  // K bytes per stage: one whole 128-byte line of every row
constexpr int kStages = 2;
constexpr int kStageBytes = (BM + kRowsB) * BKS;  // 64 KiB
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kDmaInst = BM / kWaves / 8;   // stage-load instructions (8 rows each) per operand and wave
constexpr int kGroupM = 4;
constexpr int kGatherThreads = 256;
constexpr int kCUs = 256;             // compute units of the device (gfx950)
constexpr int kMaxSplit = 8;          // workgroups per tile when K is split
constexpr int kMinSplitStages = 8;    // K stages (128 bytes) per split, at least
constexpr int kBarrierAt = 1;         // MFMA block of a stage's second unit at its barrier
constexpr int kNoGatherRows = 128;    // token rows up to which the first outlier codes are not gathered

// The tile's columns TN and the waves' grid: 256 columns as 2 x 2 waves of
// 4 x 4 blocks (32 x 32), or 224 columns as 4 x 1 waves of 2 x 7 blocks (224
// accumulators per lane), for weights whose N holds a factor 7 (the tiles of
// 256 leave the last round of CUs partly idle).  The stage layout in LDS is
// the same for both.
template <int TN>
struct Tile {
    static_assert(TN == 256 || TN == 224, "tile columns");
    static constexpr int BN = TN;
    static constexpr int WM = TN == 256 ? 2 : 4;  // waves along M
    static constexpr int WN = kWaves / WM;        // waves along N
    static constexpr int IB = BM / 32 / WM;       // 32-row blocks per wave
    static constexpr int JB = BN / 32 / WN;       // 32-column blocks per wave
    static constexpr int kWaveM = 32 * IB, kWaveN = 32 * JB;
    static constexpr int kYStride = BN * 2 + 16;  // bytes per staged Y row (padding shifts banks)
    // the stage ring (the 224-column tile: 2 A stages and 3 B stages of 224
    // rows), then (after the K loop) two block rows of Y staging, and for the
    // 224-column tile the tile rows of XO behind them
    static constexpr int kRing = TN == 224 ? 2 * BM * BKS + 3 * 224 * BKS : kStages * kStageBytes;
    static constexpr int kAfter = 2 * WM * 32 * kYStride + (TN == 224 ? BM * 16 * 2 : 0);
    static constexpr int kSmemBytes = kRing > kAfter ? kRing : kAfter;
};

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

// Two 16-bit MFMAs (16 outlier columns each): b holds the weight codes of 32
// columns as 16-bit values, a the XO values of the same columns (the low
// halves are the first 16 columns).
template <bool BF16>
__device__ __forceinline__ v16f mfma16x2(const v8i& b, const v8i& a, v16f c) {
    typedef typename Vec16<BF16>::type vec_t;
    c = mfma16<BF16>(__builtin_bit_cast(vec_t, __builtin_shufflevector(b, b, 0, 1, 2, 3)),
                     __builtin_bit_cast(vec_t, __builtin_shufflevector(a, a, 0, 1, 2, 3)), c);
    return mfma16<BF16>(__builtin_bit_cast(vec_t, __builtin_shufflevector(b, b, 4, 5, 6, 7)),
                        __builtin_bit_cast(vec_t, __builtin_shufflevector(a, a, 4, 5, 6, 7)), c);
}

// 8 weight codes (one byte each, value 0 in the low byte of w[0]) as 16-bit
// values: int8 values and E4M3 values are exact in fp16 and bf16.
template <bool BF16, bool FP8>
__device__ __forceinline__ v4i codes8_to16(v2u w) {
    v8u16 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = narrow16<BF16>(code_value<FP8>((int8_t)(w[e >> 2] >> (8 * (e & 3)))));
    return __builtin_bit_cast(v4i, r);
}

// Whether outlier_body takes the call: more than kOutLds outlier
// columns, their codes either CB's own first columns (the columns are
// 0 .. n_out-1) or gathered into the workspace (at most wo_cap of them), and
// no export of the int8 product C (asked for by tests only).
__device__ __forceinline__ bool outlier_path_takes(int n_out, const int32_t* idx, const int8_t* wo_all,
                                                     int wo_cap, bool export_c) {
    return !export_c && n_out > kOutLds &&
           (idx[n_out - 1] == n_out - 1 || (wo_all != nullptr && n_out <= wo_cap));
}

// One tile's place: its origin, its valid rows, and this workgroup's part of
// the K stages (split ks of `split`).
struct TileGeom {
    int m0, n0, rows_a, rows_b, kt_begin, nk;
    bool half_last;
};

template <int TN>
__device__ __forceinline__ TileGeom tile_geom(int tile, int ks, int split, int M, int N, int K, int tiles_m,
                                              int tiles_n) {
    TileGeom g;
    int tm, tn;
    map_tile(tile, tiles_m, tiles_n, tm, tn);
    g.m0 = tm * BM;
    g.n0 = tn * TN;
    g.rows_a = min(BM, M - g.m0);
    g.rows_b = min(TN, N - g.n0);
    // K runs in 128-byte stages; a K that is an odd multiple of 64 ends in a
    // half stage, of which only the first 64-byte unit is computed.
    const int nk_all = (K + BKS - 1) / BKS;
    g.kt_begin = ks * nk_all / split;
    g.nk = (ks + 1) * nk_all / split - g.kt_begin;
    g.half_last = (K % BKS) != 0 && ks == split - 1;
    return g;
}

// ---- LDS fragments of a stage in ring buffer u ------------------------------
// Lane l reads row (l & 31) of each 32-row block.  Fragment f < IB is A block
// f of the wave's rows, f >= IB is B block f - IB of its columns.
template <int TN>
__device__ __forceinline__ v8i read_frag8(const int8_t* smem, int u, int h, int f, int wm, int wn, int lane) {
    typedef Tile<TN> T;
    const int rr = lane & 31;
    const int a_off = wm * T::kWaveM * BKS, b_off = BM * BKS + wn * T::kWaveN * BKS;
    const int base =
        u * kStageBytes + rr * BKS + (f < T::IB ? a_off + 32 * f * BKS : b_off + 32 * (f - T::IB) * BKS);
    const int sw = (rr >> 1) & 7;
    const v4i lo = lds_load<v4i>(smem, (uint32_t)(base + (((4 * h + (lane >> 5)) ^ sw) * 16)));
    const v4i hi = lds_load<v4i>(smem, (uint32_t)(base + (((4 * h + 2 + (lane >> 5)) ^ sw) * 16)));
    return cat8(lo, hi);
}

// One block row of Y (block i of every wave: WM x 32 rows, staged row sr at
// sr * kYStride holding tile row (sr / 32) * kWaveM + 32 i + sr % 32) from its
// staging buffer to Y (after a barrier), rows past M and columns past N
// skipped: full 16-byte row-contiguous stores, non-temporal (Y is not read
// again here).  The block rows alternate between two staging buffers, so each
// is stored while the next is computed, with one barrier per block row
// (storing the whole tile after its last block row left every tile of a round
// storing 33.5 MB at once at the end).
template <int TN>
__device__ __forceinline__ void store_block(const int8_t* buf, uint16_t* __restrict__ Y, int M, int N, int m0,
                                            int n0, int i, int tid_e) {
    typedef Tile<TN> T;
    constexpr int BN = TN, kYStride = T::kYStride, kRows = T::WM * 32;
    const int rows = min(BM, M - m0), cols = min(BN, N - n0);
    auto tile_row = [&](int sr) { return (sr >> 5) * T::kWaveM + 32 * i + (sr & 31); };
    if ((N & 7) == 0) {
        const int c8 = (tid_e & 31) * 8;  // 32 lanes per staged row, 8 rows per pass
#pragma unroll
        for (int q = 0; q < kRows / (kThreads / 32); ++q) {
            const int sr = (tid_e >> 5) + (kThreads / 32) * q, tr = tile_row(sr);
            if (tr < rows && c8 < cols)
                __builtin_nontemporal_store(*reinterpret_cast<const v4i*>(buf + sr * kYStride + c8 * 2),
                                            reinterpret_cast<v4i*>(Y + (size_t)(m0 + tr) * N + n0 + c8));
        }
    } else {
        const uint16_t* ys = reinterpret_cast<const uint16_t*>(buf);
        for (int e = tid_e; e < kRows * BN; e += kThreads) {
            const int sr = e / BN, c = e - sr * BN, tr = tile_row(sr);
            if (tr < rows && c < cols) Y[(size_t)(m0 + tr) * N + n0 + c] = ys[sr * (kYStride / 2) + c];
        }
    }
}

// bytes of one block row's staging buffer (two of them alternate)
template <int TN>
constexpr int y_block_bytes() {
    return Tile<TN>::WM * 32 * Tile<TN>::kYStride;
}

// the lane index again, from v_mbcnt (opaque, so that it is not kept in a
// register across the K loop)
__device__ __forceinline__ int lane_again() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// ---- the int8 (FP8) K loop of one tile ----------------------------------------
// EXTRACT (a tile whose K is not split): the weight codes of the first
// outlier columns listed in s_xcol (ascending, ended by -BKS; at most
// kOutLds, written before the call) are taken from the B stages as they pass
// through LDS, thread t for the tile's weight row t, into s_wo (row t, column
// e at s_wo[t * kOutLds + e], as 16-bit values; the other entries are left as
// they are).  The next column's stage is compared once per stage (one scalar
// branch), so no load of the weight codes leaves the loop: gathering them
// from memory cost every tile a 128-byte line per row and column, while the
// tile's first stages wait behind those loads.
template <bool BF16, bool FP8, bool EXTRACT, int TN>
__device__ __forceinline__ void k_loop(typename TileAcc<FP8>::type (&acc)[Tile<TN>::IB][Tile<TN>::JB],
                                       v8i (&ga)[Tile<TN>::IB], v8i (&gb0)[Tile<TN>::JB], v8i (&gb1)[Tile<TN>::JB],
                                       int8_t* smem, const int8_t* __restrict__ CA, const int8_t* __restrict__ CB,
                                       int K, const TileGeom& g, int wave, int lane, uint16_t* s_wo,
                                       const int* s_xcol) {
    typedef typename TileAcc<FP8>::type acc_t;
    constexpr int IB = Tile<TN>::IB, JB = Tile<TN>::JB;
    const int wm = wave / Tile<TN>::WN, wn = wave % Tile<TN>::WN;
    // ---- stage loads: one instruction = 8 rows x 128 bytes, whole lines.  Wave
    // w fills rows [64w, 64w + 64) of A and of B, instruction i rows
    // 64w + 8i + lane/8; lane p lands in slot p%8 of its row and so fetches the
    // logical 16-byte chunk (p%8) ^ ((row/2) % 8).  Rows past M (N, or the
    // tile's columns) re-read the last valid row (their results are never
    // stored).
    const v4i rsrc_a = buffer_rsrc(CA + (size_t)g.m0 * K, (uint32_t)g.rows_a * (uint32_t)K);
    const v4i rsrc_b = buffer_rsrc(CB + (size_t)g.n0 * K, (uint32_t)g.rows_b * (uint32_t)K);
    uint32_t voff_a[kDmaInst], voff_b[kDmaInst];
#pragma unroll
    for (int i = 0; i < kDmaInst; ++i) {
        const int r = 8 * kDmaInst * wave + 8 * i + (lane >> 3);
        const int ch = ((lane & 7) ^ ((4 * i + (lane >> 4)) & 7)) * 16;
        voff_a[i] = (uint32_t)min(r, g.rows_a - 1) * (uint32_t)K + (uint32_t)g.kt_begin * BKS + ch;
        voff_b[i] = (uint32_t)min(r, g.rows_b - 1) * (uint32_t)K + (uint32_t)g.kt_begin * BKS + ch;
    }
    const uint32_t lds_base =
        __builtin_amdgcn_readfirstlane(lds_address(smem) + 8 * kDmaInst * wave * BKS);  // this wave's rows
    const int nk = g.nk;
    // stage-load instruction d (A rows for d < kDmaInst, then B rows) of stage
    // kt (relative to kt_begin) into ring buffer u
    auto dma = [&](int d, int kt, int u) {
        const uint32_t kd = (uint32_t)kt * BKS;
        if (d < kDmaInst)
            dma_line(rsrc_a, voff_a[d] + kd, lds_base + u * kStageBytes + 8 * d * BKS);
        else
            dma_line(rsrc_b, voff_b[d - kDmaInst] + kd,
                     lds_base + u * kStageBytes + BM * BKS + 8 * (d - kDmaInst) * BKS);
        static_assert(kRowsB == BM, "A and B stage rows are loaded by the same instructions");
    };
    // The prologue loads stages 0 and 1; from then on, stage kt loads stage
    // kt + 2 into the buffer it has just finished with, clamped to the last
    // stage (past K they re-read it into a buffer no wave reads again), so
    // every stage runs the same branch-free code.
#pragma unroll
    for (int d = 0; d < 2 * kDmaInst; ++d) dma(d, 0, 0);
#pragma unroll
    for (int d = 0; d < 2 * kDmaInst; ++d) dma(d, min(1, nk - 1), 1);
    wait_vmcnt<2 * kDmaInst>();  // stage 0 and everything issued before it
    if constexpr (EXTRACT) __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): s_xcol and s_wo written
    stage_barrier();

    // Fragment f of a unit is 32 bytes per lane.  FP8: one
    // v_mfma_scale_f32_32x32x64_f8f6f4 per block and unit.  int8: two
    // v_mfma_i32_32x32x32_i8, on the low halves and on the high halves.
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
    auto rf = [&](int u, int h, int f) -> v8i { return read_frag8<TN>(smem, u, h, f, wm, wn, lane); };
    // the next outlier column to take (uniform) and its place in s_xcol; its
    // stage is x_col >> 7, -1 at the list's end (no stage matches it, so the
    // loop below takes at most kOutLds columns in all)
    int x_p = 0, x_col = -BKS;
    if constexpr (EXTRACT) x_col = __builtin_amdgcn_readfirstlane(s_xcol[0]);
    auto extract = [&](int kt, int u) {
        if constexpr (EXTRACT) {
            if (kt == (x_col >> 7)) {
                const int t = wave * 64 + lane_again();  // (nothing held across the loop)
                const int row = u * kStageBytes + BM * BKS + t * BKS;
                const int sw = (t >> 1) & 7;
                do {
                    const int c = x_col & (BKS - 1);
                    const int8_t v = smem[row + ((((c >> 4) ^ sw) << 4) | (c & 15))];
                    if (t < TN) s_wo[t * kOutLds + x_p] = narrow16<BF16>(code_value<FP8>(v));
                    ++x_p;
                    x_col = __builtin_amdgcn_readfirstlane(s_xcol[x_p]);
                } while ((x_col >> 7) == kt);
            }
        }
    };
    // Unit pipeline: MFMA q of a unit is block (i, j) = (q/JB, q%JB).  A block
    // i is refilled with the next unit in place right after its last use (MFMA
    // JB i + JB-1); the B blocks have a second register set (gb1 holds unit 1
    // of every stage, gb0 unit 0).
#pragma unroll
    for (int f = 0; f < IB; ++f) ga[f] = rf(0, 0, f);
#pragma unroll
    for (int f = 0; f < JB; ++f) gb0[f] = rf(0, 0, IB + f);
    // Stage kt in ring buffer u (a compile-time constant: stages run in pairs).
    // Unit 0 reads unit 1 of the same buffer.  kBarrierAt MFMA blocks into unit
    // 1, every wave waits for its loads of stage kt+1 and for its reads of this
    // buffer, and meets the others at the barrier: stage kt+1 has landed in
    // buffer 1-u, and no wave reads buffer u again.  The rest of unit 1 reads
    // unit 0 of stage kt+1 and spreads the loads of stage kt+2 into buffer u
    // over its MFMAs, so each load has a whole stage to land.
    auto stage = [&](int kt, int u) {
        extract(kt, u);  // stage kt is in buffer u until the barrier below
#pragma unroll
        for (int q = 0; q < IB * JB; ++q) {
            const int i = q / JB, j = q % JB;
            acc[i][j] = mma(gb0[j], ga[i], acc[i][j]);
            if (q < JB) gb1[q] = rf(u, 1, IB + q);
            if (j == JB - 1) ga[i] = rf(u, 1, i);
            __builtin_amdgcn_sched_barrier(0);
        }
        const int kn = min(kt + 2, nk - 1);
#pragma unroll
        for (int q = 0; q < IB * JB; ++q) {
            const int i = q / JB, j = q % JB;
            acc[i][j] = mma(gb1[j], ga[i], acc[i][j]);
            if (q == kBarrierAt - 1) {
                __builtin_amdgcn_s_waitcnt(0);  // vmcnt, expcnt and lgkmcnt all zero
                stage_barrier();
            }
            if (q >= kBarrierAt) {
                // (at the last stage these read a stale buffer; unused)
                if (q - kBarrierAt < JB) gb0[q - kBarrierAt] = rf(1 - u, 0, IB + q - kBarrierAt);
                if (j == JB - 1) ga[i] = rf(1 - u, 0, i);
                // loads d0 .. d1-1 of the 2 kDmaInst go out with MFMA q
                constexpr int kSlots = IB * JB - kBarrierAt;
                const int d0 = (q - kBarrierAt) * 2 * kDmaInst / kSlots;
                const int d1 = (q - kBarrierAt + 1) * 2 * kDmaInst / kSlots;
#pragma unroll
                for (int d = d0; d < d1; ++d) dma(d, kn, u);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    const int nfull = g.half_last ? nk - 1 : nk;
    int kt = 0;
    for (; kt + 2 <= nfull; kt += 2) {
        stage(kt, 0);
        stage(kt + 1, 1);
    }
    if (kt < nfull) stage(kt, 0);
    if (g.half_last) {  // unit 0 of the last stage, in a buffer known at run time
        extract(nfull, nfull & 1);
#pragma unroll
        for (int q = 0; q < IB * JB; ++q) {
            const int i = q / JB, j = q % JB;
            acc[i][j] = mma(gb0[j], ga[i], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    wait_vmcnt<0>();  // the clamped loads past K have landed too
}

// ---- the 224-column tile's K loop: a deeper ring for the weights ---------------
// With M = 512 each weight byte serves only 512 rows, so the loop streams its
// weights from HBM, and one stage of lookahead leaves the MFMAs waiting.  The
// 224-column tile's B stage is 28 KiB (224 rows), so LDS holds two A stages
// (32 KiB each, at 0) and three B stages (at kDeepB), 148 KiB in all.  Stage
// kt reads A buffer kt % 2 and B buffer kt % 3; after its barrier it loads A
// stage kt + 2 and then B stage kt + 3 into the buffers it has just finished
// with.  Loads complete in order, and the barrier of stage kt needs stage
// kt + 1, whose A loads went out in stage kt - 1 just before the B loads of
// stage kt + 2: only those 7 may still be in flight, so each barrier waits
// for vmcnt <= kDmaB, and the weights get ~2.5 stages to land.  Stages run in
// groups of six so that both ring slots are compile-time constants.  The
// rest as in k_loop (the unit pipeline, the clamped loads past K, EXTRACT).
constexpr int kDeepB = 2 * BM * BKS;         // B ring offset (after the two A stages)
constexpr int kDeepBStage = 224 * BKS;       // 28 KiB
constexpr int kDmaB = 224 / kWaves / 8;      // 7 B-row instructions per wave and stage

template <bool BF16, bool FP8, bool EXTRACT>
__device__ __forceinline__ void k_loop_deep(typename TileAcc<FP8>::type (&acc)[Tile<224>::IB][Tile<224>::JB],
                                            v8i (&ga)[Tile<224>::IB], v8i (&gb0)[Tile<224>::JB],
                                            v8i (&gb1)[Tile<224>::JB], int8_t* smem, const int8_t* __restrict__ CA,
                                            const int8_t* __restrict__ CB, int K, const TileGeom& g, int wave,
                                            int lane, uint16_t* s_wo, const int* s_xcol) {
    typedef typename TileAcc<FP8>::type acc_t;
    typedef Tile<224> T;
    constexpr int IB = T::IB, JB = T::JB;
    static_assert(T::WN == 1 && kDmaB * kWaves * 8 == 224, "4 x 1 waves, 224 weight rows");
    const int wm = wave;
    // A: wave w rows [64w, 64w + 64), instruction i rows 64w + 8i + lane/8; B:
    // wave w rows [56w, 56w + 56), instruction i rows 56w + 8i + lane/8.  Lane p
    // lands in slot p%8 of its row and fetches chunk (p%8) ^ ((row/2) % 8).
    const v4i rsrc_a = buffer_rsrc(CA + (size_t)g.m0 * K, (uint32_t)g.rows_a * (uint32_t)K);
    const v4i rsrc_b = buffer_rsrc(CB + (size_t)g.n0 * K, (uint32_t)g.rows_b * (uint32_t)K);
    uint32_t voff_a[kDmaInst], voff_b[kDmaB];
#pragma unroll
    for (int i = 0; i < kDmaInst; ++i) {
        const int r = 8 * kDmaInst * wave + 8 * i + (lane >> 3);
        voff_a[i] = (uint32_t)min(r, g.rows_a - 1) * (uint32_t)K + (uint32_t)g.kt_begin * BKS +
                    ((lane & 7) ^ ((r >> 1) & 7)) * 16;
    }
#pragma unroll
    for (int i = 0; i < kDmaB; ++i) {
        const int r = 8 * kDmaB * wave + 8 * i + (lane >> 3);
        voff_b[i] = (uint32_t)min(r, g.rows_b - 1) * (uint32_t)K + (uint32_t)g.kt_begin * BKS +
                    ((lane & 7) ^ ((r >> 1) & 7)) * 16;
    }
    const uint32_t lds_a = __builtin_amdgcn_readfirstlane(lds_address(smem) + 8 * kDmaInst * wave * BKS);
    const uint32_t lds_b = __builtin_amdgcn_readfirstlane(lds_address(smem) + kDeepB + 8 * kDmaB * wave * BKS);
    const int nk = g.nk;
    // load instruction d of stage kt: A rows into A buffer ua for d < kDmaInst,
    // then B rows into B buffer ub
    auto dma = [&](int d, int kt, int ua, int ub) {
        const uint32_t kd = (uint32_t)kt * BKS;
        if (d < kDmaInst)
            dma_line(rsrc_a, voff_a[d] + kd, lds_a + ua * (BM * BKS) + 8 * d * BKS);
        else
            dma_line(rsrc_b, voff_b[d - kDmaInst] + kd, lds_b + ub * kDeepBStage + 8 * (d - kDmaInst) * BKS);
    };
    constexpr int kNd = kDmaInst + kDmaB;
    // prologue: stages 0 and 1, then B of stage 2
#pragma unroll
    for (int d = 0; d < kNd; ++d) dma(d, 0, 0, 0);
#pragma unroll
    for (int d = 0; d < kNd; ++d) dma(d, min(1, nk - 1), 1, 1);
#pragma unroll
    for (int d = kDmaInst; d < kNd; ++d) dma(d, min(2, nk - 1), 0, 2);
    wait_vmcnt<kNd + kDmaB>();  // stage 0 and everything issued before it
    if constexpr (EXTRACT) __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): s_xcol and s_wo written
    stage_barrier();

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
    // fragment f of unit h: A block f < IB of this wave's rows in A buffer ua,
    // else B block f - IB in B buffer ub (the same chunks and swizzle as read_frag8)
    auto rf = [&](int ua, int ub, int h, int f) -> v8i {
        const int rr = lane & 31;
        const int base = (f < IB ? ua * (BM * BKS) + (wm * T::kWaveM + 32 * f) * BKS
                                 : kDeepB + ub * kDeepBStage + 32 * (f - IB) * BKS) +
                         rr * BKS;
        const int sw = (rr >> 1) & 7;
        const v4i lo = lds_load<v4i>(smem, (uint32_t)(base + (((4 * h + (lane >> 5)) ^ sw) * 16)));
        const v4i hi = lds_load<v4i>(smem, (uint32_t)(base + (((4 * h + 2 + (lane >> 5)) ^ sw) * 16)));
        return cat8(lo, hi);
    };
    int x_p = 0, x_col = -BKS;
    if constexpr (EXTRACT) x_col = __builtin_amdgcn_readfirstlane(s_xcol[0]);
    auto extract = [&](int kt, int ub) {
        if constexpr (EXTRACT) {
            if (kt == (x_col >> 7)) {
                const int t = wave * 64 + lane_again();  // (nothing held across the loop)
                const int tr = min(t, 223);               // the B buffer holds 224 rows
                const int row = kDeepB + ub * kDeepBStage + tr * BKS;
                const int sw = (tr >> 1) & 7;
                do {
                    const int c = x_col & (BKS - 1);
                    const int8_t v = smem[row + ((((c >> 4) ^ sw) << 4) | (c & 15))];
                    if (t < 224) s_wo[t * kOutLds + x_p] = narrow16<BF16>(code_value<FP8>(v));
                    ++x_p;
                    x_col = __builtin_amdgcn_readfirstlane(s_xcol[x_p]);
                } while ((x_col >> 7) == kt);
            }
        }
    };
#pragma unroll
    for (int f = 0; f < IB; ++f) ga[f] = rf(0, 0, 0, f);
#pragma unroll
    for (int f = 0; f < JB; ++f) gb0[f] = rf(0, 0, 0, IB + f);
    auto stage = [&](int kt, int ua, int ub) {
        extract(kt, ub);  // stage kt is in buffers ua / ub until the barrier below
#pragma unroll
        for (int q = 0; q < IB * JB; ++q) {
            const int i = q / JB, j = q % JB;
            acc[i][j] = mma(gb0[j], ga[i], acc[i][j]);
            if (q < JB) gb1[q] = rf(ua, ub, 1, IB + q);
            if (j == JB - 1) ga[i] = rf(ua, ub, 1, i);
            __builtin_amdgcn_sched_barrier(0);
        }
        const int ka = min(kt + 2, nk - 1), kb = min(kt + 3, nk - 1);
        const int na = 1 - ua, nb = ub == 2 ? 0 : ub + 1;  // stage kt + 1's buffers
#pragma unroll
        for (int q = 0; q < IB * JB; ++q) {
            const int i = q / JB, j = q % JB;
            acc[i][j] = mma(gb1[j], ga[i], acc[i][j]);
            if (q == kBarrierAt - 1) {
                // stage kt + 1 has landed (only the B loads of stage kt + 2,
                // issued after its A loads, may be in flight), and this wave's
                // reads of buffers ua / ub are complete
                __builtin_amdgcn_s_waitcnt(kDmaB);  // vmcnt(kDmaB), expcnt and lgkmcnt 0
                stage_barrier();
            }
            if (q >= kBarrierAt) {
                // (at the last stage these read stale buffers; unused)
                if (q - kBarrierAt < JB) gb0[q - kBarrierAt] = rf(na, nb, 0, IB + q - kBarrierAt);
                if (j == JB - 1) ga[i] = rf(na, nb, 0, i);
                // loads d0 .. d1-1 (A of stage kt + 2 first, then B of stage
                // kt + 3) go out with MFMA q
                constexpr int kSlots = IB * JB - kBarrierAt;
                const int d0 = (q - kBarrierAt) * kNd / kSlots;
                const int d1 = (q - kBarrierAt + 1) * kNd / kSlots;
#pragma unroll
                for (int d = d0; d < d1; ++d) dma(d, d < kDmaInst ? ka : kb, ua, ub);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    const int nfull = g.half_last ? nk - 1 : nk;
    int kt = 0;
    for (; kt + 6 <= nfull; kt += 6) {
        stage(kt, 0, 0);
        stage(kt + 1, 1, 1);
        stage(kt + 2, 0, 2);
        stage(kt + 3, 1, 0);
        stage(kt + 4, 0, 1);
        stage(kt + 5, 1, 2);
    }
    if (kt < nfull) stage(kt, 0, 0);
    if (kt + 1 < nfull) stage(kt + 1, 1, 1);
    if (kt + 2 < nfull) stage(kt + 2, 0, 2);
    if (kt + 3 < nfull) stage(kt + 3, 1, 0);
    if (kt + 4 < nfull) stage(kt + 4, 0, 1);
    if (g.half_last) {  // unit 0 of the last stage (its fragments are in registers)
        extract(nfull, nfull % 3);
#pragma unroll
        for (int q = 0; q < IB * JB; ++q) {
            const int i = q / JB, j = q % JB;
            acc[i][j] = mma(gb0[j], ga[i], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    wait_vmcnt<0>();  // the clamped loads past K have landed too
}

// the K loop of the tile width (the FP8 variant keeps the two-stage ring at
// 224 columns: with the deep ring its loop spilled ~100 registers)
template <bool BF16, bool FP8, bool EXTRACT, int TN>
__device__ __forceinline__ void k_loop_tile(typename TileAcc<FP8>::type (&acc)[Tile<TN>::IB][Tile<TN>::JB],
                                            v8i (&ga)[Tile<TN>::IB], v8i (&gb0)[Tile<TN>::JB],
                                            v8i (&gb1)[Tile<TN>::JB], int8_t* smem, const int8_t* __restrict__ CA,
                                            const int8_t* __restrict__ CB, int K, const TileGeom& g, int wave,
                                            int lane, uint16_t* s_wo, const int* s_xcol) {
    if constexpr (TN == 224 && !FP8)
        k_loop_deep<BF16, FP8, EXTRACT>(acc, ga, gb0, gb1, smem, CA, CB, K, g, wave, lane, s_wo, s_xcol);
    else
        k_loop<BF16, FP8, EXTRACT, TN>(acc, ga, gb0, gb1, smem, CA, CB, K, g, wave, lane, s_wo, s_xcol);
}

// ---- split K: the partial sums meet in the workspace --------------------------
// Stored in register order: 16 bytes (registers 4c..4c+3 of a block) per lane,
// a wave's 64 lanes contiguous, so every access is a full 1 KiB.  The stores
// and the last arriver's loads are device-coherent (sc1: written through,
// read past a stale L2 line), so no device-scope fence has to write back or
// invalidate a whole XCD's L2: the stores complete (vmcnt) before the arrival
// count, and the loads follow it.  Returns whether this workgroup finishes the
// tile (the last to arrive); it then holds the sum of every split's part, in
// split order.  st: the tile's index among the split tiles.
template <bool FP8, int TN>
__device__ __forceinline__ bool split_sum(typename TileAcc<FP8>::type (&acc)[Tile<TN>::IB][Tile<TN>::JB], int st,
                                          int ks, int split, uint32_t* __restrict__ counters,
                                          int32_t* __restrict__ part, int wave, int lane, int tid, int* s_last) {
    typedef typename TileAcc<FP8>::type acc_t;
    constexpr int IB = Tile<TN>::IB, JB = Tile<TN>::JB;
    constexpr int kWaveWords = IB * JB * 16 * 64;  // blocks x 16 registers x 64 lanes
    constexpr int kCoherent = 16;                 // cache policy sc1: device scope
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        part + (size_t)st * split * (kWaves * kWaveWords), 0, split * (kWaves * kWaveWords) * 4, 0x00020000);
#pragma unroll
    for (int i = 0; i < IB; ++i)
#pragma unroll
        for (int j = 0; j < JB; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                // whole vectors through bit casts (a bit cast of one vector
                // element reads element 0)
                const v16i bits = __builtin_bit_cast(v16i, acc[i][j]);
                const v4i w = {bits[4 * c], bits[4 * c + 1], bits[4 * c + 2], bits[4 * c + 3]};
                __builtin_amdgcn_raw_buffer_store_b128(
                    w, rsrc, ((ks * kWaves + wave) * kWaveWords + ((i * JB + j) * 4 + c) * 256 + lane * 4) * 4, 0,
                    kCoherent);
            }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's part is stored device-wide
    __syncthreads();
    if (tid == 0) *s_last = atomicAdd(counters + st, 1u) == (unsigned)(split - 1);
    __syncthreads();
    if (!*s_last) return false;  // another workgroup finishes this tile
    // sum in split order, this workgroup's own part read back too (the same
    // result whichever workgroup arrives last)
#pragma unroll
    for (int i = 0; i < IB; ++i)
#pragma unroll
        for (int j = 0; j < JB; ++j) {
            acc_t t;
#pragma unroll
            for (int sp = 0; sp < kMaxSplit; ++sp) {
                if (sp < split) {
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const auto x = __builtin_bit_cast(
                            typename Part4<FP8>::type,
                            __builtin_amdgcn_raw_buffer_load_b128(
                                rsrc, ((sp * kWaves + wave) * kWaveWords + ((i * JB + j) * 4 + c) * 256 + lane * 4) * 4,
                                0, kCoherent));
#pragma unroll
                        for (int e = 0; e < 4; ++e) t[4 * c + e] = sp == 0 ? x[e] : t[4 * c + e] + x[e];
                    }
                }
            }
            acc[i][j] = t;
        }
    return true;
}

// The int32 (FP8: fp32) accumulators of block row i to C (tests), rows and
// columns past M, N skipped.
template <bool FP8, int TN>
__device__ __forceinline__ void export_c(const typename TileAcc<FP8>::type (&acc)[Tile<TN>::IB][Tile<TN>::JB], int i,
                                         int M, int N, int m, int n_base, int32_t* __restrict__ C_i32,
                                         float* __restrict__ C_f32) {
    // (opaque per call: the column indices and bounds of every register,
    // hoisted out of the block-row loop, would take more registers than there are)
    asm volatile("" : "+v"(n_base), "+v"(m));
#pragma unroll
    for (int j = 0; j < Tile<TN>::JB; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int n = n_base + 32 * j + 8 * (v >> 2) + (v & 3);
            if (m < M && n < N) {
                if constexpr (FP8) C_f32[(size_t)m * N + n] = acc[i][j][v];
                else C_i32[(size_t)m * N + n] = acc[i][j][v];
            }
        }
}

// The first nj of JC blocks of a block row of the wave's sub-tile, dequantized
// by the row scale (f): times SCB/127 (/448), plus bias, rounded to 16-bit,
// staged in LDS as 8-byte pieces.  Register v of lane l of block j is row
// `row` and column n_lane + 32 j + 8 (v/4) + v%4 of the tile (n_lane holds
// 4 (l/32) and the chunk's first column).
template <bool BF16, int TN, int JC>
__device__ __forceinline__ void stage_y(int8_t* smem, const float* s_sb, const float* s_bias, const v16f (&f)[JC],
                                        int nj, int row, int n_lane) {
    constexpr int kYStride = Tile<TN>::kYStride;
    uint16_t* ys = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
    for (int j = 0; j < JC; ++j)
        if (j < nj)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
            const int nl = n_lane + 32 * j + 8 * a4;
            float y[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) y[b] = f[j][4 * a4 + b] * s_sb[nl + b] + s_bias[nl + b];
            *reinterpret_cast<uint2*>(ys + row * (kYStride / 2) + nl) =
                make_uint2(pack16x2<BF16>(y[0], y[1]), pack16x2<BF16>(y[2], y[3]));
        }
}

}  // namespace

// Ahead of the GEMM: workgroup 0 zeroes the split-K arrival counters (if
// any), and the weight codes at the outlier columns are gathered (layout with
// gather_codes) when the activation kernel has not done so (codes != nullptr):
// more than min_cols columns (TiledLayout), at most cap, and not simply
// columns 0 .. n_out-1 (whose codes the product reads from CB).  plain_body
// reads the first kOutLds of them, outlier_body all.
__global__ __launch_bounds__(kGatherThreads) void gemm_prep(
    int N, int K, int cap, int min_cols, const int32_t* __restrict__ idx, const int32_t* __restrict__ n_out_ptr,
    const int8_t* __restrict__ CB, int8_t* __restrict__ codes, uint32_t* __restrict__ counters,
    int n_counters) {
    if (blockIdx.x == 0)
        for (int t = threadIdx.x; t < n_counters; t += kGatherThreads) counters[t] = 0;
    if (codes == nullptr) return;
    const int n_out = *n_out_ptr;
    if (n_out <= min_cols || n_out == 0 || n_out > cap || idx[n_out - 1] == n_out - 1) return;
    __shared__ __attribute__((aligned(16))) int8_t buf[(kGatherThreads / 16) * kGatherSeg];
    auto col = [&](int c) { return idx[c]; };
    if (n_out <= kOutLds) {
        gather_first_codes(N, K, n_out, col, CB, codes, (int64_t)blockIdx.x * kGatherThreads + threadIdx.x,
                           (int64_t)gridDim.x * kGatherThreads);
        return;
    }
    if (gather_all_sparse(K, n_out)) {
        gather_codes<kGatherThreads>(
            N, K, cap, n_out, col, (n_out + kGatherRun - 1) / kGatherRun,
            [&](int i) { return GatherChunk{kGatherRun * i, min(kGatherRun * (i + 1), n_out), -1}; }, CB, codes,
            buf, threadIdx.x, blockIdx.x, gridDim.x);
        return;
    }
    __shared__ int s_seg[kGatherSegMax + 1];
    __shared__ GatherChunks s_chunks;
    // outlier columns below each segment start: j for the starts in
    // (idx[j-1], idx[j]] of the ascending list (every start once; one pass of
    // loads, no dependent chain)
    const int nseg = (K + kGatherSeg - 1) / kGatherSeg;
    for (int j = threadIdx.x; j <= n_out; j += kGatherThreads) {
        const int s_lo = j > 0 ? idx[j - 1] / kGatherSeg + 1 : 0;
        const int s_hi = j < n_out ? min(idx[j] / kGatherSeg, nseg) : nseg;  // (clamped: stays in s_seg)
        for (int sg = s_lo; sg <= s_hi; ++sg) s_seg[sg] = j;
    }
    __syncthreads();
    if (threadIdx.x == 0) build_gather_chunks(K, n_out, [&](int sg) { return s_seg[sg]; }, s_chunks);
    __syncthreads();
    gather_codes<kGatherThreads>(
        N, K, cap, n_out, col, s_chunks.n,
        [&](int i) { return GatherChunk{s_chunks.lo[i], s_chunks.lo[i + 1], s_chunks.seg[i]}; }, CB, codes, buf,
        threadIdx.x, blockIdx.x, gridDim.x);
}

// At most kOutLds outlier columns (or a call outlier_body cannot take).  LDS:
// smem (stage ring, then the Y staging), the tile's scales and bias, s_wo
// (the weight codes of the tile's rows at the first kOutLds outlier columns,
// as 16-bit values, 0 past n_out: row r, column e at s_wo[r * kOutLds + e])
// and s_xo (the tile's rows of XO at those columns: row r at
// s_xo[r * kOutLds], 0 past n_out: XO's padding).
template <bool BF16, bool FP8, bool SPLIT, int TN>
__device__ __forceinline__ void plain_body(int8_t* smem, float* s_sa, float* s_sb, float* s_bias, uint16_t* s_wo,
                                           uint16_t* s_xo, int* s_xcol, int* s_last_p, int M, int N, int K, int tiles_m,
                                           int tiles_n, const int8_t* __restrict__ CA, const float* __restrict__ SCA,
                                           const int32_t* __restrict__ idx, const int32_t* __restrict__ n_out_ptr,
                                           const uint16_t* __restrict__ XO, const int8_t* __restrict__ CB,
                                           const float* __restrict__ SCB, const uint16_t* __restrict__ bias,
                                           uint16_t* __restrict__ Y, int32_t* __restrict__ C_i32,
                                           float* __restrict__ C_f32, const int8_t* __restrict__ wo_all,
                                           int wo_cap, int wo_min, int split, uint32_t* __restrict__ counters,
                                           int32_t* __restrict__ part) {
    typedef typename TileAcc<FP8>::type acc_t;
    typedef Tile<TN> T;
    constexpr int IB = T::IB, JB = T::JB, BN = T::BN, kWaveN = T::kWaveN;
    // The weight codes at the first kOutLds outlier columns come from the B
    // stages in the K loop (see k_loop) for the 224-column tile whose K is
    // not split; the 256-column tile's epilogue spills with the loop's extra
    // branch (measured slower), and a split tile sees only its part of K, so
    // those gather the codes from memory ahead of the loop.
    constexpr bool kExtract = TN == 224 && !SPLIT;

    const bool want_c = FP8 ? C_f32 != nullptr : C_i32 != nullptr;
    const int n_out = *n_out_ptr;

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / T::WN, wn = wave % T::WN;
    // SPLIT: workgroup b takes split ks = b % split of tile b / split
    if constexpr (!SPLIT) split = 1;
    const int tile = blockIdx.x / split, ks = blockIdx.x - tile * split;
    const TileGeom g = tile_geom<TN>(tile, ks, split, M, N, K, tiles_m, tiles_n);
    const int m0 = g.m0, n0 = g.n0;

    acc_t acc[IB][JB];
#pragma unroll
    for (int i = 0; i < IB; ++i)
#pragma unroll
        for (int j = 0; j < JB; ++j) acc[i][j] = acc_t{};

    // Epilogue operands, requested now so that their latency hides under the
    // K loop; they go to LDS after it (a use before it would make the compiler
    // wait for every load in flight, the stage loads included, which it cannot
    // see).  Every load is unconditional, from a clamped address (a load under
    // a branch is awaited where the branch rejoins).  Outlier gather: lane
    // column e = tid % 16, rows tid/16 + 16 q; lanes past n_out read column 0
    // (discarded).
    const int t8 = kThreads > 256 ? (tid & 255) : tid;  // threads 256 and on repeat 0..255
    float sa_raw = SCA[min(m0 + t8, M - 1)];
    const int n_sb = min(n0 + t8, N - 1);
    float sb_raw = SCB[n_sb];
    uint16_t bias_raw = *(bias ? bias + n_sb : XO);  // XO: any readable element
    // The weight codes at the first kOutLds outlier columns (lane column
    // e = tid % 16, rows tid/16 + 16 q; lanes past n_out read column 0 and are
    // masked): from the codes gathered once per call into the workspace when
    // it holds them (a row's 16 codes are adjacent there, and the rows too
    // when there are at most 16 columns), else from CB (a 128-byte line per
    // row and column, for every tile row of the grid again), or, with kExtract,
    // taken by the K loop into this thread's row of s_wo, zeroed first.
    const int e_out = tid & (kOutLds - 1);
    const bool e_valid = e_out < n_out;
    constexpr int kWoPasses = !kExtract ? BN * kOutLds / kThreads : 1;  // rows tid/16 + (kThreads/16) q
    int32_t wo_raw[kWoPasses];
    if constexpr (!kExtract) {
        int e_col = 0;
#pragma unroll
        for (int u = 0; u < kOutLds; ++u) {  // uniform reads; idx holds K >= 64 entries
            int c = idx[u];
            asm volatile("" : "+s"(c));  // all sixteen read, then selected without branches
            e_col = u == e_out ? c : e_col;
        }
        if (!e_valid) e_col = 0;
        // gathered for this call: the same condition as the gather's (more
        // than wo_min columns, TiledLayout::min_cols; at most the workspace's
        // columns; and not simply 0 .. n_out-1, whose codes are CB's own
        // first columns)
        const bool gathered = wo_all != nullptr && n_out > wo_min && n_out > 0 && n_out <= wo_cap &&
                              idx[max(n_out, 1) - 1] != n_out - 1;
        const int8_t* w_src = gathered ? wo_all : CB;
        const size_t w_stride = gathered ? (size_t)(n_out <= kOutLds ? kOutLds : wo_cap) : (size_t)K;
        const int w_col = gathered ? (e_valid ? e_out : 0) : e_col;
#pragma unroll
        for (int q = 0; q < kWoPasses; ++q)
            wo_raw[q] = w_src[(size_t)min(n0 + (tid >> 4) + (kThreads / 16) * q, N - 1) * w_stride + w_col];
    } else {
        if (tid < BN) {
            *reinterpret_cast<v4i*>(s_wo + tid * kOutLds) = v4i{};
            *reinterpret_cast<v4i*>(s_wo + tid * kOutLds + 8) = v4i{};
        }
        // the first min(n_out, kOutLds) columns, then the end (-BKS)
        if (tid <= kOutLds) s_xcol[tid] = tid < min(n_out, kOutLds) ? idx[tid] : -BKS;
    }
    // XO's first kOutLds columns of tile row t8 (in bounds for n_pad = 0 too:
    // XO holds M * K >= 64 elements)
    const int n_pad = (n_out + 31) & ~31;
    const v4i* xo_src = reinterpret_cast<const v4i*>(XO + (size_t)min(m0 + t8, M - 1) * n_pad);
    v4i xo_raw0 = xo_src[0], xo_raw1 = xo_src[1];

    v8i ga[IB], gb0[JB], gb1[JB];
    k_loop_tile<BF16, FP8, kExtract, TN>(acc, ga, gb0, gb1, smem, CA, CB, K, g, wave, lane, s_wo, s_xcol);

    asm volatile("" : "+v"(sa_raw), "+v"(sb_raw), "+v"(bias_raw), "+v"(xo_raw0), "+v"(xo_raw1));
    if constexpr (!kExtract) {
#pragma unroll
        for (int q = 0; q < kWoPasses; ++q) asm volatile("" : "+v"(wo_raw[q]));
    }
    // the 224-column tile keeps XO's rows in the (then dead) stage ring,
    // written after the barrier below
    constexpr bool kXoInRing = TN == 224;
    if constexpr (kXoInRing) s_xo = reinterpret_cast<uint16_t*>(smem + 2 * y_block_bytes<TN>());
    if (kThreads == 256 || tid < 256) {
        s_sa[tid] = sa_raw;
        s_sb[tid] = sb_raw / code_max<FP8>();
        s_bias[tid] = bias ? widen16<BF16>(bias_raw) : 0.0f;
        if constexpr (!kXoInRing) {
            *reinterpret_cast<v4i*>(s_xo + tid * kOutLds) = xo_raw0;
            *reinterpret_cast<v4i*>(s_xo + tid * kOutLds + 8) = xo_raw1;
        }
    }
    if constexpr (!kExtract) {
        const uint32_t e_mask = e_valid ? 0xFFFFu : 0u;  // a mask, not a select: no branches
#pragma unroll
        for (int q = 0; q < kWoPasses; ++q)
            s_wo[((tid >> 4) + (kThreads / 16) * q) * kOutLds + e_out] =
                (uint16_t)(narrow16<BF16>(code_value<FP8>((int8_t)wo_raw[q])) & e_mask);
    }

    if constexpr (SPLIT) {
        if (!split_sum<FP8, TN>(acc, tile, ks, split, counters, part, wave, lane, tid, s_last_p)) return;
    }

    // ---- epilogue, one 32-row block at a time -----------------------------------
    __syncthreads();  // every wave is done reading the stage buffers
    if constexpr (kXoInRing) {
        if (kThreads == 256 || tid < 256) {
            *reinterpret_cast<v4i*>(s_xo + tid * kOutLds) = xo_raw0;
            *reinterpret_cast<v4i*>(s_xo + tid * kOutLds + 8) = xo_raw1;
        }
        __syncthreads();
    }
    const int lane_e = lane_again();
    const int kh = lane_e >> 5, rr_e = lane_e & 31, tid_e = wave * 64 + lane_e;
    const int m_lane = wm * T::kWaveM + rr_e;        // + 32 i
    const int n_lane = wn * kWaveN + 4 * kh;       // + 32 j + 8 (v/4) + v%4
    typedef typename Vec16<BF16>::type vec_t;
    // column blocks per step of the epilogue: at most 4 (64 fp32 values per
    // lane), so the 7 blocks of a 224-column tile go in two steps
    constexpr int JC = JB < 4 ? JB : 4;
#pragma unroll
    for (int i = 0; i < IB; ++i) {
        const int m = m0 + m_lane + 32 * i;
        if (want_c) export_c<FP8, TN>(acc, i, M, N, m, n0 + n_lane, C_i32, C_f32);
        const float sa = s_sa[m_lane + 32 * i] / code_max<FP8>();
#pragma unroll
        for (int jb0 = 0; jb0 < JB; jb0 += JC) {
        const int nj = JB - jb0 < JC ? JB - jb0 : JC;
        v16f f[JC];
#pragma unroll
        for (int j = 0; j < JC; ++j)
            if (j < nj)
#pragma unroll
            for (int v = 0; v < 16; ++v) f[j][v] = (float)acc[i][jb0 + j][v] * sa;
        if (n_out > 0) {
            // the codes and XO of the first kOutLds columns, staged in LDS (XO
            // rows as the B operand: the transposed product)
            const v8u16 xraw = *reinterpret_cast<const v8u16*>(s_xo + (m_lane + 32 * i) * kOutLds + 8 * kh);
#pragma unroll
            for (int j = 0; j < JC; ++j) {
                if (j >= nj) continue;
                const v8u16 raw =
                    *reinterpret_cast<const v8u16*>(s_wo + (wn * kWaveN + 32 * (jb0 + j) + rr_e) * kOutLds + 8 * kh);
                f[j] = mfma16<BF16>(__builtin_bit_cast(vec_t, raw), __builtin_bit_cast(vec_t, xraw), f[j]);
            }
        }
        // Further columns (only when outlier_body does not take the
        // call: too many to gather and not simply columns 0 .. n_out-1, or C
        // exported): each 16-column block gathered here, as uniform (scalar)
        // column indices, lanes with kh = 1 taking the second 8.  Adjacent
        // columns from a multiple of 8 on are one 8-byte load per row;
        // otherwise one byte load each, columns past n_out reading the last
        // outlier column (no branch around a load) and masked to 0.
        for (int j0 = kOutLds; j0 < n_out; j0 += 16) {
            const vec_t xa = __builtin_bit_cast(
                vec_t, *reinterpret_cast<const v8u16*>(XO + (size_t)min(m, M - 1) * n_pad + j0 + 8 * kh));
            const int first = idx[j0], last = idx[min(j0 + 15, n_out - 1)];
            int b[JC][8];
            uint32_t keep = 0xffu;
            if (j0 + 16 <= n_out && last - first == 15 && (first & 7) == 0) {
#pragma unroll
                for (int j = 0; j < JC; ++j) {
                    const int8_t* cb = CB + (size_t)min(n0 + wn * kWaveN + 32 * (jb0 + j) + rr_e, N - 1) * K;
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
                for (int j = 0; j < JC; ++j) {
                    const int8_t* cb = CB + (size_t)min(n0 + wn * kWaveN + 32 * (jb0 + j) + rr_e, N - 1) * K;
#pragma unroll
                    for (int e = 0; e < 8; ++e) b[j][e] = cb[kcol[e]];
                }
                // all the byte loads in flight before the first wait
#pragma unroll
                for (int j = 0; j < JC; ++j)
                    asm volatile(""
                                 : "+v"(b[j][0]), "+v"(b[j][1]), "+v"(b[j][2]), "+v"(b[j][3]), "+v"(b[j][4]),
                                   "+v"(b[j][5]), "+v"(b[j][6]), "+v"(b[j][7]));
            }
#pragma unroll
            for (int j = 0; j < JC; ++j) {
                if (j >= nj) continue;
                v8u16 raw;
#pragma unroll
                for (int e = 0; e < 8; ++e)  // exact in fp16 and bf16
                    raw[e] = (uint16_t)(narrow16<BF16>(code_value<FP8>((int8_t)b[j][e])) & (0u - ((keep >> e) & 1u)));
                f[j] = mfma16<BF16>(__builtin_bit_cast(vec_t, raw), xa, f[j]);
            }
        }
        stage_y<BF16, TN, JC>(smem + (i & 1) * y_block_bytes<TN>(), s_sb, s_bias, f, nj, wm * 32 + rr_e,
                              n_lane + 32 * jb0);
        }
        __syncthreads();  // block row i staged; block row i-1's buffer read out
        store_block<TN>(smem + (i & 1) * y_block_bytes<TN>(), Y, M, N, m0, n0, i, tid_e);
    }
}

// More than kOutLds outlier columns whose codes are CB's first columns or
// gathered in the workspace.  Workgroup b takes tile b / split, split b % split
// (one tile per workgroup: a loop over tiles spills the accumulators).
template <bool BF16, bool FP8, bool SPLIT, int TN>
__device__ __forceinline__ void outlier_body(int8_t* smem, float* s_sa, float* s_sb, float* s_bias, int* s_last_p,
                                             int M, int N, int K, int tiles_m, int tiles_n,
                                             const int8_t* __restrict__ CA, const float* __restrict__ SCA,
                                             const int32_t* __restrict__ idx, const int32_t* __restrict__ n_out_ptr,
                                             const uint16_t* __restrict__ XO, const int8_t* __restrict__ CB,
                                             const float* __restrict__ SCB, const uint16_t* __restrict__ bias,
                                             uint16_t* __restrict__ Y, int32_t* __restrict__ C_i32,
                                             float* __restrict__ C_f32, const int8_t* __restrict__ wo_all,
                                             int wo_cap, int split, uint32_t* __restrict__ counters,
                                             int32_t* __restrict__ part) {
    typedef typename TileAcc<FP8>::type acc_t;
    typedef Tile<TN> T;
    constexpr int IB = T::IB, JB = T::JB, kWaveN = T::kWaveN;

    const int n_out = *n_out_ptr;
    if constexpr (!SPLIT) split = 1;
    const bool prefix = idx[n_out - 1] == n_out - 1;
    // every column an outlier (threshold 0): CA is all zero, so C = 0 and the
    // int8 loop is skipped
    const bool int8_part = n_out < K;
    const int n_pad = (n_out + 31) & ~31;
    const int no = (n_pad + 63) / 64;  // 64-column stages of the outlier loop
    const bool o_half = (n_pad & 63) != 0;
    const uint32_t cstride = prefix ? (uint32_t)K : (uint32_t)wo_cap;
    {
        const int w = blockIdx.x;
        const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int wm = wave / T::WN, wn = wave % T::WN;
        const int tile = w / split, ks = w - tile * split;
        const TileGeom g = tile_geom<TN>(tile, ks, split, M, N, K, tiles_m, tiles_n);
        const int m0 = g.m0, n0 = g.n0;

        acc_t acc[IB][JB];
#pragma unroll
        for (int i = 0; i < IB; ++i)
#pragma unroll
            for (int j = 0; j < JB; ++j) acc[i][j] = acc_t{};
        const int t8 = kThreads > 256 ? (tid & 255) : tid;
        float sa_raw = SCA[min(m0 + t8, M - 1)];
        const int n_sb = min(n0 + t8, N - 1);
        float sb_raw = SCB[n_sb];
        uint16_t bias_raw = *(bias ? bias + n_sb : XO);

        v8i ga[IB], gb0[JB], gb1[JB];
        if (int8_part)
            k_loop_tile<BF16, FP8, false, TN>(acc, ga, gb0, gb1, smem, CA, CB, K, g, wave, lane, nullptr, nullptr);

        asm volatile("" : "+v"(sa_raw), "+v"(sb_raw), "+v"(bias_raw));
        if (kThreads == 256 || tid < 256) {
            s_sa[tid] = sa_raw;
            s_sb[tid] = sb_raw / code_max<FP8>();
            s_bias[tid] = bias ? widen16<BF16>(bias_raw) : 0.0f;
        }
        if constexpr (SPLIT) {
            if (!split_sum<FP8, TN>(acc, tile, ks, split, counters, part, wave, lane, tid, s_last_p)) return;
        }
        __syncthreads();  // every wave is done reading the stage buffers; the scales are in LDS

        const int lane_e = lane_again();
        const int kh = lane_e >> 5, rr_e = lane_e & 31, tid_e = wave * 64 + lane_e;
        const int m_lane = wm * T::kWaveM + rr_e;
        const int n_lane = wn * kWaveN + 4 * kh;
        // dequantize by the row scale in place: from here on the accumulators
        // hold fp32 values (the same AGPRs)
#pragma unroll
        for (int i = 0; i < IB; ++i) {
            const float sa = s_sa[m_lane + 32 * i] / code_max<FP8>();
#pragma unroll
            for (int j = 0; j < JB; ++j) {
                v16f f;
#pragma unroll
                for (int v = 0; v < 16; ++v) f[v] = (float)acc[i][j][v] * sa;
                asm volatile("" : "+a"(f));
                acc[i][j] = __builtin_bit_cast(acc_t, f);
            }
        }

        // ---- the outlier K loop ----------------------------------------------
        // Stages of 64 outlier columns: XO's 128 bytes of each tile row (the A
        // layout of the int8 loop) and the codes' 64 bytes of each weight row,
        // at kBo in the buffer: row r at 64 r, 16-byte chunk c at slot
        // c ^ ((r/4) % 4), so a 16-lane phase of 8-byte reads (16 rows, one
        // half chunk) is conflict-free.  n_pad is a multiple of 32, so the
        // last stage may be half.
        constexpr int kBo = BM * BKS;
        constexpr int kDmaC = kRowsB / kWaves / 16;  // code-row instructions (16 rows x 64 bytes) per wave
        const int8_t* cbase = (prefix ? CB + (size_t)n0 * K : wo_all + (size_t)n0 * wo_cap);
        const v4i rsrc_x = buffer_rsrc(XO + (size_t)m0 * n_pad, (uint32_t)g.rows_a * 2u * (uint32_t)n_pad);
        const v4i rsrc_c = buffer_rsrc(cbase, (uint32_t)g.rows_b * cstride);
        uint32_t voff_x[kDmaInst], voff_c[kDmaC];
#pragma unroll
        for (int i = 0; i < kDmaInst; ++i) {
            const int r = 8 * kDmaInst * wave + 8 * i + (lane_e >> 3);
            const int ch = ((lane_e & 7) ^ ((4 * i + (lane_e >> 4)) & 7)) * 16;
            voff_x[i] = (uint32_t)min(r, g.rows_a - 1) * 2u * (uint32_t)n_pad + ch;
        }
#pragma unroll
        for (int i = 0; i < kDmaC; ++i) {
            const int r = 16 * kDmaC * wave + 16 * i + (lane_e >> 2);
            voff_c[i] = (uint32_t)min(r, g.rows_b - 1) * cstride + ((lane_e & 3) ^ ((lane_e >> 4) & 3)) * 16;
        }
        const uint32_t lbase = lds_address(smem);
        const uint32_t lds_x = __builtin_amdgcn_readfirstlane(lbase + 8 * kDmaInst * wave * BKS);
        const uint32_t lds_c = __builtin_amdgcn_readfirstlane(lbase + kBo + 16 * kDmaC * wave * 64);
        // load instruction d of stage s into buffer u: XO rows for d <
        // kDmaInst, then code rows
        auto dma_o = [&](int d, int s, int u) {
            if (d < kDmaInst)
                dma_line(rsrc_x, voff_x[d] + (uint32_t)s * 128u, lds_x + u * kStageBytes + 8 * d * BKS);
            else
                dma_line(rsrc_c, voff_c[d - kDmaInst] + (uint32_t)s * 64u,
                         lds_c + u * kStageBytes + 16 * (d - kDmaInst) * 64);
        };
        // the codes of unit h (two 16-column k-steps) of B block f as 16-bit
        // values: lane l's 8 bytes of chunks 2h and 2h+1
        auto read_codes = [&](int u, int h, int f) -> v8i {
            const int r = wn * kWaveN + 32 * f + rr_e;
            const uint32_t row = (uint32_t)(u * kStageBytes + kBo + r * 64 + 8 * kh);
            const int sw = (rr_e >> 2) & 3;
            const v2u c0 = lds_load<v2u>(smem, row + (((2 * h) ^ sw) * 16));
            const v2u c1 = lds_load<v2u>(smem, row + (((2 * h + 1) ^ sw) * 16));
            return cat8(codes8_to16<BF16, FP8>(c0), codes8_to16<BF16, FP8>(c1));
        };
        auto read_xo = [&](int u, int h, int i) -> v8i { return read_frag8<TN>(smem, u, h, i, wm, wn, lane_e); };
        constexpr int kNo = kDmaInst + kDmaC;
#pragma unroll
        for (int d = 0; d < kNo; ++d) dma_o(d, 0, 0);
#pragma unroll
        for (int d = 0; d < kNo; ++d) dma_o(d, min(1, no - 1), 1);
        wait_vmcnt<kNo>();
        stage_barrier();
#pragma unroll
        for (int f = 0; f < IB; ++f) ga[f] = read_xo(0, 0, f);
#pragma unroll
        for (int f = 0; f < JB; ++f) gb0[f] = read_codes(0, 0, f);
        // one stage, as the int8 loop's: unit 0 reads unit 1 of the same
        // buffer; kBarrierAt MFMA blocks into unit 1 the barrier, then unit 0
        // of the next stage is read and the stage after it loaded
        auto ostage = [&](int s, int u) {
#pragma unroll
            for (int q = 0; q < IB * JB; ++q) {
                const int i = q / JB, j = q % JB;
                acc[i][j] = __builtin_bit_cast(acc_t, mfma16x2<BF16>(gb0[j], ga[i], __builtin_bit_cast(v16f, acc[i][j])));
                if (q < JB) gb1[q] = read_codes(u, 1, q);
                if (j == JB - 1) ga[i] = read_xo(u, 1, i);
                __builtin_amdgcn_sched_barrier(0);
            }
            const int sn = min(s + 2, no - 1);
#pragma unroll
            for (int q = 0; q < IB * JB; ++q) {
                const int i = q / JB, j = q % JB;
                acc[i][j] = __builtin_bit_cast(acc_t, mfma16x2<BF16>(gb1[j], ga[i], __builtin_bit_cast(v16f, acc[i][j])));
                if (q == kBarrierAt - 1) {
                    __builtin_amdgcn_s_waitcnt(0);
                    stage_barrier();
                }
                if (q >= kBarrierAt) {
                    if (q - kBarrierAt < JB) gb0[q - kBarrierAt] = read_codes(1 - u, 0, q - kBarrierAt);
                    if (j == JB - 1) ga[i] = read_xo(1 - u, 0, i);
                    constexpr int kSlots = IB * JB - kBarrierAt;
                    const int d0 = (q - kBarrierAt) * kNo / kSlots, d1 = (q - kBarrierAt + 1) * kNo / kSlots;
#pragma unroll
                    for (int d = d0; d < d1; ++d) dma_o(d, sn, u);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        const int nfo = o_half ? no - 1 : no;
        int so = 0;
        for (; so + 2 <= nfo; so += 2) {
            ostage(so, 0);
            ostage(so + 1, 1);
        }
        if (so < nfo) ostage(so, 0);
        if (o_half) {
#pragma unroll
            for (int q = 0; q < IB * JB; ++q) {
                const int i = q / JB, j = q % JB;
                acc[i][j] = __builtin_bit_cast(acc_t, mfma16x2<BF16>(gb0[j], ga[i], __builtin_bit_cast(v16f, acc[i][j])));
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        wait_vmcnt<0>();
        __syncthreads();  // the ring is read out before the Y staging

        constexpr int JC = JB < 4 ? JB : 4;  // column blocks per step (registers)
#pragma unroll
        for (int i = 0; i < IB; ++i) {
#pragma unroll
            for (int jb0 = 0; jb0 < JB; jb0 += JC) {
                const int nj = JB - jb0 < JC ? JB - jb0 : JC;
                v16f f[JC];
#pragma unroll
                for (int j = 0; j < JC; ++j)
                    if (j < nj) f[j] = __builtin_bit_cast(v16f, acc[i][jb0 + j]);
                stage_y<BF16, TN, JC>(smem + (i & 1) * y_block_bytes<TN>(), s_sb, s_bias, f, nj, wm * 32 + rr_e,
                                      n_lane + 32 * jb0);
            }
            __syncthreads();  // block row i staged; block row i-1's buffer read out
            store_block<TN>(smem + (i & 1) * y_block_bytes<TN>(), Y, M, N, m0, n0, i, tid_e);
        }
    }
}

// The product's one kernel: workgroup b computes tile b / split (split b %
// split of its K stages) on one of the two paths, chosen by n_out; TN is the
// tile's columns (256 or 224).
template <bool BF16, bool FP8, bool SPLIT, int TN>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void gemm_tiled_kernel(int M, int N, int K, int tiles_m, int tiles_n,
                       const int8_t* __restrict__ CA, const float* __restrict__ SCA,
                       const int32_t* __restrict__ idx, const int32_t* __restrict__ n_out_ptr,
                       const uint16_t* __restrict__ XO, const int8_t* __restrict__ CB,
                       const float* __restrict__ SCB, const uint16_t* __restrict__ bias,
                       uint16_t* __restrict__ Y, int32_t* __restrict__ C_i32,
                       float* __restrict__ C_f32, const int8_t* __restrict__ wo_all,
                       int wo_cap, int wo_min, int split, uint32_t* __restrict__ counters,
                       int32_t* __restrict__ part) {
    __shared__ __attribute__((aligned(16))) int8_t smem[Tile<TN>::kSmemBytes];
    __shared__ float s_sa[BM], s_sb[kThreads], s_bias[kThreads];  // (entries past TN unused)
    __shared__ __attribute__((aligned(16))) uint16_t s_wo[TN * kOutLds];
    __shared__ __attribute__((aligned(16))) uint16_t s_xo[TN == 224 ? 8 : BM * kOutLds];  // (224: in smem)
    __shared__ int s_xcol[kOutLds + 1];
    __shared__ int s_last;
    const int n_out = *n_out_ptr;
    if (outlier_path_takes(n_out, idx, wo_all, wo_cap, FP8 ? C_f32 != nullptr : C_i32 != nullptr)) {
        outlier_body<BF16, FP8, SPLIT, TN>(smem, s_sa, s_sb, s_bias, &s_last, M, N, K, tiles_m, tiles_n, CA, SCA,
                                       idx, n_out_ptr, XO, CB, SCB, bias, Y, C_i32, C_f32, wo_all, wo_cap, split,
                                       counters, part);
        return;
    }
    plain_body<BF16, FP8, SPLIT, TN>(smem, s_sa, s_sb, s_bias, s_wo, s_xo, s_xcol, &s_last, M, N, K, tiles_m, tiles_n, CA, SCA,
                                 idx, n_out_ptr, XO, CB, SCB, bias, Y, C_i32, C_f32, wo_all, wo_cap, wo_min,
                                 split, counters, part);
}

// Bytes of gathered outlier codes for an N x K weight holding `cap` outlier
// columns (a multiple of 64): cap int8 codes per weight row.
static size_t gathered_codes_bytes(int64_t N, int64_t cap) { return (size_t)N * (size_t)cap; }

static int64_t tiles_of(int64_t M, int64_t N, int tn) { return ((M + BM - 1) / BM) * ((N + tn - 1) / tn); }

// Workgroups per tile: split K when the tiles fill at most half the CUs, into
// as many parts as keep one workgroup per CU, each at least kMinSplitStages
// stages long.
static int split_for(int64_t M, int64_t N, int64_t K, int tn) {
    const int64_t tiles = tiles_of(M, N, tn);
    if (tiles == 0 || tiles * 2 > kCUs) return 1;  // (no tiles: an empty call)
    int64_t s = kCUs / tiles;
    if (s > K / BKS / kMinSplitStages) s = K / BKS / kMinSplitStages;
    if (s > kMaxSplit) s = kMaxSplit;
    return s < 1 ? 1 : (int)s;
}

// The tile's columns: 224 where it takes fewer MFMA cycles per CU than 256
// (rounds of kCUs workgroups, each of tn columns and its share of the K
// stages), for instance N = 57344 or 14336 (a factor 7) at M = 512; 256
// otherwise, ties included.  A function of the shape (and of the
// environment variable LLMINT8_TILE_COLS, "256" or "224", which forces one),
// so the workspace size and the launch agree.
static int tile_cols(int64_t M, int64_t N, int64_t K) {
    if (const char* force = std::getenv("LLMINT8_TILE_COLS")) {
        if (std::strcmp(force, "256") == 0) return 256;
        if (std::strcmp(force, "224") == 0) return 224;
    }
    const int64_t nk = (K + BKS - 1) / BKS;
    int best = 256;
    int64_t best_cost = 0;
    for (int tn : {256, 224}) {
        const int split = split_for(M, N, K, tn);
        const int64_t rounds = (tiles_of(M, N, tn) * split + kCUs - 1) / kCUs;
        const int64_t cost = rounds * tn * ((nk + split - 1) / split);
        if (tn == 256 || cost < best_cost) {
            best = tn;
            best_cost = cost;
        }
    }
    return best;
}

static int split_of(int64_t M, int64_t N, int64_t K) { return split_for(M, N, K, tile_cols(M, N, K)); }

// arrival counters (padded to 256 bytes), then split x tiles partial tiles
static size_t split_bytes(int64_t M, int64_t N, int64_t K) {
    const int split = split_of(M, N, K);
    if (split <= 1) return 0;
    const int tn = tile_cols(M, N, K);
    const int64_t tiles = tiles_of(M, N, tn);
    return (((size_t)tiles * 4 + 255) & ~(size_t)255) + (size_t)split * tiles * BM * tn * 4;
}

size_t gemm_tiled_workspace(int64_t M, int64_t N, int64_t K) {
    size_t b = split_bytes(M, N, K);
    if (N > 0 && K > kOutLds) b += gathered_codes_bytes(N, K < kActGatherCols ? K : kActGatherCols);
    return b;
}

// The split region first, when the workspace holds it; the gathered codes
// take the rest: as many multiples of 64 columns as fit, at most K.
TiledLayout tiled_layout(int M, int N, int K, void* ws, size_t ws_bytes) {
    TiledLayout L;
    if (ws == nullptr || M <= 0 || N <= 0) return L;
    char* p = static_cast<char*>(ws);
    const size_t sb = split_bytes(M, N, K);
    if (sb > 0 && ws_bytes >= sb) {
        const int tiles = (int)tiles_of(M, N, tile_cols(M, N, K));
        L.split = split_of(M, N, K);
        L.counters = reinterpret_cast<uint32_t*>(p);
        L.n_counters = tiles;
        L.part = reinterpret_cast<int32_t*>(p + (((size_t)tiles * 4 + 255) & ~(size_t)255));
        p += sb;
        ws_bytes -= sb;
    }
    if (K > kOutLds) {
        const size_t fit = ws_bytes / gathered_codes_bytes(N, 64), k_blocks = (size_t)K / 64;
        L.cap = (int)(fit < k_blocks ? fit : k_blocks) * 64;
        if (L.cap > 0) L.codes = reinterpret_cast<int8_t*>(p);
    }
    // the 224-column tile whose K is not split takes its first kOutLds codes
    // from the B stages (plain_body, kExtract), and at most 128 token rows
    // (one row of tiles, each reading its rows' codes from CB once) skip the
    // gather pass; every other tile reads them from the gather
    L.min_cols = (tile_cols(M, N, K) == 224 && L.split == 1) || M <= kNoGatherRows ? kOutLds : 0;
    return L;
}

hipError_t launch_gemm_tiled(const MatmulArgs& a, hipStream_t stream, hipEvent_t ev_start,
                             hipEvent_t ev_stop) {
    const int tn = tile_cols(a.M, a.N, a.K);
    const int tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + tn - 1) / tn;
    const TiledLayout L = tiled_layout(a.M, a.N, a.K, a.ws, a.ws_bytes);
    int8_t* gather_to = a.codes_gathered ? nullptr : L.codes;
    if (gather_to != nullptr || L.split > 1) {
        // the gather's work items: a chunk of one weight row's outlier
        // columns, 16 per workgroup and pass (sized for one chunk per
        // segment; the workgroups loop over the rest)
        const int64_t items = (int64_t)a.N * ((a.K + kGatherSeg - 1) / kGatherSeg);
        const int64_t want = (items + kGatherThreads / 16 - 1) / (kGatherThreads / 16);
        const int blocks = gather_to == nullptr ? 1 : (int)(want < 2048 ? (want < 1 ? 1 : want) : 2048);
        gemm_prep<<<blocks, kGatherThreads, 0, stream>>>(a.N, a.K, L.cap, L.min_cols, a.idx, a.n_out, a.CB, gather_to,
                                                         L.counters, L.split > 1 ? L.n_counters : 0);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    typedef void (*kernel_t)(int, int, int, int, int, const int8_t*, const float*, const int32_t*,
                             const int32_t*, const uint16_t*, const int8_t*, const float*,
                             const uint16_t*, uint16_t*, int32_t*, float*, const int8_t*, int, int, int,
                             uint32_t*, int32_t*);
    // [columns 224?][split?][bf16?][fp8?]
    static const kernel_t kernels[2][2][2][2] = {
        {{{gemm_tiled_kernel<false, false, false, 256>, gemm_tiled_kernel<false, true, false, 256>},
          {gemm_tiled_kernel<true, false, false, 256>, gemm_tiled_kernel<true, true, false, 256>}},
         {{gemm_tiled_kernel<false, false, true, 256>, gemm_tiled_kernel<false, true, true, 256>},
          {gemm_tiled_kernel<true, false, true, 256>, gemm_tiled_kernel<true, true, true, 256>}}},
        {{{gemm_tiled_kernel<false, false, false, 224>, gemm_tiled_kernel<false, true, false, 224>},
          {gemm_tiled_kernel<true, false, false, 224>, gemm_tiled_kernel<true, true, false, 224>}},
         {{gemm_tiled_kernel<false, false, true, 224>, gemm_tiled_kernel<false, true, true, 224>},
          {gemm_tiled_kernel<true, false, true, 224>, gemm_tiled_kernel<true, true, true, 224>}}}};
    const kernel_t plain = kernels[tn == 224][L.split > 1][a.bf16][a.fp8];
    const int items = tiles_m * tiles_n * L.split;
    // one dispatch; the events (when given) bracket it
    dim3 block(kThreads), grid(items);
#define LLMINT8_GEMM_ARGS                                                                                     \
    a.M, a.N, a.K, tiles_m, tiles_n, a.CA, a.SCA, a.idx, a.n_out, a.XO, a.CB, a.SCB, a.bias, a.Y, a.C_i32, \
        a.C_f32, L.codes, L.cap, L.min_cols, L.split, L.counters, L.part
    if (ev_start || ev_stop) {
        hipExtLaunchKernelGGL(plain, grid, block, 0, stream, ev_start, ev_stop, 0, LLMINT8_GEMM_ARGS);
    } else {
        plain<<<grid, block, 0, stream>>>(LLMINT8_GEMM_ARGS);
    }
#undef LLMINT8_GEMM_ARGS
    return hipGetLastError();
}

}  // namespace llmint8
