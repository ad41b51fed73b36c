// Shared device helpers and kernel launchers of libllmint8 (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "llmint8.h"

namespace llmint8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned short v8u16 __attribute__((ext_vector_type(8)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---- 16-bit <-> fp32 ------------------------------------------------------
template <bool BF16>
__device__ __forceinline__ float widen16(uint16_t bits) {
    if constexpr (BF16) {
        return __builtin_bit_cast(float, (uint32_t)bits << 16);
    } else {
        return (float)__builtin_bit_cast(_Float16, bits);
    }
}

// fp32 -> 16-bit, round to nearest even (finite inputs).
template <bool BF16>
__device__ __forceinline__ uint16_t narrow16(float f) {
    if constexpr (BF16) {
        uint32_t u = __builtin_bit_cast(uint32_t, f);
        u += 0x7FFFu + ((u >> 16) & 1u);
        return (uint16_t)(u >> 16);
    } else {
        return __builtin_bit_cast(uint16_t, (_Float16)f);
    }
}

// ---- magnitudes as 16-bit patterns ----------------------------------------
// For finite fp16/bf16 values, |x| (sign bit cleared) orders like the bit
// pattern read as an unsigned integer, so maxima and threshold tests can run on
// packed u16 pairs and give exactly the fp32 results.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t abs2(uint32_t v) { return v & 0x7fff7fffu; }

__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}

// Packed 16-bit difference (wrapping) and arithmetic shift of each half.
__device__ __forceinline__ uint32_t sub_i16x2(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(i16x2, a) - __builtin_bit_cast(i16x2, b));
}
__device__ __forceinline__ uint32_t ashr16x2(uint32_t a, int s) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(i16x2, a) >> (int16_t)s);
}

// Smallest finite-or-infinite 16-bit magnitude pattern h with value(h) >= t, so
// that for finite x:  |x| >= t  <=>  bits(|x|) >= threshold_bits(t).
template <bool BF16>
__device__ __forceinline__ uint32_t threshold_bits(float t) {
    if (!(t > 0.0f)) return 0u;  // t == 0: every value qualifies
    if constexpr (BF16) {
        if (t == __builtin_inff()) return 0x7F80u;
        uint32_t h = __builtin_bit_cast(uint32_t, t) >> 16;  // truncation toward zero
        if (widen16<true>((uint16_t)h) < t) h += 1;
        return h;
    } else {
        if (t > 65504.0f) return 0x7C00u;  // above the largest finite fp16
        uint32_t h = __builtin_bit_cast(uint16_t, (_Float16)t);
        if (widen16<false>((uint16_t)h) < t) h += 1;
        return h;
    }
}

// ---- absmax quantization of one value ------------------------------------
// scale = 127.0f / absmax is computed once per vector with the correctly
// rounded fp32 divide; q = rne(x * scale) with one fp32 multiply and
// v_rndne_f32, clamped to [-127, 127].
// The int8 code of rne(x * scale) as the low byte of a 32-bit pattern, for
// |x * scale| <= 127.5: the product is rounded to fp32 first, then adding
// 1.5 * 2^23 rounds it to an integer (ties to even), which lands in the low
// mantissa bits.  Contraction must stay off: a fused multiply-add would skip
// the product's rounding and change ties.
__device__ __forceinline__ uint32_t quantize_low_byte(float x, float scale) {
#pragma clang fp contract(off)
    const float p = x * scale;
    return __builtin_bit_cast(uint32_t, p + 12582912.0f);
}

// The same code from a 16-bit value: fma(x, scale, +0) rounds the exact
// product once, as the fp32 multiply of the (exactly) widened x does, in one
// v_fma_mix_f32 that widens x itself.  A -0 product becomes +0, whose code is
// 0 as well.
__device__ __forceinline__ uint32_t quantize_low_byte_f16(_Float16 x, float scale) {
#pragma clang fp contract(off)
    const float p = __builtin_fmaf((float)x, scale, 0.0f);
    return __builtin_bit_cast(uint32_t, p + 12582912.0f);
}

__device__ __forceinline__ int quantize_value(float x, float scale) {
    float p = x * scale;
    float r = __builtin_rintf(p);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

// ---- FP8 E4M3 codes (the 8-bit floating-point variant) --------------------
// The zhichai.top summary of LLM.int8() (outlook section) names an 8-bit
// floating-point type as future work for the method.  The variant here uses
// OCP E4M3, the format gfx950's fp8 matrix instructions take: code =
// e4m3(x * scale), scale = 448.0f / absmax, one fp32 multiply and then
// v_cvt_pk_fp8_f32 (round to nearest, ties to even, subnormals kept, a result
// that rounds to zero keeps its sign).  |x * scale| <= 448 (1 + 2^-23) < 464,
// the magnitude from which the conversion would return NaN.
typedef long v2l __attribute__((ext_vector_type(2)));
typedef int v8i __attribute__((ext_vector_type(8)));

template <bool FP8>
__device__ __forceinline__ constexpr float code_max() {
    return FP8 ? 448.0f : 127.0f;
}

// four codes, value a in the lowest byte.  The first conversion's untouched
// upper half is overwritten by the second, so its "old" operand can be any
// register (here pa's own bits: no register has to be zeroed).
__device__ __forceinline__ uint32_t e4m3_pack4_products(float pa, float pb, float pc, float pd) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(pa, pb, __builtin_bit_cast(int, pa), false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(pc, pd, w, true);
    return (uint32_t)w;
}
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d, float scale) {
#pragma clang fp contract(off)
    return e4m3_pack4_products(a * scale, b * scale, c * scale, d * scale);
}
// The same codes from 16-bit values: fma(x, scale, -0) is the fp32 product of
// the exactly widened x, signed zeros included (-0 + -0 = -0, +0 + -0 = +0),
// in one v_fma_mix_f32 that widens x itself.  The -0 is passed in a register
// the compiler cannot see through (it would rewrite the fma as a multiply,
// which takes a separate widening instruction).
__device__ __forceinline__ float opaque_neg_zero() {
    uint32_t b = 0x80000000u;
    asm volatile("" : "+s"(b));
    return __builtin_bit_cast(float, b);
}
__device__ __forceinline__ uint32_t e4m3_pack4_f16(_Float16 a, _Float16 b, _Float16 c, _Float16 d, float scale,
                                                   float nz) {
    return e4m3_pack4_products(__builtin_fmaf((float)a, scale, nz), __builtin_fmaf((float)b, scale, nz),
                               __builtin_fmaf((float)c, scale, nz), __builtin_fmaf((float)d, scale, nz));
}

// value of a code byte: the int8 value, or the E4M3 value (exact in fp32)
template <bool FP8>
__device__ __forceinline__ float code_value(int8_t b) {
    if constexpr (FP8)
        return __builtin_amdgcn_cvt_f32_fp8((int)(uint8_t)b, 0);
    else
        return (float)b;
}

// ---- weight codes at the outlier columns, gathered for the tiled product ---
// The tiled product multiplies XO [M, n_pad] by the weight codes at the
// outlier columns in 64-column stages.  When those columns are not simply
// 0 .. n_out-1 (then the codes are CB's own first columns), they are gathered
// once per call into a row-major buffer of `cap` bytes per weight row (cap a
// multiple of 64, n_pad <= cap): byte c of row n is CB[n][col(c)] for
// c < n_out and 0 for n_out <= c < n_pad (code 0 is +0 in both formats).
// The product stages the codes of the first kOutLds columns in LDS for its
// epilogue, from this buffer when it holds them (any count up to cap; at
// most kOutLds columns sit in rows of kOutLds bytes: gather_first_codes).
constexpr int kOutLds = 16;

// The gather runs over chunks of the outlier list, the same for every weight
// row: a dense chunk is every outlier column of one kGatherSeg-byte segment
// of the row holding at least kGatherDense of them (the segment is read whole,
// coalesced, and the codes picked from LDS); a sparse chunk is up to
// kGatherRun consecutive outlier columns from sparser segments (one byte load
// each).
// Chunk i covers outlier columns lo[i] .. lo[i+1]-1; seg[i] is its segment
// (dense) or -1.
constexpr int kGatherSeg = 1024, kGatherDense = 16, kGatherRun = 64;
constexpr int kGatherSegMax = (LLMINT8_K_MAX + kGatherSeg - 1) / kGatherSeg;
// Chunks: at most one dense chunk per segment; the sparse columns (under
// kGatherDense per segment) fill a chunk every kGatherRun, plus one cut short
// at each dense segment: under 3 per segment.
constexpr int kGatherChunksMax = 3 * kGatherSegMax + 1;
struct GatherChunks {
    int n;
    int lo[kGatherChunksMax + 1];
    short seg[kGatherChunksMax];
};
struct GatherChunk {
    int lo, hi, seg;
};

// Whether every chunk may be sparse without a look at the segments: fewer
// than kGatherDense outlier columns per segment on average (a dense segment
// among them is then gathered with byte loads, the same codes).  Chunk i is
// then columns kGatherRun i .. kGatherRun (i+1) - 1.
__device__ __forceinline__ bool gather_all_sparse(int K, int n_out) {
    return (int64_t)n_out * kGatherSeg < (int64_t)kGatherDense * K;
}

// One thread builds the chunk list (seg_count(s): the number of outlier
// columns below kGatherSeg s, seg_count(nseg) = n_out).
template <typename SegCount>
__device__ __forceinline__ void build_gather_chunks(int K, int n_out, SegCount seg_count, GatherChunks& g) {
    const int nseg = (K + kGatherSeg - 1) / kGatherSeg;
    int n = 0, run = -1;  // run: first column of the open sparse chunk
    int next = seg_count(0);
    for (int sg = 0; sg < nseg; ++sg) {
        const int lo = next, hi = seg_count(sg + 1);
        next = hi;
        if (hi - lo >= kGatherDense) {
            if (run >= 0) {
                g.lo[n] = run;
                g.seg[n++] = -1;
                run = -1;
            }
            g.lo[n] = lo;
            g.seg[n++] = (short)sg;
        } else if (hi > lo) {
            if (run < 0) run = lo;
            for (; hi - run > kGatherRun; run += kGatherRun) {  // the open chunk is full
                g.lo[n] = run;
                g.seg[n++] = -1;
            }
        }
    }
    if (run >= 0) {
        g.lo[n] = run;
        g.seg[n++] = -1;
    }
    g.lo[n] = n_out;
    g.n = n;
}

// At most kOutLds outlier columns: their codes in rows of kOutLds bytes
// instead (byte e of row n is CB[n][col(e)] for e < n_out, 0 after), which
// the product reads 16 adjacent bytes per weight row.  One (row, column) item
// per thread of the t0 / nt grid share, four items per thread in flight at
// once; no barriers.
template <typename Col>
__device__ __forceinline__ void gather_first_codes(int N, int K, int n_out, Col col, const int8_t* __restrict__ CB,
                                                   int8_t* __restrict__ out, int64_t t0, int64_t nt) {
    const int64_t items = (int64_t)N * kOutLds;
    for (int64_t base = t0; base < items; base += 4 * nt) {
        int8_t v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = min(base + u * nt, items - 1);  // (past the end: re-read the last item)
            const int e = (int)(i & (kOutLds - 1)), n = (int)(i / kOutLds);
            v[u] = CB[(size_t)n * K + col(min(e, n_out - 1))];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = base + u * nt;
            if (i < items) out[i] = (int)(i & (kOutLds - 1)) < n_out ? v[u] : (int8_t)0;
        }
    }
}

// Work items (weight row n, chunk i < nch; chunk(i) its columns and segment),
// one per 16-lane group of a THREADS-thread
// workgroup, THREADS / 16 per workgroup and pass (wg = this workgroup's rank
// among n_wg).  A group writes its chunk's codes to out[n * cap + j], 16
// consecutive j per store instruction; the group of chunk 0 also writes the
// zeros at n_out .. n_pad-1.  buf: kGatherSeg bytes per group.  Every thread
// of the workgroup calls it (it holds barriers).
template <int THREADS, typename Col, typename Chunk>
__device__ __forceinline__ void gather_codes(int N, int K, int cap, int n_out, Col col, int nch, Chunk chunk,
                                             const int8_t* __restrict__ CB, int8_t* __restrict__ out,
                                             int8_t* buf, int tid, int wg, int n_wg) {
    constexpr int kGroups = THREADS / 16;
    const int n_pad = (n_out + 31) & ~31;
    const int grp = tid >> 4, q = tid & 15;
    int8_t* gb = buf + grp * kGatherSeg;
    const int64_t items = (int64_t)N * nch;
    for (int64_t base = (int64_t)wg * kGroups; base < items; base += (int64_t)n_wg * kGroups) {
        const int64_t e = base + grp;
        const bool ok = e < items;
        const int n = ok ? (int)(e / nch) : 0, ch = ok ? (int)(e - (int64_t)n * nch) : 0;
        const GatherChunk c_ = ok ? chunk(ch) : GatherChunk{0, 0, -1};
        const int lo = c_.lo, hi = c_.hi, sg = c_.seg;
        const int8_t* row = CB + (size_t)n * K;
        if (sg >= 0) {
            v4i v[kGatherSeg / 256];
#pragma unroll
            for (int u = 0; u < kGatherSeg / 256; ++u) {
                const int o = sg * kGatherSeg + 256 * u + 16 * q;
                v[u] = o < K ? *reinterpret_cast<const v4i*>(row + o) : v4i{0, 0, 0, 0};
            }
#pragma unroll
            for (int u = 0; u < kGatherSeg / 256; ++u) *reinterpret_cast<v4i*>(gb + 256 * u + 16 * q) = v[u];
        }
        __syncthreads();
        // 64 codes per round, 4 per lane, every read issued before the stores
        // (reads past the chunk re-read its last column and are not stored)
        int8_t* orow = out + (size_t)n * cap;
        for (int j0 = lo; j0 < hi; j0 += 64) {
            int8_t b[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int c = col(min(j0 + q + 16 * t, hi - 1));
                b[t] = sg >= 0 ? gb[c - sg * kGatherSeg] : row[c];
            }
#pragma unroll
            for (int t = 0; t < 4; ++t)
                if (j0 + q + 16 * t < hi) orow[j0 + q + 16 * t] = b[t];
        }
        if (ok && ch == 0)
            for (int j = n_out + q; j < n_pad; j += 16) orow[j] = 0;
        __syncthreads();  // the group's buffer is read out before the next pass
    }
}

// ---- cross-lane reductions and scans with DPP (no LDS round trips) --------
// DPP controls of the gfx9 family: quad_perm, row_shr:n (0x110 + n), row_mirror
// (0x140), row_half_mirror (0x141), row_bcast:15 (0x142), row_bcast:31 (0x143).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i(int old, int v) {
    return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xF, false);
}

// max over the 64 lanes, returned to every lane (v >= 0 or any finite value)
// max over 16-lane rows of packed u16 pairs: afterwards lanes 0, 16, 32 and 48
// hold their row's maxima (every lane of a row holds the same value)
__device__ __forceinline__ uint32_t row16_max_u16x2(uint32_t v) {
    v = max_u16x2(v, (uint32_t)dpp_i<0xB1>(0, (int)v));
    v = max_u16x2(v, (uint32_t)dpp_i<0x4E>(0, (int)v));
    v = max_u16x2(v, (uint32_t)dpp_i<0x141>(0, (int)v));
    v = max_u16x2(v, (uint32_t)dpp_i<0x140>(0, (int)v));
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, __builtin_bit_cast(float, dpp_i<0xB1>(0, __builtin_bit_cast(int, v))));   // xor 1
    v = fmaxf(v, __builtin_bit_cast(float, dpp_i<0x4E>(0, __builtin_bit_cast(int, v))));   // xor 2
    v = fmaxf(v, __builtin_bit_cast(float, dpp_i<0x141>(0, __builtin_bit_cast(int, v))));  // half-row
    v = fmaxf(v, __builtin_bit_cast(float, dpp_i<0x140>(0, __builtin_bit_cast(int, v))));  // row
    const int b = __builtin_bit_cast(int, v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// inclusive prefix sum over the 64 lanes
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += dpp_i<0x111>(0, v);        // row_shr:1 (lanes without a source add 0)
    v += dpp_i<0x112>(0, v);        // row_shr:2
    v += dpp_i<0x114>(0, v);        // row_shr:4
    v += dpp_i<0x118>(0, v);        // row_shr:8
    v += dpp_i<0x142, 0xA>(0, v);   // row_bcast:15 into rows 1 and 3
    v += dpp_i<0x143, 0xC>(0, v);   // row_bcast:31 into rows 2 and 3
    return v;
}

// max over the 64 lanes (unsigned), returned to every lane
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)dpp_i<0xB1>(0, (int)v));
    v = max(v, (uint32_t)dpp_i<0x4E>(0, (int)v));
    v = max(v, (uint32_t)dpp_i<0x141>(0, (int)v));
    v = max(v, (uint32_t)dpp_i<0x140>(0, (int)v));
    const uint32_t r0 = __builtin_amdgcn_readlane((int)v, 0), r1 = __builtin_amdgcn_readlane((int)v, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane((int)v, 32), r3 = __builtin_amdgcn_readlane((int)v, 48);
    return max(max(r0, r1), max(r2, r3));
}

__device__ __forceinline__ int wave_sum(int v) {
    return __builtin_amdgcn_readlane(wave_incl_scan(v), 63);
}

// ---- LDS-DMA and explicit waits -------------------------------------------
// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// workgroup barrier without the memory fence of __syncthreads (the LDS-DMA
// completions are awaited explicitly with vmcnt); the empty asm keeps the
// compiler from moving LDS accesses across it
__device__ __forceinline__ void stage_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// One global_load_lds_dwordx4: lane p's 16 bytes at gptr land in LDS at
// lds_addr + 16 p.  Issued through asm so the compiler does not treat later LDS
// reads as possibly aliasing it (it would wait for every load in flight); the
// waits are explicit (wait_vmcnt + stage_barrier).  M0 is saved and restored.
__device__ __forceinline__ void dma16(const int8_t* gptr, uint32_t lds_addr) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_addr), "v"(gptr)
        : "memory");
}

// A raw buffer descriptor (stride 0, 32-bit data format) for `bytes` bytes
// from `base`, in scalar registers.  Loads through it at offsets >= bytes
// return 0 and touch no memory.
__device__ __forceinline__ v4i buffer_rsrc(const void* base, uint32_t bytes) {
    const uint64_t b = (uint64_t)(uintptr_t)base;
    v4i r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));  // base[47:32], stride 0
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);                // num_records
    r[3] = 0x00020000;                                                // data format 32
    return r;
}

// One buffer_load_dwordx4 ... lds: lane p's 16 bytes at byte offset voff of
// the buffer land in LDS at lds_addr + 16 p (offsets past the buffer's size
// read 0).  Issued through asm for the same reasons as dma16; M0 is saved and
// restored.
__device__ __forceinline__ void dma_line(const v4i& rsrc, uint32_t voff, uint32_t lds_addr) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_addr), "v"(voff), "s"(rsrc)
        : "memory");
}

__device__ __forceinline__ uint32_t lds_address(const int8_t* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) int8_t*)p;
}

// LDS accesses with 32-bit addressing: base + byte offset in address space 3.
// (Generic-pointer arithmetic on an LDS array can be done in 64 bits, with an
// operand register that may still be the target of a load in flight, which
// then forces a wait for that load.)
template <typename T>
__device__ __forceinline__ T lds_load(const void* base, uint32_t byte_off) {
    typedef const __attribute__((address_space(3))) char* lds_cptr;
    return *(const __attribute__((address_space(3))) T*)((lds_cptr)base + byte_off);
}
template <typename T>
__device__ __forceinline__ void lds_store(void* base, uint32_t byte_off, T v) {
    typedef __attribute__((address_space(3))) char* lds_ptr;
    *(__attribute__((address_space(3))) T*)((lds_ptr)base + byte_off) = v;
}

// ---- launchers (each returns hipGetLastError() after its launches) --------
// fp8: E4M3 codes (scale 448/absmax) instead of int8 (127/absmax)
hipError_t launch_quantize_weight(const void* W, bool bf16, bool fp8, int N, int K, int8_t* CB,
                                  float* SCB, hipStream_t stream);

// Per-tensor absmax quantization (one scale for the whole tensor, written to
// every row's scale); workspace of quantize_tensor_workspace() bytes.
size_t quantize_tensor_workspace();
hipError_t launch_quantize_tensor(const void* A, bool bf16, int64_t rows, int64_t cols, int8_t* Q,
                                  float* scale, void* ws, hipStream_t stream);

// Weight codes the activation kernel gathers (layout above) for the tiled
// product that follows it, at most kActGatherCols columns, and only for more
// than min_cols of them; out == nullptr: none.  The launcher clears out when
// it did not gather.
constexpr int kActGatherCols = 1024;
struct CodeGather {
    const int8_t* CB = nullptr;
    int N = 0, cap = 0, min_cols = 0;
    int8_t* out = nullptr;
};

size_t quantize_act_workspace(int64_t M, int64_t K);
hipError_t launch_quantize_act(const void* X, bool bf16, bool fp8, int M, int K, float threshold,
                               int8_t* CA, float* SCA, int32_t* idx, int32_t* n_out, void* XO,
                               void* ws, hipStream_t stream, CodeGather* gather = nullptr);

// CA / CB hold int8 codes, or E4M3 code bytes when fp8 is set; the product is
// exported to C_i32 (int8) or C_f32 (fp8, the fp32 accumulation) when given.
struct MatmulArgs {
    bool bf16;
    bool fp8;
    int M, N, K;
    const int8_t* CA;
    const float* SCA;
    const int32_t* idx;
    const int32_t* n_out;
    const uint16_t* XO;
    const int8_t* CB;
    const float* SCB;
    const uint16_t* bias;
    uint16_t* Y;
    int32_t* C_i32;
    float* C_f32;
    void* ws;
    size_t ws_bytes;
    bool codes_gathered = false;  // the activation kernel filled the workspace's codes
};

size_t matmul_workspace(int64_t M, int64_t N, int64_t K);
size_t gemm_tiled_workspace(int64_t M, int64_t N, int64_t K);
// How the tiled product uses a workspace: split-K arrival counters and
// partial tiles (split > 1), then the gathered outlier codes (cap columns),
// gathered when there are more than min_cols outlier columns (kOutLds for the
// tile that takes its first kOutLds codes from its own K loop, else 0).
struct TiledLayout {
    int split = 1;
    uint32_t* counters = nullptr;
    int n_counters = 0;
    int32_t* part = nullptr;
    int8_t* codes = nullptr;
    int cap = 0;
    int min_cols = 0;
};
TiledLayout tiled_layout(int M, int N, int K, void* ws, size_t ws_bytes);
hipError_t launch_matmul(const MatmulArgs& a, hipStream_t stream, hipEvent_t ev_start,
                         hipEvent_t ev_stop);

// Fused one-launch forward for small M (activation quantization + product).
bool linear_small_m_supported(int M, int K);
hipError_t launch_linear_small_m(const void* X, bool bf16, int M, int N, int K, float t,
                                 const int8_t* CB, const float* SCB, const void* bias, void* Y,
                                 int8_t* CA, float* SCA, int32_t* idx, int32_t* n_out, void* XO,
                                 int32_t* C_i32, hipStream_t stream, hipEvent_t ev_start,
                                 hipEvent_t ev_stop);

// Fused one-launch forward for decode batches (M <= 8, M*K <= 32768), int8
// or FP8 codes (the product to C_i32 or C_f32).  Preferred over
// launch_linear_small_m.
bool linear_decode_supported(int M, int K);
hipError_t launch_linear_decode(const void* X, bool bf16, bool fp8, int M, int N, int K, float t,
                                const int8_t* CB, const float* SCB, const void* bias, void* Y,
                                int8_t* CA, float* SCA, int32_t* idx, int32_t* n_out, void* XO,
                                int32_t* C_i32, float* C_f32, hipStream_t stream,
                                hipEvent_t ev_start, hipEvent_t ev_stop);

// Kernel families used by launch_matmul.
constexpr int kSmallM = 16;  // M <= kSmallM takes the streaming kernel
// More than 8 rows with at least 256 x 64 output channels: workgroups of 64
// channels (four groups of 16), each reading the M x K activations once for
// 64 weight rows instead of 16. Up to 8 rows those re-reads are small and
// the finer grid of 16-channel workgroups balances better (4 x 28672 x 16384:
// 135 us in workgroups of 64 channels, 123 in workgroups of 16).
inline bool small_m_wide(int64_t M, int64_t N) { return M > 8 && N >= 64 * 256; }
// Whether the streaming kernel's grid is one round of the chip: up to 32
// rows, 512 workgroups of 64 or of 16 channels (two per CU); above, 256 of
// 64 (one per CU). Workgroups of 16 channels with four groups of 16 rows lost
// to the tiled product even in one round (64 x 8192 x 28672 150 against
// 140 us).
inline bool small_m_one_round(int64_t M, int64_t N) {
    if (M <= 32) return (N + (small_m_wide(M, N) ? 63 : 15)) / (small_m_wide(M, N) ? 64 : 16) <= 512;
    return small_m_wide(M, N) && (N + 63) / 64 <= 256;
}
// Up to 64 rows the streaming kernel (1, 2 or 4 groups of 16 rows) also takes
// shapes whose M * N * K is at most kSmallMWork, and any whose grid is one
// round: each workgroup's time grows with K and every further round adds one,
// while the tiled product runs one row of 256-row tiles over the whole weight
// (measured, against the tiled product: 17 x 28672 x 8192 68 against 76 us,
// 64 x 16384 x 4096 49 against 66, 64 x 16384 x 16384 100 against 126,
// 32 x 16384 x 8192 46 against 63, 32 x 8192 x 28672 95 against 136; above
// both, 64 x 20480 x 8192 113 against 90 and 32 x 57344 x 8192 183 against
// 121)
constexpr int64_t kSmallMMaxRows = 64;
constexpr int64_t kSmallMWork = 6000000000LL;
inline bool small_m_product(int64_t M, int64_t N, int64_t K) {
    return M <= kSmallM ||
           (M <= kSmallMMaxRows && (M * N * K <= kSmallMWork || small_m_one_round(M, N)));
}
hipError_t launch_gemm_small_m(const MatmulArgs& a, hipStream_t stream, hipEvent_t ev_start,
                               hipEvent_t ev_stop);
hipError_t launch_gemm_tiled(const MatmulArgs& a, hipStream_t stream, hipEvent_t ev_start,
                             hipEvent_t ev_stop);

}  // namespace llmint8
