// Tiled LLM.int8() product for prefill shapes, bound by int8 MFMA throughput.
//
// "A Gentle Introduction to 8-bit Matrix Multiplication for transformers at
// scale": section "LLM.int8() summary" (non-outliers in int8, outliers in
// 16-bit, dequantize and add), section "inside the MatMul" (row-wise scales
// for the hidden states, per-output-channel scales for the weight), section
// "absmax quantization" (denormalize by the outer product of the two absmax
// vectors), section "Usage" (recovered weight CB * SCB / 127).
//
// Design (gfx950, 256 CUs in 8 XCDs, 160 KiB LDS per CU):
//  * Workgroup tile 256 x 256, K step 128 bytes; 4 waves in a 2 x 2 grid, each
//    wave owns a 128 x 128 sub-tile = 4 x 4 v_mfma_i32_32x32x32_i8 blocks
//    (256 int32 accumulators per lane, kept in AGPRs).  One workgroup per CU.
//  * CA [M,K] and CB [N,K] are both K-contiguous.  Each K step loads 2 x 32 KiB
//    with 16-byte global loads (8 lanes cover one 128-byte row slice) into
//    registers while the MFMAs run on the other LDS buffer (2 x 64 KiB double
//    buffer, one barrier per step).  LDS rows are 128 bytes with the 16-byte
//    slots XOR-swizzled by (row & 7), so both the 16-byte stores and the
//    16-byte fragment reads of 8 consecutive rows hit distinct banks.
//  * Tile order: blocks are dispatched round-robin over the 8 XCDs; block b is
//    remapped so that each XCD walks a contiguous range of a grouped raster
//    (8 tile rows per group), which keeps an XCD's tiles on shared CA/CB
//    panels in its own L2.
//  * Epilogue, fused: int32 -> fp32 times SCA[m]/127; the outlier columns
//    (n_out read from device memory, no host sync) run as
//    v_mfma_f32_32x32x16_{f16,bf16} of XO against the int8 weights gathered
//    at idx and converted exactly to 16-bit, accumulating into the same
//    registers; then times SCB[n]/127, plus bias, round to 16-bit, store.
#include "common.h"

namespace llmint8 {

namespace {

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int kThreads = 256;
constexpr int kGroupM = 8;

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

template <bool BF16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_tiled_kernel(int M, int N, int K, int tiles_m, int tiles_n,
                       const int8_t* __restrict__ CA, const float* __restrict__ SCA,
                       const int32_t* __restrict__ idx, const int32_t* __restrict__ n_out_ptr,
                       const uint16_t* __restrict__ XO, const int8_t* __restrict__ CB,
                       const float* __restrict__ SCB, const uint16_t* __restrict__ bias,
                       uint16_t* __restrict__ Y, int32_t* __restrict__ C_i32) {
    __shared__ __attribute__((aligned(16))) int8_t smem[2][2][BM * BK];
    __shared__ float s_sa[BM], s_sb[BN];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    int tm, tn;
    map_tile(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    // global -> LDS: thread owns rows lrow + 32 i (i < 8), 16-byte slot lchk
    const int lrow = tid >> 3, lchk = tid & 7;
    const int lslot = (lchk ^ (lrow & 7)) * 16;
    const int8_t* pA = CA + (size_t)(m0 + lrow) * K + lchk * 16;
    const int8_t* pB = CB + (size_t)(n0 + lrow) * K + lchk * 16;
    const int a_rows = M - m0 - lrow;  // row i valid iff 32 i < a_rows
    const int b_rows = N - n0 - lrow;
    v4i ra[8], rb[8];

    auto gload = [&](int kt) {
        const bool kok = kt * BK + lchk * 16 < K;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            ra[i] = (kok && 32 * i < a_rows)
                        ? *reinterpret_cast<const v4i*>(pA + (size_t)(32 * i) * K + kt * BK)
                        : v4i{0, 0, 0, 0};
            rb[i] = (kok && 32 * i < b_rows)
                        ? *reinterpret_cast<const v4i*>(pB + (size_t)(32 * i) * K + kt * BK)
                        : v4i{0, 0, 0, 0};
        }
    };
    auto lstore = [&](int buf) {
        int8_t* sA = smem[buf][0];
        int8_t* sB = smem[buf][1];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            *reinterpret_cast<v4i*>(sA + (lrow + 32 * i) * BK + lslot) = ra[i];
            *reinterpret_cast<v4i*>(sB + (lrow + 32 * i) * BK + lslot) = rb[i];
        }
    };

    v16i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v16i{};

    const int r32 = lane & 31, kh = lane >> 5;
    auto compute = [&](int buf) {
        const int8_t* sA = smem[buf][0] + (wm * 128 + r32) * BK;
        const int8_t* sB = smem[buf][1] + (wn * 128 + r32) * BK;
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            const int slot = ((2 * ks + kh) ^ (r32 & 7)) * 16;
            v4i a[4], b[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                a[t] = *reinterpret_cast<const v4i*>(sA + t * 32 * BK + slot);
                b[t] = *reinterpret_cast<const v4i*>(sB + t * 32 * BK + slot);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    };

    const int nk = (K + BK - 1) / BK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
        compute(buf);
        if (kt + 1 < nk) lstore(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue ----------------------------------------------------------
    if (tid < BM) {
        const int m = m0 + tid;
        s_sa[tid] = m < M ? SCA[m] / 127.0f : 0.0f;
        const int n = n0 + tid;
        s_sb[tid] = n < N ? SCB[n] / 127.0f : 0.0f;
    }
    __syncthreads();

    // accumulator register v of lane l in a 32x32 block: row 8(v/4) + 4(l/32) + v%4, col l%32
    const int row_base = wm * 128 + 4 * kh;  // + 32 i + 8 (v/4) + v%4
    const int col_base = wn * 128 + r32;     // + 32 j

    if (C_i32) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int m = m0 + row_base + 32 * i + 8 * (v >> 2) + (v & 3);
                    const int n = n0 + col_base + 32 * j;
                    if (m < M && n < N) C_i32[(size_t)m * N + n] = acc[i][j][v];
                }
    }

    v16f f[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float sa = s_sa[row_base + 32 * i + 8 * (v >> 2) + (v & 3)];
#pragma unroll
            for (int j = 0; j < 4; ++j) f[i][j][v] = (float)acc[i][j][v] * sa;
        }

    const int n_out = *n_out_ptr;
    if (n_out > 0) {
        typedef typename Vec16<BF16>::type vec_t;
        const int n_pad = (n_out + 31) & ~31;
        for (int j0 = 0; j0 < n_out; j0 += 16) {
            vec_t xa[4], xb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = m0 + wm * 128 + 32 * i + r32;
                v8u16 raw = m < M ? *reinterpret_cast<const v8u16*>(XO + (size_t)m * n_pad + j0 + 8 * kh)
                                  : v8u16{0, 0, 0, 0, 0, 0, 0, 0};
                xa[i] = __builtin_bit_cast(vec_t, raw);
            }
            int kcol[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int j = j0 + 8 * kh + e;
                kcol[e] = j < n_out ? idx[j] : -1;
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int n = n0 + col_base + 32 * jj;
                const int8_t* cb = CB + (size_t)(n < N ? n : 0) * K;
                v8u16 raw;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float w = (kcol[e] >= 0 && n < N) ? (float)cb[kcol[e]] : 0.0f;
                    raw[e] = narrow16<BF16>(w);  // |w| <= 127: exact in fp16 and bf16
                }
                xb[jj] = __builtin_bit_cast(vec_t, raw);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) f[i][jj] = mfma16<BF16>(xa[i], xb[jj], f[i][jj]);
        }
    }

#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int nl = col_base + 32 * j;
        const int n = n0 + nl;
        if (n >= N) continue;
        const float sb = s_sb[nl];
        const float bv = bias ? widen16<BF16>(bias[n]) : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = m0 + row_base + 32 * i + 8 * (v >> 2) + (v & 3);
                if (m < M) Y[(size_t)m * N + n] = narrow16<BF16>(f[i][j][v] * sb + bv);
            }
    }
}

}  // namespace

hipError_t launch_gemm_tiled(const MatmulArgs& a, hipStream_t stream, hipEvent_t ev_start,
                             hipEvent_t ev_stop) {
    const int tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
    dim3 grid(tiles_m * tiles_n), block(kThreads);
    void (*fn)(int, int, int, int, int, const int8_t*, const float*, const int32_t*,
               const int32_t*, const uint16_t*, const int8_t*, const float*, const uint16_t*,
               uint16_t*, int32_t*) = a.bf16 ? gemm_tiled_kernel<true> : gemm_tiled_kernel<false>;
    if (ev_start || ev_stop) {
        hipExtLaunchKernelGGL(fn, grid, block, 0, stream, ev_start, ev_stop, 0, a.M, a.N, a.K,
                              tiles_m, tiles_n, a.CA, a.SCA, a.idx, a.n_out, a.XO, a.CB, a.SCB,
                              a.bias, a.Y, a.C_i32);
    } else {
        fn<<<grid, block, 0, stream>>>(a.M, a.N, a.K, tiles_m, tiles_n, a.CA, a.SCA, a.idx, a.n_out,
                                       a.XO, a.CB, a.SCB, a.bias, a.Y, a.C_i32);
    }
    return hipGetLastError();
}

}  // namespace llmint8
