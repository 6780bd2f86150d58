// nm_spmm.hip -- product of activations with 2:4 weights kept in the packed form, on gfx950's
// sparse matrix cores (v_smfmac_f32_32x32x32_bf16).
//
// "Accelerating Sparse Deep Neural Networks" summary page, sections 3.1-3.2: the sparse operand
// stays compressed (the kept values plus 2-bit positions) and the matrix unit skips the pruned
// products.  Here Y[t, o] = sum_i X[t, i] * W[o, i] for a linear layer W [out, in] pruned 2:4
// along `in`, read straight from nm_mask_harden_pack's output.
//
// Operand layout of v_smfmac_f32_32x32x32_bf16 (32 x 32 output tile, 32 dense k per
// instruction), measured on the part with one-hot and random operands:
//   A (sparse, 32 x 32 dense = 32 x 16 kept): lane L holds row L%32 and the 8 kept values of the
//     dense groups 4*(L/32) .. 4*(L/32)+3; bits [4g + 2u, 4g + 2u + 2) of the index operand give
//     the position of kept value u of the lane's group g (the upper 16 bits are not read).
//   B (dense, 32 x 32): lane l holds column l%32; element e < 8 is k = 8*(l/32) + e, element
//     e >= 8 is k = 16 + 8*(l/32) + e - 8.
//   D (32 x 32 fp32): lane l, element r is row 8*(r/4) + 4*(l/32) + r%4, column l%32.
// So one lane's index operand is 16 consecutive bits of a packed row's index stream and its A
// values are 8 consecutive packed values: the packed form feeds the instruction unchanged.
//
// Tiling: a block of 512 threads computes a 256 (out) x 256 (token) tile of Y^T (the last tile
// along either side may be partial), each of its 8
// waves a 128 x 64 part as 4 x 2 instruction tiles with fp32 accumulators.  Per stage of 64
// dense k the block stages the packed values (256 rows x 64 B), their index words (256 x 8 B)
// and X (256 tokens x 128 B) in LDS, double buffered: the next stage is loaded from memory into
// registers while the current one runs on the matrix cores, then written to the other buffer,
// with one barrier per stage.  Blocks are numbered so that each XCD (block id mod 8) works on a
// contiguous run of tiles, which share W rows in that XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nm_kernels.hpp"

namespace nm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16_t __attribute__((ext_vector_type(16)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int SP_BM = 256;  // W rows (outputs) per block
constexpr int SP_BN = 256;  // tokens per block
constexpr int SP_AP = 40;   // LDS pitch of a packed-value row, in bf16 (32 kept + 8 padding)
constexpr int SP_BP = 72;   // LDS pitch of an X row, in bf16 (64 + 8 padding)
constexpr int SP_ABUF = SP_BM * SP_AP;
constexpr int SP_BBUF = SP_BN * SP_BP;

constexpr int SP_THREADS = 512;  // 8 waves: 2 along W rows x 4 along tokens, 128 x 64 each

__global__ __launch_bounds__(SP_THREADS) void k_spmm24(SpmmArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    uint16_t* As = smem;                                          // [2][SP_ABUF]
    uint16_t* Bs = smem + 2 * SP_ABUF;                            // [2][SP_BBUF]
    uint32_t* Is = reinterpret_cast<uint32_t*>(smem + 2 * SP_ABUF + 2 * SP_BBUF);  // [2][SP_BM*2]

    // XCD-aware tile order: block b runs on XCD b % 8 and takes tile (b % 8) * chunk + b / 8
    const int64_t ntok = (a.tokens + SP_BN - 1) / SP_BN, nout = (a.out + SP_BM - 1) / SP_BM;
    const int64_t C = ntok % 4 == 0 ? 4 : (ntok % 2 == 0 ? 2 : 1), R = 8 / C;
    const int64_t rt = (ntok + C - 1) / C, ro = (nout + R - 1) / R;   // region size in tiles
    const int64_t x = blockIdx.x % 8, p = blockIdx.x / 8;
    const int64_t ot = (x / C) * ro + p / rt, tt = (x % C) * rt + p % rt;
    if (p >= ro * rt || ot >= nout || tt >= ntok) return;  // whole block
    const int64_t bo = ot * SP_BM, bt = tt * SP_BN;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wo = (wv >> 2) * 128, wt = (wv & 3) * 64;

    // staging: per thread 2 x 16 B of packed values, 4 B of index words, 4 x 16 B of X.  In the
    // last tile of a ragged count, W rows past the end read the last row and tokens past the end
    // the last token; their outputs are computed but not stored.
    const int64_t olast = a.out - 1, o0 = bo + (tid >> 2), o1 = bo + (tid >> 1);
    const uint16_t* va0 = a.values + (o0 < olast ? o0 : olast) * a.vstride + (tid & 3) * 8;
    const uint16_t* va1 = a.values + (o0 + 128 < olast ? o0 + 128 : olast) * a.vstride + (tid & 3) * 8;
    const uint32_t* ia = a.indices + (o1 < olast ? o1 : olast) * a.istride + (tid & 1);
    const int64_t tlast = a.tokens - 1, t0 = bt + (tid >> 3);
    const uint16_t* xa0 = a.x + (t0 < tlast ? t0 : tlast) * a.xstride + (tid & 7) * 8;
    const uint16_t* xa1 = a.x + (t0 + 64 < tlast ? t0 + 64 : tlast) * a.xstride + (tid & 7) * 8;
    const uint16_t* xa2 = a.x + (t0 + 128 < tlast ? t0 + 128 : tlast) * a.xstride + (tid & 7) * 8;
    const uint16_t* xa3 = a.x + (t0 + 192 < tlast ? t0 + 192 : tlast) * a.xstride + (tid & 7) * 8;
    const int la = (tid >> 2) * SP_AP + (tid & 3) * 8;          // + 128 * SP_AP for the second
    const int lx = (tid >> 3) * SP_BP + (tid & 7) * 8;          // + 64 * SP_BP per step
    uint4 ra0, ra1, rx0, rx1, rx2, rx3;
    uint32_t ri;

    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int64_t nk = a.in / 64;
    const int r32 = lane & 31, kg = lane >> 5;

#define NM_SP_GLOAD(ks)                                                                 \
    do {                                                                                \
        ra0 = *reinterpret_cast<const uint4*>(va0 + (ks) * 32);                         \
        ra1 = *reinterpret_cast<const uint4*>(va1 + (ks) * 32);                         \
        ri = ia[(ks) * 2];                                                              \
        rx0 = *reinterpret_cast<const uint4*>(xa0 + (ks) * 64);                         \
        rx1 = *reinterpret_cast<const uint4*>(xa1 + (ks) * 64);                         \
        rx2 = *reinterpret_cast<const uint4*>(xa2 + (ks) * 64);                         \
        rx3 = *reinterpret_cast<const uint4*>(xa3 + (ks) * 64);                         \
    } while (0)
#define NM_SP_LSTORE(buf)                                                               \
    do {                                                                                \
        uint16_t* as_ = As + (buf) * SP_ABUF + la;                                      \
        uint16_t* bs_ = Bs + (buf) * SP_BBUF + lx;                                      \
        *reinterpret_cast<uint4*>(as_) = ra0;                                           \
        *reinterpret_cast<uint4*>(as_ + 128 * SP_AP) = ra1;                             \
        Is[(buf) * SP_BM * 2 + tid] = ri; /* row tid/2, word tid%2 */                   \
        *reinterpret_cast<uint4*>(bs_) = rx0;                                           \
        *reinterpret_cast<uint4*>(bs_ + 64 * SP_BP) = rx1;                              \
        *reinterpret_cast<uint4*>(bs_ + 128 * SP_BP) = rx2;                             \
        *reinterpret_cast<uint4*>(bs_ + 192 * SP_BP) = rx3;                             \
    } while (0)

    NM_SP_GLOAD(0);
    NM_SP_LSTORE(0);
    __syncthreads();
    if (nk > 1) NM_SP_GLOAD(1);
    for (int64_t ks = 0; ks < nk; ++ks) {
        const int cur = (int)(ks & 1);
        const uint16_t* A = As + cur * SP_ABUF;
        const uint16_t* B = Bs + cur * SP_BBUF;
        const uint32_t* I = Is + cur * SP_BM * 2;
#pragma unroll
        for (int h = 0; h < 2; ++h) {  // two instructions of 32 dense k per stage
            bf16x8_t af[4];
            int ai[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = wo + i * 32 + r32;
                af[i] = *reinterpret_cast<const bf16x8_t*>(A + row * SP_AP + h * 16 + kg * 8);
                ai[i] = (int)(I[row * 2 + h] >> (kg * 16));
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int tok = wt + j * 32 + r32;
                const bf16x8_t lo = *reinterpret_cast<const bf16x8_t*>(B + tok * SP_BP + h * 32 + kg * 8);
                const bf16x8_t hi = *reinterpret_cast<const bf16x8_t*>(B + tok * SP_BP + h * 32 + 16 + kg * 8);
                const bf16x16_t bf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(af[i], bf, acc[i][j], ai[i], 0, 0);
            }
        }
        if (ks + 1 < nk) NM_SP_LSTORE(cur ^ 1);
        if (ks + 2 < nk) NM_SP_GLOAD(ks + 2);
        __syncthreads();
    }
#undef NM_SP_GLOAD
#undef NM_SP_LSTORE

    // epilogue: element r of tile (i, j) is W row bo + wo + 32 i + 8 (r/4) + 4 (lane/32) + r%4 and
    // token bt + wt + 32 j + lane%32; four consecutive r are consecutive outputs of one Y row
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t t = bt + wt + j * 32 + r32;
            if (t >= a.tokens) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t o = bo + wo + i * 32 + q * 8 + kg * 4;  // out % 4 == 0: o..o+3 all in or out
                if (o >= a.out) continue;
                const f32x16_t v = acc[i][j];
                if (a.ytype == 0) {
                    *reinterpret_cast<float4*>(static_cast<float*>(a.y) + t * a.ystride + o) =
                        make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
                } else {
                    const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[4 * q]) |
                                        ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[4 * q + 1]) << 16);
                    const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[4 * q + 2]) |
                                        ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[4 * q + 3]) << 16);
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.y) + t * a.ystride + o) = make_uint2(lo, hi);
                }
            }
        }
    }
}

constexpr size_t SP_SMEM = (2 * SP_ABUF + 2 * SP_BBUF) * sizeof(uint16_t) + 2 * SP_BM * 2 * sizeof(uint32_t);

hipError_t launch_spmm24(const SpmmArgs& a, hipStream_t s) {
    // the block's LDS (116 KB) is above the default dynamic limit: allow it for this kernel
    const hipError_t e = hipFuncSetAttribute((const void*)k_spmm24, hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)SP_SMEM);
    if (e != hipSuccess) return e;
    const int64_t ntok = (a.tokens + SP_BN - 1) / SP_BN, nout = (a.out + SP_BM - 1) / SP_BM;
    const int64_t C = ntok % 4 == 0 ? 4 : (ntok % 2 == 0 ? 2 : 1), R = 8 / C;
    const int64_t grid = 8 * ((ntok + C - 1) / C) * ((nout + R - 1) / R);
    k_spmm24<<<dim3((unsigned)grid), SP_THREADS, SP_SMEM, s>>>(a);
    return hipGetLastError();
}

}  // namespace nm
