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
// Tiling (the largest tile of the family, SpTile<8>): a block of 512 threads computes a 256 (out)
// x 256 (token) tile of Y^T (the last tile along either side may be partial), each of its 8 waves
// a 128 x 64 part as 4 x 2 instruction tiles with fp32 accumulators.  A stage covers 64 dense k:
// the packed values (256 rows x 64 B), their index words (256 x 8 B) and X (256 tokens x 128 B),
// 50 KB in LDS.  The 4- and 2-wave tiles (128 and 64 square) scale every stage region with the
// tile, so each wave's share of the loads stays the same.  Three stages live in
// LDS at once and are filled by LDS DMA loads (global_load_lds), which write LDS without passing
// through registers: stage s + 3 is requested once stage s has been read, so memory has about
// two stages of matrix work to answer, and the LDS fragment reads of each half stage overlap the
// matrix instructions of the previous half.  One barrier per stage.  Blocks are numbered so that
// each XCD (block id mod 8) works on a rectangle of tiles, which share W rows and X rows in that
// XCD's L2.
//
// LDS layout.  A DMA load writes its 64 lanes' 16 B chunks to 1 KB of consecutive LDS, lane by
// lane, so the layout in LDS is chosen through the global address each lane loads.  Rows are
// stored unpadded with their 16 B chunks permuted by an XOR of row bits (swz_a, swz_x), so that
// the fragment reads of 8 or 16 consecutive lanes (consecutive rows, one chunk column) fall on
// distinct banks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nm_kernels.hpp"

namespace nm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Tile family.  A block of WAVES waves owns a T x T tile of Y^T with T = 32 * WAVES (256, 128
// or 64), so that every wave's share of a stage's DMA loads is the same: 2 KB of packed values,
// 4 KB of X and 256 B of index words (7 loads).  Waves are laid out WR along W rows by WT along
// tokens, each computing TI x TJ instruction tiles of 32 x 32.
template <int WAVES>
struct SpTile {
    static constexpr int T = 32 * WAVES;             // W rows and tokens per block
    static constexpr int WR = 2;                     // waves along W rows
    static constexpr int WT = WAVES / 2;             // waves along tokens
    static constexpr int TI = T / (32 * WR);         // instruction tiles per wave along W rows
    static constexpr int TJ = T / (32 * WT);         // ... along tokens
    static constexpr int ABYTES = T * 64;            // packed values of a stage: 32 kept bf16 per row
    static constexpr int XBYTES = T * 128;           // X of a stage: 64 bf16 per token
    static constexpr int IBYTES = T * 8;             // index words of a stage: 2 per row
    static constexpr int STAGE = ABYTES + XBYTES + IBYTES;
    static constexpr size_t SMEM = 3 * (size_t)STAGE;  // three stages: 150, 75 or 37.5 KB
    static_assert(WAVES == 2 || WAVES == 4 || WAVES == 8, "tile family");
};

// chunk permutations: 16 B chunk c of packed-value row r sits at chunk c ^ swz_a(r); chunk c of
// X row t at c ^ swz_x(t)
__device__ __forceinline__ int swz_a(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }
__device__ __forceinline__ int swz_x(int t) { return (t ^ (t >> 3)) & 7; }

// SPLIT > 1: the k range is split into SPLIT consecutive parts, part sp taken by blocks
// sp * base .. sp * base + base - 1 (so a block's XCD, its id mod 8, is that of its tile), and
// each part's fp32 tile goes to its own slice of `ws` ([SPLIT][tokens][out]) for
// k_spmm_combine to add in part order.
template <int WAVES, int SPLIT>
__global__ __launch_bounds__(64 * WAVES) void k_spmm24(SpmmArgs a, int64_t base, float* ws) {
    using TL = SpTile<WAVES>;
    constexpr int T = TL::T, TI = TL::TI, TJ = TL::TJ;
    constexpr int SP_ABYTES = TL::ABYTES, SP_XBYTES = TL::XBYTES, SP_STAGE = TL::STAGE;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    // XCD-aware tile order: block b runs on XCD b % 8 and takes tile (b % 8) * chunk + b / 8
    const int64_t ntok = (a.tokens + T - 1) / T, nout = (a.out + T - 1) / T;
    const int64_t C = ntok % 4 == 0 ? 4 : (ntok % 2 == 0 ? 2 : 1), R = 8 / C;
    const int64_t rt = (ntok + C - 1) / C, ro = (nout + R - 1) / R;   // region size in tiles
    const int64_t bx = SPLIT > 1 ? (int64_t)blockIdx.x % base : (int64_t)blockIdx.x;
    const int sp = SPLIT > 1 ? (int)((int64_t)blockIdx.x / base) : 0;
    const int64_t x = bx % 8, p = bx / 8;
    const int64_t ot = (x / C) * ro + p / rt, tt = (x % C) * rt + p % rt;
    if (p >= ro * rt || ot >= nout || tt >= ntok) return;  // whole block
    const int64_t bo = ot * T, bt = tt * T;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wo = (wv / TL::WT) * (32 * TI), wt = (wv % TL::WT) * (32 * TJ);

    // DMA sources.  Per stage each wave fills 2 KB of packed values, 4 KB of X and 256 B of
    // index words; lane `lane` of the wave's k-th 1 KB piece fills 16 B slot piece * 64 + lane
    // of the region.  In the last tile of a ragged count, W rows past the end load the last row
    // and tokens past the end the last token; their outputs are computed but not stored.
    const int64_t olast = a.out - 1, tlast = a.tokens - 1;
    auto orow = [&](int r) { const int64_t o = bo + r; return o < olast ? o : olast; };
    auto trow = [&](int t) { const int64_t u = bt + t; return u < tlast ? u : tlast; };
    auto asrc = [&](int s) {  // slot = row * 4 + stored chunk
        return a.values + orow(s >> 2) * a.vstride + (((s & 3) ^ swz_a(s >> 2)) << 3);
    };
    auto xsrc = [&](int s) {  // slot = token * 8 + stored chunk
        return a.x + trow(s >> 3) * a.xstride + (((s & 7) ^ swz_x(s >> 3)) << 3);
    };
    const int sa = wv * 128 + lane, sx = wv * 256 + lane, si = wv * 64 + lane;
    // this part's stages (64 dense k each): k0 .. k0 + nk - 1 (the whole row without a split)
    const int64_t nall = a.in / 64, k0 = sp * nall / SPLIT, nk = (sp + 1) * nall / SPLIT - k0;
    const uint16_t* ga0 = asrc(sa) + k0 * 32;
    const uint16_t* ga1 = asrc(sa + 64) + k0 * 32;
    const uint16_t* gx0 = xsrc(sx) + k0 * 64;
    const uint16_t* gx1 = xsrc(sx + 64) + k0 * 64;
    const uint16_t* gx2 = xsrc(sx + 128) + k0 * 64;
    const uint16_t* gx3 = xsrc(sx + 192) + k0 * 64;
    const uint32_t* gi = a.indices + orow(si >> 1) * a.istride + (si & 1) + k0 * 2;  // word slot = row * 2 + word

    // LDS destinations of this wave's pieces, relative to a stage
    const int da = wv * 2048, dx = SP_ABYTES + wv * 4096, di = SP_ABYTES + SP_XBYTES + wv * 256;

#define NM_SP_DMA(ks, buf)                                                                         \
    do {                                                                                           \
        unsigned char* st_ = smem + (buf) * SP_STAGE;                                              \
        __builtin_amdgcn_global_load_lds(ga0 + (ks) * 32, st_ + da, 16, 0, 0);                     \
        __builtin_amdgcn_global_load_lds(ga1 + (ks) * 32, st_ + da + 1024, 16, 0, 0);              \
        __builtin_amdgcn_global_load_lds(gx0 + (ks) * 64, st_ + dx, 16, 0, 0);                     \
        __builtin_amdgcn_global_load_lds(gx1 + (ks) * 64, st_ + dx + 1024, 16, 0, 0);              \
        __builtin_amdgcn_global_load_lds(gx2 + (ks) * 64, st_ + dx + 2048, 16, 0, 0);              \
        __builtin_amdgcn_global_load_lds(gx3 + (ks) * 64, st_ + dx + 3072, 16, 0, 0);              \
        __builtin_amdgcn_global_load_lds(gi + (ks) * 2, st_ + di, 4, 0, 0);                        \
    } while (0)

    // fragment offsets within a stage (lane constants; the rest folds into immediates)
    const int r32 = lane & 31, kg = lane >> 5;
    const int sw = swz_a(r32);  // rows wo + 32 i + r32 share r32's bits 1-4
    int aoff[2], xoff[2][TJ][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        aoff[h] = (wo + r32) * 64 + (((2 * h + kg) ^ sw) << 4);
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            const int t = wt + j * 32 + r32, s = swz_x(t);
            xoff[h][j][0] = SP_ABYTES + t * 128 + (((4 * h + kg) ^ s) << 4);
            xoff[h][j][1] = SP_ABYTES + t * 128 + (((4 * h + 2 + kg) ^ s) << 4);
        }
    }
    const int ioff = SP_ABYTES + SP_XBYTES + (wo + r32) * 8;

    f32x16_t acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // fragments of one instruction column (32 dense k) of a stage: 4 A tiles with their index
    // words and 2 B tiles
    struct Frag {
        bf16x8_t a[TI], lo[TJ], hi[TJ];
        uint32_t i[TI];  // the index word of the tile's rows; this lane's half is taken at use
    };
#define NM_SP_READ(F, st, h)                                                                       \
    do {                                                                                           \
        _Pragma("unroll") for (int i_ = 0; i_ < TI; ++i_) {                                        \
            (F).a[i_] = *reinterpret_cast<const bf16x8_t*>((st) + aoff[h] + i_ * 32 * 64);         \
            (F).i[i_] = *reinterpret_cast<const uint32_t*>((st) + ioff + i_ * 32 * 8 + (h) * 4);   \
        }                                                                                          \
        _Pragma("unroll") for (int j_ = 0; j_ < TJ; ++j_) {                                        \
            (F).lo[j_] = *reinterpret_cast<const bf16x8_t*>((st) + xoff[h][j_][0]);                \
            (F).hi[j_] = *reinterpret_cast<const bf16x8_t*>((st) + xoff[h][j_][1]);                \
        }                                                                                          \
    } while (0)
#define NM_SP_MMA(F)                                                                               \
    do {                                                                                           \
        _Pragma("unroll") for (int j_ = 0; j_ < TJ; ++j_) {                                        \
            const bf16x16_t bf_ = __builtin_shufflevector((F).lo[j_], (F).hi[j_], 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15); \
            _Pragma("unroll") for (int i_ = 0; i_ < TI; ++i_)                                      \
                acc[i_][j_] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16((F).a[i_], bf_, acc[i_][j_],     \
                                                                        (int)((F).i[i_] >> (kg * 16)), 0, 0); \
        }                                                                                          \
    } while (0)

    // Pipeline.  Stages s, s + 1 and s + 2 occupy the three buffers.  While the first half (32
    // dense k) of stage s is multiplied, the second half's fragments are read from LDS; then,
    // after one barrier, the buffer of stage s is refilled with stage s + 3 and the first half of
    // stage s + 1 is read while the second half of stage s is multiplied.  The barrier carries
    // no fence (a fence would wait for every outstanding DMA load, the later stages' too): each
    // wave waits explicitly for its own loads of stage s + 1 (7 per stage; those of stage s + 2
    // may stay in flight) and for its own LDS reads, then all waves meet.
    NM_SP_DMA(0, 0);
    if (nk > 1) NM_SP_DMA(1, 1);
    if (nk > 2) NM_SP_DMA(2, 2);
    if (nk > 2)
        asm volatile("s_waitcnt vmcnt(14)" ::: "memory");
    else if (nk > 1)
        asm volatile("s_waitcnt vmcnt(7)" ::: "memory");
    else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    // the loop runs every stage but the last, the same instructions each time (no merge of paths
    // with different LDS reads in flight, which would force a wait for all of them); the
    // scheduling barriers keep each half stage's fragment reads ahead of the matrix instructions
    // they overlap
    // the epilogue's scalars are loaded before the loop: a scalar load still in flight at the
    // loop head would make every wait there a wait for all LDS reads (scalar loads return out of
    // order on the same counter)
    int64_t ystride = a.ystride;
    int32_t ytype = a.ytype;
    void* yp = a.y;
    asm volatile("" : "+s"(ystride), "+s"(ytype), "+s"(yp));
    Frag f0, f1;
    NM_SP_READ(f0, smem, 0);
    int cur = 0;  // buffer of stage ks
    for (int64_t ks = 0; ks + 1 < nk; ++ks) {
        NM_SP_READ(f1, smem + cur * SP_STAGE, 1);
        __builtin_amdgcn_sched_barrier(0);
        NM_SP_MMA(f0);
        if (ks + 2 < nk)
            asm volatile("s_waitcnt vmcnt(7) lgkmcnt(0)" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (ks + 3 < nk) NM_SP_DMA(ks + 3, cur);
        cur = cur == 2 ? 0 : cur + 1;
        NM_SP_READ(f0, smem + cur * SP_STAGE, 0);
        __builtin_amdgcn_sched_barrier(0);
        NM_SP_MMA(f1);
    }
    NM_SP_READ(f1, smem + cur * SP_STAGE, 1);
    NM_SP_MMA(f0);
    NM_SP_MMA(f1);
#undef NM_SP_READ
#undef NM_SP_MMA
#undef NM_SP_DMA

    // epilogue: element r of tile (i, j) is W row bo + wo + 32 i + 8 (r/4) + 4 (lane/32) + r%4 and
    // token bt + wt + 32 j + lane%32; four consecutive r are consecutive outputs of one Y row
#pragma unroll
    for (int i = 0; i < TI; ++i) {
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            const int64_t t = bt + wt + j * 32 + r32;
            if (t >= a.tokens) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t o = bo + wo + i * 32 + q * 8 + kg * 4;  // out % 4 == 0: o..o+3 all in or out
                if (o >= a.out) continue;
                const f32x16_t v = acc[i][j];
                if constexpr (SPLIT > 1) {
                    *reinterpret_cast<float4*>(ws + ((int64_t)sp * a.tokens + t) * a.out + o) =
                        make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
                } else if (ytype == 0) {
                    *reinterpret_cast<float4*>(static_cast<float*>(yp) + t * ystride + o) =
                        make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
                } else {
                    const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[4 * q]) |
                                        ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[4 * q + 1]) << 16);
                    const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[4 * q + 2]) |
                                        ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[4 * q + 3]) << 16);
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(yp) + t * ystride + o) = make_uint2(lo, hi);
                }
            }
        }
    }
}

// Few tokens (a decode-sized batch): the 256 x 256 tiles above would leave most CUs idle, and
// the product is bound by reading W once.  This path uses v_smfmac_f32_16x16x64_bf16, whose
// operands were measured the same way as above (random integer operands, exact comparison):
//   A (16 x 64 dense = 16 x 32 kept): lane L holds row L%16 and the 8 kept values of the dense
//     groups 4*(L/16) .. 4*(L/16)+3; index bits [4g + 2u, 4g + 2u + 2) give the position of kept
//     value u of the lane's group g (the upper 16 bits are not read);
//   B (64 x 16): lane l holds column l%16; element e < 8 is k = 8*(l/16) + e, element e >= 8 is
//     k = 32 + 8*(l/16) + e - 8;
//   D (16 x 16): lane l, element r is row 4*(l/16) + r, column l%16.
// A block owns 16 W rows x 16 J tokens; its waves split k (wave w takes the 64-k blocks w,
// w + WAVES, ...) and load their fragments straight from memory into registers, U blocks ahead
// (the packed rows feed the instruction as laid out; X, small, comes from L2).  The block then
// sums the waves' partial tiles in LDS in a fixed order, so the result is deterministic.
template <int J, int WAVES, int U>
__global__ __launch_bounds__(64 * WAVES) void k_spmm24_skinny(SpmmArgs a) {
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    constexpr int THREADS = 64 * WAVES;
    __shared__ float part[WAVES * J * 4 * 64];  // the waves' partial tiles
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int r16 = lane & 15, q = lane >> 4;
    const int64_t bo = (int64_t)blockIdx.x * 16, bt = (int64_t)blockIdx.y * 16 * J;
    const int64_t olast = a.out - 1, tlast = a.tokens - 1;
    const int64_t orow = bo + r16 < olast ? bo + r16 : olast;  // rows past the end: the last row
    const uint16_t* va = a.values + orow * a.vstride + q * 8;    // + 32 per 64-k block
    const uint32_t* ia = a.indices + orow * a.istride + (q >> 1);  // + 2 words per 64-k block
    const int ish = 16 * (q & 1);
    const uint16_t* xb[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int64_t t = bt + 16 * j + r16;
        xb[j] = a.x + (t < tlast ? t : tlast) * a.xstride + q * 8;  // + 64 per 64-k block
    }
    f32x4_t acc[J];
#pragma unroll
    for (int j = 0; j < J; ++j) acc[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    const int64_t nkb = a.in / 64;
    for (int64_t kb0 = wv; kb0 < nkb; kb0 += U * WAVES) {
        bf16x8_t av[U], lo[U][J], hi[U][J];
        uint32_t iv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t kb = kb0 + u * WAVES;
            if (kb < nkb) {
                av[u] = *reinterpret_cast<const bf16x8_t*>(va + kb * 32);
                iv[u] = ia[kb * 2];
#pragma unroll
                for (int j = 0; j < J; ++j) {
                    lo[u][j] = *reinterpret_cast<const bf16x8_t*>(xb[j] + kb * 64);
                    hi[u][j] = *reinterpret_cast<const bf16x8_t*>(xb[j] + kb * 64 + 32);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (kb0 + u * WAVES < nkb) {
#pragma unroll
                for (int j = 0; j < J; ++j) {
                    const bf16x16_t bf = __builtin_shufflevector(lo[u][j], hi[u][j], 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10,
                                                                 11, 12, 13, 14, 15);
                    acc[j] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(av[u], bf, acc[j], (int)(iv[u] >> ish), 0, 0);
                }
            }
        }
    }

#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) part[((wv * J + j) * 4 + r) * 64 + lane] = acc[j][r];
    __syncthreads();
    // output (token bt + tl, row bo + ol), rows fastest so that consecutive threads store
    // consecutive outputs; element r of lane l holds row 4 (l/16) + r, token l%16
    for (int e = tid; e < 16 * 16 * J; e += THREADS) {
        const int ol = e & 15, tl = e >> 4, j = tl >> 4;
        const int l = (tl & 15) + 16 * (ol >> 2), r = ol & 3;
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) sum += part[((w * J + j) * 4 + r) * 64 + l];
        const int64_t t = bt + tl, o = bo + ol;
        if (t < a.tokens && o < a.out) {
            if (a.ytype == 0)
                static_cast<float*>(a.y)[t * a.ystride + o] = sum;
            else
                static_cast<__bf16*>(a.y)[t * a.ystride + o] = (__bf16)sum;
        }
    }
}

// One to four tokens: the product is a matrix-vector product bound by reading the packed rows
// once, and 16-row matrix-core fragments would make each wave gather 64-byte pieces of 16
// rows.  Here each wave streams whole packed rows instead: lane L takes the 16-byte chunks
// L, L + 64, ... of a row (chunk c holds the kept values 8c .. 8c + 7, that is the dense
// groups 4c .. 4c + 3 and the index bits [16c, 16c + 16) of the row, the upper or lower half
// of index word c/2).  X, its tokens (at most J) of `in` bf16, is staged once per block in
// LDS; one byte permute per group and token picks the two kept columns out of the group's two
// X words as a bf16 pair, and one two-term bf16 dot product (fp32 accumulate) takes it with
// the kept pair as stored.  The next chunks are loaded before the current ones are used (the first before the X barrier), and
// each row ends with a fixed-order wave reduction, so the result is deterministic.
template <int J>
__global__ __launch_bounds__(512) void k_spmv24(SpmmArgs a, int64_t rows_per_block) {
    constexpr int U = 4;  // 16-byte chunks per lane in flight
    extern __shared__ uint4 xs[];  // [tokens][in / 8] 16-byte pieces of X
    const int nt = (int)a.tokens;  // J when J <= 2, else 3 or 4
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t nch = a.in / 16, xch = a.in / 8;
    const int64_t rend = (int64_t)(blockIdx.x + 1) * rows_per_block;
    const int64_t r1 = rend < a.out ? rend : a.out;
    int64_t r = (int64_t)blockIdx.x * rows_per_block + wv, c0 = 0;

    uint4 v[U];
    uint32_t iw[U];
    auto fetch = [&](int64_t rr, int64_t cc, uint4* vv, uint32_t* ii) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = cc + 64 * u + lane;
            vv[u] = make_uint4(0u, 0u, 0u, 0u);
            ii[u] = 0u;
            if (rr < r1 && c < nch) {
                vv[u] = *reinterpret_cast<const uint4*>(a.values + rr * a.vstride + c * 8);
                ii[u] = a.indices[rr * a.istride + (c >> 1)];
            }
        }
    };
    fetch(r, c0, v, iw);
    for (int64_t c = tid; c < nt * xch; c += 512) {
        const int64_t t = c / xch, k = c - t * xch;
        xs[c] = *reinterpret_cast<const uint4*>(a.x + t * a.xstride + k * 8);
    }
    __syncthreads();

    float acc[J];
#pragma unroll
    for (int t = 0; t < J; ++t) acc[t] = 0.0f;
    while (r < r1) {  // uniform over the wave
        int64_t rn = r, cn = c0 + 64 * U;
        if (cn >= nch) {
            rn = r + 8;
            cn = 0;
        }
        uint4 vn[U];
        uint32_t iwn[U];
        fetch(rn, cn, vn, iwn);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t c = c0 + 64 * u + lane;
            if (c < nch) {
                const uint32_t bits = iw[u] >> (16 * (int)(c & 1));
                const uint32_t vw[4] = {v[u].x, v[u].y, v[u].z, v[u].w};  // kept pair of group g
                // group g keeps positions pa, pb: bytes 2pa, 2pa + 1, 2pb, 2pb + 1 of the group's
                // eight X bytes {xd[2g + 1], xd[2g]} form the bf16 pair (x[pa], x[pb]), which
                // lines up with the kept pair as stored
                uint32_t sel[4];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const uint32_t pa = (bits >> (4 * g)) & 3u, pb = (bits >> (4 * g + 2)) & 3u;
                    sel[g] = 0x01000100u + pa * 0x0202u + ((pb * 0x0202u) << 16);
                }
#pragma unroll
                for (int t = 0; t < J; ++t) {
                    if (J > 2 && t >= nt) break;  // uniform
                    const uint4 xa = xs[t * xch + 2 * c], xb = xs[t * xch + 2 * c + 1];
                    const uint32_t xd[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const uint32_t xp = __builtin_amdgcn_perm(xd[2 * g + 1], xd[2 * g], sel[g]);
                        acc[t] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, vw[g]),
                                                                 __builtin_bit_cast(bf16x2_t, xp), acc[t], false);
                    }
                }
            }
        }
        if (cn == 0) {  // the row is done
#pragma unroll
            for (int t = 0; t < J; ++t) {
                float s = acc[t];
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
                if (lane == 0 && (J <= 2 || t < nt)) {
                    if (a.ytype == 0)
                        static_cast<float*>(a.y)[t * a.ystride + r] = s;
                    else
                        static_cast<__bf16*>(a.y)[t * a.ystride + r] = (__bf16)s;
                }
                acc[t] = 0.0f;
            }
        }
        r = rn;
        c0 = cn;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            v[u] = vn[u];
            iw[u] = iwn[u];
        }
    }
}

// The parts of a split k range, added in part order: y[t, o] = ws[0][t][o] + ws[1][t][o] + ...,
// rounded once to the output type.  One thread per four consecutive outputs.
template <int SPLIT>
__global__ __launch_bounds__(256) void k_spmm_combine(SpmmArgs a, const float* __restrict__ ws) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= a.tokens * (a.out / 4)) return;
    const int64_t t = i / (a.out / 4), o = (i % (a.out / 4)) * 4;
    const int64_t slice = a.tokens * a.out;
    float4 v = *reinterpret_cast<const float4*>(ws + t * a.out + o);
#pragma unroll
    for (int sp = 1; sp < SPLIT; ++sp) {
        const float4 u = *reinterpret_cast<const float4*>(ws + sp * slice + t * a.out + o);
        v.x += u.x;
        v.y += u.y;
        v.z += u.z;
        v.w += u.w;
    }
    if (a.ytype == 0) {
        *reinterpret_cast<float4*>(static_cast<float*>(a.y) + t * a.ystride + o) = v;
    } else {
        const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v.x) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v.y) << 16);
        const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v.z) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v.w) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.y) + t * a.ystride + o) = make_uint2(lo, hi);
    }
}

template <int WAVES, int SPLIT>
static hipError_t launch_tile(const SpmmArgs& a, float* ws, hipStream_t s) {
    using TL = SpTile<WAVES>;
    // the 150 KB of the largest tile are above the default dynamic LDS limit: allow the size
    const hipError_t e = hipFuncSetAttribute((const void*)k_spmm24<WAVES, SPLIT>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)TL::SMEM);
    if (e != hipSuccess) return e;
    const int64_t ntok = (a.tokens + TL::T - 1) / TL::T, nout = (a.out + TL::T - 1) / TL::T;
    const int64_t C = ntok % 4 == 0 ? 4 : (ntok % 2 == 0 ? 2 : 1), R = 8 / C;
    const int64_t grid = 8 * ((ntok + C - 1) / C) * ((nout + R - 1) / R);
    k_spmm24<WAVES, SPLIT><<<dim3((unsigned)(grid * SPLIT)), 64 * WAVES, TL::SMEM, s>>>(a, grid, ws);
    if constexpr (SPLIT > 1) {
        const int64_t quads = a.tokens * (a.out / 4);
        k_spmm_combine<SPLIT><<<dim3((unsigned)((quads + 255) / 256)), 256, 0, s>>>(a, ws);
    }
    return hipGetLastError();
}

// Up to this many tokens the 16-row kernel can run (its J = 4 variant holds 64 tokens).
constexpr int64_t SP_SKINNY_MAX_TOKENS = 64;

// Up to this many bf16 of X (all tokens, 48 KB) the row-streaming kernel stages X in LDS.
constexpr int64_t SP_SPMV_MAX_X = 24576;

int spmm_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
        (void)hipGetLastError();
        cus = 256;  // MI355X
    }
    return cus;
}

namespace {

// Cost model of the tiled kernel, in microseconds.  A CU moves its blocks' stages from L2 into
// LDS at about 35 KB per microsecond with one block resident, 10% faster per further resident
// block (up to the blocks whose three stages fit in 160 KB of LDS: 1, 2 or 4 for the 256, 128
// and 64 tiles), plus 4 us per round of resident blocks (filling the pipeline from HBM); the CU
// with the most blocks sets the time.  A split adds the combine pass: 2 us plus 0.5 us per MB
// of fp32 parts (written by the product and read back).  The constants were fitted to the
// measured time of every (tile, parts) candidate on q/o (4096 x 4096), gate (11008 x 4096) and
// down (4096 x 11008) weights at 5 to 4096 tokens, each call reading its weights from HBM (a
// rotation of copies larger than the 256 MB last-level cache, as a model's layers run); on
// seven other shapes (1024 x 4096 to 24576 x 6144, 5 to 2048 tokens) the plan it picks was
// 1.1% slower than the fastest candidate on average and 12% at worst, where taking the largest
// tile that fills the CUs was 47% slower on average.
template <int WAVES>
double tile_cost_us(int64_t out, int64_t in, int64_t tokens, int cus, int parts) {
    using TL = SpTile<WAVES>;
    constexpr int64_t occ = (160 * 1024) / (int64_t)TL::SMEM;
    const int64_t blocks = ((out + TL::T - 1) / TL::T) * ((tokens + TL::T - 1) / TL::T) * parts;
    const int64_t per_cu = (blocks + cus - 1) / cus;
    const int64_t resident = per_cu < occ ? per_cu : occ;
    const int64_t rounds = (per_cu + resident - 1) / resident;
    const int64_t stages = (in / 64 + parts - 1) / parts;
    const double stage_kb = (double)TL::STAGE / 1024.0;
    double t = (double)rounds * (4.0 + (double)(resident * stages) * stage_kb / (35.0 * (1.0 + 0.1 * (double)(resident - 1))));
    if (parts > 1) t += 2.0 + 0.5 * (double)parts * (double)tokens * (double)out * 4e-6;
    return t;
}

// The 16-row kernel (blocks of 16 W rows reading W once, X from L2): 2.9 us plus a cost per
// weight of the busiest CU that grows with the tokens; fitted to the same measurements.
double skinny_cost_us(int64_t out, int64_t in, int64_t tokens, int cus) {
    const int64_t blocks = (out + 15) / 16;
    const double w = (double)((blocks + cus - 1) / cus) * 16.0 * (double)in * (double)cus * 1e-6;
    return 2.945 + w * (0.2469 + 0.01329 * (double)tokens);
}

}  // namespace

// The kernel of a product.  One to four tokens whose X fits in LDS stream rows (tile 0); else
// every candidate is costed: the 16-row kernel (tile 16, up to 64 tokens) and the 256, 128 and
// 64 tiles with the k range whole or split into 2, 4 or 8 parts (8 not for the 256 tile), the
// parts only with a workspace and at least one 64-wide k stage each.  The cheapest is taken; on
// a tie, the larger tile and the fewer parts.  Candidates whose grid would pass 2^31 - 1 blocks
// are skipped (the entry points admit only sizes whose 256 tiles stay below it; the 16-row
// kernel has one block per 16 W rows), and so are splits of outputs above 2^41 elements (their
// workspace size and combine grid).
SpmmPlan spmm_plan(int64_t out, int64_t in, int64_t tokens, int cus, bool allow_split) {
    if (tokens <= 4 && tokens * in <= SP_SPMV_MAX_X) return {0, 1};
    SpmmPlan best{256, 1};
    double cost = 0.0;
    bool have = false;
    for (int tile : {256, 128, 64}) {
        for (int parts : {1, 2, 4, 8}) {
            if (parts > 1 && (!allow_split || in / 64 < parts || (tile == 256 && parts == 8))) continue;
            if (parts > 1 && tokens > ((int64_t)1 << 41) / out) continue;
            if (((out + tile - 1) / tile + 8) * ((tokens + tile - 1) / tile + 4) > (int64_t)INT32_MAX / parts) continue;
            const double c = tile == 256   ? tile_cost_us<8>(out, in, tokens, cus, parts)
                             : tile == 128 ? tile_cost_us<4>(out, in, tokens, cus, parts)
                                           : tile_cost_us<2>(out, in, tokens, cus, parts);
            if (!have || c < cost) {
                best = {tile, parts};
                cost = c;
                have = true;
            }
        }
    }
    if (tokens <= SP_SKINNY_MAX_TOKENS && (out + 15) / 16 <= (int64_t)INT32_MAX &&
        skinny_cost_us(out, in, tokens, cus) < cost)
        best = {16, 1};
    return best;
}

int64_t spmm_workspace_bytes(int64_t out, int64_t in, int64_t tokens) {
    const SpmmPlan pl = spmm_plan(out, in, tokens, spmm_cus(), true);
    return pl.parts > 1 ? 4 * pl.parts * tokens * out : 0;
}

hipError_t launch_spmm24(const SpmmArgs& a, float* ws, int64_t ws_bytes, hipStream_t s) {
    const int cus = spmm_cus();
    // A split needs the caller's workspace; without it (or with too little) the best plan
    // without one runs.
    SpmmPlan pl = spmm_plan(a.out, a.in, a.tokens, cus, ws != nullptr);
    if (pl.parts > 1 && ws_bytes < 4 * pl.parts * a.tokens * a.out) pl = spmm_plan(a.out, a.in, a.tokens, cus, false);
    if (pl.tile == 0) {
        // about two blocks of eight waves per CU; every wave ends its row loop, then the block
        const int64_t target = 2 * (int64_t)cus;
        const int64_t rpb = (a.out + target - 1) / target;
        const int64_t grid = (a.out + rpb - 1) / rpb;
        const size_t smem = (size_t)(a.tokens * a.in * 2);
        if (a.tokens == 1)
            k_spmv24<1><<<dim3((unsigned)grid), 512, smem, s>>>(a, rpb);
        else if (a.tokens == 2)
            k_spmv24<2><<<dim3((unsigned)grid), 512, smem, s>>>(a, rpb);
        else
            k_spmv24<4><<<dim3((unsigned)grid), 512, smem, s>>>(a, rpb);
        return hipGetLastError();
    }
    if (pl.tile == 16) {
        const unsigned gx = (unsigned)((a.out + 15) / 16);
        if (a.tokens <= 16)
            k_spmm24_skinny<1, 8, 4><<<dim3(gx, 1), 512, 0, s>>>(a);
        else if (a.tokens <= 32)
            k_spmm24_skinny<2, 8, 2><<<dim3(gx, 1), 512, 0, s>>>(a);
        else
            k_spmm24_skinny<4, 8, 4><<<dim3(gx, 1), 512, 0, s>>>(a);
        return hipGetLastError();
    }
    // Deeper pipelines (6 or 9 stages per block instead of 3) were measured no faster.
    if (pl.tile == 256) {
        if (pl.parts == 2) return launch_tile<8, 2>(a, ws, s);
        if (pl.parts == 4) return launch_tile<8, 4>(a, ws, s);
        return launch_tile<8, 1>(a, nullptr, s);
    }
    if (pl.tile == 128) {
        if (pl.parts == 2) return launch_tile<4, 2>(a, ws, s);
        if (pl.parts == 4) return launch_tile<4, 4>(a, ws, s);
        if (pl.parts == 8) return launch_tile<4, 8>(a, ws, s);
        return launch_tile<4, 1>(a, nullptr, s);
    }
    if (pl.parts == 2) return launch_tile<2, 2>(a, ws, s);
    if (pl.parts == 4) return launch_tile<2, 4>(a, ws, s);
    if (pl.parts == 8) return launch_tile<2, 8>(a, ws, s);
    return launch_tile<2, 1>(a, nullptr, s);
}

}  // namespace nm
