// nm_pack.hip -- hard mask, pack and unpack kernels, diagnostic kernels, and their launchers.
#include "nm_layer.hpp"

namespace nm {

template <int N, int M, typename T>
struct TileShape {
    static constexpr int K = Candidates<N, M>::K;
    static constexpr int BITS = PackTiling<N, M>::BITS;
    static constexpr int GT = M * T::bytes >= 16 ? 1 : 16 / (M * T::bytes);  // groups per thread
    static constexpr int TILE = kThreads * GT;                               // groups per block
    static constexpr int TBITS = GT * N * BITS;                               // a thread's index bits
    static_assert(TILE * N * BITS % 32 == 0 && TBITS <= 32, "tiles start on words; <= 2 words per thread");
};

template <int N, int M, typename T>
__global__ __launch_bounds__(kThreads) void k_pack(PackArgs a) {
    // Index fields are assembled per wave: a wave's 64 * GT groups fill whole 32-bit words, so
    // each wave ORs its lanes' fields into its own LDS word tile and stores those words itself.
    // LDS operations of one wave complete in order, so wave-scope fences replace block barriers.
    using TS = TileShape<N, M, T>;
    constexpr int K = TS::K, GT = TS::GT, BITS = TS::BITS;
    constexpr int WW = 64 * GT * N * BITS / 32;                // index words of a wave's groups
    static_assert(64 * GT * N * BITS % 32 == 0, "a wave's fields fill whole words");
    __shared__ uint32_t words[kThreads / 64 * WW];
    const int lane = threadIdx.x & 63, wq = (threadIdx.x >> 6) * 64 * GT;  // wave's first group
    uint32_t* ww = words + (threadIdx.x >> 6) * WW;
    const int64_t q_begin = (int64_t)blockIdx.x * TS::TILE;
    const int ng = (int)(a.gpr - q_begin < TS::TILE ? a.gpr - q_begin : TS::TILE);
    const int ngw = ng - wq < 0 ? 0 : (ng - wq < 64 * GT ? ng - wq : 64 * GT);
    if (ngw == 0) return;  // a whole wave past the row's end (no block barrier is used)
    const int nwords = (ngw * N * BITS + 31) / 32;
    const int lq = threadIdx.x * GT;                        // first group of this thread in the tile
    const int mine = ng - lq < 0 ? 0 : (ng - lq < GT ? ng - lq : GT);
    const bool vec = a.aligned != 0 && mine == GT;
    const int lb = lane * GT * N * BITS;                    // the thread's first bit in the wave's words
    for (int64_t r = blockIdx.y; r < a.rows; r += gridDim.y) {
        const int64_t g0 = r * a.gpr + q_begin + lq;        // flat index of the thread's first group
        float l[GT * K];
        uint32_t raw[GT * M];
        if (mine > 0) {
            if (vec) load_logit_unit<GT * K>(a.logits + g0 * K, true, GT * K, l);
            else load_logit_unit<GT * K>(a.logits + g0 * K, false, mine * K, l);
            load_group_raw<T, GT * M>(reinterpret_cast<const typename T::storage*>(a.w) + g0 * M, vec, raw, mine * M);
        }
        for (int i = lane; i < WW; i += 64) ww[i] = 0u;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        if (mine > 0) {
            uint32_t v[GT * N], hard[GT];
            uint32_t acc = 0;  // TBITS <= 32
#pragma unroll
            for (int i = 0; i < GT; ++i) {
                const float* li = l + i * K;
                // first largest logit; a NaN never compares greater, so it never displaces candidate 0
                float best = li[0];
                int bk = 0;
                uint32_t keep = cand_keep<N, M, 0>();
                static_for<1, K>([&](auto kc) NM_INLINE {
                    constexpr int k = decltype(kc)::value;
                    const bool up = li[k] > best;
                    best = up ? li[k] : best;
                    bk = up ? k : bk;
                    keep = up ? cand_keep<N, M, k>() : keep;
                });
                hard[i] = (uint32_t)bk;
#pragma unroll
                for (int tt = 0; tt < N; ++tt) {
                    const int p = __builtin_ctz(keep);  // kept positions in ascending order
                    keep &= keep - 1;
                    uint32_t x = raw[i * M];
#pragma unroll
                    for (int j = 1; j < M; ++j) x = p == j ? raw[i * M + j] : x;
                    v[i * N + tt] = x;
                    if (i < mine) acc |= (uint32_t)p << ((i * N + tt) * BITS);
                }
            }
            auto* vp = reinterpret_cast<typename T::storage*>(a.values) + g0 * N;
            if (vec) {
                store_group_raw<T, GT * N>(vp, true, v);
            } else {
                for (int e = 0; e < mine * N; ++e) store_bits<T>(vp, e, v[e]);
            }
            if (a.hard) {
#pragma unroll
                for (int i = 0; i < GT; ++i)
                    if (i < mine) st_store(a.hard + g0 + i, (uint8_t)hard[i]);
            }
            // a thread's fields fit one word (TBITS <= 32); at bit lb % 32 they may straddle two
            const uint32_t f = acc, s = (uint32_t)(lb % 32);
            atomicOr(&ww[lb / 32], shl_lo(f, s));
            if ((lb % 32) + TS::TBITS > 32) atomicOr(&ww[lb / 32 + 1], shl_carry(f, s));
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();
        uint32_t* idx = a.indices + r * a.words_per_row + (q_begin + wq) * N * BITS / 32;
        for (int i = lane; i < nwords; i += 64) st_store(idx + i, ww[i]);
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");  // the words are read before the next row clears them
        __builtin_amdgcn_wave_barrier();
    }
}

// Groups of eight whose rows' index bits fill whole 32-bit words: one group per thread on a flat
// grid.  A full block reads its logits as one coalesced span through the sampling kernels' LDS
// tile (lanes on consecutive vectors instead of 112- or 280-byte runs per lane), and each wave
// assembles its 64 groups' fields, 6N whole words, in its own LDS words.  Lanes past the end take
// part in the wave's word assembly with no fields; only the last block has such lanes, and it is
// not staged, so no block barrier is reached by a subset of the block.
template <int N, typename T>
__global__ __launch_bounds__(kThreads) void k_pack_flat8(PackArgs a) {
    constexpr int M = 8, BITS = 3;
    using S = Sample<N, M>;
    constexpr int K = S::K;
    static_assert(S::P == 1 && S::PK == K, "one group per thread");
    constexpr int WW = 64 * N * BITS / 32;
    static_assert(64 * N * BITS % 32 == 0, "a wave's fields fill whole words");
    __shared__ typename StageTile<N, M>::vec tile[StageTile<N, M>::VEC];
    __shared__ uint32_t words[kThreads / 64 * WW];
    const int64_t groups = a.rows * a.gpr;
    const int64_t g0 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int nvalid = g0 < groups ? 1 : 0;
    const bool full = nvalid == 1;
    const bool staged = block_full<N, M>(groups);  // uniform over the block
    float l[K];
    load_logits<N, M>(a.logits, g0, threadIdx.x, full, nvalid, staged, tile, l);  // consecutive groups per wave
    uint32_t raw[M];
    if (full) load_group_raw<T, M>(reinterpret_cast<const typename T::storage*>(a.w) + g0 * M, true, raw);
    const int lane = threadIdx.x & 63;
    uint32_t* ww = words + (threadIdx.x >> 6) * WW;
    for (int i = lane; i < WW; i += 64) ww[i] = 0u;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (full) {
        // first largest logit; a NaN never compares greater, so it never displaces candidate 0
        float best = l[0];
        int bk = 0;
        uint32_t keep = cand_keep<N, M, 0>();
        static_for<1, K>([&](auto kc) NM_INLINE {
            constexpr int k = decltype(kc)::value;
            const bool up = l[k] > best;
            best = up ? l[k] : best;
            bk = up ? k : bk;
            keep = up ? cand_keep<N, M, k>() : keep;
        });
        uint32_t v[N];
        uint32_t acc = 0;  // N * BITS <= 21
#pragma unroll
        for (int tt = 0; tt < N; ++tt) {
            const int p = __builtin_ctz(keep);  // kept positions in ascending order
            keep &= keep - 1;
            uint32_t x = raw[0];
#pragma unroll
            for (int j = 1; j < M; ++j) x = p == j ? raw[j] : x;
            v[tt] = x;
            acc |= (uint32_t)p << (tt * BITS);
        }
        store_group_raw<T, N>(reinterpret_cast<typename T::storage*>(a.values) + g0 * N, true, v);
        if (a.hard) st_store(a.hard + g0, (uint8_t)bk);
        const int lb = lane * N * BITS;  // the thread's first bit in the wave's words
        const uint32_t f = acc, s = (uint32_t)(lb % 32);
        atomicOr(&ww[lb / 32], shl_lo(f, s));
        if ((lb % 32) + N * BITS > 32) atomicOr(&ww[lb / 32 + 1], shl_carry(f, s));
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const int64_t gw0 = g0 - lane;  // the wave's first group, a multiple of 64
    if (gw0 < groups) {
        const int ngw = (int)(groups - gw0 < 64 ? groups - gw0 : 64);
        const int nwords = (ngw * N * BITS + 31) / 32;
        uint32_t* idx = a.indices + gw0 * N * BITS / 32;
        for (int i = lane; i < nwords; i += 64) st_store(idx + i, ww[i]);
    }
}

// Unpack of groups of eight on the same flat stream: one group per thread, its fields read
// straight from the index words (a wave's fields are 6N consecutive words).
template <int N, typename T>
__global__ __launch_bounds__(kThreads) void k_unpack_flat8(UnpackArgs a) {
    constexpr int M = 8, BITS = 3;
    const int64_t g0 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (g0 >= a.rows * a.gpr) return;
    uint32_t v[N], o[M];
    load_group_raw<T, N>(reinterpret_cast<const typename T::storage*>(a.values) + g0 * N, true, v);
    const int64_t lb = g0 * N * BITS;  // the group's first bit in the flat stream
    const uint32_t* idx = a.indices + lb / 32;
    const uint32_t w1 = (lb % 32) + N * BITS > 32 ? idx[1] : 0u;  // read only when the fields straddle
    const uint32_t acc = funnel_right(w1, idx[0], (uint32_t)(lb % 32));
    uint32_t pos[N];
#pragma unroll
    for (int tt = 0; tt < N; ++tt) pos[tt] = (uint32_t)(acc >> (tt * BITS)) & 7u;
#pragma unroll
    for (int j = 0; j < M; ++j) {
        uint32_t x = 0u;  // +0.0 where nothing is kept
#pragma unroll
        for (int tt = 0; tt < N; ++tt) x = pos[tt] == (uint32_t)j ? v[tt] : x;  // later field wins
        o[j] = x;
    }
    store_group_raw<T, M, true>(reinterpret_cast<typename T::storage*>(a.dense) + g0 * M, true, o);
}

template <int N, int M, typename T>
__global__ __launch_bounds__(kThreads) void k_unpack(UnpackArgs a) {
    // Each thread reads the one or two index words that hold its fields straight from memory
    // (a wave's fields are a few consecutive words, so its lanes share cache lines): no LDS tile
    // and no barrier.  The second word is read only when the fields straddle into it, so every
    // read stays within the row's words.
    using TS = TileShape<N, M, T>;
    constexpr int GT = TS::GT, BITS = TS::BITS;
    const int64_t q_begin = (int64_t)blockIdx.x * TS::TILE;
    const int ng = (int)(a.gpr - q_begin < TS::TILE ? a.gpr - q_begin : TS::TILE);
    const int lq = threadIdx.x * GT;
    const int mine = ng - lq < 0 ? 0 : (ng - lq < GT ? ng - lq : GT);
    if (mine == 0) return;
    const bool vec = a.aligned != 0 && mine == GT;
    const int64_t lb = (q_begin + lq) * N * BITS;  // the thread's first bit in its row's stream
    for (int64_t r = blockIdx.y; r < a.rows; r += gridDim.y) {
        const int64_t g0 = r * a.gpr + q_begin + lq;
        uint32_t v[GT * N], o[GT * M];
        const auto* vp = reinterpret_cast<const typename T::storage*>(a.values) + g0 * N;
        if (vec) {
            load_group_raw<T, GT * N>(vp, true, v);
        } else {
#pragma unroll
            for (int e = 0; e < GT * N; ++e) v[e] = e < mine * N ? load_bits<T>(vp, e) : 0u;
        }
        const uint32_t* idx = a.indices + r * a.words_per_row + lb / 32;
        const uint32_t w1 = (lb % 32) + mine * N * BITS > 32 ? idx[1] : 0u;
        const uint32_t acc = funnel_right(w1, idx[0], (uint32_t)(lb % 32));
#pragma unroll
        for (int i = 0; i < GT; ++i) {
            uint32_t pos[N];
#pragma unroll
            for (int tt = 0; tt < N; ++tt) pos[tt] = (uint32_t)(acc >> ((i * N + tt) * BITS)) & ((1u << BITS) - 1u);
#pragma unroll
            for (int j = 0; j < M; ++j) {
                uint32_t x = 0u;  // +0.0 where nothing is kept
#pragma unroll
                for (int tt = 0; tt < N; ++tt) x = pos[tt] == (uint32_t)j ? v[i * N + tt] : x;  // later field wins
                o[i * M + j] = x;
            }
        }
        auto* dp = reinterpret_cast<typename T::storage*>(a.dense) + g0 * M;
        if (vec) {
            store_group_raw<T, GT * M, true>(dp, true, o);
        } else {
            for (int e = 0; e < mine * M; ++e) store_bits<T>(dp, e, o[e]);
        }
    }
}

// ------------------------------------------------------------------------------------------
// Fast path of pack/unpack for groups of four keeping one or two (2 bits per kept value), when
// every row's index bits fill whole words: a thread owns the U = 8/(2N) groups of one index
// byte, so the index bytes, packed values, hard indices and dense weights of consecutive threads
// are contiguous and every store instruction of a wave writes whole cache lines.

template <int N, typename T>
struct ByteTiling {
    static constexpr int M = 4;
    static constexpr int K = Candidates<N, M>::K;
    static constexpr int U = 8 / (2 * N);  // groups per index byte
    static_assert(N == 1 || N == 2, "one index byte holds whole groups");
};

// The logits of a full block's threads form one contiguous span of kThreads * CNT floats: it is
// read with consecutive lanes on consecutive 16-byte vectors (non-temporally: each is read
// once) and handed to the threads through an LDS tile.
template <int CNT>
__device__ __forceinline__ void load_block_logits(const float* __restrict__ block_base, float4* tile,
                                                  float (&l)[CNT]) {
    static_assert(CNT % 4 == 0, "whole float4 vectors per thread");
    constexpr int PER = CNT / 4;
    const float4* src = reinterpret_cast<const float4*>(block_base);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const uint4 u = nt_load4(src + threadIdx.x + i * kThreads);
        tile[threadIdx.x + i * kThreads] =
            make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i) vec_to_floats(tile[threadIdx.x * PER + i], l + 4 * i);
}

template <int N, typename T>
__global__ __launch_bounds__(kThreads) void k_pack_bytes(PackArgs a) {
    using BT = ByteTiling<N, T>;
    constexpr int M = 4, K = BT::K, U = BT::U;
    __shared__ float4 tile[kThreads * U * K / 4];
    const int64_t groups = a.rows * a.gpr;
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t g0 = t * U;
    const bool staged = ((int64_t)blockIdx.x + 1) * kThreads * U <= groups;  // uniform: a full block
    if (g0 >= groups) return;  // only in the last block, which is not staged
    float l[U * K];
    if (staged) load_block_logits<U * K>(a.logits + (int64_t)blockIdx.x * kThreads * U * K, tile, l);
    else load_logit_unit<U * K>(a.logits + g0 * K, true, U * K, l);
    uint32_t raw[U * M];
    load_raw<T, U * M, U * M * T::bytes == 16>(reinterpret_cast<const typename T::storage*>(a.w) + g0 * M, true,
                                                U * M, raw);
    uint32_t vals[U * N];
    uint32_t byte = 0u, hard = 0u;
#pragma unroll
    for (int q = 0; q < U; ++q) {
        const float* lq = l + q * K;
        float best = lq[0];
        int bk = 0;
        uint32_t keep = cand_keep<N, M, 0>();
        static_for<1, K>([&](auto kc) NM_INLINE {
            constexpr int k = decltype(kc)::value;
            const bool up = lq[k] > best;  // a NaN never wins: candidate 0 keeps its place
            best = up ? lq[k] : best;
            bk = up ? k : bk;
            keep = up ? cand_keep<N, M, k>() : keep;
        });
        hard |= (uint32_t)bk << (8 * q);
#pragma unroll
        for (int tt = 0; tt < N; ++tt) {
            const int p = __builtin_ctz(keep);
            keep &= keep - 1;
            uint32_t v = raw[q * M];
#pragma unroll
            for (int j = 1; j < M; ++j) v = p == j ? raw[q * M + j] : v;
            vals[q * N + tt] = v;
            byte |= (uint32_t)p << (2 * (q * N + tt));
        }
    }
    auto* vp = reinterpret_cast<typename T::storage*>(a.values) + g0 * N;
    if constexpr (U * N * T::bytes == 16) {
        store_raw<T, U * N>(vp, true, U * N, vals);
    } else {  // 8 bytes: four bf16 values
        st_store(vp, make_uint2(vals[0] | (vals[1] << 16), vals[2] | (vals[3] << 16)));
    }
    st_store(reinterpret_cast<uint8_t*>(a.indices) + t, (uint8_t)byte);  // byte t
    if (a.hard) {
        if constexpr (U == 2) st_store(reinterpret_cast<uint16_t*>(a.hard + g0), (uint16_t)hard);
        else st_store(a.hard + g0, hard);
    }
}

template <int N, typename T>
__global__ __launch_bounds__(kThreads) void k_unpack_bytes(UnpackArgs a) {
    using BT = ByteTiling<N, T>;
    constexpr int M = 4, U = BT::U;
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t g0 = t * U;
    if (g0 >= a.rows * a.gpr) return;
    const uint32_t byte = reinterpret_cast<const uint8_t*>(a.indices)[t];
    const auto* vp = reinterpret_cast<const typename T::storage*>(a.values) + g0 * N;
    uint32_t v[U * N];
    if constexpr (U * N * T::bytes == 16) {
        load_raw<T, U * N>(vp, true, U * N, v);
    } else {
        const uint2 d = reinterpret_cast<const uint2*>(vp)[0];
        v[0] = d.x & 0xFFFFu; v[1] = d.x >> 16; v[2] = d.y & 0xFFFFu; v[3] = d.y >> 16;
    }
    if constexpr (T::bytes == 2) {
        // a group's four bf16 outputs are two 32-bit words: each kept value goes to its
        // position, replacing what an earlier field put there (later field wins)
        uint32_t w[2 * U];
#pragma unroll
        for (int q = 0; q < U; ++q) {
            uint32_t w0 = 0u, w1 = 0u;  // +0.0 where nothing is kept
#pragma unroll
            for (int tt = 0; tt < N; ++tt) put16(w0, w1, (byte >> (2 * (q * N + tt))) & 3u, v[q * N + tt]);
            w[2 * q] = w0;
            w[2 * q + 1] = w1;
        }
        auto* dp = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.dense) + g0 * M);
#pragma unroll
        for (int i = 0; i < U / 2; ++i) nt_store(dp + i, make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]));
    } else {
        uint32_t dense[U * M];
#pragma unroll
        for (int q = 0; q < U; ++q) {
#pragma unroll
            for (int j = 0; j < M; ++j) {
                uint32_t o = 0u;  // +0.0 where nothing is kept
#pragma unroll
                for (int tt = 0; tt < N; ++tt)
                    o = ((byte >> (2 * (q * N + tt))) & 3u) == (uint32_t)j ? v[q * N + tt] : o;  // later field wins
                dense[q * M + j] = o;
            }
        }
        store_raw<T, U * M, true>(reinterpret_cast<typename T::storage*>(a.dense) + g0 * M, true, U * M, dense);
    }
}

// 1:4 unpack with 16 bytes of dense output per thread (two bf16 groups or one fp32 group), so
// that every store instruction writes one contiguous span: a whole index byte per thread (the
// byte kernel's tiling) would give each thread 32 or 64 bytes in strided 16-byte pieces.  The
// rows' 2-bit fields form one flat stream here (each row fills whole words), so group g's field
// is bits 2g mod 8 of byte g / 4.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_unpack_1of4(UnpackArgs a) {
    constexpr int G = 16 / (4 * T::bytes);  // groups per thread
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t g0 = t * G;
    if (g0 >= a.rows * a.gpr) return;
    const uint32_t byte = reinterpret_cast<const uint8_t*>(a.indices)[g0 >> 2];
    const uint32_t f = byte >> (2 * (g0 & 3));  // field of group g0 + q at bits 2q
    auto* dp = reinterpret_cast<uint4*>(reinterpret_cast<typename T::storage*>(a.dense) + g0 * 4);
    if constexpr (T::bytes == 2) {
        const uint32_t v = reinterpret_cast<const uint32_t*>(a.values)[t];  // the two kept values
        uint32_t a0 = 0u, a1 = 0u, b0 = 0u, b1 = 0u;
        put16(a0, a1, f & 3u, v & 0xFFFFu);
        put16(b0, b1, (f >> 2) & 3u, v >> 16);
        nt_store(dp, make_uint4(a0, a1, b0, b1));
    } else {
        const uint32_t v = reinterpret_cast<const uint32_t*>(a.values)[t];
        const uint32_t p = f & 3u;
        nt_store(dp, make_uint4(p == 0 ? v : 0u, p == 1 ? v : 0u, p == 2 ? v : 0u, p == 3 ? v : 0u));
    }
}

// ------------------------------------------------------------------------------------------
// Diagnostics: raw noise words and the base-2 Gumbel exponent, from the same device functions.

__global__ __launch_bounds__(kThreads) void k_debug_noise(NoiseArgs a) {
    const int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x;  // one Philox block
    if (b * 4 >= a.slots) return;
    const Philox4 blk = noise_block(a.nk, (uint64_t)b);
#pragma unroll
    for (int q = 0; q < 4; ++q)
        if (b * 4 + q < a.slots) a.words[b * 4 + q] = blk.v[q];
}

// A plain flat copy with the path kernels' access pattern (one 16-byte vector per thread, one
// tile per thread, non-temporal load and store): the streaming ceiling the path is compared
// with.  Of the copy shapes measured (1, 2, 4 or 8 vectors per thread, ordinary or
// non-temporal loads), this one is the fastest on MI355X.
__global__ __launch_bounds__(kThreads) void k_debug_copy(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                        int64_t vecs) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < vecs) nt_store(dst + i, nt_load4(src + i));
}

__global__ __launch_bounds__(kThreads) void k_debug_gumbel(GumbelArgs a) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= a.count) return;
    a.h[i] = gumbel_log2(a.words[i]);
}

// ------------------------------------------------------------------------------------------
// Launchers.

// Tile grid of the general pack/unpack: x = tiles per row, y = rows (capped; the kernels loop).
template <int N, int M, typename T>
static dim3 tile_grid(int64_t rows, int64_t gpr) {
    const int64_t tiles = (gpr + TileShape<N, M, T>::TILE - 1) / TileShape<N, M, T>::TILE;
    return dim3((unsigned)tiles, (unsigned)(rows < 65535 ? rows : 65535), 1);
}

// The byte path needs whole-word rows (no padding bits) so that index byte t of the whole
// stream belongs to groups U*t .. U*t+U-1; all its accesses are then 16-byte aligned given the
// 16-byte aligned base pointers the entry points require.
template <int N, int M>
static bool byte_path(int64_t gpr) {
    if constexpr (M == 4 && (N == 1 || N == 2)) return (gpr * N * 2) % 32 == 0;
    else return false;
}

template <int N, int M, typename T>
static hipError_t pack_nmt(PackArgs a, hipStream_t s) {
    if constexpr (M == 4 && (N == 1 || N == 2)) {
        if (byte_path<N, M>(a.gpr)) {
            k_pack_bytes<N, T><<<grid_for(a.rows * a.gpr / ByteTiling<N, T>::U), kThreads, 0, s>>>(a);
            return hipGetLastError();
        }
    }
    if constexpr (M == 8) {
        if ((a.gpr * N * 3) % 32 == 0) {  // every row's fields fill whole words: one flat stream
            k_pack_flat8<N, T><<<grid_for(a.rows * a.gpr), kThreads, 0, s>>>(a);
            return hipGetLastError();
        }
    }
    k_pack<N, M, T><<<tile_grid<N, M, T>(a.rows, a.gpr), kThreads, 0, s>>>(a);
    return hipGetLastError();
}
template <int N, int M, typename T>
static hipError_t unpack_nmt(UnpackArgs a, hipStream_t s) {
    if constexpr (M == 4 && N == 1) {
        if (byte_path<N, M>(a.gpr)) {
            constexpr int G = 16 / (4 * T::bytes);
            k_unpack_1of4<T><<<grid_for(a.rows * a.gpr / G), kThreads, 0, s>>>(a);
            return hipGetLastError();
        }
    }
    if constexpr (M == 4 && N == 2) {
        if (byte_path<N, M>(a.gpr)) {
            k_unpack_bytes<N, T><<<grid_for(a.rows * a.gpr / ByteTiling<N, T>::U), kThreads, 0, s>>>(a);
            return hipGetLastError();
        }
    }
    if constexpr (M == 8) {
        if ((a.gpr * N * 3) % 32 == 0) {  // every row's fields fill whole words: one flat stream
            k_unpack_flat8<N, T><<<grid_for(a.rows * a.gpr), kThreads, 0, s>>>(a);
            return hipGetLastError();
        }
    }
    k_unpack<N, M, T><<<tile_grid<N, M, T>(a.rows, a.gpr), kThreads, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_pack(int n, int m, int wtype, const PackArgs& a, hipStream_t s) {
    NM_DISPATCH(pack_nmt, n, m, wtype, a, s);
}
hipError_t launch_unpack(int n, int m, int wtype, const UnpackArgs& a, hipStream_t s) {
    NM_DISPATCH(unpack_nmt, n, m, wtype, a, s);
}
hipError_t launch_debug_noise(const NoiseArgs& a, hipStream_t s) {
    k_debug_noise<<<grid_for((a.slots + 3) / 4), kThreads, 0, s>>>(a);
    return hipGetLastError();
}
hipError_t launch_debug_copy(const void* src, void* dst, int64_t vecs, hipStream_t s) {
    k_debug_copy<<<grid_for(vecs), kThreads, 0, s>>>(static_cast<const uint4*>(src), static_cast<uint4*>(dst), vecs);
    return hipGetLastError();
}
hipError_t launch_debug_gumbel(const GumbelArgs& a, hipStream_t s) {
    k_debug_gumbel<<<grid_for(a.count), kThreads, 0, s>>>(a);
    return hipGetLastError();
}

int groups_per_thread(int n, int m) {
    const int K = binom(m, n);
    if (K % 4 == 0 || K == 70) return 1;
    return K % 2 == 0 ? 2 : 4;
}


}  // namespace nm
