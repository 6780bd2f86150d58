// nm_layer.hpp -- device code shared by the kernels of the N:M mask layer (internal).
//
// Every kernel is a single coalesced pass over HBM with one tile per thread and a flat grid
// (no grid-stride loop): the layer is bandwidth-bound and independent per group, nothing is
// contracted, so there is no MFMA work.  Noise is regenerated in registers from a counter-based
// generator in both passes and is never stored.  The kernels live in nm_forward.hip (forward,
// monitored forward, magnitude prior), nm_backward.hip and nm_pack.hip (hard mask, pack,
// unpack, diagnostics); each translation unit instantiates only what its launchers use.
#pragma once
#include "nm_device.hpp"
#include "nm_kernels.hpp"

namespace nm {

constexpr int kThreads = 256;

// ------------------------------------------------------------------------------------------
// Loads of logits / stores of logit gradients: CNT floats, 16- or 8-byte vectors.

template <int CNT, int ALIGN>
__device__ __forceinline__ void load_f32(const float* __restrict__ p, bool vec, int valid, float (&out)[CNT]) {
    if (vec) {
        if constexpr (ALIGN == 16 && CNT % 4 == 0) {
#pragma unroll
            for (int i = 0; i < CNT / 4; ++i) {
                const uint4 v = nt_load4(reinterpret_cast<const float4*>(p) + i);
                out[4 * i] = __uint_as_float(v.x); out[4 * i + 1] = __uint_as_float(v.y);
                out[4 * i + 2] = __uint_as_float(v.z); out[4 * i + 3] = __uint_as_float(v.w);
            }
        } else {
            static_assert(CNT % 2 == 0, "even count");
#pragma unroll
            for (int i = 0; i < CNT / 2; ++i) {
                const uint2 v = nt_load2(reinterpret_cast<const float2*>(p) + i);
                out[2 * i] = __uint_as_float(v.x); out[2 * i + 1] = __uint_as_float(v.y);
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < CNT; ++i) out[i] = i < valid ? p[i] : 0.0f;
}

template <int CNT, int ALIGN>
__device__ __forceinline__ void store_f32(float* p, bool vec, int valid, const float (&in)[CNT]) {
    if (vec) {
        if constexpr (ALIGN == 16 && CNT % 4 == 0) {
#pragma unroll
            for (int i = 0; i < CNT / 4; ++i)
                nt_store(reinterpret_cast<uint4*>(p) + i,
                         make_uint4(__float_as_uint(in[4 * i]), __float_as_uint(in[4 * i + 1]),
                                    __float_as_uint(in[4 * i + 2]), __float_as_uint(in[4 * i + 3])));
        } else {
#pragma unroll
            for (int i = 0; i < CNT / 2; ++i) reinterpret_cast<float2*>(p)[i] = make_float2(in[2 * i], in[2 * i + 1]);
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < CNT; ++i)
        if (i < valid) p[i] = in[i];
}

// ------------------------------------------------------------------------------------------
// The sample of a thread's P groups: probabilities up to the normaliser.
//
// MaskLLM project page, Fig. 3 caption (Gumbel softmax over the candidates of each group) and
// Fig. 5 caption (kappa scales the logits): y_k = softmax_k((kappa*l_k + g_k)/tau).  In base 2,
// z'_k = A*l_k - B*h_k (see gumbel_log2).  A*|l| reaches several hundred at kappa = 100 while the
// differences between candidates that matter are small, so z'_k is carried as an fp32 head
// hi_k = fl(A*l_k - B*h_k) plus the remainder rem_k = (A*l_k - hi_k) - B*h_k that the fma leaves
// (exact up to the rounding of B*h_k).  With mu = max_k hi_k, e_k = 2^((hi_k - mu) + rem_k): the
// rounding errors are relative to |z'_k - mu| rather than to |A*l_k|, and mu cancels in y.

template <int N, int M>
struct Sample {
    static constexpr int K = Candidates<N, M>::K;
    static constexpr int P = SlotTiling<K>::P;
    static constexpr int PK = P * K;
    static constexpr int PH = SlotTiling<K>::phased ? 2 : 0;  // extra words of a phased tile
    static constexpr int NB = (PK + PH + 3) / 4;              // Philox blocks per thread
    static constexpr int LALIGN = (PK * 4) % 16 == 0 ? 16 : 8; // byte alignment of a thread's logits
    // Stage a block's logits (and logit gradients) through LDS when a thread's share is more than
    // one vector: then neighbouring lanes are more than a vector apart and direct accesses leave
    // partly used cache lines in every instruction.  Tile: kThreads * PK floats (<= 70 KB).
    static constexpr bool STAGE = PK * 4 > LALIGN;
};


// The group a thread of a sampling kernel owns.  A thread owns P consecutive groups, block by
// block.  For K = 70 (one group per thread; 70 slots are 17.5 Philox blocks) an even group's
// slots start at word 0 of a block and an odd group's at word 2, so within each block the
// waves take groups of one parity (waves 0-1 the even groups, waves 2-3 the odd ones): the
// phase is then uniform over a wave, and the noise is read through compile-time word indices
// on either side of a scalar branch.  `q` is the thread's place in the block's logit tile.
template <int N, int M>
struct ThreadGroup {
    int64_t g0;  // first group
    int q;       // index of the thread's P-group tile within the block (for LDS staging)
};
template <int N, int M>
__device__ __forceinline__ ThreadGroup<N, M> thread_group() {
    using S = Sample<N, M>;
    const int tid = threadIdx.x;
    int q = tid;
    if constexpr (S::PH != 0) {
        static_assert(S::P == 1 && kThreads == 256, "four waves, one group per thread");
        q = 2 * ((tid & 63) + 64 * ((tid >> 6) & 1)) + (tid >> 7);
    }
    return ThreadGroup<N, M>{((int64_t)blockIdx.x * kThreads + q) * S::P, q};
}

// h[i] for slots i = 0 .. PK-1 when slot 0 is word SH of Philox block b0: each block is turned
// into Gumbel exponents as soon as it is generated.
template <int N, int M, int SH>
__device__ __forceinline__ void noise_run(const NoiseKey& nk, uint64_t b0, float (&h)[Sample<N, M>::PK]) {
    using S = Sample<N, M>;
    constexpr int NB = (S::PK + SH + 3) / 4;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const Philox4 blk = noise_block(nk, b0 + j);
#pragma unroll
        for (int i = 0; i < S::PK; ++i)
            if ((i + SH) / 4 == j) h[i] = gumbel_log2(blk.v[(i + SH) % 4]);  // slot i is word i + SH
    }
}

// h[i] for the thread's slots i = 0 .. PK-1 (slot index relative to g0*K).
template <int N, int M>
__device__ __forceinline__ void thread_noise(const NoiseKey& nk, int64_t g0, float (&h)[Sample<N, M>::PK]) {
    using S = Sample<N, M>;
    const uint64_t slot0 = (uint64_t)g0 * S::K;
    if constexpr (S::PH == 0) {
        noise_run<N, M, 0>(nk, slot0 >> 2, h);
    } else {
        // K = 70: word 2 for an odd group; the same for every lane of the wave (thread_group)
        if (__builtin_amdgcn_readfirstlane((int)(slot0 & 3)) != 0) noise_run<N, M, 2>(nk, slot0 >> 2, h);
        else noise_run<N, M, 0>(nk, slot0 >> 2, h);
    }
}

// For group p of the thread: t[k] = z'_k - mu, the base-2 scores relative to their maximum.
template <int N, int M>
__device__ __forceinline__ void group_scores(const float* l, const float* h, float A, float B,
                                             float (&t)[Candidates<N, M>::K]) {
    constexpr int K = Candidates<N, M>::K;
    float hi[K], rem[K];
    float mu = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const float bh = B * h[k];
        hi[k] = fmaf(A, l[k], -bh);
        rem[k] = fmaf(A, l[k], -hi[k]) - bh;
        mu = fmaxf(mu, hi[k]);
    }
#pragma unroll
    for (int k = 0; k < K; ++k) t[k] = (hi[k] - mu) + rem[k];
}

// e[k] = 2^(z'_k - mu) (unnormalised probabilities).
template <int N, int M>
__device__ __forceinline__ void group_exp(const float* l, const float* h, float A, float B,
                                          float (&e)[Candidates<N, M>::K]) {
    constexpr int K = Candidates<N, M>::K;
    float t[K];
    group_scores<N, M>(l, h, A, B, t);
#pragma unroll
    for (int k = 0; k < K; ++k) e[k] = exp2_fast(t[k]);
}

// Soft-mask sums s_j = sum over candidates k keeping j of e_k, and 1/S with S = sum_k e_k:
// every candidate keeps N positions, so sum_j s_j = N * S.  Sums start from -0.0, which the
// compiler drops (-0.0 + x is x for every x), so a sum of n terms costs n - 1 additions.
//
// Groups of eight go through the halves of the group: R[A] sums e_k over the candidates whose
// kept positions among 0-3 are exactly the set A, C[B] likewise among 4-7; then s_j is the sum
// of R[A] over the sets A that contain j (j < 4), or of C[B] over the B that contain j - 4.
// For 4:8 that is 164 additions instead of 280 (each of the 70 candidates adds into 4 positions).
template <int N, int M>
__device__ __forceinline__ float group_soft(const float (&e)[Candidates<N, M>::K], float (&sj)[M]) {
    constexpr int K = Candidates<N, M>::K;
    if constexpr (M == 8) {
        float R[16], C[16];
        static_for<0, 16>([&](auto ac) NM_INLINE {
            R[decltype(ac)::value] = -0.0f;
            C[decltype(ac)::value] = -0.0f;
        });
        static_for<0, K>([&](auto kc) NM_INLINE {
            constexpr int k = decltype(kc)::value;
            constexpr uint32_t lo = cand_keep<N, M, k>() & 15u, hi = cand_keep<N, M, k>() >> 4;
            if constexpr (lo != 0) R[lo] += e[k];
            if constexpr (hi != 0) C[hi] += e[k];
        });
        static_for<0, 4>([&](auto jc) NM_INLINE {
            constexpr int j = decltype(jc)::value;
            float lo = -0.0f, hi = -0.0f;
            static_for<1, 16>([&](auto ac) NM_INLINE {
                constexpr int a = decltype(ac)::value;
                if constexpr ((a >> j) & 1) {
                    lo += R[a];
                    hi += C[a];
                }
            });
            sj[j] = lo;
            sj[4 + j] = hi;
        });
    } else {
        static_for<0, M>([&](auto jc) NM_INLINE {
            constexpr int j = decltype(jc)::value;
            float acc = -0.0f;
            static_for<0, K>([&](auto kc) NM_INLINE {
                constexpr int k = decltype(kc)::value;
                if constexpr ((cand_keep<N, M, k>() >> j) & 1u) acc += e[k];
            });
            sj[j] = acc;
        });
    }
    float tot = sj[0];
#pragma unroll
    for (int j = 1; j < M; ++j) tot += sj[j];
    return __builtin_amdgcn_rcpf(tot * (1.0f / N));  // S >= 1 (the largest e_k is ~1): rcp within 1 ulp
}

// Candidate sums d_k = sum over the positions j kept by candidate k of a_j.  Groups of eight
// build them from the subset sums of the two halves (a subset's sum is a smaller subset's plus
// one term, 11 additions per half), then d_k = DL[low part] + DH[high part]: for 4:8, 90
// additions instead of 210.  Groups of four add their N terms directly.
constexpr int top_bit(int a) { return a < 2 ? 0 : 1 + top_bit(a >> 1); }

template <int N, int M, typename F>
__device__ __forceinline__ void candidate_sums(const float (&aj)[M], F&& use) {
    constexpr int K = Candidates<N, M>::K;
    if constexpr (M == 8) {
        float DL[16], DH[16];
        static_for<1, 16>([&](auto ac) NM_INLINE {
            constexpr int a = decltype(ac)::value, t = top_bit(a), rest = a & ~(1 << t);
            if constexpr (rest == 0) {
                DL[a] = aj[t];
                DH[a] = aj[4 + t];
            } else {
                DL[a] = DL[rest] + aj[t];
                DH[a] = DH[rest] + aj[4 + t];
            }
        });
        static_for<0, K>([&](auto kc) NM_INLINE {
            constexpr int k = decltype(kc)::value;
            constexpr uint32_t lo = cand_keep<N, M, k>() & 15u, hi = cand_keep<N, M, k>() >> 4;
            if constexpr (lo == 0) use(kc, DH[hi]);
            else if constexpr (hi == 0) use(kc, DL[lo]);
            else use(kc, DL[lo] + DH[hi]);
        });
    } else {
        static_for<0, K>([&](auto kc) NM_INLINE {
            constexpr int k = decltype(kc)::value;
            float dk = -0.0f;
            static_for<0, M>([&](auto jc) NM_INLINE {
                constexpr int j = decltype(jc)::value;
                if constexpr ((cand_keep<N, M, k>() >> j) & 1u) dk += aj[j];
            });
            use(kc, dk);
        });
    }
}

// ------------------------------------------------------------------------------------------
// Block staging of logits and logit gradients through LDS.  A thread's PK floats are contiguous,
// but lanes are PK*4 bytes apart, so direct 16-byte accesses would touch partly used cache lines
// in every instruction.  In a block whose tiles are all present, the block's logits are moved as
// one contiguous span with every lane on consecutive 16-byte vectors, and exchanged through an
// LDS tile.  Partial blocks (the last one) use direct accesses.

template <int N, int M>
struct StageTile {
    using S = Sample<N, M>;
    using vec = float4;                                    // LDS element: the span moves in 16-byte vectors
    static constexpr int G16 = kThreads * S::PK / 4;       // 16-byte vectors of a block's span
    static constexpr int ROUNDS = (G16 + kThreads - 1) / kThreads;  // per thread (the last guarded)
    static constexpr bool EVEN = G16 % kThreads == 0;
    static constexpr int VEC = S::STAGE ? G16 : 1;         // vectors per tile
    static_assert(kThreads * S::PK % 4 == 0, "a block's span is whole 16-byte vectors");
};

// The HBM side of a staged span, held in registers between the loads and the LDS exchange.
template <int N, int M>
struct StagedSpan {
    uint4 v[StageTile<N, M>::ROUNDS];
};

template <int N, int M>
__device__ __forceinline__ bool block_full(int64_t groups) {
    return ((int64_t)blockIdx.x + 1) * kThreads * Sample<N, M>::P <= groups;
}

template <typename V>
__device__ __forceinline__ void vec_to_floats(const V& v, float* out) {
    if constexpr (sizeof(V) == 16) { out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w; }
    else { out[0] = v.x; out[1] = v.y; }
}
template <typename V>
__device__ __forceinline__ V floats_to_vec(const float* in) {
    if constexpr (sizeof(V) == 16) return make_float4(in[0], in[1], in[2], in[3]);
    else return make_float2(in[0], in[1]);
}

// Logits in two steps, so that work independent of them (the noise) can run while the loads are
// in flight.  logits_issue: a staged block's span is loaded into registers, 16-byte vectors with
// consecutive lanes on consecutive vectors; a thread of an unstaged block loads its own logits
// directly into l.  logits_exchange: the staged span goes through the LDS tile, and each thread
// reads its PK floats at float offset q * PK (q: its place in the block, thread_group).
template <int N, int M>
__device__ __forceinline__ void logits_issue(const float* logits, int64_t g0, bool full, int nvalid, bool staged,
                                             StagedSpan<N, M>& st, float (&l)[Sample<N, M>::PK]) {
    using S = Sample<N, M>;
    using ST = StageTile<N, M>;
    if constexpr (S::STAGE) {
        if (staged) {
            const uint4* src = reinterpret_cast<const uint4*>(logits + (int64_t)blockIdx.x * kThreads * S::PK);
#pragma unroll
            for (int r = 0; r < ST::ROUNDS; ++r) {
                const int i = threadIdx.x + r * kThreads;
                if (ST::EVEN || r + 1 < ST::ROUNDS || i < ST::G16) st.v[r] = nt_load4(src + i);
            }
            return;
        }
    }
    load_f32<S::PK, S::LALIGN>(logits + g0 * S::K, full, nvalid * S::K, l);
}

template <int N, int M>
__device__ __forceinline__ void logits_exchange(int q, bool staged, float4* tile, const StagedSpan<N, M>& st,
                                                float (&l)[Sample<N, M>::PK]) {
    using S = Sample<N, M>;
    using ST = StageTile<N, M>;
    if constexpr (S::STAGE) {
        if (staged) {
#pragma unroll
            for (int r = 0; r < ST::ROUNDS; ++r) {
                const int i = threadIdx.x + r * kThreads;
                if (ST::EVEN || r + 1 < ST::ROUNDS || i < ST::G16)
                    tile[i] = make_float4(__uint_as_float(st.v[r].x), __uint_as_float(st.v[r].y),
                                          __uint_as_float(st.v[r].z), __uint_as_float(st.v[r].w));
            }
            __syncthreads();
            const float* mine = reinterpret_cast<const float*>(tile) + q * S::PK;
            if constexpr (S::LALIGN == 16) {
#pragma unroll
                for (int i = 0; i < S::PK / 4; ++i) vec_to_floats(reinterpret_cast<const float4*>(mine)[i], l + 4 * i);
            } else {
#pragma unroll
                for (int i = 0; i < S::PK / 2; ++i) vec_to_floats(reinterpret_cast<const float2*>(mine)[i], l + 2 * i);
            }
        }
    }
}

// Both steps at once.
template <int N, int M>
__device__ __forceinline__ void load_logits(const float* logits, int64_t g0, int q, bool full, int nvalid, bool staged,
                                            float4* tile, float (&l)[Sample<N, M>::PK]) {
    StagedSpan<N, M> st;
    logits_issue<N, M>(logits, g0, full, nvalid, staged, st, l);
    logits_exchange<N, M>(q, staged, tile, st, l);
}

template <int N, int M>
__device__ __forceinline__ void store_dlogits(float* dlogits, int64_t g0, int q, bool full, int nvalid, bool staged,
                                              float4* tile, const float (&dl)[Sample<N, M>::PK]) {
    using S = Sample<N, M>;
    using ST = StageTile<N, M>;
    if constexpr (S::STAGE) {
        if (staged) {
            __syncthreads();  // every thread has read its logits out of the tile
            float* mine = reinterpret_cast<float*>(tile) + q * S::PK;
            if constexpr (S::LALIGN == 16) {
#pragma unroll
                for (int i = 0; i < S::PK / 4; ++i) reinterpret_cast<float4*>(mine)[i] = floats_to_vec<float4>(dl + 4 * i);
            } else {
#pragma unroll
                for (int i = 0; i < S::PK / 2; ++i) reinterpret_cast<float2*>(mine)[i] = floats_to_vec<float2>(dl + 2 * i);
            }
            __syncthreads();
            uint4* dst = reinterpret_cast<uint4*>(dlogits + (int64_t)blockIdx.x * kThreads * S::PK);
#pragma unroll
            for (int r = 0; r < ST::ROUNDS; ++r) {
                const int i = threadIdx.x + r * kThreads;
                if (ST::EVEN || r + 1 < ST::ROUNDS || i < ST::G16) {
                    const float4 v = tile[i];
                    nt_store(dst + i, make_uint4(__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                                                 __float_as_uint(v.w)));
                }
            }
            return;
        }
    }
    store_f32<S::PK, S::LALIGN>(dlogits + g0 * S::K, full, nvalid * S::K, dl);
}

// ------------------------------------------------------------------------------------------
// Hard mask and compressed storage ("Accelerating Sparse Deep Neural Networks" summary page,
// section 3.1).  A thread owns a chunk of consecutive groups of one row whose index fields fill
// whole 32-bit words (2:4: 8 groups -> 1 word; 2:8 and 4:8: 16 and 8 groups -> 3 words), so the
// metadata is written with plain stores and no atomics.

template <int N, int M>
struct PackTiling {
    static constexpr int BITS = M <= 2 ? 1 : (M <= 4 ? 2 : (M <= 8 ? 3 : 4));  // ceil(log2 M)
};

// Groups per 16-byte-multiple unit when a group occupies `bytes` bytes (8 B -> 2 groups).
constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }
constexpr int unit_groups(int bytes) { return 16 / gcd_c(16, bytes); }

// One element's raw bits (zero-extended to 32 for bf16).
template <typename T>
__device__ __forceinline__ uint32_t load_bits(const typename T::storage* p, int64_t i) {
    if constexpr (T::bytes == 4) return reinterpret_cast<const uint32_t*>(p)[i];
    else return (uint32_t)p[i];
}
template <typename T>
__device__ __forceinline__ void store_bits(typename T::storage* p, int64_t i, uint32_t v) {
    if constexpr (T::bytes == 4) st_store(reinterpret_cast<uint32_t*>(p) + i, v);
    else st_store(reinterpret_cast<uint16_t*>(p) + i, (uint16_t)v);
}

// Raw element bits (bit copies: packed values keep NaN payloads and signed zeros).  CNT elements
// of T, each zero-extended into a uint32.  vec: the caller guarantees 16-byte alignment, that
// CNT * bytes is a multiple of 16 and that all CNT elements exist; otherwise element i is read
// or written only if i < valid.
template <typename T, int CNT, bool NTL = false>
__device__ __forceinline__ void load_raw(const typename T::storage* __restrict__ p, bool vec, int valid,
                                         uint32_t* out) {
    static_assert(CNT * T::bytes % 16 == 0, "whole 16-byte vectors");
    if (vec) {
#pragma unroll
        for (int i = 0; i < CNT * T::bytes / 16; ++i) {
            const uint4 v = NTL ? nt_load4(reinterpret_cast<const uint4*>(p) + i) : reinterpret_cast<const uint4*>(p)[i];
            const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if constexpr (T::bytes == 4) {
                    out[4 * i + q] = d[q];
                } else {
                    out[8 * i + 2 * q] = d[q] & 0xFFFFu;
                    out[8 * i + 2 * q + 1] = d[q] >> 16;
                }
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
        if constexpr (T::bytes == 4) out[i] = i < valid ? reinterpret_cast<const uint32_t*>(p)[i] : 0u;
        else out[i] = i < valid ? (uint32_t)p[i] : 0u;
    }
}

// NTS: the 16-byte vectors are stored non-temporally (the unpack's dense output); otherwise
// every store is an ordinary one (the pack's compressed storage).
template <typename T, int CNT, bool NTS = false>
__device__ __forceinline__ void store_raw(typename T::storage* p, bool vec, int valid,
                                          const uint32_t* in) {
    static_assert(CNT * T::bytes % 16 == 0, "whole 16-byte vectors");
    if (vec) {
#pragma unroll
        for (int i = 0; i < CNT * T::bytes / 16; ++i) {
            uint32_t d[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if constexpr (T::bytes == 4) d[q] = in[4 * i + q];
                else d[q] = in[8 * i + 2 * q] | (in[8 * i + 2 * q + 1] << 16);
            }
            if constexpr (NTS) nt_store(reinterpret_cast<uint4*>(p) + i, make_uint4(d[0], d[1], d[2], d[3]));
            else st_store(reinterpret_cast<uint4*>(p) + i, make_uint4(d[0], d[1], d[2], d[3]));
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
        if (i < valid) {
            if constexpr (T::bytes == 4) reinterpret_cast<uint32_t*>(p)[i] = in[i];
            else p[i] = (uint16_t)in[i];
        }
    }
}

// Logits of `cnt` groups starting at p (scalar path reads only the first `valid` floats).
template <int CNT>
__device__ __forceinline__ void load_logit_unit(const float* __restrict__ p, bool vec, int valid, float* out) {
    if (vec) {
        if constexpr (CNT % 4 == 0) {
#pragma unroll
            for (int i = 0; i < CNT / 4; ++i) {
                const float4 v = reinterpret_cast<const float4*>(p)[i];
                out[4 * i] = v.x; out[4 * i + 1] = v.y; out[4 * i + 2] = v.z; out[4 * i + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < CNT / 2; ++i) {
                const float2 v = reinterpret_cast<const float2*>(p)[i];
                out[2 * i] = v.x; out[2 * i + 1] = v.y;
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < CNT; ++i) out[i] = i < valid ? p[i] : 0.0f;
}

// One group's raw weights (M elements) and the store of N kept values / M dense values, with
// the widest single access the group's byte size allows when `vec` (rows 16-byte aligned, so a
// group of 2^i bytes is 2^i-byte aligned); element accesses otherwise, of the first `valid`
// elements only (the rest read as 0): a thread whose last groups lie past the end of its row
// reads nothing beyond its own groups.
template <typename T, int CNT>
__device__ __forceinline__ void load_group_raw(const typename T::storage* __restrict__ p, bool vec, uint32_t* out,
                                               int valid = CNT) {
    constexpr int BYTES = CNT * T::bytes;
    if constexpr (BYTES % 16 == 0) {
        if (vec) {
            load_raw<T, CNT>(p, true, CNT, out);
            return;
        }
    } else if constexpr (BYTES == 8) {
        if (vec) {
            const uint2 d = *reinterpret_cast<const uint2*>(p);
            if constexpr (T::bytes == 2) {
                out[0] = d.x & 0xFFFFu; out[1] = d.x >> 16; out[2] = d.y & 0xFFFFu; out[3] = d.y >> 16;
            } else {
                out[0] = d.x; out[1] = d.y;
            }
            return;
        }
    }
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
        if constexpr (T::bytes == 4) out[i] = i < valid ? reinterpret_cast<const uint32_t*>(p)[i] : 0u;
        else out[i] = i < valid ? (uint32_t)p[i] : 0u;
    }
}

template <typename T, int CNT, bool NTS = false>
__device__ __forceinline__ void store_group_raw(typename T::storage* p, bool vec, const uint32_t* in) {
    constexpr int BYTES = CNT * T::bytes;
    if constexpr (BYTES % 16 == 0) {
        if (vec) {
            store_raw<T, CNT, NTS>(p, true, CNT, in);
            return;
        }
    } else if constexpr (BYTES == 8) {
        if (vec) {
            if constexpr (T::bytes == 2) st_store(p, make_uint2(in[0] | (in[1] << 16), in[2] | (in[3] << 16)));
            else st_store(p, make_uint2(in[0], in[1]));
            return;
        }
    } else if constexpr (BYTES == 4) {
        if (vec) {
            if constexpr (T::bytes == 2) st_store(p, in[0] | (in[1] << 16));
            else st_store(p, in[0]);
            return;
        }
    }
#pragma unroll
    for (int i = 0; i < CNT; ++i) store_bits<T>(p, i, in[i]);
}

// ------------------------------------------------------------------------------------------
// Bit-field and 16-bit slot helpers in 32-bit operations only.  MI355X was measured to compute
// v_lshlrev_b64 (and its right-shift forms) wrongly, now and then, when the shift amount is a
// VGPR at the end of an 8-register allocation block: an unpack whose two such shifts placed the
// second group's kept values produced wrong dense groups in about one in 10^5 threads (the
// other group of the same thread, shifted by amounts in other registers, never).  The pack and
// unpack kernels therefore never shift a 64-bit value by a register amount.

// Low 32 bits of the 64-bit value (hi:lo) shifted right by s, 0 <= s < 32 (one v_alignbit).
__device__ __forceinline__ uint32_t funnel_right(uint32_t hi, uint32_t lo, uint32_t s) {
    return __builtin_amdgcn_alignbit(hi, lo, s);
}
// (lo << s) as a 64-bit value, 0 <= s < 32: the low word and the bits shifted out of it.
__device__ __forceinline__ uint32_t shl_lo(uint32_t lo, uint32_t s) { return lo << s; }
__device__ __forceinline__ uint32_t shl_carry(uint32_t lo, uint32_t s) { return (lo >> 1) >> (31u - s); }

// Put the 16-bit value v at position p (0..3) of four 16-bit elements held as two 32-bit words
// (w0: positions 0-1, w1: positions 2-3), replacing what is there.
__device__ __forceinline__ void put16(uint32_t& w0, uint32_t& w1, uint32_t p, uint32_t v) {
    const uint32_t sh = (p & 1u) << 4;
    const uint32_t m = 0xFFFFu << sh, x = v << sh;
    const uint32_t n0 = (w0 & ~m) | x, n1 = (w1 & ~m) | x;
    w0 = p < 2u ? n0 : w0;
    w1 = p < 2u ? w1 : n1;
}

// General pack/unpack: a block owns a tile of consecutive groups of one row (grid x = tile within
// the row, grid y = row, looping over rows beyond the grid's y limit).  A thread owns GT
// consecutive groups, GT chosen so that its weights / dense output are one 16-byte vector
// (2 groups of four bf16, else 1), so weights, packed values, hard indices and dense output of
// neighbouring lanes are contiguous.  Index fields, which straddle words for 3-bit positions,
// are assembled in LDS (ds_or of at most two words per thread) and stored as whole words after
// a barrier; every tile starts on a word boundary because kThreads * GT * N * BITS is a
// multiple of 32.  The host sets `aligned` when every row of w, logits, values and dense starts
// on a 16-byte boundary (then every thread's vector is aligned to its size).

// ------------------------------------------------------------------------------------------
// Launch helpers.  Grids are flat, one tile per thread; the host has checked that every count fits.

static inline unsigned grid_for(int64_t threads) { return (unsigned)((threads + kThreads - 1) / kThreads); }

// (n, m, wtype) -> template instance.  The caller has validated the triple.
#define NM_DISPATCH(FN, n, m, wt, ...)                                            \
    do {                                                                          \
        const bool bf = (wt) == 1;                                                \
        switch ((m) * 16 + (n)) {                                                 \
        case 4 * 16 + 1: return bf ? FN<1, 4, BF16>(__VA_ARGS__) : FN<1, 4, F32>(__VA_ARGS__); \
        case 4 * 16 + 2: return bf ? FN<2, 4, BF16>(__VA_ARGS__) : FN<2, 4, F32>(__VA_ARGS__); \
        case 4 * 16 + 3: return bf ? FN<3, 4, BF16>(__VA_ARGS__) : FN<3, 4, F32>(__VA_ARGS__); \
        case 8 * 16 + 1: return bf ? FN<1, 8, BF16>(__VA_ARGS__) : FN<1, 8, F32>(__VA_ARGS__); \
        case 8 * 16 + 2: return bf ? FN<2, 8, BF16>(__VA_ARGS__) : FN<2, 8, F32>(__VA_ARGS__); \
        case 8 * 16 + 3: return bf ? FN<3, 8, BF16>(__VA_ARGS__) : FN<3, 8, F32>(__VA_ARGS__); \
        case 8 * 16 + 4: return bf ? FN<4, 8, BF16>(__VA_ARGS__) : FN<4, 8, F32>(__VA_ARGS__); \
        case 8 * 16 + 5: return bf ? FN<5, 8, BF16>(__VA_ARGS__) : FN<5, 8, F32>(__VA_ARGS__); \
        case 8 * 16 + 6: return bf ? FN<6, 8, BF16>(__VA_ARGS__) : FN<6, 8, F32>(__VA_ARGS__); \
        case 8 * 16 + 7: return bf ? FN<7, 8, BF16>(__VA_ARGS__) : FN<7, 8, F32>(__VA_ARGS__); \
        default: return hipErrorInvalidValue;                                     \
        }                                                                         \
    } while (0)

}  // namespace nm
