// nm_forward.hip -- forward, monitored forward and magnitude-prior kernels, and their launchers.
#include "nm_layer.hpp"

namespace nm {

// ------------------------------------------------------------------------------------------
// Forward: w_masked = w * m (MODE 0), or the soft mask m itself in fp32 (MODE 1, diagnostic).
// Soft mask (Fig. 3 caption, weighted averaging): m_j = sum over candidates k keeping j of y_k.
// MODE 2 (2:4 only) also writes the packed form of the hard mask from the weights and logits the
// forward has already loaded, so a step that needs both reads them once: per thread two groups,
// whose 2-bit fields make one index byte ("Accelerating Sparse Deep Neural Networks" summary
// page, section 3.1), with the hard mask the first argmax of the logits, as nm_mask_harden_pack.

template <int N, int M, typename T, int MODE>
__global__ __launch_bounds__(kThreads) void k_forward(FwdArgs a) {
    using S = Sample<N, M>;
    constexpr int K = S::K, P = S::P, PK = S::PK;
    const ThreadGroup<N, M> tg = thread_group<N, M>();
    const int64_t g0 = tg.g0;
    if (g0 >= a.groups) return;
    const int nvalid = (int)(a.groups - g0 < P ? a.groups - g0 : P);
    const bool full = nvalid == P;

    __shared__ typename StageTile<N, M>::vec tile[StageTile<N, M>::VEC];
    const bool staged = block_full<N, M>(a.groups);  // uniform over the block
    // Groups of eight: the noise (hundreds of instructions per group) is generated while the
    // logit loads are in flight, and the logits go through LDS afterwards.
    constexpr bool EARLY = M == 8;
    float l[PK];
    StagedSpan<N, M> span;
    logits_issue<N, M>(a.logits, g0, full, nvalid, staged, span, l);
    if constexpr (!EARLY) logits_exchange<N, M>(tg.q, staged, tile, span, l);
    float w[P * M];
    if constexpr (MODE != 1)
        load_as_float<T, P * M>(reinterpret_cast<const typename T::storage*>(a.w) + g0 * M, full, nvalid * M, w);
    float h[PK];
    thread_noise<N, M>(step_key(a.nk, a.offset_dev), g0, h);
    if constexpr (EARLY) logits_exchange<N, M>(tg.q, staged, tile, span, l);

    float out[P * M];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        float e[K], sj[M];
        group_exp<N, M>(l + p * K, h + p * K, a.A, a.B, e);
        const float inv = group_soft<N, M>(e, sj);
#pragma unroll
        for (int j = 0; j < M; ++j) {
            const float mj = sj[j] * inv;
            out[p * M + j] = MODE != 1 ? w[p * M + j] * mj : mj;
        }
    }
    if constexpr (MODE != 1)
        store_from_float<T, P * M>(reinterpret_cast<typename T::storage*>(a.out) + g0 * M, full, nvalid * M, out);
    else
        store_f32<P * M, (P * M * 4) % 16 == 0 ? 16 : 8>(reinterpret_cast<float*>(a.out) + g0 * M, full, nvalid * M, out);
    if constexpr (MODE == 2) {
        static_assert(N == 2 && M == 4 && P == 2, "two groups of four fill one index byte");
        // every thread is full here: the host takes this path only when cols/4 is a multiple of 8
        uint32_t vals[P * N], byte = 0u, hard = 0u;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const float* lp = l + p * K;
            float best = lp[0];
            int bk = 0;
            uint32_t keep = cand_keep<N, M, 0>();
            static_for<1, K>([&](auto kc) NM_INLINE {
                constexpr int k = decltype(kc)::value;
                const bool up = lp[k] > best;  // a NaN never wins: candidate 0 keeps its place
                best = up ? lp[k] : best;
                bk = up ? k : bk;
                keep = up ? cand_keep<N, M, k>() : keep;
            });
            hard |= (uint32_t)bk << (8 * p);
#pragma unroll
            for (int tt = 0; tt < N; ++tt) {
                const int pos = __builtin_ctz(keep);  // kept positions in ascending order
                keep &= keep - 1;
                float x = w[p * M];
#pragma unroll
                for (int j = 1; j < M; ++j) x = pos == j ? w[p * M + j] : x;
                // the weight's own bits: a bf16 widened to fp32 keeps them in the upper half
                vals[p * N + tt] = T::bytes == 2 ? __float_as_uint(x) >> 16 : __float_as_uint(x);
                byte |= (uint32_t)pos << (2 * (p * N + tt));
            }
        }
        // the compressed storage with ordinary stores, as nm_mask_harden_pack writes it
        if constexpr (T::bytes == 2) {
            st_store(reinterpret_cast<uint16_t*>(a.values) + g0 * N,
                     make_uint2(vals[0] | (vals[1] << 16), vals[2] | (vals[3] << 16)));
        } else {
            st_store(reinterpret_cast<uint32_t*>(a.values) + g0 * N, make_uint4(vals[0], vals[1], vals[2], vals[3]));
        }
        st_store(reinterpret_cast<uint8_t*>(a.indices) + g0 / P, (uint8_t)byte);  // the byte of groups g0, g0 + 1
        if (a.hard) st_store(reinterpret_cast<uint16_t*>(a.hard + g0), (uint16_t)hard);
    }
}

// ------------------------------------------------------------------------------------------
// Forward with the convergence monitors fused in (MaskLLM project page, Fig. 5 caption: the L1
// distance between the masks sampled at adjacent training steps, and the largest probability of
// the mask distribution).  Besides w * m, per group:
//   sample: the first k with the largest score t_k of this step's noise (Gumbel-max: the hard
//           sample of the distribution that the soft mask relaxes);
//   p_max:  1 / sum_k 2^(A0 (l_k - l_max)) with A0 = kappa*log2(e), the largest probability of
//           softmax(kappa * l), which carries no noise;
//   l1:     popcount(mask(sample) xor mask(prev)), a prev index >= K standing for the empty mask.
// No thread returns early: every lane of the block takes part in the block sums of p_max and
// l1 (fp32, in LDS, then across the first wave; the l1 sums are exact integers).  The sums over
// the whole matrix are taken in the same launch, with integer arithmetic so that they do not
// depend on the order in which blocks finish: a block's p_max sum becomes an integer count of
// 2^-F (F chosen by the host so that the matrix total stays below 2^56), its l1 sum is an
// integer already.  The blocks are the leaves of a 64-ary tree whose nodes are two 64-bit words
// in the workspace, each holding (arrivals << 57) + sum; node i of a level of c nodes has parent
// i % ceil(c / 64), so that blocks that run at the same time add to different words (children
// of one parent, adding in a burst, measured several times slower).  A block adds
// (1 << 57) + its sum to its parent's word with one atomic fetch-and-add; the add that brings
// the arrivals to the parent's child count returns every other child's contribution, so that
// block holds the parent's complete sum, sets the word back to zero and carries the sum one
// level up; the block that completes the root writes the stat.  Every exchange is a
// read-modify-write of a single word, whose updates all happen in one order, so no fence is
// needed (a device-scope fence per block, which writes back and invalidates L2, measured
// twenty times slower), and no block waits for another.  The p_max and l1 words are carried
// independently (their roots may be completed by different blocks).

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

constexpr unsigned long long kTreeOne = 1ull << 57, kTreeSum = kTreeOne - 1ull;

// Lane 0 of a block with the block's sums bp (p_max) and bl (l1): both as integers, carried up
// the tree (the adds of the two words in flight together); a completed root is a stat.
__device__ __forceinline__ void block_sums(const MonitorArgs& a, float bp, float bl) {
    // every p_max is at most 1, so the matrix total stays below 2^56 units: a block sum that is
    // not (a NaN) adds nothing
    const double x = (double)bp * a.pscale;
    unsigned long long pv = (x >= 0.0 && x < 0x1p56) ? (unsigned long long)__builtin_rint(x) : 0ull;
    unsigned long long lv = (unsigned long long)bl;  // popcounts: an exact integer <= 4096
    bool cp = true, cl = true;
    uint32_t node = blockIdx.x, below = gridDim.x;
    unsigned long long* level = a.tree;
    while (below > 1 && (cp || cl)) {
        const uint32_t nodes = (below + 63) / 64, parent = node % nodes;
        const uint32_t expect = (below - parent + nodes - 1) / nodes;  // children of `parent`
        unsigned long long* wp = level + 2 * parent;
        unsigned long long op = 0, ol = 0;
        if (cp) op = __hip_atomic_fetch_add(wp, kTreeOne | pv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (cl) ol = __hip_atomic_fetch_add(wp + 1, kTreeOne | lv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (cp) {
            cp = (op >> 57) + 1 == expect;
            if (cp) {
                pv += op & kTreeSum;
                __hip_atomic_store(wp, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        if (cl) {
            cl = (ol >> 57) + 1 == expect;
            if (cl) {
                lv += ol & kTreeSum;
                __hip_atomic_store(wp + 1, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        level += 2 * nodes;
        node = parent;
        below = nodes;
    }
    if (cp) a.stats[0] = (double)pv * a.pinv;
    if (cl) a.stats[1] = (double)lv;
}

// Candidate bit patterns of groups of four packed as nibbles of one constant (K <= 6).
template <int N, int M>
constexpr uint32_t packed_nibbles() {
    uint32_t v = 0;
    for (int k = 0; k < Candidates<N, M>::K; ++k) v |= (uint32_t)Candidates<N, M>{}.keep[k] << (4 * k);
    return v;
}

// Bit pattern of candidate k for a run-time k; 0 (the empty mask) for k >= K.  Groups of four
// extract a nibble of a constant; groups of eight read a K-byte table the block put in LDS.
template <int N, int M>
__device__ __forceinline__ uint32_t cand_bits_rt(uint32_t k, const uint8_t* lds_table) {
    constexpr int K = Candidates<N, M>::K;
    if constexpr (M == 4) {
        const uint32_t b = __builtin_amdgcn_ubfe(packed_nibbles<N, M>(), 4 * k, 4);
        return k < (uint32_t)K ? b : 0u;
    } else {
        return k < (uint32_t)K ? (uint32_t)lds_table[k] : 0u;
    }
}

// A thread's outputs of the monitored forward: its masked weights and sampled candidates.
template <int N, int M, typename T>
__device__ __forceinline__ void monitor_store(const MonitorArgs& a, int64_t g0, bool full, int nvalid,
                                              const float (&out)[Sample<N, M>::P * M],
                                              const uint32_t (&ksv)[Sample<N, M>::P]) {
    constexpr int P = Sample<N, M>::P;
    store_from_float<T, P * M>(reinterpret_cast<typename T::storage*>(a.f.out) + g0 * M, full, nvalid * M, out);
    if (a.sample) {
        if (P == 2 && full && ((uintptr_t)a.sample & 1u) == 0) {
            st_store(reinterpret_cast<uint16_t*>(a.sample + g0), (uint16_t)(ksv[0] | (ksv[P - 1] << 8)));
        } else {
#pragma unroll
            for (int p = 0; p < P; ++p)
                if (p < nvalid) a.sample[g0 + p] = (uint8_t)ksv[p];
        }
    }
}

template <int N, int M, typename T>
__global__ __launch_bounds__(kThreads) void k_forward_monitor(MonitorArgs a) {
    using S = Sample<N, M>;
    constexpr int K = S::K, P = S::P, PK = S::PK;
    const ThreadGroup<N, M> tg = thread_group<N, M>();
    const int64_t g0 = tg.g0;
    const int64_t left = a.f.groups - g0;
    const int nvalid = left <= 0 ? 0 : (left < P ? (int)left : P);
    const bool full = nvalid == P;

    __shared__ typename StageTile<N, M>::vec tile[StageTile<N, M>::VEC];
    __shared__ float2 red[kThreads];
    __shared__ uint8_t table[M == 4 ? 1 : K];
    if constexpr (M != 4) {
        if (threadIdx.x < K) {
            uint32_t b = 0;
            static_for<0, K>([&](auto kc) NM_INLINE {
                constexpr int k = decltype(kc)::value;
                b = threadIdx.x == (unsigned)k ? cand_keep<N, M, k>() : b;
            });
            table[threadIdx.x] = (uint8_t)b;
        }
    }
    const bool staged = block_full<N, M>(a.f.groups);  // uniform over the block
    // as k_forward: groups of eight generate their noise while the logit loads are in flight
    constexpr bool EARLY = M == 8;
    float l[PK];
    StagedSpan<N, M> span;
    logits_issue<N, M>(a.f.logits, g0, full, nvalid, staged, span, l);
    if constexpr (!EARLY) logits_exchange<N, M>(tg.q, staged, tile, span, l);
    float w[P * M];
    load_as_float<T, P * M>(reinterpret_cast<const typename T::storage*>(a.f.w) + g0 * M, full, nvalid * M, w);
    // the previous samples, issued with the other loads so that their latency overlaps the
    // noise; a thread's P bytes in one load when they are aligned (P = 2: g0 is even)
    const bool pair = P == 2 && full && ((uintptr_t)a.prev & 1u) == 0;
    uint32_t prev[P];
    if (pair && a.prev) {
        const uint32_t v = *reinterpret_cast<const uint16_t*>(a.prev + g0);
        prev[0] = v & 0xFFu;
        prev[P - 1] = v >> 8;
    } else {
#pragma unroll
        for (int p = 0; p < P; ++p) prev[p] = (a.prev && p < nvalid) ? a.prev[g0 + p] : 0u;
    }
    float h[PK];
    thread_noise<N, M>(step_key(a.f.nk, a.f.offset_dev), g0, h);
    if constexpr (EARLY) logits_exchange<N, M>(tg.q, staged, tile, span, l);
    if constexpr (M != 4) __syncthreads();  // the candidate table is in LDS

    float out[P * M];
    uint32_t ksv[P];
    float psum = 0.0f, lsum = 0.0f;
#pragma unroll
    for (int p = 0; p < P; ++p) {
        // in the order that frees registers soonest: the scores, their first maximum (the
        // sampled candidate), the largest probability (the last use of the logits), then the
        // exponentials of the scores (in their place) and the soft mask
        float e[K], sj[M];
        group_scores<N, M>(l + p * K, h + p * K, a.f.A, a.f.B, e);
        float best = e[0];
        uint32_t ks = 0;
#pragma unroll
        for (int k = 1; k < K; ++k) {
            const bool up = e[k] > best;
            best = up ? e[k] : best;
            ks = up ? (uint32_t)k : ks;
        }
        // largest probability of softmax(kappa * l): 1 / sum_k 2^(A0 (l_k - l_max)), whose
        // largest term is exactly 1 (a fused A0 l_k - A0 l_max would not be)
        float lmax = l[p * K];
#pragma unroll
        for (int k = 1; k < K; ++k) lmax = fmaxf(lmax, l[p * K + k]);
        float z = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) z += exp2_fast(a.A0 * (l[p * K + k] - lmax));
#pragma unroll
        for (int k = 0; k < K; ++k) e[k] = exp2_fast(e[k]);
        const float inv = group_soft<N, M>(e, sj);
#pragma unroll
        for (int j = 0; j < M; ++j) out[p * M + j] = w[p * M + j] * (sj[j] * inv);
        const bool live = p < nvalid;
        psum += live ? __builtin_amdgcn_rcpf(z) : 0.0f;
        if (a.prev) {
            const uint32_t d = cand_bits_rt<N, M>(ks, table) ^ cand_bits_rt<N, M>(prev[p], table);
            lsum += live ? (float)__builtin_popcount(d) : 0.0f;
        }
        ksv[p] = ks;
    }

    // Every thread issues its stores, then leaves its sums in LDS; the first wave adds them up
    // and lane 0 takes the block's sums up the tree.  (Measured: letting the first wave climb
    // before its own stores, or combining the waves through LDS atomics without a barrier, or
    // wave sums in DPP steps, was no faster.)
    monitor_store<N, M, T>(a, g0, full, nvalid, out, ksv);
    red[threadIdx.x] = make_float2(psum, lsum);
    __syncthreads();
    if (threadIdx.x < 64) {
        float2 b = red[threadIdx.x];
#pragma unroll
        for (int i = 1; i < kThreads / 64; ++i) {
            const float2 v = red[threadIdx.x + 64 * i];
            b.x += v.x;
            b.y += v.y;
        }
        b.x = wave_sum(b.x);
        b.y = wave_sum(b.y);
        if (threadIdx.x == 0) block_sums(a, b.x, b.y);
    }
}

// ------------------------------------------------------------------------------------------
// Magnitude prior ("Accelerating Sparse Deep Neural Networks" summary page, section 4.1:
// magnitude pruning keeps the largest magnitudes of each group; MaskLLM project page, Table 2
// caption: prior masks initialise the learnable logits).  Per group the candidate that keeps the
// N largest |w| is found in N rounds, each taking the first free position whose magnitude no
// earlier free position reaches (ties keep the lower position; a NaN is taken only as the first
// free position, since no comparison favours it).  Its logit is alpha, the others 0.

template <int N, int M>
__device__ __forceinline__ int prior_candidate(const float* w) {
    constexpr int K = Candidates<N, M>::K;
    float mag[M];
#pragma unroll
    for (int j = 0; j < M; ++j) mag[j] = fabsf(w[j]);
    uint32_t chosen = 0u;
#pragma unroll
    for (int t = 0; t < N; ++t) {
        int best = -1;
        float bm = 0.0f;
#pragma unroll
        for (int j = 0; j < M; ++j) {
            const bool take = !((chosen >> j) & 1u) && (best < 0 || mag[j] > bm);
            best = take ? j : best;
            bm = take ? mag[j] : bm;
        }
        chosen |= 1u << best;
    }
    int kstar = 0;
    static_for<0, K>([&](auto kc) NM_INLINE {
        constexpr int k = decltype(kc)::value;
        kstar = chosen == cand_keep<N, M, k>() ? k : kstar;
    });
    return kstar;
}

// A thread finds the prior candidates of its P consecutive groups from its weights (one
// coalesced load) and leaves them in LDS (one byte per group).  After one barrier the block
// writes its groups' logits as one contiguous span, consecutive threads on consecutive 16-byte
// vectors, so no logit tile is staged.  A vector holds floats of at most two groups (K >= 4);
// a float is alpha where it is its group's prior candidate, +0 elsewhere.  The group of a
// thread's next vector follows from the previous one by a constant step, so there is one
// division per thread.
template <int N, int M, typename T>
__global__ __launch_bounds__(kThreads) void k_prior(PriorArgs a) {
    using S = Sample<N, M>;
    constexpr int K = S::K, P = S::P, BG = kThreads * P;
    static_assert(K >= 4, "a 16-byte vector holds floats of at most two groups");
    __shared__ uint8_t ks[BG];
    const int64_t bg0 = (int64_t)blockIdx.x * BG;  // the block's first group (< groups)
    const int64_t g0 = bg0 + (int64_t)threadIdx.x * P;
    if (g0 < a.groups) {
        const int nvalid = (int)(a.groups - g0 < P ? a.groups - g0 : P);
        float w[P * M];
        load_as_float<T, P * M>(reinterpret_cast<const typename T::storage*>(a.w) + g0 * M, nvalid == P,
                                nvalid * M, w);
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int kstar = prior_candidate<N, M>(w + p * M);
            ks[threadIdx.x * P + p] = (uint8_t)kstar;
            if (a.idx && p < nvalid) a.idx[g0 + p] = (uint8_t)kstar;
        }
    }
    __syncthreads();
    const int ng = a.groups - bg0 < BG ? (int)(a.groups - bg0) : BG;
    float* dst = a.logits + bg0 * K;  // 16-byte aligned: bg0 * K * 4 is a multiple of 1024
    const int nf = ng * K, nv = nf / 4;
    constexpr int STEP = 4 * kThreads, SQ = STEP / K, SR = STEP % K;
    int f = 4 * (int)threadIdx.x, qa = f / K, ra = f - qa * K;  // group of the vector's first float
    for (int v = threadIdx.x; v < nv; v += kThreads) {
        const int qb = qa + (ra + 3 >= K ? 1 : 0);  // group of its last float
        const int pa = qa * K + ks[qa], pb = qb * K + ks[qb];
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (f + e == pa || f + e == pb) ? a.alpha : 0.0f;
        nt_store(dst + f, make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                                     __float_as_uint(x[3])));
        f += STEP;
        qa += SQ;
        ra += SR;
        if (ra >= K) {
            ra -= K;
            ++qa;
        }
    }
    for (int t = 4 * nv + (int)threadIdx.x; t < nf; t += kThreads) {  // a span that ends inside a vector
        const int gt = t / K;
        dst[t] = t == gt * K + ks[gt] ? a.alpha : 0.0f;
    }
}

// ------------------------------------------------------------------------------------------
// Launchers.

template <int N, int M, typename T>
static hipError_t fwd_nmt(const FwdArgs& a, bool soft, hipStream_t s) {
    const int64_t threads = (a.groups + Sample<N, M>::P - 1) / Sample<N, M>::P;
    if (soft) k_forward<N, M, T, 1><<<grid_for(threads), kThreads, 0, s>>>(a);
    else k_forward<N, M, T, 0><<<grid_for(threads), kThreads, 0, s>>>(a);
    return hipGetLastError();
}
hipError_t launch_forward(int n, int m, int wtype, const FwdArgs& a, bool soft, hipStream_t s) {
    NM_DISPATCH(fwd_nmt, n, m, wtype, a, soft, s);
}
hipError_t launch_forward_pack(int wtype, const FwdArgs& a, hipStream_t s) {
    const int64_t threads = (a.groups + Sample<2, 4>::P - 1) / Sample<2, 4>::P;
    if (wtype == 1) k_forward<2, 4, BF16, 2><<<grid_for(threads), kThreads, 0, s>>>(a);
    else k_forward<2, 4, F32, 2><<<grid_for(threads), kThreads, 0, s>>>(a);
    return hipGetLastError();
}
MonitorLayout monitor_layout(int n, int m, int64_t groups) {
    const int P = groups_per_thread(n, m);
    MonitorLayout L;
    L.blocks = ((groups + P - 1) / P + kThreads - 1) / kThreads;
    L.words = 0;
    for (int64_t below = L.blocks; below > 1; below = (below + 63) / 64) L.words += 2 * ((below + 63) / 64);
    L.bytes = 8 * (L.words > 2 ? L.words : 2);
    int bits = 0;  // bit length of the group count: the p_max total is below 2^bits
    while (bits < 62 && (groups >> bits) != 0) ++bits;
    L.frac_bits = 56 - bits;
    return L;
}

template <int N, int M, typename T>
static hipError_t monitor_nmt(const MonitorArgs& a, hipStream_t s) {
    const int64_t threads = (a.f.groups + Sample<N, M>::P - 1) / Sample<N, M>::P;
    k_forward_monitor<N, M, T><<<grid_for(threads), kThreads, 0, s>>>(a);
    return hipGetLastError();
}
hipError_t launch_forward_monitor(int n, int m, int wtype, const MonitorArgs& a, hipStream_t s) {
    NM_DISPATCH(monitor_nmt, n, m, wtype, a, s);
}

// The prior writes K floats of logits per group from M weights: nearly a pure write stream, of a
// contiguous span of kThreads * P * K * 4 bytes per block.  Measured on 4096 x 11008 (bf16),
// the write rate falls once a CU holds more than about 200 KB of such spans at a time: 2:8
// (28 KB per block) ran at 70.1% of 8 TB/s with 8 blocks per CU and 75.1% with 7, 4:8 (70 KB)
// at 60.8% with 8, 71.1% with 4 and 75.6% with 3, while 2:4 (12 KB) is best at 8.  So a block
// whose span is large reserves LDS it does not use, capping the blocks a CU holds (160 KB of
// LDS per CU) at 210 KB / span; the reservation is rounded down to whole KB and leaves 1 KB
// per block for the hardware's allocation granularity, so that the cap is met exactly.
constexpr int kLdsPerCu = 160 * 1024;
template <int N, int M>
constexpr size_t prior_lds_reserve() {
    constexpr int span = kThreads * Sample<N, M>::P * Sample<N, M>::K * 4;
    constexpr int cap = 210 * 1024 / span;
    if constexpr (cap >= 8) {
        return 0;
    } else {
        constexpr int blocks = cap < 1 ? 1 : cap;
        constexpr int total = (kLdsPerCu / blocks - 1024) / 1024 * 1024;
        return (size_t)(total - kThreads * Sample<N, M>::P);  // less the static ks[]
    }
}

template <int N, int M, typename T>
static hipError_t prior_nmt(const PriorArgs& a, hipStream_t s) {
    const int64_t threads = (a.groups + Sample<N, M>::P - 1) / Sample<N, M>::P;
    k_prior<N, M, T><<<grid_for(threads), kThreads, prior_lds_reserve<N, M>(), s>>>(a);
    return hipGetLastError();
}
hipError_t launch_prior(int n, int m, int wtype, const PriorArgs& a, hipStream_t s) {
    NM_DISPATCH(prior_nmt, n, m, wtype, a, s);
}

}  // namespace nm
