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
// l1, which go to part[blockIdx.x]; k_monitor_reduce adds the block sums in double.

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
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
    float l[PK];
    load_logits<N, M>(a.f.logits, g0, tg.q, full, nvalid, staged, tile, l);
    float w[P * M];
    load_as_float<T, P * M>(reinterpret_cast<const typename T::storage*>(a.f.w) + g0 * M, full, nvalid * M, w);
    uint32_t prev[P];  // issued with the other loads so that its latency overlaps the noise
#pragma unroll
    for (int p = 0; p < P; ++p) prev[p] = (a.prev && p < nvalid) ? a.prev[g0 + p] : 0u;
    float h[PK];
    thread_noise<N, M>(step_key(a.f.nk, a.f.offset_dev), g0, h);
    if constexpr (M != 4) __syncthreads();  // the candidate table is in LDS

    float out[P * M];
    float psum = 0.0f, lsum = 0.0f;
#pragma unroll
    for (int p = 0; p < P; ++p) {
        float sc[K], e[K], sj[M];
        group_scores<N, M>(l + p * K, h + p * K, a.f.A, a.f.B, sc);
#pragma unroll
        for (int k = 0; k < K; ++k) e[k] = exp2_fast(sc[k]);
        const float inv = group_soft<N, M>(e, sj);
#pragma unroll
        for (int j = 0; j < M; ++j) out[p * M + j] = w[p * M + j] * (sj[j] * inv);

        // sampled candidate: first maximum of the scores
        float best = sc[0];
        uint32_t ks = 0;
#pragma unroll
        for (int k = 1; k < K; ++k) {
            const bool up = sc[k] > best;
            best = up ? sc[k] : best;
            ks = up ? (uint32_t)k : ks;
        }
        // largest probability of softmax(kappa * l)
        float lmax = l[p * K];
#pragma unroll
        for (int k = 1; k < K; ++k) lmax = fmaxf(lmax, l[p * K + k]);
        float z = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) z += exp2_fast(a.A0 * (l[p * K + k] - lmax));
        const bool live = p < nvalid;
        psum += live ? __builtin_amdgcn_rcpf(z) : 0.0f;
        if (a.prev) {
            const uint32_t d = cand_bits_rt<N, M>(ks, table) ^ cand_bits_rt<N, M>(prev[p], table);
            lsum += live ? (float)__builtin_popcount(d) : 0.0f;
        }
        if (a.sample && live) a.sample[g0 + p] = (uint8_t)ks;
    }
    store_from_float<T, P * M>(reinterpret_cast<typename T::storage*>(a.f.out) + g0 * M, full, nvalid * M, out);

    // block sums: every thread leaves its pair in LDS, the first wave adds them up
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
        if (threadIdx.x == 0) a.part[blockIdx.x] = b;
    }
}

// One block of 1024 threads adds the per-block sums in a fixed order (deterministic).  Each
// thread issues U loads before it adds, so the block keeps many loads in flight.
__global__ __launch_bounds__(1024) void k_monitor_reduce(const float2* __restrict__ part, int64_t nparts,
                                                        double* __restrict__ stats) {
    constexpr int U = 8;
    double s0 = 0.0, s1 = 0.0;
    for (int64_t base = 0; base < nparts; base += 1024 * U) {
        float2 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + u * 1024 + threadIdx.x;
            v[u] = i < nparts ? part[i] : make_float2(0.0f, 0.0f);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            s0 += v[u].x;
            s1 += v[u].y;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        s0 += __shfl_xor(s0, o);
        s1 += __shfl_xor(s1, o);
    }
    __shared__ double red[2][16];
    if ((threadIdx.x & 63) == 0) {
        red[0][threadIdx.x >> 6] = s0;
        red[1][threadIdx.x >> 6] = s1;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double a = 0.0, b = 0.0;
        for (int i = 0; i < 16; ++i) { a += red[0][i]; b += red[1][i]; }
        stats[0] = a;
        stats[1] = b;
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

template <int N, int M, typename T>
__global__ __launch_bounds__(kThreads) void k_prior(PriorArgs a) {
    using S = Sample<N, M>;
    constexpr int K = S::K, P = S::P, PK = S::PK;
    const ThreadGroup<N, M> tg = thread_group<N, M>();
    const int64_t g0 = tg.g0;
    if (g0 >= a.groups) return;
    const int nvalid = (int)(a.groups - g0 < P ? a.groups - g0 : P);
    const bool full = nvalid == P;

    __shared__ typename StageTile<N, M>::vec tile[StageTile<N, M>::VEC];
    const bool staged = block_full<N, M>(a.groups);  // uniform over the block
    float w[P * M];
    load_as_float<T, P * M>(reinterpret_cast<const typename T::storage*>(a.w) + g0 * M, full, nvalid * M, w);
    float l[PK];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const int kstar = prior_candidate<N, M>(w + p * M);
#pragma unroll
        for (int k = 0; k < K; ++k) l[p * K + k] = k == kstar ? a.alpha : 0.0f;
        if (a.idx && p < nvalid) a.idx[g0 + p] = (uint8_t)kstar;
    }
    store_dlogits<N, M>(a.logits, g0, tg.q, full, nvalid, staged, tile, l);
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
int64_t monitor_parts(int n, int m, int64_t groups) {
    const int P = groups_per_thread(n, m);
    return ((groups + P - 1) / P + kThreads - 1) / kThreads;
}

template <int N, int M, typename T>
static hipError_t monitor_nmt(const MonitorArgs& a, hipStream_t s) {
    const int64_t threads = (a.f.groups + Sample<N, M>::P - 1) / Sample<N, M>::P;
    const unsigned blocks = grid_for(threads);
    k_forward_monitor<N, M, T><<<blocks, kThreads, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    k_monitor_reduce<<<1, 1024, 0, s>>>(a.part, (int64_t)blocks, a.stats);
    return hipGetLastError();
}
hipError_t launch_forward_monitor(int n, int m, int wtype, const MonitorArgs& a, hipStream_t s) {
    NM_DISPATCH(monitor_nmt, n, m, wtype, a, s);
}

template <int N, int M, typename T>
static hipError_t prior_nmt(const PriorArgs& a, hipStream_t s) {
    const int64_t threads = (a.groups + Sample<N, M>::P - 1) / Sample<N, M>::P;
    k_prior<N, M, T><<<grid_for(threads), kThreads, 0, s>>>(a);
    return hipGetLastError();
}
hipError_t launch_prior(int n, int m, int wtype, const PriorArgs& a, hipStream_t s) {
    NM_DISPATCH(prior_nmt, n, m, wtype, a, s);
}

}  // namespace nm
