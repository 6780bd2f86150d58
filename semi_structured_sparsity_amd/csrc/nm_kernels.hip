// nm_kernels.hip -- HIP kernels of the N:M mask layer for gfx950 (MI355X) and their launchers.
//
// Every kernel is a single coalesced pass over HBM with one tile per thread and a flat grid
// (no grid-stride loop): the layer is bandwidth-bound and independent per group, nothing is
// contracted, so there is no MFMA work.  Noise is regenerated in registers from a counter-based
// generator in both passes and is never stored.
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
__device__ __forceinline__ void store_f32(float* __restrict__ p, bool vec, int valid, const float (&in)[CNT]) {
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

template <int VW> struct StageVec;
template <> struct StageVec<16> { using type = float4; };
template <> struct StageVec<8> { using type = float2; };

// h[i] for the thread's slots i = 0 .. PK-1 (slot index relative to g0*K).  Each Philox block
// is turned into Gumbel exponents as soon as it is generated; only the last two words of the
// previous block are carried, for a phased tile (K = 70) whose first slot may sit at word 2.
template <int N, int M>
__device__ __forceinline__ void thread_noise(const NoiseKey& nk, int64_t g0, float (&h)[Sample<N, M>::PK]) {
    using S = Sample<N, M>;
    const uint64_t slot0 = (uint64_t)g0 * S::K;
    const uint64_t b0 = slot0 >> 2;
    const bool shifted = S::PH != 0 && (slot0 & 3) != 0;  // K = 70, odd group: starts at word 2
    uint32_t carry2 = 0u, carry3 = 0u;
#pragma unroll
    for (int j = 0; j < S::NB; ++j) {
        const Philox4 blk = noise_block(nk, b0 + j);
#pragma unroll
        for (int i = 0; i < S::PK; ++i) {
            if ((i + S::PH) / 4 != j) continue;  // slot i becomes available with block j
            uint32_t x;
            if constexpr (S::PH == 0) {
                x = blk.v[i - 4 * j];
            } else {
                // shifted: word i+2, always in this block; else word i, in this block or the last
                const uint32_t own = i >= 4 * j ? blk.v[i - 4 * j] : (i - 4 * j + 4 == 2 ? carry2 : carry3);
                x = shifted ? blk.v[i + 2 - 4 * j] : own;
            }
            h[i] = gumbel_log2(x);
        }
        carry2 = blk.v[2];
        carry3 = blk.v[3];
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
// every candidate keeps N positions, so sum_j s_j = N * S.
template <int N, int M>
__device__ __forceinline__ float group_soft(const float (&e)[Candidates<N, M>::K], float (&sj)[M]) {
    constexpr int K = Candidates<N, M>::K;
    float tot = 0.0f;
    static_for<0, M>([&](auto jc) NM_INLINE {
        constexpr int j = decltype(jc)::value;
        float acc = 0.0f;
        static_for<0, K>([&](auto kc) NM_INLINE {
            constexpr int k = decltype(kc)::value;
            if constexpr ((cand_keep<N, M, k>() >> j) & 1u) acc += e[k];
        });
        sj[j] = acc;
        tot += acc;
    });
    return __builtin_amdgcn_rcpf(tot * (1.0f / N));  // S >= 1 (the largest e_k is ~1): rcp within 1 ulp
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
    using vec = typename StageVec<S::LALIGN>::type;
    static constexpr int PER = S::PK * 4 / S::LALIGN;               // vectors per thread
    static constexpr int VEC = S::STAGE ? kThreads * PER : 1;       // vectors per tile
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
template <typename V>
__device__ __forceinline__ void nt_store_vec(V* p, const V& v) {
    if constexpr (sizeof(V) == 16)
        nt_store(p, make_uint4(__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)));
    else
        nt_store(p, make_uint2(__float_as_uint(v.x), __float_as_uint(v.y)));
}

template <int N, int M>
__device__ __forceinline__ void load_logits(const float* logits, int64_t g0, bool full, int nvalid, bool staged,
                                            typename StageTile<N, M>::vec* tile, float (&l)[Sample<N, M>::PK]) {
    using S = Sample<N, M>;
    using ST = StageTile<N, M>;
    using V = typename ST::vec;
    constexpr int PK = S::PK, PER = ST::PER, W = S::LALIGN / 4;
    if constexpr (S::STAGE) {
        if (staged) {
            const V* src = reinterpret_cast<const V*>(logits + (int64_t)blockIdx.x * kThreads * PK);
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                if constexpr (sizeof(V) == 16) {
                    const uint4 u = nt_load4(src + threadIdx.x + i * kThreads);
                    tile[threadIdx.x + i * kThreads] = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
                } else {
                    const uint2 u = nt_load2(src + threadIdx.x + i * kThreads);
                    tile[threadIdx.x + i * kThreads] = make_float2(__uint_as_float(u.x), __uint_as_float(u.y));
                }
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < PER; ++i) vec_to_floats(tile[threadIdx.x * PER + i], l + W * i);
            return;
        }
    }
    load_f32<PK, S::LALIGN>(logits + g0 * S::K, full, nvalid * S::K, l);
}

template <int N, int M>
__device__ __forceinline__ void store_dlogits(float* dlogits, int64_t g0, bool full, int nvalid, bool staged,
                                              typename StageTile<N, M>::vec* tile,
                                              const float (&dl)[Sample<N, M>::PK]) {
    using S = Sample<N, M>;
    using ST = StageTile<N, M>;
    using V = typename ST::vec;
    constexpr int PK = S::PK, PER = ST::PER, W = S::LALIGN / 4;
    if constexpr (S::STAGE) {
        if (staged) {
            __syncthreads();  // every thread has read its logits out of the tile
#pragma unroll
            for (int i = 0; i < PER; ++i) tile[threadIdx.x * PER + i] = floats_to_vec<V>(dl + W * i);
            __syncthreads();
            V* dst = reinterpret_cast<V*>(dlogits + (int64_t)blockIdx.x * kThreads * PK);
#pragma unroll
            for (int i = 0; i < PER; ++i) nt_store_vec(dst + threadIdx.x + i * kThreads, tile[threadIdx.x + i * kThreads]);
            return;
        }
    }
    store_f32<PK, S::LALIGN>(dlogits + g0 * S::K, full, nvalid * S::K, dl);
}

// ------------------------------------------------------------------------------------------
// Forward: w_masked = w * m (MODE 0), or the soft mask m itself in fp32 (MODE 1, diagnostic).
// Soft mask (Fig. 3 caption, weighted averaging): m_j = sum over candidates k keeping j of y_k.

template <int N, int M, typename T, int MODE>
__global__ __launch_bounds__(kThreads) void k_forward(FwdArgs a) {
    using S = Sample<N, M>;
    constexpr int K = S::K, P = S::P, PK = S::PK;
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t g0 = t * P;
    if (g0 >= a.groups) return;
    const int nvalid = (int)(a.groups - g0 < P ? a.groups - g0 : P);
    const bool full = nvalid == P;

    __shared__ typename StageTile<N, M>::vec tile[StageTile<N, M>::VEC];
    const bool staged = block_full<N, M>(a.groups);  // uniform over the block
    float l[PK];
    load_logits<N, M>(a.logits, g0, full, nvalid, staged, tile, l);
    float w[P * M];
    if constexpr (MODE == 0)
        load_as_float<T, P * M>(reinterpret_cast<const typename T::storage*>(a.w) + g0 * M, full, nvalid * M, w);
    float h[PK];
    thread_noise<N, M>(a.nk, g0, h);

    float out[P * M];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        float e[K], sj[M];
        group_exp<N, M>(l + p * K, h + p * K, a.A, a.B, e);
        const float inv = group_soft<N, M>(e, sj);
#pragma unroll
        for (int j = 0; j < M; ++j) {
            const float mj = sj[j] * inv;
            out[p * M + j] = MODE == 0 ? w[p * M + j] * mj : mj;
        }
    }
    if constexpr (MODE == 0)
        store_from_float<T, P * M>(reinterpret_cast<typename T::storage*>(a.out) + g0 * M, full, nvalid * M, out);
    else
        store_f32<P * M, (P * M * 4) % 16 == 0 ? 16 : 8>(reinterpret_cast<float*>(a.out) + g0 * M, full, nvalid * M, out);
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
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t g0 = t * P;
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
    load_logits<N, M>(a.f.logits, g0, full, nvalid, staged, tile, l);
    float w[P * M];
    load_as_float<T, P * M>(reinterpret_cast<const typename T::storage*>(a.f.w) + g0 * M, full, nvalid * M, w);
    uint32_t prev[P];  // issued with the other loads so that its latency overlaps the noise
#pragma unroll
    for (int p = 0; p < P; ++p) prev[p] = (a.prev && p < nvalid) ? a.prev[g0 + p] : 0u;
    float h[PK];
    thread_noise<N, M>(a.f.nk, g0, h);
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
// Backward to the logits (Fig. 3 caption: all steps differentiable).  Upstream G = dL/dw_masked:
//   dL/dy_k = d_k = sum_{j kept by k} G_j w_j,  s = sum_k y_k d_k,
//   dL/dl_k = (kappa/tau) * y_k * (d_k - s).
// The noise is regenerated from the same (seed, offset) as the forward.

template <int N, int M, typename T>
__global__ __launch_bounds__(kThreads) void k_backward(BwdArgs a) {
    using S = Sample<N, M>;
    constexpr int K = S::K, P = S::P, PK = S::PK;
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t g0 = t * P;
    if (g0 >= a.groups) return;
    const int nvalid = (int)(a.groups - g0 < P ? a.groups - g0 : P);
    const bool full = nvalid == P;

    __shared__ typename StageTile<N, M>::vec tile[StageTile<N, M>::VEC];
    const bool staged = block_full<N, M>(a.groups);  // uniform over the block
    float l[PK];
    load_logits<N, M>(a.logits, g0, full, nvalid, staged, tile, l);
    float w[P * M], gw[P * M];
    load_as_float<T, P * M>(reinterpret_cast<const typename T::storage*>(a.w) + g0 * M, full, nvalid * M, w);
    load_as_float<T, P * M>(reinterpret_cast<const typename T::storage*>(a.grad) + g0 * M, full, nvalid * M, gw);
    float h[PK];
    thread_noise<N, M>(a.nk, g0, h);

    float dl[PK];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        float e[K], sj[M];
        group_exp<N, M>(l + p * K, h + p * K, a.A, a.B, e);
        const float inv = group_soft<N, M>(e, sj);
        float aj[M];
#pragma unroll
        for (int j = 0; j < M; ++j) aj[j] = gw[p * M + j] * w[p * M + j];
        float d[K];
        float es = 0.0f;
        static_for<0, K>([&](auto kc) NM_INLINE {
            constexpr int k = decltype(kc)::value;
            float dk = 0.0f;
            static_for<0, M>([&](auto jc) NM_INLINE {
                constexpr int j = decltype(jc)::value;
                if constexpr ((cand_keep<N, M, k>() >> j) & 1u) dk += aj[j];
            });
            d[k] = dk;
            es = fmaf(e[k], dk, es);
        });
        const float s = es * inv;
        const float ci = a.C * inv;
#pragma unroll
        for (int k = 0; k < K; ++k) dl[p * K + k] = (ci * e[k]) * (d[k] - s);
    }
    store_dlogits<N, M>(a.dlogits, g0, full, nvalid, staged, tile, dl);
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
    if constexpr (T::bytes == 4) reinterpret_cast<uint32_t*>(p)[i] = v;
    else p[i] = (uint16_t)v;
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

template <typename T, int CNT>
__device__ __forceinline__ void store_raw(typename T::storage* __restrict__ p, bool vec, int valid,
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
            nt_store(reinterpret_cast<uint4*>(p) + i, make_uint4(d[0], d[1], d[2], d[3]));
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
// group of 2^i bytes is 2^i-byte aligned); element accesses otherwise.
template <typename T, int CNT>
__device__ __forceinline__ void load_group_raw(const typename T::storage* __restrict__ p, bool vec, uint32_t* out) {
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
        if constexpr (T::bytes == 4) out[i] = reinterpret_cast<const uint32_t*>(p)[i];
        else out[i] = (uint32_t)p[i];
    }
}

template <typename T, int CNT>
__device__ __forceinline__ void store_group_raw(typename T::storage* __restrict__ p, bool vec, const uint32_t* in) {
    constexpr int BYTES = CNT * T::bytes;
    if constexpr (BYTES % 16 == 0) {
        if (vec) {
            store_raw<T, CNT>(p, true, CNT, in);
            return;
        }
    } else if constexpr (BYTES == 8) {
        if (vec) {
            if constexpr (T::bytes == 2) nt_store(p, make_uint2(in[0] | (in[1] << 16), in[2] | (in[3] << 16)));
            else nt_store(p, make_uint2(in[0], in[1]));
            return;
        }
    } else if constexpr (BYTES == 4) {
        if (vec) {
            if constexpr (T::bytes == 2) nt_store(p, in[0] | (in[1] << 16));
            else nt_store(p, in[0]);
            return;
        }
    }
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
        if constexpr (T::bytes == 4) reinterpret_cast<uint32_t*>(p)[i] = in[i];
        else p[i] = (uint16_t)in[i];
    }
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

template <int N, int M, typename T>
struct TileShape {
    static constexpr int K = Candidates<N, M>::K;
    static constexpr int BITS = PackTiling<N, M>::BITS;
    static constexpr int GT = M * T::bytes >= 16 ? 1 : 16 / (M * T::bytes);  // groups per thread
    static constexpr int TILE = kThreads * GT;                               // groups per block
    static constexpr int WORDS = TILE * N * BITS / 32;                        // index words per tile
    static constexpr int TBITS = GT * N * BITS;                               // a thread's index bits
    static_assert(TILE * N * BITS % 32 == 0 && TBITS <= 32, "tiles start on words; <= 2 words per thread");
};

template <int N, int M, typename T>
__global__ __launch_bounds__(kThreads) void k_pack(PackArgs a) {
    using TS = TileShape<N, M, T>;
    constexpr int K = TS::K, GT = TS::GT, BITS = TS::BITS;
    __shared__ uint32_t words[TS::WORDS];
    const int64_t q_begin = (int64_t)blockIdx.x * TS::TILE;
    const int ng = (int)(a.gpr - q_begin < TS::TILE ? a.gpr - q_begin : TS::TILE);
    const int nwords = (ng * N * BITS + 31) / 32;
    const int lq = threadIdx.x * GT;                        // first group of this thread in the tile
    const int mine = ng - lq < 0 ? 0 : (ng - lq < GT ? ng - lq : GT);
    const bool vec = a.aligned != 0 && mine == GT;
    for (int64_t r = blockIdx.y; r < a.rows; r += gridDim.y) {
        for (int i = threadIdx.x; i < TS::WORDS; i += kThreads) words[i] = 0u;
        __syncthreads();
        if (mine > 0) {
            const int64_t g0 = r * a.gpr + q_begin + lq;    // flat index of the thread's first group
            float l[GT * K];
            if (vec) load_logit_unit<GT * K>(a.logits + g0 * K, true, GT * K, l);
            else load_logit_unit<GT * K>(a.logits + g0 * K, false, mine * K, l);
            uint32_t raw[GT * M], v[GT * N], hard[GT];
            load_group_raw<T, GT * M>(reinterpret_cast<const typename T::storage*>(a.w) + g0 * M, vec, raw);
            uint64_t acc = 0;
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
                    if (i < mine) acc |= (uint64_t)p << ((i * N + tt) * BITS);
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
                    if (i < mine) a.hard[g0 + i] = (uint8_t)hard[i];
            }
            const int lb = lq * N * BITS;                   // the thread's first bit in the tile
            atomicOr(&words[lb / 32], (uint32_t)(acc << (lb % 32)));
            if ((lb % 32) + TS::TBITS > 32) atomicOr(&words[lb / 32 + 1], (uint32_t)((acc << (lb % 32)) >> 32));
        }
        __syncthreads();
        uint32_t* idx = a.indices + r * a.words_per_row + q_begin * N * BITS / 32;
        for (int i = threadIdx.x; i < nwords; i += kThreads) nt_store(idx + i, words[i]);
        __syncthreads();  // the next row reuses the tile
    }
}

template <int N, int M, typename T>
__global__ __launch_bounds__(kThreads) void k_unpack(UnpackArgs a) {
    using TS = TileShape<N, M, T>;
    constexpr int GT = TS::GT, BITS = TS::BITS;
    __shared__ uint32_t words[TS::WORDS];
    const int64_t q_begin = (int64_t)blockIdx.x * TS::TILE;
    const int ng = (int)(a.gpr - q_begin < TS::TILE ? a.gpr - q_begin : TS::TILE);
    const int nwords = (ng * N * BITS + 31) / 32;
    const int lq = threadIdx.x * GT;
    const int mine = ng - lq < 0 ? 0 : (ng - lq < GT ? ng - lq : GT);
    const bool vec = a.aligned != 0 && mine == GT;
    for (int64_t r = blockIdx.y; r < a.rows; r += gridDim.y) {
        const uint32_t* idx = a.indices + r * a.words_per_row + q_begin * N * BITS / 32;
        for (int i = threadIdx.x; i < nwords; i += kThreads) words[i] = idx[i];
        __syncthreads();
        if (mine > 0) {
            const int64_t g0 = r * a.gpr + q_begin + lq;
            const int lb = lq * N * BITS;
            uint64_t acc = words[lb / 32];
            if ((lb % 32) + TS::TBITS > 32) acc |= (uint64_t)words[lb / 32 + 1] << 32;
            acc >>= lb % 32;
            uint32_t v[GT * N], o[GT * M];
            const auto* vp = reinterpret_cast<const typename T::storage*>(a.values) + g0 * N;
            if (vec) {
                load_group_raw<T, GT * N>(vp, true, v);
            } else {
#pragma unroll
                for (int e = 0; e < GT * N; ++e) v[e] = e < mine * N ? load_bits<T>(vp, e) : 0u;
            }
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
                store_group_raw<T, GT * M>(dp, true, o);
            } else {
                for (int e = 0; e < mine * M; ++e) store_bits<T>(dp, e, o[e]);
            }
        }
        __syncthreads();  // the next row reuses the tile
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
        nt_store(vp, make_uint2(vals[0] | (vals[1] << 16), vals[2] | (vals[3] << 16)));
    }
    __builtin_nontemporal_store((uint8_t)byte, reinterpret_cast<uint8_t*>(a.indices) + t);  // byte t
    if (a.hard) {
        if constexpr (U == 2) __builtin_nontemporal_store((uint16_t)hard, reinterpret_cast<uint16_t*>(a.hard + g0));
        else nt_store(a.hard + g0, hard);
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
        // a group's four bf16 outputs form one 64-bit word: each kept value is shifted to its
        // position, clearing what an earlier field put there (later field wins)
        uint32_t w[2 * U];
#pragma unroll
        for (int q = 0; q < U; ++q) {
            uint64_t o = 0u;  // +0.0 where nothing is kept
#pragma unroll
            for (int tt = 0; tt < N; ++tt) {
                const uint32_t sh = 16u * ((byte >> (2 * (q * N + tt))) & 3u);
                o = (o & ~(0xFFFFull << sh)) | ((uint64_t)v[q * N + tt] << sh);
            }
            w[2 * q] = (uint32_t)o;
            w[2 * q + 1] = (uint32_t)(o >> 32);
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
        store_raw<T, U * M>(reinterpret_cast<typename T::storage*>(a.dense) + g0 * M, true, U * M, dense);
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
        const uint64_t o0 = (uint64_t)(v & 0xFFFFu) << (16u * (f & 3u));
        const uint64_t o1 = (uint64_t)(v >> 16) << (16u * ((f >> 2) & 3u));
        nt_store(dp, make_uint4((uint32_t)o0, (uint32_t)(o0 >> 32), (uint32_t)o1, (uint32_t)(o1 >> 32)));
    } else {
        const uint32_t v = reinterpret_cast<const uint32_t*>(a.values)[t];
        const uint32_t p = f & 3u;
        nt_store(dp, make_uint4(p == 0 ? v : 0u, p == 1 ? v : 0u, p == 2 ? v : 0u, p == 3 ? v : 0u));
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
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t g0 = t * P;
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
    store_dlogits<N, M>(a.logits, g0, full, nvalid, staged, tile, l);
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
// Launchers.  Grids are flat, one tile per thread; the host has checked that every count fits.

static inline unsigned grid_for(int64_t threads) { return (unsigned)((threads + kThreads - 1) / kThreads); }

template <int N, int M, typename T>
static hipError_t fwd_nmt(const FwdArgs& a, bool soft, hipStream_t s) {
    const int64_t threads = (a.groups + Sample<N, M>::P - 1) / Sample<N, M>::P;
    if (soft) k_forward<N, M, T, 1><<<grid_for(threads), kThreads, 0, s>>>(a);
    else k_forward<N, M, T, 0><<<grid_for(threads), kThreads, 0, s>>>(a);
    return hipGetLastError();
}
template <int N, int M, typename T>
static hipError_t bwd_nmt(const BwdArgs& a, hipStream_t s) {
    const int64_t threads = (a.groups + Sample<N, M>::P - 1) / Sample<N, M>::P;
    k_backward<N, M, T><<<grid_for(threads), kThreads, 0, s>>>(a);
    return hipGetLastError();
}
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
    k_unpack<N, M, T><<<tile_grid<N, M, T>(a.rows, a.gpr), kThreads, 0, s>>>(a);
    return hipGetLastError();
}

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

hipError_t launch_forward(int n, int m, int wtype, const FwdArgs& a, bool soft, hipStream_t s) {
    NM_DISPATCH(fwd_nmt, n, m, wtype, a, soft, s);
}
hipError_t launch_backward(int n, int m, int wtype, const BwdArgs& a, hipStream_t s) {
    NM_DISPATCH(bwd_nmt, n, m, wtype, a, s);
}
hipError_t launch_pack(int n, int m, int wtype, const PackArgs& a, hipStream_t s) {
    NM_DISPATCH(pack_nmt, n, m, wtype, a, s);
}
hipError_t launch_unpack(int n, int m, int wtype, const UnpackArgs& a, hipStream_t s) {
    NM_DISPATCH(unpack_nmt, n, m, wtype, a, s);
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
