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
                const float4 v = reinterpret_cast<const float4*>(p)[i];
                out[4 * i] = v.x; out[4 * i + 1] = v.y; out[4 * i + 2] = v.z; out[4 * i + 3] = v.w;
            }
        } else {
            static_assert(CNT % 2 == 0, "even count");
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

template <int CNT, int ALIGN>
__device__ __forceinline__ void store_f32(float* __restrict__ p, bool vec, int valid, const float (&in)[CNT]) {
    if (vec) {
        if constexpr (ALIGN == 16 && CNT % 4 == 0) {
#pragma unroll
            for (int i = 0; i < CNT / 4; ++i)
                reinterpret_cast<float4*>(p)[i] = make_float4(in[4 * i], in[4 * i + 1], in[4 * i + 2], in[4 * i + 3]);
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
// z'_k = A*l_k - B*h_k (see gumbel_log2).  The exponent of each candidate is formed as a
// difference to a reference candidate r (the largest z'):
//     d_k = A*(l_k - l_r) + B*(h_r - h_k),
// so its rounding error is relative to |d_k| rather than to |A*l_k|; A*|l| reaches several
// hundred at kappa = 100 while the differences that matter are small.  e_k = 2^(d_k) <= 1 up to
// rounding, S = sum e_k >= 1, y_k = e_k / S.

template <int N, int M>
struct Sample {
    static constexpr Candidates<N, M> C{};
    static constexpr int K = Candidates<N, M>::K;
    static constexpr int P = SlotTiling<K>::P;
    static constexpr int PK = P * K;
    static constexpr int PH = SlotTiling<K>::phased ? 2 : 0;  // extra words of a phased tile
    static constexpr int NB = (PK + PH + 3) / 4;              // Philox blocks per thread
    static constexpr int LALIGN = (PK * 4) % 16 == 0 ? 16 : 8; // byte alignment of a thread's logits
};

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

// For group p of the thread: e[k] = 2^(d_k) and the inverse normaliser.
template <int N, int M>
__device__ __forceinline__ float group_exp(const float* l, const float* h, float A, float B,
                                           float (&e)[Candidates<N, M>::K]) {
    constexpr int K = Candidates<N, M>::K;
    float zr = fmaf(A, l[0], -B * h[0]);
    float lr = l[0], hr = h[0];
#pragma unroll
    for (int k = 1; k < K; ++k) {
        const float z = fmaf(A, l[k], -B * h[k]);
        const bool up = z > zr;
        zr = up ? z : zr;
        lr = up ? l[k] : lr;
        hr = up ? h[k] : hr;
    }
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const float d = fmaf(A, l[k] - lr, B * (hr - h[k]));
        e[k] = exp2_fast(d);
        s += e[k];
    }
    return __builtin_amdgcn_rcpf(s);  // s in [1, K]: v_rcp_f32 is within 1 ulp
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

    float l[PK];
    load_f32<PK, S::LALIGN>(a.logits + g0 * K, full, nvalid * K, l);
    float w[P * M];
    if constexpr (MODE == 0)
        load_as_float<T, P * M>(reinterpret_cast<const typename T::storage*>(a.w) + g0 * M, full, nvalid * M, w);
    float h[PK];
    thread_noise<N, M>(a.nk, g0, h);

    float out[P * M];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        float e[K];
        const float inv = group_exp<N, M>(l + p * K, h + p * K, a.A, a.B, e);
#pragma unroll
        for (int j = 0; j < M; ++j) {
            float sj = 0.0f;
#pragma unroll
            for (int k = 0; k < K; ++k)
                if (S::C.kept(k, j)) sj += e[k];
            const float mj = sj * inv;
            out[p * M + j] = MODE == 0 ? w[p * M + j] * mj : mj;
        }
    }
    if constexpr (MODE == 0)
        store_from_float<T, P * M>(reinterpret_cast<typename T::storage*>(a.out) + g0 * M, full, nvalid * M, out);
    else
        store_f32<P * M, (P * M * 4) % 16 == 0 ? 16 : 8>(reinterpret_cast<float*>(a.out) + g0 * M, full, nvalid * M, out);
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

    float l[PK];
    load_f32<PK, S::LALIGN>(a.logits + g0 * K, full, nvalid * K, l);
    float w[P * M], gw[P * M];
    load_as_float<T, P * M>(reinterpret_cast<const typename T::storage*>(a.w) + g0 * M, full, nvalid * M, w);
    load_as_float<T, P * M>(reinterpret_cast<const typename T::storage*>(a.grad) + g0 * M, full, nvalid * M, gw);
    float h[PK];
    thread_noise<N, M>(a.nk, g0, h);

    float dl[PK];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        float e[K];
        const float inv = group_exp<N, M>(l + p * K, h + p * K, a.A, a.B, e);
        float aj[M];
#pragma unroll
        for (int j = 0; j < M; ++j) aj[j] = gw[p * M + j] * w[p * M + j];
        float d[K];
        float es = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            float dk = 0.0f;
#pragma unroll
            for (int j = 0; j < M; ++j)
                if (S::C.kept(k, j)) dk += aj[j];
            d[k] = dk;
            es = fmaf(e[k], dk, es);
        }
        const float s = es * inv;
        const float ci = a.C * inv;
#pragma unroll
        for (int k = 0; k < K; ++k) dl[p * K + k] = (ci * e[k]) * (d[k] - s);
    }
    store_f32<PK, S::LALIGN>(a.dlogits + g0 * K, full, nvalid * K, dl);
}

// ------------------------------------------------------------------------------------------
// Hard mask and compressed storage ("Accelerating Sparse Deep Neural Networks" summary page,
// section 3.1).  A thread owns a chunk of consecutive groups of one row whose index fields fill
// whole 32-bit words (2:4: 8 groups -> 1 word; 2:8 and 4:8: 16 and 8 groups -> 3 words), so the
// metadata is written with plain stores and no atomics.

template <int N, int M>
struct PackTiling {
    static constexpr int BITS = M <= 2 ? 1 : (M <= 4 ? 2 : (M <= 8 ? 3 : 4));  // ceil(log2 M)
    static constexpr int GBITS = N * BITS;                                    // bits per group
    static constexpr int gcd(int a, int b) { return b == 0 ? a : gcd(b, a % b); }
    static constexpr int CHUNK_BITS = GBITS / gcd(GBITS, 32) * 32;            // lcm(GBITS, 32)
    static constexpr int GPC = CHUNK_BITS / GBITS;                            // groups per chunk
    static constexpr int WPC = CHUNK_BITS / 32;                               // words per chunk
};

// Raw element bits (bit copies: the packed values keep NaN payloads and signed zeros).
template <typename T>
__device__ __forceinline__ uint32_t load_bits(const typename T::storage* p, int64_t i) {
    if constexpr (T::bytes == 4) return __float_as_uint(reinterpret_cast<const float*>(p)[i]);
    else return (uint32_t)p[i];
}
template <typename T>
__device__ __forceinline__ void store_bits(typename T::storage* p, int64_t i, uint32_t v) {
    if constexpr (T::bytes == 4) reinterpret_cast<uint32_t*>(p)[i] = v;
    else p[i] = (uint16_t)v;
}

template <int N, int M, typename T>
__global__ __launch_bounds__(kThreads) void k_pack(PackArgs a) {
    using PT = PackTiling<N, M>;
    constexpr Candidates<N, M> C{};
    constexpr int K = Candidates<N, M>::K;
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (t >= a.rows * a.chunks_per_row) return;
    const int64_t r = t / a.chunks_per_row;
    const int64_t c = t - r * a.chunks_per_row;
    const int64_t q0 = c * PT::GPC;                       // first group of the chunk in its row
    const int ng = (int)(a.gpr - q0 < PT::GPC ? a.gpr - q0 : PT::GPC);
    const int64_t grow = r * a.gpr;                       // flat index of the row's first group
    const auto* w = reinterpret_cast<const typename T::storage*>(a.w) + (grow + q0) * M;
    const float* lg = a.logits + (grow + q0) * K;
    auto* vals = reinterpret_cast<typename T::storage*>(a.values) + (grow + q0) * N;

    uint32_t acc[PT::WPC];
#pragma unroll
    for (int i = 0; i < PT::WPC; ++i) acc[i] = 0u;

#pragma unroll
    for (int q = 0; q < PT::GPC; ++q) {
        if (q < ng) {  // predicated, so the loop unrolls and bit positions stay compile-time
            // first largest logit; a NaN never compares greater, so it never displaces candidate 0
            float best = lg[q * K];
            int bk = 0;
            uint32_t keep = C.keep[0];
#pragma unroll
            for (int k = 1; k < K; ++k) {
                const float v = lg[q * K + k];
                const bool up = v > best;
                best = up ? v : best;
                bk = up ? k : bk;
                keep = up ? (uint32_t)C.keep[k] : keep;
            }
            if (a.hard) a.hard[grow + q0 + q] = (uint8_t)bk;
            uint32_t raw[M];
#pragma unroll
            for (int j = 0; j < M; ++j) raw[j] = load_bits<T>(w, q * M + j);
#pragma unroll
            for (int tt = 0; tt < N; ++tt) {
                const int p = __builtin_ctz(keep);  // kept positions in ascending order
                keep &= keep - 1;
                uint32_t v = raw[0];
#pragma unroll
                for (int j = 1; j < M; ++j) v = p == j ? raw[j] : v;
                store_bits<T>(vals, q * N + tt, v);
                const int bit = (q * N + tt) * PT::BITS;  // compile-time position inside the chunk
                acc[bit / 32] |= (uint32_t)p << (bit % 32);
                if ((bit % 32) + PT::BITS > 32) acc[bit / 32 + 1] |= (uint32_t)p >> (32 - bit % 32);
            }
        }
    }
    uint32_t* idx = a.indices + r * a.words_per_row + c * PT::WPC;
#pragma unroll
    for (int i = 0; i < PT::WPC; ++i)
        if (c * PT::WPC + i < a.words_per_row) idx[i] = acc[i];
}

template <int N, int M, typename T>
__global__ __launch_bounds__(kThreads) void k_unpack(UnpackArgs a) {
    using PT = PackTiling<N, M>;
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (t >= a.rows * a.chunks_per_row) return;
    const int64_t r = t / a.chunks_per_row;
    const int64_t c = t - r * a.chunks_per_row;
    const int64_t q0 = c * PT::GPC;
    const int ng = (int)(a.gpr - q0 < PT::GPC ? a.gpr - q0 : PT::GPC);
    const int64_t grow = r * a.gpr;
    const uint32_t* idx = a.indices + r * a.words_per_row + c * PT::WPC;
    uint32_t acc[PT::WPC];
#pragma unroll
    for (int i = 0; i < PT::WPC; ++i) acc[i] = c * PT::WPC + i < a.words_per_row ? idx[i] : 0u;
    const auto* vals = reinterpret_cast<const typename T::storage*>(a.values) + (grow + q0) * N;
    auto* dense = reinterpret_cast<typename T::storage*>(a.dense) + (grow + q0) * M;
#pragma unroll
    for (int q = 0; q < PT::GPC; ++q) {
        if (q < ng) {
            uint32_t pos[N], v[N];
#pragma unroll
            for (int tt = 0; tt < N; ++tt) {
                const int bit = (q * N + tt) * PT::BITS;
                uint32_t f = acc[bit / 32] >> (bit % 32);
                if ((bit % 32) + PT::BITS > 32) f |= acc[bit / 32 + 1] << (32 - bit % 32);
                pos[tt] = f & ((1u << PT::BITS) - 1u);
                v[tt] = load_bits<T>(vals, q * N + tt);
            }
#pragma unroll
            for (int j = 0; j < M; ++j) {
                uint32_t o = 0u;  // +0.0 where nothing is kept
#pragma unroll
                for (int tt = 0; tt < N; ++tt) o = pos[tt] == (uint32_t)j ? v[tt] : o;  // later field wins
                store_bits<T>(dense, q * M + j, o);
            }
        }
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
template <int N, int M, typename T>
static hipError_t pack_nmt(PackArgs a, hipStream_t s) {
    a.chunks_per_row = (a.gpr + PackTiling<N, M>::GPC - 1) / PackTiling<N, M>::GPC;
    k_pack<N, M, T><<<grid_for(a.rows * a.chunks_per_row), kThreads, 0, s>>>(a);
    return hipGetLastError();
}
template <int N, int M, typename T>
static hipError_t unpack_nmt(UnpackArgs a, hipStream_t s) {
    a.chunks_per_row = (a.gpr + PackTiling<N, M>::GPC - 1) / PackTiling<N, M>::GPC;
    k_unpack<N, M, T><<<grid_for(a.rows * a.chunks_per_row), kThreads, 0, s>>>(a);
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
hipError_t launch_debug_noise(const NoiseArgs& a, hipStream_t s) {
    k_debug_noise<<<grid_for((a.slots + 3) / 4), kThreads, 0, s>>>(a);
    return hipGetLastError();
}
hipError_t launch_debug_gumbel(const GumbelArgs& a, hipStream_t s) {
    k_debug_gumbel<<<grid_for(a.count), kThreads, 0, s>>>(a);
    return hipGetLastError();
}

int pack_groups_per_chunk(int n, int m) {
    switch (m * 16 + n) {
#define NM_GPC(nn, mm) case mm * 16 + nn: return PackTiling<nn, mm>::GPC;
        NM_GPC(1, 4) NM_GPC(2, 4) NM_GPC(3, 4) NM_GPC(1, 8) NM_GPC(2, 8) NM_GPC(3, 8) NM_GPC(4, 8)
        NM_GPC(5, 8) NM_GPC(6, 8) NM_GPC(7, 8)
#undef NM_GPC
    default: return 0;
    }
}
int groups_per_thread(int n, int m) {
    const int K = binom(m, n);
    if (K % 4 == 0 || K == 70) return 1;
    return K % 2 == 0 ? 2 : 4;
}

}  // namespace nm
