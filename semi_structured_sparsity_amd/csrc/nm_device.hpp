// nm_device.hpp -- device building blocks of the N:M mask kernels for gfx950 (MI355X):
// compile-time candidate tables, Philox4x32-10 noise, the Gumbel transform in base 2, and
// vector load/store helpers.  Everything here is header-only and inlined into the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "nm_kernels.hpp"

namespace nm {

// ------------------------------------------------------------------------------------------
// Candidate masks (MaskLLM project page, Fig. 3 caption: each group of M weights has a
// categorical distribution over the masks that keep N of them).  Order: lexicographic in the
// ascending list of kept positions.  With position j mapped to bit M-1-j, that order is the
// descending numeric order of the bit patterns, which is how the table is generated.

constexpr int binom(int m, int n) {
    int c = 1;
    for (int i = 0; i < n; ++i) c = c * (m - i) / (i + 1);
    return c;
}

constexpr int popcount_c(unsigned v) {
    int c = 0;
    for (; v; v &= v - 1) ++c;
    return c;
}

template <int N, int M>
struct Candidates {
    static constexpr int K = binom(M, N);
    uint8_t keep[K];  // bit j set: position j kept
    constexpr Candidates() : keep{} {
        int k = 0;
        for (int r = (1 << M) - 1; r >= 0; --r) {
            if (popcount_c((unsigned)r) != N) continue;
            unsigned bits = 0;
            for (int j = 0; j < M; ++j)
                if (r >> (M - 1 - j) & 1) bits |= 1u << j;
            keep[k++] = (uint8_t)bits;
        }
    }
    constexpr bool kept(int k, int j) const { return (keep[k] >> j & 1) != 0; }
    // t-th kept position of candidate k
    constexpr int pos(int k, int t) const {
        int seen = 0;
        for (int j = 0; j < M; ++j)
            if (kept(k, j)) {
                if (seen == t) return j;
                ++seen;
            }
        return -1;
    }
};

// Compile-time loop: f(std::integral_constant<int, I>) for I = B .. E-1.  Candidate membership
// tests inside it are constant expressions, so they vanish from the generated code instead of
// becoming run-time bit tests and selects.
template <int I>
using ic = std::integral_constant<int, I>;

// Lambda bodies of static_for are always inlined, so the arrays they reach stay in registers.
#define NM_INLINE __attribute__((always_inline))

template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(ic<B>{});
        static_for<B + 1, E>(f);
    }
}

// Bit pattern of candidate k (k-th n-subset in lexicographic order) as a constant expression.
template <int N, int M, int k>
constexpr uint32_t cand_keep() {
    constexpr uint32_t bits = Candidates<N, M>{}.keep[k];  // evaluated by the compiler
    return bits;
}

// Groups per thread in the sampling kernels: enough for the thread's candidate slots to fill
// whole Philox blocks when K is not a multiple of 4 (K = 6 -> 2 groups = 3 blocks).  K = 70 is
// handled with one group per thread and a 0-or-2 word phase instead (2 groups would keep 280
// values live per thread).
template <int K>
struct SlotTiling {
    static constexpr int P = (K % 4 == 0 || K == 70) ? 1 : (K % 2 == 0 ? 2 : 4);
    static constexpr bool phased = (P * K) % 4 != 0;  // block boundary may fall inside a group
};

// ------------------------------------------------------------------------------------------
// Philox4x32 (Salmon, Moraes, Dror, Shaw, SC'11, section 3.3): 10 rounds; each multiplies words
// 0 and 2 by fixed odd constants, the high halves are xored into the other two words with the
// round key, and the key is advanced by two Weyl increments between rounds.  The key (the seed)
// and the high counter half (the offset) are uniform across a launch and stay in SGPRs.  Each
// three-way xor is one gfx950 v_bitop3_b32 (truth table 0x96: odd number of ones).

__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
    return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

struct Philox4 {
    uint32_t v[4];
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = xor3((uint32_t)(p1 >> 32), c1, k0);
        const uint32_t n2 = xor3((uint32_t)(p0 >> 32), c3, k1);
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return Philox4{{c0, c1, c2, c3}};
}

// Block b of the noise stream: slots 4b .. 4b+3.
__device__ __forceinline__ Philox4 noise_block(const NoiseKey& nk, uint64_t b) {
    return philox4x32_10((uint32_t)b, (uint32_t)(b >> 32), nk.off0, nk.off1, nk.k0, nk.k1);
}

// ------------------------------------------------------------------------------------------
// Gumbel noise in base 2.  The sample is g = -ln(-ln u) with u = (j + 1/2) 2^-23, j = x >> 9.
// Writing a = -log2(u) gives g = -ln2 * (log2(a) + log2(ln2)); the constant cancels in the
// softmax, so the kernels work with h = log2(a) and z' = z * log2(e) = A*l - B*h + const, with
// A = kappa*log2(e)/tau and B = 1/tau.  u = (2j + 1) 2^-24 is exact in fp32, and v_log_f32 is
// within about 1 ulp (relative) for normal inputs, also just below 1 where a is tiny, so
// h is accurate to a few ulp everywhere.
//
// u is formed in two instructions: one v_alignbit_b32 places j under the exponent of 1.0
// (the float 1 + j 2^-23, in [1, 2)), and subtracting 1 - 2^-24 leaves (2j + 1) 2^-24, which is
// representable, so the subtraction is exact.
__device__ __forceinline__ float gumbel_u(uint32_t x) {
    const float one_j = __uint_as_float(__builtin_amdgcn_alignbit(0x7Fu, x, 9));  // 0x3F800000 | (x >> 9)
    return one_j - 0x1.fffffep-1f;
}
__device__ __forceinline__ float gumbel_log2(uint32_t x) {
    return __builtin_amdgcn_logf(-__builtin_amdgcn_logf(gumbel_u(x)));
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------------------------------------
// Element types: W and its gradient are fp32 or bf16; arithmetic is fp32.

struct F32 {
    using storage = float;
    static constexpr int bytes = 4;
};
struct BF16 {
    using storage = uint16_t;
    static constexpr int bytes = 2;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Streaming stores: outputs are written once and not read again by the same kernel, so they
// are stored non-temporally (they are not kept in the caches at the expense of the inputs).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void nt_store(void* p, uint4 v) {
    const u32x4_t x = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(x, reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ void nt_store(void* p, uint2 v) {
    const u32x2_t x = {v.x, v.y};
    __builtin_nontemporal_store(x, reinterpret_cast<u32x2_t*>(p));
}
__device__ __forceinline__ void nt_store(void* p, uint32_t v) {
    __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p));
}

// Ordinary (write-back) stores of the compressed storage: the packed values, index words and
// hard indices of the pack.  These outputs are the next kernel's inputs (unpack reads what pack
// wrote), so they are written with the default cache policy rather than the streaming hint; the
// byte and short stores of index bytes and hard indices in particular stay plain.  Measured on
// MI355X, the pack is as fast this way; the unpack's 16-byte dense stores stay non-temporal
// (ordinary stores made the LLaMA-7B-shaped unpack 30% slower).
__device__ __forceinline__ void st_store(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }
__device__ __forceinline__ void st_store(void* p, uint2 v) { *reinterpret_cast<uint2*>(p) = v; }
__device__ __forceinline__ void st_store(void* p, uint32_t v) { *reinterpret_cast<uint32_t*>(p) = v; }
__device__ __forceinline__ void st_store(void* p, uint16_t v) { *reinterpret_cast<uint16_t*>(p) = v; }
__device__ __forceinline__ void st_store(void* p, uint8_t v) { *reinterpret_cast<uint8_t*>(p) = v; }

// Streaming loads: every input element is read once per launch, so the sampling kernels load
// their inputs non-temporally as well (measured: backward 6% and forward 5% faster on MI355X).
// Only for accesses whose lanes cover whole cache lines together: when lanes are further apart
// than their vector (the pack kernels' per-thread logit runs), each instruction touches partial
// lines, and with non-temporal loads those lines are fetched again by the next instruction.
__device__ __forceinline__ uint4 nt_load4(const void* p) {
    const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ uint2 nt_load2(const void* p) {
    const u32x2_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    return make_uint2(x[0], x[1]);
}

// Round-to-nearest-even fp32 -> bf16 pair (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const __bf16 a = (__bf16)lo, b = (__bf16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Load CNT consecutive elements of type T (F32/BF16) as floats.  `vec` selects 16-byte vector
// loads (the caller guarantees alignment and that all CNT elements exist); otherwise only the
// first `valid` elements are read and the rest are zero.
template <typename T, int CNT>
__device__ __forceinline__ void load_as_float(const typename T::storage* __restrict__ p, bool vec,
                                              int valid, float (&out)[CNT]) {
    if constexpr (T::bytes == 4) {
        if (vec && CNT % 4 == 0) {
#pragma unroll
            for (int i = 0; i < CNT / 4; ++i) {
                const uint4 u = nt_load4(reinterpret_cast<const float4*>(p) + i);
                const float4 v = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
                out[4 * i + 0] = v.x;
                out[4 * i + 1] = v.y;
                out[4 * i + 2] = v.z;
                out[4 * i + 3] = v.w;
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < CNT; ++i) out[i] = (vec || i < valid) ? p[i] : 0.0f;
    } else {
        if (vec && CNT % 8 == 0) {
#pragma unroll
            for (int i = 0; i < CNT / 8; ++i) {
                const uint4 v = nt_load4(reinterpret_cast<const uint4*>(p) + i);
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    out[8 * i + 2 * q] = bf16_lo(w[q]);
                    out[8 * i + 2 * q + 1] = bf16_hi(w[q]);
                }
            }
            return;
        }
        if (vec && CNT % 4 == 0) {
#pragma unroll
            for (int i = 0; i < CNT / 4; ++i) {
                const uint2 v = nt_load2(reinterpret_cast<const uint2*>(p) + i);
                out[4 * i + 0] = bf16_lo(v.x);
                out[4 * i + 1] = bf16_hi(v.x);
                out[4 * i + 2] = bf16_lo(v.y);
                out[4 * i + 3] = bf16_hi(v.y);
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < CNT; ++i) out[i] = (vec || i < valid) ? __uint_as_float((uint32_t)p[i] << 16) : 0.0f;
    }
}

// Store CNT floats rounded to T.  Same `vec` / `valid` contract as load_as_float.
template <typename T, int CNT>
__device__ __forceinline__ void store_from_float(typename T::storage* p, bool vec,
                                                 int valid, const float (&in)[CNT]) {
    if constexpr (T::bytes == 4) {
        if (vec && CNT % 4 == 0) {
#pragma unroll
            for (int i = 0; i < CNT / 4; ++i)
                nt_store(reinterpret_cast<uint4*>(p) + i,
                         make_uint4(__float_as_uint(in[4 * i]), __float_as_uint(in[4 * i + 1]),
                                    __float_as_uint(in[4 * i + 2]), __float_as_uint(in[4 * i + 3])));
            return;
        }
#pragma unroll
        for (int i = 0; i < CNT; ++i)
            if (vec || i < valid) p[i] = in[i];
    } else {
        if (vec && CNT % 8 == 0) {
#pragma unroll
            for (int i = 0; i < CNT / 8; ++i)
                nt_store(reinterpret_cast<uint4*>(p) + i,
                         make_uint4(pack_bf16x2(in[8 * i], in[8 * i + 1]), pack_bf16x2(in[8 * i + 2], in[8 * i + 3]),
                                    pack_bf16x2(in[8 * i + 4], in[8 * i + 5]), pack_bf16x2(in[8 * i + 6], in[8 * i + 7])));
            return;
        }
        if (vec && CNT % 4 == 0) {
#pragma unroll
            for (int i = 0; i < CNT / 4; ++i)
                nt_store(reinterpret_cast<uint2*>(p) + i,
                         make_uint2(pack_bf16x2(in[4 * i], in[4 * i + 1]), pack_bf16x2(in[4 * i + 2], in[4 * i + 3])));
            return;
        }
#pragma unroll
        for (int i = 0; i < CNT; ++i)
            if (vec || i < valid) p[i] = __builtin_bit_cast(uint16_t, (__bf16)in[i]);
    }
}

}  // namespace nm
