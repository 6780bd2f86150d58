// nm_backward.hpp -- the backward kernel template (internal), instantiated by nm_backward.hip
// (plain) and nm_backward_wreg.hip (with the weight regulariser) in two translation units that
// compile in parallel.
#pragma once
#include "nm_layer.hpp"

namespace nm {

// ------------------------------------------------------------------------------------------
// Backward to the logits (Fig. 3 caption: all steps differentiable).  Upstream G = dL/dw_masked:
//   dL/dy_k = d_k = sum_{j kept by k} G_j w_j,  s = sum_k y_k d_k,
//   dL/dl_k = (kappa/tau) * y_k * (d_k - s).
// The noise is regenerated from the same (seed, offset) as the forward.
//
// REG adds the weight regulariser lambda * sum (w_j m_j)^2 to the loss (MaskLLM project page,
// Table 3: weight regularisation helps mask learning; the squared norm of the masked weights is
// the reading taken, the page gives no formula).  Its gradient on w_masked is 2 lambda w_j m_j,
// so G_j becomes G_j + 2 lambda w_j m_j, with m_j the soft mask this pass already has.
//   REG 0: task gradient only;  1: task gradient + regulariser;  2: regulariser only (no G read).

template <int N, int M, typename T, int REG>
__global__ __launch_bounds__(kThreads) void k_backward(BwdArgs a) {
    using S = Sample<N, M>;
    constexpr int K = S::K, P = S::P, PK = S::PK;
    const ThreadGroup<N, M> tg = thread_group<N, M>();
    const int64_t g0 = tg.g0;
    if (g0 >= a.groups) return;
    const int nvalid = (int)(a.groups - g0 < P ? a.groups - g0 : P);
    const bool full = nvalid == P;

    __shared__ typename StageTile<N, M>::vec tile[StageTile<N, M>::VEC];
    const bool staged = block_full<N, M>(a.groups);  // uniform over the block
    // The logits go through LDS before the noise is generated (generating the noise while they
    // are in flight, as k_forward does for groups of eight, measured slower here: the backward
    // already overlaps its weight and gradient loads with that work).
    constexpr bool EARLY = false;
    float l[PK];
    StagedSpan<N, M> span;
    logits_issue<N, M>(a.logits, g0, full, nvalid, staged, span, l);
    if constexpr (!EARLY) logits_exchange<N, M>(tg.q, staged, tile, span, l);
    float w[P * M], gw[P * M];
    load_as_float<T, P * M>(reinterpret_cast<const typename T::storage*>(a.w) + g0 * M, full, nvalid * M, w);
    if constexpr (REG != 2)
        load_as_float<T, P * M>(reinterpret_cast<const typename T::storage*>(a.grad) + g0 * M, full, nvalid * M, gw);
    float h[PK];
    thread_noise<N, M>(step_key(a.nk, a.offset_dev), g0, h);
    if constexpr (EARLY) logits_exchange<N, M>(tg.q, staged, tile, span, l);

    float dl[PK];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        float e[K], sj[M];
        group_exp<N, M>(l + p * K, h + p * K, a.A, a.B, e);
        const float inv = group_soft<N, M>(e, sj);
        float aj[M];
#pragma unroll
        for (int j = 0; j < M; ++j) {
            const float wj = w[p * M + j];
            if constexpr (REG == 0) {
                aj[j] = gw[p * M + j] * wj;
            } else {
                const float mj = sj[j] * inv;
                const float up = REG == 1 ? fmaf(a.lam2 * wj, mj, gw[p * M + j]) : (a.lam2 * wj) * mj;
                aj[j] = up * wj;
            }
        }
        // s = sum_k y_k d_k: four interleaved fma chains, added at the end, so a K-term sum
        // rounds about K/4 + 2 times on any path instead of K (K = 70 for 4:8)
        float d[K];
        float es[4] = {-0.0f, -0.0f, -0.0f, -0.0f};
        candidate_sums<N, M>(aj, [&](auto kc, float dk) NM_INLINE {
            constexpr int k = decltype(kc)::value;
            d[k] = dk;
            es[k & 3] = k < 4 ? e[k] * dk : fmaf(e[k], dk, es[k & 3]);
        });
        const float s = ((es[0] + es[1]) + (es[2] + es[3])) * inv;
        const float ci = a.C * inv;
#pragma unroll
        for (int k = 0; k < K; ++k) dl[p * K + k] = (ci * e[k]) * (d[k] - s);
    }
    store_dlogits<N, M>(a.dlogits, g0, tg.q, full, nvalid, staged, tile, dl);
}

}  // namespace nm
