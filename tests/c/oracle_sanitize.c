/* A C driver of every oracle entry point, for builds with AddressSanitizer + UndefinedBehavior-
 * Sanitizer (and, on its own, ThreadSanitizer).  Every buffer is allocated with exactly the size
 * the call's row window needs, so a read or write past a window's end is an ASan report; the
 * windows are ragged (rows 1..4 of 5, a row length that is not a multiple of 32 groups) and the
 * worker counts are 1, 3 and 8, so that the threaded row split is exercised and TSan sees the
 * workers.  Results must be identical for every worker count, the soft masks of a group must
 * add up to n, unpack(pack(w)) must keep exactly the hard mask's weights, and the argument checks
 * must reject what the header says they reject.  Prints one line per failure, then a summary. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "nm_oracle.h"

static int failures = 0;
#define CHECK(cond)                                                \
    do {                                                           \
        if (!(cond)) {                                             \
            printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                            \
        }                                                          \
    } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) { /* xorshift64*: inputs only */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static float next_f(void) { return (float)((int32_t)(next_u32() % 2001u) - 1000) / 500.0f; }

static void *xmalloc(size_t bytes) {
    void *p = malloc(bytes ? bytes : 1);
    if (!p) {
        printf("out of memory\n");
        exit(2);
    }
    return p;
}

/* weights of the window in wtype (bf16 = the upper half of an fp32, exact for these values) */
static void *make_w(int32_t wtype, int64_t count) {
    if (wtype == REF_F32) {
        float *w = (float *)xmalloc((size_t)count * 4);
        for (int64_t i = 0; i < count; ++i) w[i] = next_f();
        return w;
    }
    uint16_t *w = (uint16_t *)xmalloc((size_t)count * 2);
    for (int64_t i = 0; i < count; ++i) {
        const float f = (float)((int32_t)(next_u32() % 17u) - 8) / 4.0f;
        uint32_t b;
        memcpy(&b, &f, 4);
        w[i] = (uint16_t)(b >> 16);
    }
    return w;
}

static double w_at(const void *w, int32_t wtype, int64_t i) {
    if (wtype == REF_F32) return ((const float *)w)[i];
    const uint32_t b = (uint32_t)((const uint16_t *)w)[i] << 16;
    float f;
    memcpy(&f, &b, 4);
    return f;
}

static const int32_t THREADS[] = {1, 3, 8};

static void one_layout(int32_t n, int32_t m, int32_t wtype) {
    const int32_t K = ref_num_candidates(n, m);
    CHECK(K > 0);
    const int64_t rows = 5, gpr = 37, cols = gpr * m, rb = 1, re = 4, wr = re - rb;
    const ref_shape s = {rows, cols, n, m, wtype};
    const int64_t wcount = wr * cols, lcount = wr * gpr * K, groups = wr * gpr;
    const double kappa = 30.0, tau = 0.4;
    const uint64_t seed = 77, offset = 5;

    uint8_t cand[70];
    CHECK(ref_candidate_bits(n, m, cand) == 0);
    void *w = make_w(wtype, wcount), *grad = make_w(wtype, wcount);
    float *logits = (float *)xmalloc((size_t)lcount * 4);
    for (int64_t i = 0; i < lcount; ++i) logits[i] = next_f();

    double *first_soft = NULL, *first_fwd = NULL, *first_bwd = NULL, *first_reg = NULL, *first_probs = NULL,
           *first_mp = NULL;
    uint8_t *first_smp = NULL;
    for (size_t t = 0; t < sizeof THREADS / sizeof THREADS[0]; ++t) {
        const int32_t nt = THREADS[t];
        double *soft = (double *)xmalloc((size_t)wcount * 8), *fwd = (double *)xmalloc((size_t)wcount * 8);
        double *bwd = (double *)xmalloc((size_t)lcount * 8), *reg = (double *)xmalloc((size_t)lcount * 8);
        double *probs = (double *)xmalloc((size_t)lcount * 8), *mp = (double *)xmalloc((size_t)groups * 8);
        uint8_t *smp = (uint8_t *)xmalloc((size_t)groups), *prev = (uint8_t *)xmalloc((size_t)groups);
        uint8_t *l1 = (uint8_t *)xmalloc((size_t)groups);
        CHECK(ref_soft_mask(&s, kappa, tau, seed, offset, rb, re, logits, soft, nt) == 0);
        CHECK(ref_forward(&s, kappa, tau, seed, offset, rb, re, w, logits, fwd, nt) == 0);
        CHECK(ref_backward(&s, kappa, tau, seed, offset, rb, re, w, logits, grad, bwd, nt) == 0);
        CHECK(ref_backward_wreg(&s, kappa, tau, seed, offset, 0.25, rb, re, w, logits, NULL, reg, nt) == 0);
        CHECK(ref_probs(&s, kappa, tau, seed, offset, rb, re, logits, probs, nt) == 0);
        for (int64_t g = 0; g < groups; ++g) prev[g] = (uint8_t)(g % (K + 1)); /* K: the empty mask */
        CHECK(ref_monitor(&s, kappa, tau, seed, offset, rb, re, logits, prev, mp, smp, l1, nt) == 0);
        CHECK(ref_monitor(&s, kappa, tau, seed, offset, rb, re, logits, NULL, mp, smp, NULL, nt) == 0);
        for (int64_t g = 0; g < groups; ++g) {
            double sum = 0.0, ps = 0.0;
            for (int32_t j = 0; j < m; ++j) sum += soft[g * m + j];
            for (int32_t k = 0; k < K; ++k) ps += probs[g * K + k];
            CHECK(fabs(sum - n) < 1e-12);
            CHECK(fabs(ps - 1.0) < 1e-12);
            CHECK(smp[g] < K && mp[g] > 0.0 && mp[g] <= 1.0);
        }
        if (t == 0) {
            first_soft = soft, first_fwd = fwd, first_bwd = bwd, first_reg = reg, first_probs = probs, first_mp = mp;
            first_smp = smp;
        } else {
            CHECK(memcmp(soft, first_soft, (size_t)wcount * 8) == 0);
            CHECK(memcmp(fwd, first_fwd, (size_t)wcount * 8) == 0);
            CHECK(memcmp(bwd, first_bwd, (size_t)lcount * 8) == 0);
            CHECK(memcmp(reg, first_reg, (size_t)lcount * 8) == 0);
            CHECK(memcmp(probs, first_probs, (size_t)lcount * 8) == 0);
            CHECK(memcmp(mp, first_mp, (size_t)groups * 8) == 0);
            CHECK(memcmp(smp, first_smp, (size_t)groups) == 0);
            free(soft), free(fwd), free(bwd), free(reg), free(probs), free(mp), free(smp);
        }
        free(prev), free(l1);

        /* hard mask, pack, unpack */
        const int64_t wpr = ref_index_words_per_row(&s), vcount = wr * (cols / m) * n;
        const size_t esz = wtype == REF_F32 ? 4 : 2;
        uint8_t *hard = (uint8_t *)xmalloc((size_t)groups), *hard2 = (uint8_t *)xmalloc((size_t)groups);
        void *values = xmalloc((size_t)vcount * esz), *dense = xmalloc((size_t)wcount * esz);
        uint32_t *idx = (uint32_t *)xmalloc((size_t)(wr * wpr) * 4);
        CHECK(ref_harden(&s, rb, re, logits, hard, nt) == 0);
        CHECK(ref_pack(&s, rb, re, w, logits, values, idx, hard2, nt) == 0);
        CHECK(memcmp(hard, hard2, (size_t)groups) == 0);
        CHECK(ref_unpack(&s, rb, re, values, idx, dense, nt) == 0);
        for (int64_t g = 0; g < groups; ++g)
            for (int32_t j = 0; j < m; ++j) {
                const double want = (cand[hard[g]] >> j & 1) ? w_at(w, wtype, g * m + j) : 0.0;
                CHECK(w_at(dense, wtype, g * m + j) == want);
            }

        /* magnitude prior */
        float *pl = (float *)xmalloc((size_t)lcount * 4);
        uint8_t *pidx = (uint8_t *)xmalloc((size_t)groups);
        CHECK(ref_prior_init(&s, rb, re, w, 3.0f, pl, pidx, nt) == 0);
        for (int64_t g = 0; g < groups; ++g) {
            CHECK(pidx[g] < K && pl[g * K + pidx[g]] == 3.0f);
            double kept = 1e300, dropped = 0.0; /* every kept |w| >= every dropped |w| */
            for (int32_t j = 0; j < m; ++j) {
                const double a = fabs(w_at(w, wtype, g * m + j));
                if (cand[pidx[g]] >> j & 1)
                    kept = a < kept ? a : kept;
                else
                    dropped = a > dropped ? a : dropped;
            }
            CHECK(kept >= dropped);
        }

        /* product with the packed weights: y equals the dense dot product of the unpacked rows */
        const int64_t tokens = 3;
        float *x = (float *)xmalloc((size_t)(tokens * cols) * 4);
        for (int64_t i = 0; i < tokens * cols; ++i) x[i] = next_f();
        double *y = (double *)xmalloc((size_t)(tokens * wr) * 8);
        CHECK(ref_sparse_matmul(&s, rb, re, values, idx, x, REF_F32, tokens, y, nt) == 0);
        for (int64_t tk = 0; tk < tokens; ++tk)
            for (int64_t o = 0; o < wr; ++o) {
                double acc = 0.0, mag = 0.0;
                for (int64_t c = 0; c < cols; ++c) {
                    acc += w_at(dense, wtype, o * cols + c) * (double)x[tk * cols + c];
                    mag += fabs(w_at(dense, wtype, o * cols + c) * (double)x[tk * cols + c]);
                }
                CHECK(fabs(y[tk * wr + o] - acc) <= 1e-13 * (mag + 1.0));
            }
        free(hard), free(hard2), free(values), free(dense), free(idx), free(pl), free(pidx), free(x), free(y);
    }
    free(first_soft), free(first_fwd), free(first_bwd), free(first_reg), free(first_probs), free(first_mp), free(first_smp);
    free(w), free(grad), free(logits);
}

static void argument_checks(void) {
    const ref_shape s = {4, 8, 2, 4, REF_F32};
    float l[4 * 2 * 6] = {0};
    double out[4 * 8];
    uint8_t hard[8];
    CHECK(ref_num_candidates(0, 4) == -1 && ref_num_candidates(5, 4) == -1 && ref_num_candidates(2, 9) == -1);
    CHECK(ref_candidate_bits(2, 4, NULL) == -1);
    CHECK(ref_soft_mask(NULL, 1.0, 1.0, 0, 0, 0, 4, l, out, 1) == -1);
    CHECK(ref_soft_mask(&s, 1.0, 1.0, 0, 0, 0, 5, l, out, 1) == -1);    /* window past the rows */
    CHECK(ref_soft_mask(&s, 1.0, 1.0, 0, 0, 3, 2, l, out, 1) == -1);    /* reversed window */
    CHECK(ref_soft_mask(&s, 1.0, 0.0, 0, 0, 0, 4, l, out, 1) == -1);    /* tau = 0 */
    CHECK(ref_soft_mask(&s, 1.0, 1.0, 0, 0, 0, 4, NULL, out, 1) == -1);
    CHECK(ref_soft_mask(&s, 1.0, 1.0, 0, 0, 2, 2, NULL, NULL, 1) == 0); /* empty window */
    CHECK(ref_backward_wreg(&s, 1.0, 1.0, 0, 0, NAN, 0, 4, l, l, NULL, out, 1) == -1);
    CHECK(ref_harden(&s, 0, 4, l, NULL, 1) == -1);
    CHECK(ref_harden(&s, 0, 4, l, hard, 1) == 0);
    const ref_shape ragged = {4, 6, 2, 4, REF_F32}; /* cols not a multiple of m */
    CHECK(ref_harden(&ragged, 0, 4, l, hard, 1) == -1);
    CHECK(ref_sparse_matmul(&s, 0, 4, l, (const uint32_t *)l, l, 7, 1, out, 1) == -1);
    CHECK(ref_sparse_matmul(&s, 0, 4, l, (const uint32_t *)l, l, REF_F32, -1, out, 1) == -1);
    CHECK(ref_threads_used(3) == 3 && ref_threads_used(0) >= 1);
    uint32_t words[9];
    ref_noise_words(1, 2, 3, 0, NULL); /* count 0 writes nothing */
    ref_noise_words(1, 2, 3, 9, words);
    for (int i = 0; i < 9; ++i) CHECK(words[i] == ref_noise_word(1, 2, 3 + (uint64_t)i));
    double g[9];
    ref_gumbel_many(words, 9, g);
    for (int i = 0; i < 9; ++i) CHECK(isfinite(g[i]));
    CHECK(ref_uniform(0u) > 0.0 && ref_uniform(0xFFFFFFFFu) < 1.0);
}

int main(void) {
    argument_checks();
    const int32_t layouts[][2] = {{1, 4}, {2, 4}, {2, 8}, {4, 8}};
    for (size_t i = 0; i < sizeof layouts / sizeof layouts[0]; ++i) {
        one_layout(layouts[i][0], layouts[i][1], REF_F32);
        one_layout(layouts[i][0], layouts[i][1], REF_BF16);
    }
    printf(failures ? "oracle sanitize check: %d failure(s)\n" : "oracle sanitize check: ok\n", failures);
    return failures ? 1 : 0;
}
