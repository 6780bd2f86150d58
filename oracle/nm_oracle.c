/*
 * nm_oracle.c -- plain CPU oracle for the differentiable N:M mask layer.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the package smoke check and the CPU-baseline
 * leg of the benchmark, never by the product path.  It is written from the pages and from the
 * Philox paper, group by group, with no blocking, fusion or reordering beyond the definitions
 * stated at each function; all floating point is IEEE binary64 and the file is compiled without
 * fast-math and without floating-point contraction.  See nm_oracle.h for the sources.
 */
#define _GNU_SOURCE
#include "nm_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define MAX_M 8
#define MAX_K 70 /* C(8,4) */

/* ------------------------------------------------------------------------------------------ */
/* Candidates.  MaskLLM project page, Fig. 3 caption: the distribution of each group ranges over
 * the candidate masks, i.e. all ways to keep n of the m weights.  Order (a reading, the pages
 * are silent): lexicographic order of the ascending kept-position lists, so for 2:4 the
 * candidates are {0,1},{0,2},{0,3},{1,2},{1,3},{2,3}. */

int32_t ref_num_candidates(int32_t n, int32_t m) {
    if (m < 1 || m > MAX_M || n < 1 || n > m) return -1;
    int64_t c = 1;
    for (int32_t i = 0; i < n; ++i) c = c * (m - i) / (i + 1);
    return (int32_t)c;
}

/* Recursive lexicographic enumeration: choose the next kept position after `start`. */
static void enumerate(int32_t n, int32_t m, int32_t start, int32_t depth, uint8_t bits,
                      uint8_t *out, int32_t *count) {
    if (depth == n) {
        out[(*count)++] = bits;
        return;
    }
    for (int32_t p = start; p <= m - (n - depth); ++p)
        enumerate(n, m, p + 1, depth + 1, (uint8_t)(bits | (1u << p)), out, count);
}

int32_t ref_candidate_bits(int32_t n, int32_t m, uint8_t *out_bits) {
    int32_t k = ref_num_candidates(n, m);
    if (k < 0 || !out_bits) return -1;
    int32_t count = 0;
    enumerate(n, m, 0, 0, 0, out_bits, &count);
    return count == k ? 0 : -1;
}

/* ------------------------------------------------------------------------------------------ */
/* Philox4x32 (Salmon et al., SC'11, section 3.3).  One round multiplies words 0 and 2 by the
 * two round multipliers, and the new state is (hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0); between
 * rounds the key is bumped by the Weyl constants (golden ratio and sqrt(3)-1, as 32-bit
 * fractions). */

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

void ref_philox4x32(const uint32_t ctr[4], const uint32_t key[2], int32_t rounds, uint32_t out[4]) {
    uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int32_t r = 0; r < rounds; ++r) {
        if (r > 0) {
            k0 += PHILOX_W0;
            k1 += PHILOX_W1;
        }
        uint64_t p0 = (uint64_t)PHILOX_M0 * x0;
        uint64_t p1 = (uint64_t)PHILOX_M1 * x2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ x1 ^ k0;
        uint32_t n2 = hi0 ^ x3 ^ k1;
        x0 = n0;
        x1 = lo1;
        x2 = n2;
        x3 = lo0;
    }
    out[0] = x0;
    out[1] = x1;
    out[2] = x2;
    out[3] = x3;
}

/* Noise for candidate slot i = g*K + k (a reading: the pages only say "Gumbel Softmax
 * sampling").  Four consecutive slots share one 10-round block; the seed is the key and the
 * offset (the training step) fills the upper half of the counter, so each step draws fresh
 * noise and the backward pass of a step can regenerate exactly the noise of its forward. */
uint32_t ref_noise_word(uint64_t seed, uint64_t offset, uint64_t i) {
    uint64_t b = i >> 2;
    uint32_t ctr[4] = {(uint32_t)b, (uint32_t)(b >> 32), (uint32_t)offset, (uint32_t)(offset >> 32)};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    ref_philox4x32(ctr, key, 10, out);
    return out[i & 3];
}

void ref_noise_words(uint64_t seed, uint64_t offset, uint64_t first, int64_t count,
                     uint32_t *words) {
    for (int64_t j = 0; j < count; ++j) words[j] = ref_noise_word(seed, offset, first + (uint64_t)j);
}

/* Uniform in (0,1) from the top 23 bits j of a word, at the midpoint of its 2^-23 cell:
 * u = (2j + 1) / 2^24 (a reading: the pages fix no bit width; 23 bits make every u exactly
 * representable in binary32 as well).  Never 0 or 1, so both logarithms below are finite. */
double ref_uniform(uint32_t x) { return ((double)(x >> 9) + 0.5) * 0x1p-23; }

/* Gumbel(0,1) by inverting its CDF F(g) = exp(-exp(-g)). */
double ref_gumbel(uint32_t x) {
    double u = ref_uniform(x);
    return -log(-log(u));
}

void ref_gumbel_many(const uint32_t *x, int64_t count, double *g) {
    for (int64_t j = 0; j < count; ++j) g[j] = ref_gumbel(x[j]);
}

/* ------------------------------------------------------------------------------------------ */
/* element access */

static double load_w(const void *base, int32_t wtype, int64_t idx) {
    if (wtype == REF_F32) return (double)((const float *)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static void copy_w(const void *src, int64_t si, void *dst, int64_t di, int32_t wtype) {
    if (wtype == REF_F32)
        ((uint32_t *)dst)[di] = ((const uint32_t *)src)[si];
    else
        ((uint16_t *)dst)[di] = ((const uint16_t *)src)[si];
}

static void zero_w(void *dst, int64_t di, int32_t wtype) {
    if (wtype == REF_F32)
        ((uint32_t *)dst)[di] = 0u; /* +0.0 */
    else
        ((uint16_t *)dst)[di] = 0u;
}

static int shape_ok(const ref_shape *s) {
    if (!s || s->rows < 0 || s->cols < 0) return 0;
    if (ref_num_candidates(s->n, s->m) < 0) return 0;
    if (s->cols % s->m != 0) return 0;
    if (s->wtype != REF_F32 && s->wtype != REF_BF16) return 0;
    return 1;
}

static int window_ok(const ref_shape *s, int64_t rb, int64_t re) {
    return shape_ok(s) && rb >= 0 && rb <= re && re <= s->rows;
}

/* ------------------------------------------------------------------------------------------ */
/* One group's sample.  MaskLLM project page, Fig. 3 caption (Gumbel softmax over the candidate
 * logits) and Fig. 5 caption (kappa scales the logits and so sets the randomness): with
 * Gumbel noise g_k,
 *      z_k = (kappa * l_k + g_k) / tau,   y = softmax(z),
 * and the softmax subtracts the largest z first so that no exponential overflows. */
typedef struct {
    int32_t n, m, K;
    uint8_t cand[MAX_K];
    double kappa, tau;
    uint64_t seed, offset;
} group_ctx;

static void group_probs(const group_ctx *c, int64_t g, const float *l, double *y) {
    double z[MAX_K];
    for (int32_t k = 0; k < c->K; ++k) {
        uint32_t x = ref_noise_word(c->seed, c->offset, (uint64_t)g * (uint64_t)c->K + (uint64_t)k);
        double gk = ref_gumbel(x);
        z[k] = (c->kappa * (double)l[k] + gk) / c->tau;
    }
    double mu = -INFINITY;
    for (int32_t k = 0; k < c->K; ++k)
        if (z[k] > mu) mu = z[k];
    double sum = 0.0;
    for (int32_t k = 0; k < c->K; ++k) {
        y[k] = exp(z[k] - mu);
        sum += y[k];
    }
    for (int32_t k = 0; k < c->K; ++k) y[k] /= sum;
}

/* Weighted averaging of the candidates (Fig. 3 caption): m_j = sum_k y_k [candidate k keeps j]. */
static void group_soft_mask(const group_ctx *c, const double *y, double *mask) {
    for (int32_t j = 0; j < c->m; ++j) {
        mask[j] = 0.0;
        for (int32_t k = 0; k < c->K; ++k)
            if (c->cand[k] >> j & 1u) mask[j] += y[k];
    }
}

/* ------------------------------------------------------------------------------------------ */
/* Row-parallel driver: rows [rb, re) are split into contiguous blocks, one per thread. */

typedef struct job job;
typedef void (*row_fn)(const job *, int64_t r);
struct job {
    const ref_shape *s;
    group_ctx ctx;
    int64_t rb;
    const void *w;
    const float *logits;
    const void *grad;
    void *out;
    void *out2;
    uint8_t *hard;
    int64_t tokens;  /* sparse product: rows of X */
    int64_t ystride; /* sparse product: row stride of Y (the window's W rows) */
    int32_t xtype;   /* sparse product: element type of X */
    double lambda;   /* regularised backward: weight of sum (w_masked)^2 in the loss */
    row_fn fn;
};

typedef struct {
    const job *jb;
    int64_t r0, r1;
} slice;

static void *run_slice(void *arg) {
    const slice *sl = (const slice *)arg;
    for (int64_t r = sl->r0; r < sl->r1; ++r) sl->jb->fn(sl->jb, r);
    return NULL;
}

int32_t ref_threads_used(int32_t nthreads) {
    if (nthreads > 0) return nthreads;
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int32_t)n : 1;
}

static void run_rows(const job *jb, int64_t rb, int64_t re, int32_t nthreads) {
    int32_t t = ref_threads_used(nthreads);
    int64_t rows = re - rb;
    if (rows <= 0) return;
    if (t > rows) t = (int32_t)rows;
    if (t <= 1) {
        slice one = {jb, rb, re};
        run_slice(&one);
        return;
    }
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)t);
    slice *sl = (slice *)malloc(sizeof(slice) * (size_t)t);
    int32_t started = 0;
    for (int32_t i = 0; i < t; ++i) {
        sl[i].jb = jb;
        sl[i].r0 = rb + rows * i / t;
        sl[i].r1 = rb + rows * (i + 1) / t;
        if (pthread_create(&th[i], NULL, run_slice, &sl[i]) != 0) {
            run_slice(&sl[i]); /* could not start a thread: do the slice here */
            th[i] = 0;
        } else {
            ++started;
        }
    }
    for (int32_t i = 0; i < t; ++i)
        if (th[i]) pthread_join(th[i], NULL);
    (void)started;
    free(th);
    free(sl);
}

static int init_ctx(group_ctx *c, const ref_shape *s, double kappa, double tau, uint64_t seed,
                    uint64_t offset) {
    c->n = s->n;
    c->m = s->m;
    c->K = ref_num_candidates(s->n, s->m);
    if (c->K < 0 || ref_candidate_bits(s->n, s->m, c->cand) != 0) return 0;
    if (!(isfinite(kappa) && isfinite(tau) && tau > 0.0)) return 0; /* z = (kappa l + g) / tau */
    c->kappa = kappa;
    c->tau = tau;
    c->seed = seed;
    c->offset = offset;
    return 1;
}

/* ------------------------------------------------------------------------------------------ */
/* Soft mask, forward, probabilities. */

static void row_soft(const job *jb, int64_t r) {
    const ref_shape *s = jb->s;
    int64_t gpr = s->cols / s->m;
    double y[MAX_K];
    for (int64_t q = 0; q < gpr; ++q) {
        int64_t g = r * gpr + q;
        const float *l = jb->logits + ((r - jb->rb) * gpr + q) * jb->ctx.K;
        group_probs(&jb->ctx, g, l, y);
        double *mask = (double *)jb->out + (r - jb->rb) * s->cols + q * s->m;
        group_soft_mask(&jb->ctx, y, mask);
    }
}

int32_t ref_soft_mask(const ref_shape *shape, double kappa, double tau, uint64_t seed,
                      uint64_t offset, int64_t row_begin, int64_t row_end, const float *logits,
                      double *soft, int32_t nthreads) {
    job jb;
    memset(&jb, 0, sizeof jb);
    if (!window_ok(shape, row_begin, row_end) || !init_ctx(&jb.ctx, shape, kappa, tau, seed, offset))
        return -1;
    if (row_end > row_begin && (!logits || !soft)) return -1;
    jb.s = shape;
    jb.rb = row_begin;
    jb.logits = logits;
    jb.out = soft;
    jb.fn = row_soft;
    run_rows(&jb, row_begin, row_end, nthreads);
    return 0;
}

/* Frozen weights (MaskLLM abstract): the layer output is w * m, with no weight update. */
static void row_forward(const job *jb, int64_t r) {
    const ref_shape *s = jb->s;
    int64_t gpr = s->cols / s->m;
    double y[MAX_K], mask[MAX_M];
    for (int64_t q = 0; q < gpr; ++q) {
        int64_t g = r * gpr + q;
        const float *l = jb->logits + ((r - jb->rb) * gpr + q) * jb->ctx.K;
        group_probs(&jb->ctx, g, l, y);
        group_soft_mask(&jb->ctx, y, mask);
        int64_t base = (r - jb->rb) * s->cols + q * s->m;
        for (int32_t j = 0; j < s->m; ++j)
            ((double *)jb->out)[base + j] = load_w(jb->w, s->wtype, base + j) * mask[j];
    }
}

int32_t ref_forward(const ref_shape *shape, double kappa, double tau, uint64_t seed,
                    uint64_t offset, int64_t row_begin, int64_t row_end, const void *w,
                    const float *logits, double *w_masked, int32_t nthreads) {
    job jb;
    memset(&jb, 0, sizeof jb);
    if (!window_ok(shape, row_begin, row_end) || !init_ctx(&jb.ctx, shape, kappa, tau, seed, offset))
        return -1;
    if (row_end > row_begin && (!w || !logits || !w_masked)) return -1;
    jb.s = shape;
    jb.rb = row_begin;
    jb.w = w;
    jb.logits = logits;
    jb.out = w_masked;
    jb.fn = row_forward;
    run_rows(&jb, row_begin, row_end, nthreads);
    return 0;
}

static void row_probs(const job *jb, int64_t r) {
    const ref_shape *s = jb->s;
    int64_t gpr = s->cols / s->m;
    for (int64_t q = 0; q < gpr; ++q) {
        int64_t g = r * gpr + q;
        int64_t local = (r - jb->rb) * gpr + q;
        group_probs(&jb->ctx, g, jb->logits + local * jb->ctx.K, (double *)jb->out + local * jb->ctx.K);
    }
}

int32_t ref_probs(const ref_shape *shape, double kappa, double tau, uint64_t seed,
                  uint64_t offset, int64_t row_begin, int64_t row_end, const float *logits,
                  double *probs, int32_t nthreads) {
    job jb;
    memset(&jb, 0, sizeof jb);
    if (!window_ok(shape, row_begin, row_end) || !init_ctx(&jb.ctx, shape, kappa, tau, seed, offset))
        return -1;
    if (row_end > row_begin && (!logits || !probs)) return -1;
    jb.s = shape;
    jb.rb = row_begin;
    jb.logits = logits;
    jb.out = probs;
    jb.fn = row_probs;
    run_rows(&jb, row_begin, row_end, nthreads);
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Backward to the logits (Fig. 3 caption: every step is differentiable).  With upstream
 * gradient G = dL/d(w_masked):
 *     dL/dm_j = G_j w_j,   dL/dy_k = d_k = sum_{j kept by k} G_j w_j,
 *     softmax:  dL/dz_k = y_k (d_k - s),  s = sum_i y_i d_i,
 *     dz_k/dl_k = kappa / tau,
 * and the weights get no gradient (they are frozen). */
/* From a_j = dL/dm_j of one group to its logit gradient. */
static void group_backward(const group_ctx *c, const double *y, const double *a, double *out) {
    double d[MAX_K];
    double sdot = 0.0;
    for (int32_t k = 0; k < c->K; ++k) {
        d[k] = 0.0;
        for (int32_t j = 0; j < c->m; ++j)
            if (c->cand[k] >> j & 1u) d[k] += a[j];
        sdot += y[k] * d[k];
    }
    for (int32_t k = 0; k < c->K; ++k) out[k] = (c->kappa / c->tau) * y[k] * (d[k] - sdot);
}

static void row_backward(const job *jb, int64_t r) {
    const ref_shape *s = jb->s;
    const group_ctx *c = &jb->ctx;
    int64_t gpr = s->cols / s->m;
    double y[MAX_K], a[MAX_M];
    for (int64_t q = 0; q < gpr; ++q) {
        int64_t g = r * gpr + q;
        int64_t local = (r - jb->rb) * gpr + q;
        group_probs(c, g, jb->logits + local * c->K, y);
        int64_t base = (r - jb->rb) * s->cols + q * s->m;
        for (int32_t j = 0; j < s->m; ++j)
            a[j] = load_w(jb->grad, s->wtype, base + j) * load_w(jb->w, s->wtype, base + j);
        group_backward(c, y, a, (double *)jb->out + local * c->K);
    }
}

int32_t ref_backward(const ref_shape *shape, double kappa, double tau, uint64_t seed,
                     uint64_t offset, int64_t row_begin, int64_t row_end, const void *w,
                     const float *logits, const void *grad, double *dlogits, int32_t nthreads) {
    job jb;
    memset(&jb, 0, sizeof jb);
    if (!window_ok(shape, row_begin, row_end) || !init_ctx(&jb.ctx, shape, kappa, tau, seed, offset))
        return -1;
    if (row_end > row_begin && (!w || !logits || !grad || !dlogits)) return -1;
    jb.s = shape;
    jb.rb = row_begin;
    jb.w = w;
    jb.logits = logits;
    jb.grad = grad;
    jb.out = dlogits;
    jb.fn = row_backward;
    run_rows(&jb, row_begin, row_end, nthreads);
    return 0;
}

/* Backward with a weight regulariser in the loss (MaskLLM project page, Table 3: weight
 * regularisation helps mask learning).  The page states no formula; the reading here is the
 * squared norm of the masked weights, R = lambda * sum_j (w_j m_j)^2, whose gradient with
 * respect to w_masked_j is 2 lambda w_j m_j.  The loss is then the caller's task loss (upstream
 * gradient G, or none) plus R, and dL/dm_j = (G_j + 2 lambda w_j m_j) w_j; from there the
 * chain through the softmax is the one of the plain backward.  A negative lambda rewards large
 * kept weights, a positive one penalises them. */
static void row_backward_wreg(const job *jb, int64_t r) {
    const ref_shape *s = jb->s;
    const group_ctx *c = &jb->ctx;
    int64_t gpr = s->cols / s->m;
    double y[MAX_K], mask[MAX_M], a[MAX_M];
    for (int64_t q = 0; q < gpr; ++q) {
        int64_t g = r * gpr + q;
        int64_t local = (r - jb->rb) * gpr + q;
        group_probs(c, g, jb->logits + local * c->K, y);
        group_soft_mask(c, y, mask);
        int64_t base = (r - jb->rb) * s->cols + q * s->m;
        for (int32_t j = 0; j < s->m; ++j) {
            double wj = load_w(jb->w, s->wtype, base + j);
            double gj = jb->grad ? load_w(jb->grad, s->wtype, base + j) : 0.0;
            double up = gj + 2.0 * jb->lambda * wj * mask[j]; /* dL/dw_masked_j */
            a[j] = up * wj;                                   /* dL/dm_j */
        }
        group_backward(c, y, a, (double *)jb->out + local * c->K);
    }
}

int32_t ref_backward_wreg(const ref_shape *shape, double kappa, double tau, uint64_t seed,
                          uint64_t offset, double lambda, int64_t row_begin, int64_t row_end,
                          const void *w, const float *logits, const void *grad, double *dlogits,
                          int32_t nthreads) {
    job jb;
    memset(&jb, 0, sizeof jb);
    if (!window_ok(shape, row_begin, row_end) || !init_ctx(&jb.ctx, shape, kappa, tau, seed, offset))
        return -1;
    if (!isfinite(lambda)) return -1;
    if (row_end > row_begin && (!w || !logits || !dlogits)) return -1;
    jb.s = shape;
    jb.rb = row_begin;
    jb.w = w;
    jb.logits = logits;
    jb.grad = grad; /* NULL: no task loss, the regulariser alone */
    jb.lambda = lambda;
    jb.out = dlogits;
    jb.fn = row_backward_wreg;
    run_rows(&jb, row_begin, row_end, nthreads);
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Hard mask: the mode of the learned distribution, i.e. the candidate with the largest logit
 * (a reading: the project page speaks of applying the learned masks for lossless 2:4
 * sparsity; the mode carries no sampling noise).  The scan keeps the first maximum, so exact
 * ties go to the lower candidate index and a NaN logit never replaces candidate 0. */
static int32_t group_argmax(const float *l, int32_t K) {
    int32_t best = 0;
    for (int32_t k = 1; k < K; ++k)
        if (l[k] > l[best]) best = k;
    return best;
}

static void row_harden(const job *jb, int64_t r) {
    const ref_shape *s = jb->s;
    int64_t gpr = s->cols / s->m;
    for (int64_t q = 0; q < gpr; ++q) {
        int64_t local = (r - jb->rb) * gpr + q;
        jb->hard[local] = (uint8_t)group_argmax(jb->logits + local * jb->ctx.K, jb->ctx.K);
    }
}

int32_t ref_harden(const ref_shape *shape, int64_t row_begin, int64_t row_end,
                   const float *logits, uint8_t *hard, int32_t nthreads) {
    job jb;
    memset(&jb, 0, sizeof jb);
    if (!window_ok(shape, row_begin, row_end) || !init_ctx(&jb.ctx, shape, 1.0, 1.0, 0, 0)) return -1;
    if (row_end > row_begin && (!logits || !hard)) return -1;
    jb.s = shape;
    jb.rb = row_begin;
    jb.logits = logits;
    jb.hard = hard;
    jb.fn = row_harden;
    run_rows(&jb, row_begin, row_end, nthreads);
    return 0;
}

/* Compressed storage ("Accelerating Sparse Deep Neural Networks", section 3.1): only the kept
 * values are stored, and each kept value's position inside its group goes to separate
 * metadata, 2 bits for groups of four.  Readings: kept values in ascending position order;
 * bits = ceil(log2 m) per field; field f = q*n + t of a row sits at bit f*bits of the row's
 * little-endian stream of 32-bit words (so for 2:4 it is word q/8, bits 4*(q%8) + 2t); each row
 * starts on a new word and unused high bits of its last word are zero. */
static int32_t index_bits(int32_t m) {
    int32_t b = 0;
    while ((1 << b) < m) ++b;
    return b;
}

int64_t ref_index_words_per_row(const ref_shape *shape) {
    if (!shape_ok(shape)) return -1;
    int64_t fields = shape->cols / shape->m * shape->n;
    int64_t bits = fields * index_bits(shape->m);
    return (bits + 31) / 32;
}

static void put_bits(uint32_t *row, int64_t bitpos, uint32_t value, int32_t nbits) {
    for (int32_t i = 0; i < nbits; ++i) {
        int64_t p = bitpos + i;
        if (value >> i & 1u) row[p / 32] |= 1u << (p % 32);
    }
}

static uint32_t get_bits(const uint32_t *row, int64_t bitpos, int32_t nbits) {
    uint32_t v = 0;
    for (int32_t i = 0; i < nbits; ++i) {
        int64_t p = bitpos + i;
        v |= ((row[p / 32] >> (p % 32)) & 1u) << i;
    }
    return v;
}

static void row_pack(const job *jb, int64_t r) {
    const ref_shape *s = jb->s;
    int64_t gpr = s->cols / s->m;
    int64_t wpr = ref_index_words_per_row(s);
    int32_t nb = index_bits(s->m);
    int64_t lr = r - jb->rb;
    uint32_t *idx = (uint32_t *)jb->out2 + lr * wpr;
    for (int64_t i = 0; i < wpr; ++i) idx[i] = 0u;
    for (int64_t q = 0; q < gpr; ++q) {
        int64_t local = lr * gpr + q;
        int32_t k = group_argmax(jb->logits + local * jb->ctx.K, jb->ctx.K);
        if (jb->hard) jb->hard[local] = (uint8_t)k;
        int32_t t = 0;
        for (int32_t j = 0; j < s->m; ++j) {
            if (!(jb->ctx.cand[k] >> j & 1u)) continue;
            copy_w(jb->w, lr * s->cols + q * s->m + j, jb->out, lr * (s->cols / s->m * s->n) + q * s->n + t,
                   s->wtype);
            put_bits(idx, (q * s->n + t) * nb, (uint32_t)j, nb);
            ++t;
        }
    }
}

int32_t ref_pack(const ref_shape *shape, int64_t row_begin, int64_t row_end, const void *w,
                 const float *logits, void *values, uint32_t *indices, uint8_t *hard,
                 int32_t nthreads) {
    job jb;
    memset(&jb, 0, sizeof jb);
    if (!window_ok(shape, row_begin, row_end) || !init_ctx(&jb.ctx, shape, 1.0, 1.0, 0, 0)) return -1;
    if (row_end > row_begin && (!w || !logits || !values || !indices)) return -1;
    jb.s = shape;
    jb.rb = row_begin;
    jb.w = w;
    jb.logits = logits;
    jb.out = values;
    jb.out2 = indices;
    jb.hard = hard;
    jb.fn = row_pack;
    run_rows(&jb, row_begin, row_end, nthreads);
    return 0;
}

/* Decompression: each kept value goes back to the position its metadata names; every other
 * position holds +0.0. */
static void row_unpack(const job *jb, int64_t r) {
    const ref_shape *s = jb->s;
    int64_t gpr = s->cols / s->m;
    int64_t wpr = ref_index_words_per_row(s);
    int32_t nb = index_bits(s->m);
    int64_t lr = r - jb->rb;
    const uint32_t *idx = (const uint32_t *)jb->grad + lr * wpr;
    for (int64_t c = 0; c < s->cols; ++c) zero_w(jb->out, lr * s->cols + c, s->wtype);
    for (int64_t q = 0; q < gpr; ++q) {
        for (int32_t t = 0; t < s->n; ++t) {
            uint32_t p = get_bits(idx, (q * s->n + t) * nb, nb);
            if ((int32_t)p >= s->m) continue; /* malformed metadata: position outside the group */
            copy_w(jb->w, lr * (gpr * s->n) + q * s->n + t, jb->out, lr * s->cols + q * s->m + p, s->wtype);
        }
    }
}

int32_t ref_unpack(const ref_shape *shape, int64_t row_begin, int64_t row_end,
                   const void *values, const uint32_t *indices, void *dense, int32_t nthreads) {
    job jb;
    memset(&jb, 0, sizeof jb);
    if (!window_ok(shape, row_begin, row_end) || !init_ctx(&jb.ctx, shape, 1.0, 1.0, 0, 0)) return -1;
    if (row_end > row_begin && (!values || !indices || !dense)) return -1;
    jb.s = shape;
    jb.rb = row_begin;
    jb.w = values;
    jb.grad = indices;
    jb.out = dense;
    jb.fn = row_unpack;
    run_rows(&jb, row_begin, row_end, nthreads);
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Magnitude prior ("Accelerating Sparse Deep Neural Networks" summary page, section 4.1:
 * magnitude pruning keeps the largest magnitudes of each group; MaskLLM project page, Table 2
 * caption: prior masks initialise the logits of the learned masks).  Selection (a reading that
 * fixes ties): n rounds, each taking the first unchosen position with the largest |w| (a strictly
 * larger magnitude replaces the current choice, so ties keep the lower position and a NaN is
 * taken only when it is the first unchosen position).  Logits: alpha on the prior candidate,
 * 0 elsewhere. */
static int32_t prior_candidate(const group_ctx *c, const double *mag) {
    uint32_t chosen = 0;
    for (int32_t t = 0; t < c->n; ++t) {
        int32_t best = -1;
        for (int32_t j = 0; j < c->m; ++j) {
            if (chosen >> j & 1u) continue;
            if (best < 0 || mag[j] > mag[best]) best = j;
        }
        chosen |= 1u << best;
    }
    for (int32_t k = 0; k < c->K; ++k)
        if (c->cand[k] == chosen) return k;
    return -1; /* not reached: every n-subset is a candidate */
}

static void row_prior(const job *jb, int64_t r) {
    const ref_shape *s = jb->s;
    int64_t gpr = s->cols / s->m;
    double mag[MAX_M];
    for (int64_t q = 0; q < gpr; ++q) {
        int64_t local = (r - jb->rb) * gpr + q;
        for (int32_t j = 0; j < s->m; ++j)
            mag[j] = fabs(load_w(jb->w, s->wtype, (r - jb->rb) * s->cols + q * s->m + j));
        int32_t k = prior_candidate(&jb->ctx, mag);
        float *l = (float *)jb->out + local * jb->ctx.K;
        for (int32_t i = 0; i < jb->ctx.K; ++i) l[i] = i == k ? (float)jb->ctx.kappa : 0.0f;
        if (jb->hard) jb->hard[local] = (uint8_t)k;
    }
}

int32_t ref_prior_init(const ref_shape *shape, int64_t row_begin, int64_t row_end, const void *w,
                       float alpha, float *logits, uint8_t *prior_idx, int32_t nthreads) {
    job jb;
    memset(&jb, 0, sizeof jb);
    /* alpha travels in the kappa slot of the context */
    if (!window_ok(shape, row_begin, row_end) || !init_ctx(&jb.ctx, shape, (double)alpha, 1.0, 0, 0))
        return -1;
    if (row_end > row_begin && (!w || !logits)) return -1;
    jb.s = shape;
    jb.rb = row_begin;
    jb.w = w;
    jb.out = logits;
    jb.hard = prior_idx;
    jb.fn = row_prior;
    run_rows(&jb, row_begin, row_end, nthreads);
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Convergence monitors (MaskLLM project page, Fig. 5 caption): (a) the L1 distance between the
 * masks sampled at adjacent training steps, (b) the largest probability of the mask
 * distribution.  Readings: the distribution is p = softmax(kappa * l) (the one the Gumbel
 * softmax relaxes, no noise); the step's sampled mask is the candidate with the largest
 * perturbed score (kappa*l_k + g_k)/tau of that step's noise (Gumbel-max, first one on exact
 * ties); the L1 distance of two 0/1 masks counts the positions where they differ.  A previous
 * index outside [0, K) stands for the empty mask. */
static double group_max_prob(const group_ctx *c, const float *l) {
    double lmax = -INFINITY;
    for (int32_t k = 0; k < c->K; ++k)
        if ((double)l[k] > lmax) lmax = (double)l[k];
    double sum = 0.0;
    for (int32_t k = 0; k < c->K; ++k) sum += exp(c->kappa * ((double)l[k] - lmax));
    return 1.0 / sum; /* p_max = exp(0) / sum */
}

static int32_t group_sample(const group_ctx *c, int64_t g, const float *l) {
    int32_t best = 0;
    double zbest = 0.0;
    for (int32_t k = 0; k < c->K; ++k) {
        uint32_t x = ref_noise_word(c->seed, c->offset, (uint64_t)g * (uint64_t)c->K + (uint64_t)k);
        double z = (c->kappa * (double)l[k] + ref_gumbel(x)) / c->tau;
        if (k == 0 || z > zbest) {
            best = k;
            zbest = z;
        }
    }
    return best;
}

static int32_t mask_l1(const group_ctx *c, int32_t k, int32_t prev) {
    uint32_t a = c->cand[k], b = (prev >= 0 && prev < c->K) ? c->cand[prev] : 0u;
    int32_t d = 0;
    for (int32_t j = 0; j < c->m; ++j) d += (int32_t)((a >> j & 1u) != (b >> j & 1u));
    return d;
}

static void row_monitor(const job *jb, int64_t r) {
    const ref_shape *s = jb->s;
    int64_t gpr = s->cols / s->m;
    for (int64_t q = 0; q < gpr; ++q) {
        int64_t g = r * gpr + q;
        int64_t local = (r - jb->rb) * gpr + q;
        const float *l = jb->logits + local * jb->ctx.K;
        ((double *)jb->out)[local] = group_max_prob(&jb->ctx, l);
        int32_t k = group_sample(&jb->ctx, g, l);
        jb->hard[local] = (uint8_t)k;
        if (jb->grad)
            ((uint8_t *)jb->out2)[local] = (uint8_t)mask_l1(&jb->ctx, k, ((const uint8_t *)jb->grad)[local]);
    }
}

int32_t ref_monitor(const ref_shape *shape, double kappa, double tau, uint64_t seed, uint64_t offset,
                    int64_t row_begin, int64_t row_end, const float *logits, const uint8_t *prev_sample,
                    double *max_prob, uint8_t *sample, uint8_t *l1, int32_t nthreads) {
    job jb;
    memset(&jb, 0, sizeof jb);
    if (!window_ok(shape, row_begin, row_end) || !init_ctx(&jb.ctx, shape, kappa, tau, seed, offset))
        return -1;
    if (row_end > row_begin && (!logits || !max_prob || !sample || (prev_sample && !l1))) return -1;
    jb.s = shape;
    jb.rb = row_begin;
    jb.logits = logits;
    jb.grad = prev_sample;
    jb.out = max_prob;
    jb.out2 = l1;
    jb.hard = sample;
    jb.fn = row_monitor;
    run_rows(&jb, row_begin, row_end, nthreads);
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Deployment product with the compressed weights ("Accelerating Sparse Deep Neural Networks"
 * summary page, sections 3.1-3.2: the sparse operand is used in its compressed form, kept
 * values plus their positions, against a dense operand).  For a linear layer with weights
 * W [out, in] (groups of m along in, packed as above) and activations X [tokens, in]:
 *     Y[t, o] = sum over groups q and kept values u of values[o, q*n + u] * X[t, q*m + p_u]
 * with p_u the position field of (o, q, u): X times the transpose of the unpacked W.  Binary64
 * products and sums, groups and kept values in ascending order.  Work is split over W rows;
 * y is [tokens, window rows] (column o - row_begin holds W row o). */
static void row_sparse_matmul(const job *jb, int64_t o) {
    const ref_shape *s = jb->s;
    int64_t gpr = s->cols / s->m;
    int64_t wpr = ref_index_words_per_row(s);
    int32_t nb = index_bits(s->m);
    int64_t lo = o - jb->rb;
    const uint32_t *idx = (const uint32_t *)jb->grad + lo * wpr;
    for (int64_t t = 0; t < jb->tokens; ++t) {
        double acc = 0.0;
        for (int64_t q = 0; q < gpr; ++q) {
            for (int32_t u = 0; u < s->n; ++u) {
                uint32_t p = get_bits(idx, (q * s->n + u) * nb, nb);
                if ((int32_t)p >= s->m) continue; /* malformed metadata: nothing kept there */
                double v = load_w(jb->w, s->wtype, lo * (gpr * s->n) + q * s->n + u);
                acc += v * load_w(jb->out2, jb->xtype, t * s->cols + q * s->m + p);
            }
        }
        ((double *)jb->out)[t * jb->ystride + lo] = acc;
    }
}

int32_t ref_sparse_matmul(const ref_shape *shape, int64_t row_begin, int64_t row_end,
                          const void *values, const uint32_t *indices, const void *x,
                          int32_t xtype, int64_t tokens, double *y, int32_t nthreads) {
    job jb;
    memset(&jb, 0, sizeof jb);
    if (!window_ok(shape, row_begin, row_end) || !init_ctx(&jb.ctx, shape, 1.0, 1.0, 0, 0)) return -1;
    if (tokens < 0 || (xtype != REF_F32 && xtype != REF_BF16)) return -1;
    if (row_end > row_begin && tokens > 0 && (!values || !indices || !x || !y)) return -1;
    jb.s = shape;
    jb.rb = row_begin;
    jb.w = values;
    jb.grad = indices;
    jb.out2 = (void *)x; /* read only */
    jb.out = y;
    jb.tokens = tokens;
    jb.ystride = row_end - row_begin;
    jb.xtype = xtype;
    jb.fn = row_sparse_matmul;
    run_rows(&jb, row_begin, row_end, nthreads);
    return 0;
}
