/*
 * nm_oracle.h -- plain CPU oracle for the differentiable N:M mask layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the CPU-baseline
 * leg of the benchmark may load this library.  It shares no code, header, table or constant
 * with the HIP library under semi_structured_sparsity_amd/csrc, and it never includes it.
 *
 * What it computes (every floating-point step in IEEE binary64 unless a comment says otherwise):
 *
 *   MaskLLM project page ("MaskLLM: Learnable Semi-Structured Sparsity for Large Language
 *   Models"), Fig. 3 caption: each run of M consecutive weights owns a learnable categorical
 *   distribution over the candidate N:M masks; a Gumbel-softmax sample of that distribution is
 *   turned into a soft mask by weighted averaging of the candidates, and every step is
 *   differentiable.  Fig. 5 caption: a scaling factor kappa sets how random the sampling is.
 *   Abstract: the weights stay frozen, only the masks are learned.
 *
 *   "Accelerating Sparse Deep Neural Networks" summary page, section 3.1: the compressed 2:4
 *   format keeps the two non-zero values of every four and stores each one's position inside
 *   its group in 2 bits of separate metadata.  Section 4.1: magnitude pruning keeps the largest
 *   magnitudes of each group of four.
 *
 *   Philox4x32: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel Random Numbers:
 *   As Easy as 1, 2, 3", SC'11, section 3.3 (the Philox S-box and key schedule).
 *
 * Readings of points the pages leave open (N = number kept; groups along the contiguous input
 * dimension; lexicographic candidate order; fp32 logits [rows, cols/M, K]; z = (kappa*l+g)/tau;
 * Philox counter map; 23-bit midpoint uniforms; argmax of the logits for the hard mask with the
 * first maximum winning; little-endian per-row index bitstream) are listed with each function.
 *
 * Parity pins: every function below is pinned by tests/test_oracle_*.py against library
 * routines, closed forms, brute force or invariants; none is "parity unpinned".
 */
#ifndef NM_ORACLE_H
#define NM_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* weight element types (the oracle's own numbering, matched by value in oracle.py) */
#define REF_F32 0
#define REF_BF16 1

typedef struct {
    int64_t rows, cols; /* W is [rows, cols] row-major; groups of m run along cols */
    int32_t n, m;       /* n kept of every m */
    int32_t wtype;      /* REF_F32 or REF_BF16 */
} ref_shape;

/* Return codes: 0 ok, -1 bad argument (among them a non-finite kappa or tau, or tau <= 0). */

/* --- candidates ------------------------------------------------------------------------- */
/* C(m, n), or -1 if not 1 <= n <= m <= 8. */
int32_t ref_num_candidates(int32_t n, int32_t m);
/* The C(m,n) n-subsets of {0..m-1} in lexicographic order of their ascending position lists;
 * out_bits[k] has bit j set iff position j is kept by candidate k. */
int32_t ref_candidate_bits(int32_t n, int32_t m, uint8_t *out_bits);

/* --- counter-based noise ---------------------------------------------------------------- */
/* One Philox4x32 block with `rounds` rounds: out = Philox(ctr, key). */
void ref_philox4x32(const uint32_t ctr[4], const uint32_t key[2], int32_t rounds, uint32_t out[4]);
/* The raw noise word of candidate slot i = g*K + k: word (i & 3) of the 10-round block with
 * key (seed lo, seed hi) and counter ((i>>2) lo, (i>>2) hi, offset lo, offset hi). */
uint32_t ref_noise_word(uint64_t seed, uint64_t offset, uint64_t i);
/* words[j] = ref_noise_word(seed, offset, first + j) for j < count */
void ref_noise_words(uint64_t seed, uint64_t offset, uint64_t first, int64_t count,
                     uint32_t *words);
/* u = ((x >> 9) + 1/2) / 2^23, exact in binary64 (and in binary32), in (0, 1). */
double ref_uniform(uint32_t x);
/* Standard Gumbel(0,1) sample by the inverse CDF: g = -ln(-ln u). */
double ref_gumbel(uint32_t x);
/* g[j] = ref_gumbel(x[j]) */
void ref_gumbel_many(const uint32_t *x, int64_t count, double *g);

/* --- the layer -------------------------------------------------------------------------- *
 * All layer functions work on the row window [row_begin, row_end) of a matrix of shape
 * `shape`.  Pointers point at the data of row `row_begin` (not of row 0), so a caller can pass
 * a window copied out of a large matrix; the noise still uses the global group index
 * g = r*(cols/m) + q.  nthreads <= 0 means all online CPUs.
 *
 *   w, grad      [rows, cols] in shape->wtype (bf16 = upper 16 bits of an fp32)
 *   logits       fp32 [rows, cols/m, K], K contiguous
 *   soft/w_masked/dlogits  binary64 results, same layout as their fp32/wtype counterparts   */

/* y_k = softmax_k((kappa*l_k + g_k)/tau), m_j = sum over candidates k that keep j of y_k. */
int32_t ref_soft_mask(const ref_shape *shape, double kappa, double tau, uint64_t seed,
                      uint64_t offset, int64_t row_begin, int64_t row_end, const float *logits,
                      double *soft, int32_t nthreads);
/* w_masked = w * soft_mask (frozen weights, no rounding to wtype). */
int32_t ref_forward(const ref_shape *shape, double kappa, double tau, uint64_t seed,
                    uint64_t offset, int64_t row_begin, int64_t row_end, const void *w,
                    const float *logits, double *w_masked, int32_t nthreads);
/* dlogits_k = d loss / d l_k for an upstream gradient grad = d loss / d w_masked. */
int32_t ref_backward(const ref_shape *shape, double kappa, double tau, uint64_t seed,
                     uint64_t offset, int64_t row_begin, int64_t row_end, const void *w,
                     const float *logits, const void *grad, double *dlogits, int32_t nthreads);
/* dlogits of the task loss (upstream grad, may be NULL for none) plus the weight regulariser
 * lambda * sum (w * soft_mask)^2: the upstream gradient becomes grad + 2 lambda w_masked. */
int32_t ref_backward_wreg(const ref_shape *shape, double kappa, double tau, uint64_t seed,
                          uint64_t offset, double lambda, int64_t row_begin, int64_t row_end,
                          const void *w, const float *logits, const void *grad, double *dlogits,
                          int32_t nthreads);
/* Per-group probabilities y [groups, K] (a by-product of the soft mask, used for statistics). */
int32_t ref_probs(const ref_shape *shape, double kappa, double tau, uint64_t seed,
                  uint64_t offset, int64_t row_begin, int64_t row_end, const float *logits,
                  double *probs, int32_t nthreads);

/* --- hard mask and compressed storage ---------------------------------------------------- */
/* Words per row of the index bitstream: ceil((cols/m) * n * bits / 32), bits = ceil(log2 m). */
int64_t ref_index_words_per_row(const ref_shape *shape);
/* hard[g] = first k with the largest logit (no noise). */
int32_t ref_harden(const ref_shape *shape, int64_t row_begin, int64_t row_end,
                   const float *logits, uint8_t *hard, int32_t nthreads);
/* values [rows, cols*n/m] (wtype, bit copies of the kept weights, ascending position);
 * indices [rows, words_per_row] little-endian bit fields, field f = q*n + t at bit f*bits. */
int32_t ref_pack(const ref_shape *shape, int64_t row_begin, int64_t row_end, const void *w,
                 const float *logits, void *values, uint32_t *indices, uint8_t *hard,
                 int32_t nthreads);
/* dense [rows, cols] = +0.0 everywhere, then the kept values scattered back. */
int32_t ref_unpack(const ref_shape *shape, int64_t row_begin, int64_t row_end,
                   const void *values, const uint32_t *indices, void *dense, int32_t nthreads);

/* --- magnitude prior -------------------------------------------------------------------- */
/* logits [rows, cols/m, K] fp32 (overwritten): alpha on the candidate that keeps the n largest
 * |w| of the group (n rounds of "first largest |w| among unchosen positions"), 0 elsewhere;
 * prior_idx [rows, cols/m] (optional) gets that candidate's index. */
int32_t ref_prior_init(const ref_shape *shape, int64_t row_begin, int64_t row_end, const void *w,
                       float alpha, float *logits, uint8_t *prior_idx, int32_t nthreads);

/* --- convergence monitors ------------------------------------------------------------------ */
/* Per group of the window: max_prob = max_k softmax(kappa*l)_k (no noise); sample = the index of
 * the largest (kappa*l_k + g_k)/tau with the noise of (seed, offset), first one on exact ties;
 * if prev_sample is given, l1 = number of positions where the masks of sample and prev_sample
 * differ (a prev_sample entry >= K stands for the empty mask).  All three are [window groups]. */
int32_t ref_monitor(const ref_shape *shape, double kappa, double tau, uint64_t seed, uint64_t offset,
                    int64_t row_begin, int64_t row_end, const float *logits, const uint8_t *prev_sample,
                    double *max_prob, uint8_t *sample, uint8_t *l1, int32_t nthreads);

/* --- product with the compressed weights ------------------------------------------------ */
/* y [tokens, row_end - row_begin] binary64 (overwritten): y[t, o - row_begin] = sum over the
 * kept values of W row o (values, indices in the packed layout, rows of the window) times the
 * matching elements of X row t.  x [tokens, cols] of type xtype (REF_F32 or REF_BF16 bits). */
int32_t ref_sparse_matmul(const ref_shape *shape, int64_t row_begin, int64_t row_end,
                          const void *values, const uint32_t *indices, const void *x,
                          int32_t xtype, int64_t tokens, double *y, int32_t nthreads);

/* number of worker threads a call with this nthreads argument uses */
int32_t ref_threads_used(int32_t nthreads);

#ifdef __cplusplus
}
#endif
#endif
