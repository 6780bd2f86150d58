/*
 * nm_mask.h -- C ABI of the MI355X (gfx950) library for learnable N:M semi-structured sparsity:
 * the differentiable Gumbel-softmax mask layer, its backward pass to the logits, hard-mask
 * extraction and the compressed N:M storage format; around it, the magnitude-prior
 * initialisation of the logits, the forward with the convergence monitors fused in, and the
 * product of activations with the packed 2:4 weights on the sparse matrix cores.
 *
 * Method (MaskLLM project page, "MaskLLM: Learnable Semi-Structured Sparsity for Large Language
 * Models", Fig. 3 caption): each run of M consecutive weights owns a learnable categorical
 * distribution over the C(M,N) candidate masks that keep N of the M weights.  A Gumbel-softmax
 * sample of that distribution, weighted-averaged over the candidates, is a differentiable soft
 * mask.  Fig. 5 caption: a scaling factor kappa sets the randomness of the sampling.  Abstract:
 * the weights stay frozen and only the masks are learned.
 * Compressed storage ("Accelerating Sparse Deep Neural Networks" summary page, section 3.1):
 * only the kept values are stored, plus the position of each kept value inside its group as
 * separate metadata (2 bits per kept value for groups of four).
 *
 * Conventions used by every entry point
 *   W          [rows, cols] row-major, element type shape->wtype (NM_F32 or NM_BF16); groups of
 *              m consecutive elements run along cols (the contiguous, input dimension), so group
 *              g = r*(cols/m) + q holds W[r, q*m .. q*m+m-1].
 *   candidates the K = C(m,n) subsets of n kept positions, in lexicographic order of their
 *              ascending position lists (2:4: {0,1},{0,2},{0,3},{1,2},{1,3},{2,3}); see
 *              nm_candidate_table.
 *   logits     fp32 [rows, cols/m, K], K contiguous: logit k of group g is logits[g*K + k].
 *   noise      candidate slot i = g*K + k uses word (i & 3) of the Philox4x32-10 block (Salmon et
 *              al., SC'11) with key (seed lo, seed hi) and counter ((i>>2) lo, (i>>2) hi,
 *              offset lo, offset hi).  Its top 23 bits j give u = (j + 1/2) / 2^23 (exact in
 *              fp32) and the Gumbel sample g = -ln(-ln u).  offset is the training step:
 *              forward and backward of one step pass the same (seed, offset), and the backward
 *              regenerates the noise instead of reading it from memory.
 *   sample     y_k = softmax_k((kappa*l_k + g_k) / tau); soft mask m_j = sum of y_k over the
 *              candidates k that keep position j (so m_j is in [0,1] and sums to n per group).
 *   hard mask  the candidate with the largest logit (no noise; the first one on exact ties).
 *   packed     values [rows, cols*n/m] in wtype: the kept weights of each group in ascending
 *              position order.  indices: per row, a little-endian stream of 32-bit words holding
 *              b = ceil(log2 m) bits per kept value (2 for m = 4, 3 for m = 8); field
 *              f = q*n + t of a row (kept value t of group q) sits at bit f*b.  Each row starts
 *              on a new word; unused bits of its last word are zero.  Words per row:
 *              nm_index_words_per_row.
 *
 * Supported: m in {4, 8}, 1 <= n < m (K = 4, 6, 4 for m = 4; 8, 28, 56, 70, 56, 28, 8 for
 * m = 8); wtype NM_F32 or NM_BF16; all arithmetic is fp32.
 *
 * Ownership and execution: every pointer is device memory owned by the caller (a torch tensor,
 * a hipMalloc buffer).  An output must not overlap an input or another output.  The library
 * allocates nothing, keeps no mutable global state other than the fixed device array of
 * nm_mask_forward_monitor_static, and may be called from several host threads.  Calls are asynchronous and ordered on `stream` (a
 * hipStream_t passed as void*; NULL is the default stream).  The return value reports argument
 * validation and launch only; execution errors surface at the caller's next synchronisation.
 * Calls can be captured into a HIP graph on `stream` (none allocates, synchronises or records a
 * memset); the sample is a launch argument, so a captured forward or backward replays the noise
 * of the step it was captured with, unless the step offset is read from device memory
 * (nm_mask_forward_offset_dev, nm_mask_backward_offset_dev).
 *
 * Errors: arguments are checked on the host before any HIP call; on an error nothing is
 * launched and no output is touched.  An empty matrix (rows == 0 or cols == 0) is valid and
 * launches nothing.  Outputs are unspecified for non-finite weights, logits or gradients, except
 * that the hard mask and the packed data are always well formed (a NaN logit never wins over
 * logit 0 of its group).
 *   NM_EINVAL       null shape/sample/required pointer, rows or cols < 0, cols % m != 0,
 *                   kappa < 0 or non-finite, tau <= 0 or non-finite, size overflow
 *   NM_EUNSUPPORTED (n, m) or wtype outside the supported set
 *   NM_EALIGN       a data pointer that is not 16-byte aligned
 *   NM_EHIP         the HIP launch failed (hipGetLastError is consumed)
 *   NM_ESCRATCH     the shape needs more scratch memory than nm_mask_forward_monitor_static's
 *                   fixed array holds
 */
#ifndef NM_MASK_H
#define NM_MASK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NM_OK = 0,
    NM_EINVAL = 1,
    NM_EALIGN = 2,
    NM_EUNSUPPORTED = 3,
    NM_EHIP = 4,
    NM_ESCRATCH = 5
} nm_status;

enum { NM_F32 = 0, NM_BF16 = 1 };

typedef struct {
    int64_t rows, cols; /* W is [rows, cols] row-major */
    int32_t n, m;       /* keep n of every m consecutive weights along cols */
    int32_t wtype;      /* NM_F32 or NM_BF16: type of W, of its gradient and of packed values */
} nm_shape;

typedef struct {
    float kappa;     /* logit scale (MaskLLM project page, Fig. 5 caption), >= 0 */
    float tau;       /* Gumbel-softmax temperature, > 0 */
    uint64_t seed;   /* Philox key */
    uint64_t offset; /* Philox counter high half: the training step */
} nm_sample;

/* Forward of the differentiable mask (MaskLLM project page, Fig. 3 caption; frozen weights per
 * its Abstract): w_masked = W * m, rounded to wtype, with m the soft mask of the sample.
 *   w         [rows, cols] wtype, read
 *   logits    [rows, cols/m, K] fp32, read
 *   w_masked  [rows, cols] wtype, written (may not alias the inputs) */
nm_status nm_mask_forward(const nm_shape *shape, const nm_sample *sample, const void *w,
                          const float *logits, void *w_masked, void *stream);

/* Forward with the convergence monitors of MaskLLM project page, Fig. 5 caption fused in: (a) the
 * L1 distance between the masks sampled at adjacent training steps, (b) the largest probability
 * of the mask distribution.  w_masked is the same as nm_mask_forward's (same sample); besides it,
 * per group g:
 *   sampled candidate  s_g = the first k with the largest (kappa*l_k + g_k)/tau for this step's
 *                      noise (the Gumbel-max hard sample; the decision is taken in fp32, so on
 *                      near-ties within the fp32 rounding of the scores either candidate may win;
 *                      with non-finite logits it is unspecified)
 *   max probability    p_g = max_k softmax(kappa * l)_k (the distribution itself, no noise)
 *   L1 distance        d_g = number of positions where the masks of s_g and prev_sample[g]
 *                      differ; a prev_sample entry >= K stands for the empty mask
 *   w, logits, w_masked  as nm_mask_forward
 *   prev_sample  [rows, cols/m] uint8, read, may be NULL (then no L1 distance is taken)
 *   sample_idx   [rows, cols/m] uint8, written with s_g, may be NULL; pass it as the next step's
 *                prev_sample (no alignment requirement for either)
 *   stats        2 doubles, written: stats[0] = sum of p_g, stats[1] = sum of d_g (0 without
 *                prev_sample); divide by the group count rows*cols/m for the means.  Left
 *                untouched for an empty matrix (nothing is launched).
 *   workspace    device memory of at least nm_monitor_workspace_bytes(shape) bytes, 16-byte
 *                aligned, holding arrival counters and partial sums; it must be zero-filled
 *                before its first use, and every call leaves it zero-filled again, so one
 *                workspace serves any number of calls (of any shapes it is large enough for)
 *                and any number of replays of a captured graph; workspace_bytes is its size
 *                (NM_EINVAL if short).  Calls whose executions overlap must not share one.
 * One kernel launch, with no fence and no waiting between blocks: the sums are integers (the
 * p_max sum in units of 2^-F, F = 56 minus the bit length of the group count, after an fp32
 * sum per block of 256 threads), added up a 64-ary tree over the blocks by atomic adds, so
 * repeated calls give identical stats whatever the order in which blocks finish.  With
 * non-finite logits stats[0] is unspecified. */
nm_status nm_mask_forward_monitor(const nm_shape *shape, const nm_sample *sample, const void *w,
                                  const float *logits, void *w_masked, const uint8_t *prev_sample,
                                  uint8_t *sample_idx, double *stats, void *workspace,
                                  int64_t workspace_bytes, void *stream);

/* nm_mask_forward_monitor for callers that cannot allocate device memory (code being captured
 * into a HIP graph, tight serving loops, harnesses that forbid hipMalloc): the same kernels and
 * results, with the counters and partial sums of the in-launch sums kept in a fixed array of
 * NM_MONITOR_SCRATCH_BYTES in device memory that the library owns (one per GPU, held until the
 * process ends) instead of a caller workspace.  Nothing is allocated: the array's address is
 * looked up once per device, on the first call with that device current.  64 KiB holds the
 * sums of up to 262,144 blocks of 256 threads: 134 million groups at 2:4 (two per thread),
 * 67 million at the other patterns.
 *   arguments   as nm_mask_forward_monitor, without the workspace
 *   NM_ESCRATCH the shape needs more than NM_MONITOR_SCRATCH_BYTES (nm_monitor_workspace_bytes
 *               tells how much it needs), checked before any HIP call
 *   NM_EHIP     the array's address could not be looked up, or the launch failed
 * The array starts zero-filled (a static device array) and every call leaves it so; it is
 * shared by every call on the same GPU: calls on one GPU whose executions overlap (on
 * different streams, or from different host threads) race and must be ordered by the caller.
 * The stream's device must be the calling thread's current device. */
#define NM_MONITOR_SCRATCH_BYTES (1 << 16)
nm_status nm_mask_forward_monitor_static(const nm_shape *shape, const nm_sample *sample, const void *w,
                                         const float *logits, void *w_masked, const uint8_t *prev_sample,
                                         uint8_t *sample_idx, double *stats, void *stream);

/* Backward to the logits (Fig. 3 caption: every step is differentiable).  With the upstream
 * gradient G = dL/dw_masked, d_k = sum over positions j kept by candidate k of G_j * w_j,
 * s = sum_k y_k d_k and grad_logits_k = (kappa/tau) * y_k * (d_k - s).  The noise is
 * regenerated from (seed, offset), so pass the sample of the matching forward.  The weights
 * are frozen and get no gradient.
 *   w, grad_w_masked  [rows, cols] wtype, read
 *   logits            [rows, cols/m, K] fp32, read
 *   grad_logits       [rows, cols/m, K] fp32, overwritten (not accumulated) */
nm_status nm_mask_backward(const nm_shape *shape, const nm_sample *sample, const void *w,
                           const float *logits, const void *grad_w_masked, float *grad_logits,
                           void *stream);

/* nm_mask_forward and nm_mask_backward with the step offset read from device memory when the
 * kernels run, for a training step captured once into a HIP graph and replayed at every step:
 * the caller updates *offset_dev (for instance with a stream-ordered copy or a one-element
 * kernel) before each replay, and each replay samples that step's noise.  The results are those
 * of nm_mask_forward / nm_mask_backward with sample->offset = *offset_dev (sample->offset is
 * not used).
 *   offset_dev  one uint64_t in device memory, 8-byte aligned (NM_EALIGN otherwise), read
 *               on the stream; NULL is NM_EINVAL
 *   the other arguments and errors  as nm_mask_forward / nm_mask_backward */
nm_status nm_mask_forward_offset_dev(const nm_shape *shape, const nm_sample *sample,
                                     const uint64_t *offset_dev, const void *w, const float *logits,
                                     void *w_masked, void *stream);
nm_status nm_mask_backward_offset_dev(const nm_shape *shape, const nm_sample *sample,
                                      const uint64_t *offset_dev, const void *w, const float *logits,
                                      const void *grad_w_masked, float *grad_logits, void *stream);

/* Backward with a weight regulariser in the loss (MaskLLM project page, Table 3: weight
 * regularisation helps mask learning).  The page gives no formula; this entry point takes it as
 * R = lambda * sum_j (w_j m_j)^2 over the masked weights, added to the caller's task loss.  The
 * gradient of R on w_masked is 2 lambda w_masked, so the result is nm_mask_backward's with the
 * upstream gradient G_j + 2 lambda w_j m_j, m the step's soft mask (regenerated here, as the
 * noise is).  It saves the caller a pass that would read w_masked and G and write G + 2 lambda
 * w_masked.  A negative lambda rewards large kept weights, a positive one penalises them.
 *   lambda         finite (NM_EINVAL otherwise); 0 gives the plain backward up to signed zeros
 *   grad_w_masked  [rows, cols] wtype, read; may be NULL: the regulariser alone (no task loss)
 *   w, logits, grad_logits, errors  as nm_mask_backward */
nm_status nm_mask_backward_wreg(const nm_shape *shape, const nm_sample *sample, float lambda,
                                const void *w, const float *logits, const void *grad_w_masked,
                                float *grad_logits, void *stream);

/* Forward and hard-mask pack of the same weights and logits in one call, for a step that needs
 * both (for instance a training step that also exports the current hard mask): the outputs are
 * exactly those of nm_mask_forward and nm_mask_harden_pack with the same arguments.  For 2:4
 * with cols/4 a multiple of 8 (every row's index bits fill whole words) one kernel reads w and
 * the logits once for both, moving 2*wb + 6 + wb/2 + 1/8 bytes per weight instead of
 * 3*wb + 12 + wb/2 + 1/8; other shapes run the two passes one after the other.
 *   w, logits, w_masked           as nm_mask_forward
 *   values, indices, hard_idx     as nm_mask_harden_pack (hard_idx may be NULL)
 * Errors: those of both entry points, checked before anything is launched. */
nm_status nm_mask_forward_pack(const nm_shape *shape, const nm_sample *sample, const void *w,
                               const float *logits, void *w_masked, void *values, uint32_t *indices,
                               uint8_t *hard_idx, void *stream);

/* Hard mask and compressed storage ("Accelerating Sparse Deep Neural Networks" summary page,
 * section 3.1).  Per group: k* = first argmax of its logits; the kept weights of candidate k*
 * go to `values` and their positions to `indices` (layout above).
 *   w        [rows, cols] wtype, read;  logits [rows, cols/m, K] fp32, read
 *   values   [rows, cols*n/m] wtype, written (bit copies of the kept weights)
 *   indices  [rows, nm_index_words_per_row] uint32, written
 *   hard_idx [rows, cols/m] uint8, written with k*; may be NULL */
nm_status nm_mask_harden_pack(const nm_shape *shape, const void *w, const float *logits,
                              void *values, uint32_t *indices, uint8_t *hard_idx, void *stream);

/* Decompression: w_dense = +0.0 everywhere except the kept values at their positions.
 * Positions >= m in malformed metadata are skipped.
 *   values  [rows, cols*n/m] wtype, read;  indices [rows, nm_index_words_per_row] uint32, read
 *   w_dense [rows, cols] wtype, written */
nm_status nm_unpack(const nm_shape *shape, const void *values, const uint32_t *indices,
                    void *w_dense, void *stream);

/* Magnitude-prior initialisation of the logits, the step before the learnable layer
 * (MaskLLM project page, Table 2 caption: prior masks initialise the logits; "Accelerating
 * Sparse Deep Neural Networks" summary page, section 4.1: magnitude pruning keeps the largest
 * magnitudes of each group).  Per group the prior candidate keeps the n largest |w|: n rounds,
 * each taking the first not yet taken position whose |w| no earlier free position reaches, so
 * equal magnitudes keep the lower position and a NaN is taken only as the first free position.
 * Its logit is alpha, every other logit of the group +0.0.
 *   w          [rows, cols] wtype, read
 *   alpha      finite (any sign), else NM_EINVAL
 *   logits     [rows, cols/m, K] fp32, overwritten
 *   prior_idx  [rows, cols/m] uint8, written with the prior candidate's index; may be NULL
 *              (no alignment requirement) */
nm_status nm_prior_init(const nm_shape *shape, float alpha, const void *w, float *logits,
                        uint8_t *prior_idx, void *stream);

/* Product with the packed weights on gfx950's sparse matrix cores, the deployment step after
 * the path ("Accelerating Sparse Deep Neural Networks" summary page, sections 3.1-3.2: the
 * compressed operand, values plus 2-bit positions, is multiplied as is and the pruned products
 * are skipped).  For a linear layer W [out, in] pruned 2:4 along `in` and packed by
 * nm_mask_harden_pack:  Y[t, o] = sum_i X[t, i] * W[o, i], accumulated in fp32.
 *   w_shape   rows = out, cols = in, n = 2, m = 4, wtype = NM_BF16 (else NM_EUNSUPPORTED)
 *   values    [out, in/2] bf16, indices [out, in/32] uint32: the packed form, read
 *   x         [tokens, in] bf16, read
 *   y         [tokens, out], ytype NM_F32 or NM_BF16 (round to nearest even), overwritten
 * Supported sizes: in a positive multiple of 64 and out a multiple of 4 (else NM_EUNSUPPORTED),
 * any tokens >= 0; out = 0 or tokens = 0 launches nothing.  Pointers 16-byte aligned.  Above
 * 64 tokens the product runs on square tiles of 256, 128 or 64 W rows and tokens, the largest
 * that still gives every compute unit a block (a partial last tile costs a whole one); from 5
 * to 64 tokens, on blocks of 16 W rows that split k and read the packed weights once; at 1 to 4
 * tokens whose X is at most 24576 bf16 in all (48 KB), without the matrix cores, each wave
 * streaming whole packed rows against X held in LDS (larger X takes the 16-row blocks).
 * Deterministic: every output is accumulated in a fixed order. */
nm_status nm_sparse_matmul(const nm_shape *w_shape, const void *values, const uint32_t *indices,
                           const void *x, int64_t tokens, void *y, int32_t ytype, void *stream);

/* nm_sparse_matmul with a caller-provided workspace, which lets the product split each tile's k
 * range into 2, 4 or 8 parts run by separate blocks where that is estimated faster (batches too
 * small to give every compute unit enough tiles, long k): each part's fp32 sums go to the
 * workspace, and a second kernel adds the parts in part order and rounds once to ytype
 * (deterministic; the sum order differs from an unsplit product's, so results may differ from
 * nm_sparse_matmul's by rounding).  Same result otherwise.
 *   workspace        device memory, 16-byte aligned, of at least
 *                    nm_sparse_matmul_workspace_bytes(w_shape, tokens) bytes (may be NULL when
 *                    that is 0); its contents on entry do not matter and are left unspecified.
 *                    It must not overlap values, indices, x or y, and calls whose executions
 *                    overlap must not share one.
 *   workspace_bytes  its size (NM_EINVAL if short)
 *   other arguments  as nm_sparse_matmul */
nm_status nm_sparse_matmul_ws(const nm_shape *w_shape, const void *values, const uint32_t *indices,
                              const void *x, int64_t tokens, void *y, int32_t ytype, void *workspace,
                              int64_t workspace_bytes, void *stream);
/* Workspace bytes nm_sparse_matmul_ws needs for these sizes on the calling thread's current
 * device (whose compute-unit count the plan depends on; 256 if it cannot be asked): 0 when
 * the product is not split, else 4 * parts * tokens * out; -1 for sizes nm_sparse_matmul
 * rejects. */
int64_t nm_sparse_matmul_workspace_bytes(const nm_shape *w_shape, int64_t tokens);
/* The kernel these sizes run on, on the calling thread's current device (host only, no device
 * work): *tile = 0 for the row-streaming kernel (1 to 4 tokens whose X fits in 48 KB), 16 for
 * the kernel of 16-row blocks, 64, 128 or 256 for the tiles of that many W rows x tokens per
 * block; *parts = the parts the k range is split into (1 unless with_workspace is non-zero, as
 * for nm_sparse_matmul_ws).  The choice is the cheapest under a cost model of the candidates
 * fitted to MI355X measurements.  Empty products give *tile = -1, *parts = 0.  NM_EINVAL for
 * NULL outputs, otherwise the size checks of nm_sparse_matmul. */
nm_status nm_sparse_matmul_plan(const nm_shape *w_shape, int64_t tokens, int32_t with_workspace, int32_t *tile,
                                int32_t *parts);

/* ---- host-only helpers (no device work, no HIP call) ---------------------------------- */
/* K = C(m, n) for a supported (n, m), else -1. */
int32_t nm_num_candidates(int32_t n, int32_t m);
/* out_bits[k] (K bytes, caller-owned host memory): bit j set iff candidate k keeps j. */
nm_status nm_candidate_table(int32_t n, int32_t m, uint8_t *out_bits);
/* rows * cols * n / m, or -1 for an invalid shape. */
int64_t nm_packed_value_elems(const nm_shape *shape);
/* ceil((cols/m) * n * ceil(log2 m) / 32), or -1 for an invalid shape. */
int64_t nm_index_words_per_row(const nm_shape *shape);
/* rows * nm_index_words_per_row, or -1. */
int64_t nm_packed_index_words(const nm_shape *shape);
/* Workspace bytes nm_mask_forward_monitor needs for this shape (two 8-byte words per node of a
 * 64-ary tree over the blocks of its grid, at least 16), or -1 for an invalid shape. */
int64_t nm_monitor_workspace_bytes(const nm_shape *shape);
/* Static description of a status code; any other value gives "unknown status".  The argument
 * is a plain int32_t so that a value outside the enumeration is well defined on both sides. */
const char *nm_status_str(int32_t status);

/* ---- diagnostic exports: the same device functions the kernels use ------------------- */
/* Raw noise words [rows*cols/m, K] (uint32) of a sample; kappa and tau are not used. */
nm_status nm_debug_noise(const nm_shape *shape, const nm_sample *sample, uint32_t *words,
                         void *stream);
/* Base-2 Gumbel exponent of noise words: h = log2(-log2(u)), u = ((x >> 9) + 1/2) / 2^23, so
 * that the Gumbel sample is g = -ln(2) * (h + log2(ln 2)).  words and h hold count elements. */
nm_status nm_debug_gumbel_log2(const uint32_t *words, float *h, int64_t count, void *stream);
/* Plain device copy of `bytes` (a multiple of 16) with the access pattern of the path kernels
 * (one 16-byte vector per thread, non-temporal loads and stores): the streaming ceiling the
 * path's bandwidth is compared with.  src and dst 16-byte aligned, not overlapping. */
nm_status nm_debug_copy(const void *src, void *dst, int64_t bytes, void *stream);
/* Soft mask [rows, cols] fp32 of a sample (the forward's m before the multiply). */
nm_status nm_debug_soft_mask(const nm_shape *shape, const nm_sample *sample,
                             const float *logits, float *soft_mask, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* NM_MASK_H */
