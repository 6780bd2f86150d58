/* A plain C99 caller of the library's C ABI: the header needs no HIP or C++ headers, and the
 * host helpers and argument validation answer without a GPU (no device work is requested:
 * every call below either is a host helper or is rejected before any HIP call).  Prints one
 * line per check and exits non-zero on the first failure. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "nm_mask.h"

static int failures = 0;
#define CHECK(cond)                                                   \
    do {                                                              \
        if (!(cond)) {                                                \
            printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);    \
            ++failures;                                               \
        }                                                             \
    } while (0)

int main(void) {
    /* candidate counts C(m, n) */
    CHECK(nm_num_candidates(2, 4) == 6);
    CHECK(nm_num_candidates(1, 4) == 4);
    CHECK(nm_num_candidates(2, 8) == 28);
    CHECK(nm_num_candidates(4, 8) == 70);
    CHECK(nm_num_candidates(2, 6) < 0);

    /* 2:4 candidates in lexicographic order of their kept positions */
    uint8_t bits[70];
    const uint8_t want24[6] = {0x3, 0x5, 0x9, 0x6, 0xA, 0xC};
    CHECK(nm_candidate_table(2, 4, bits) == NM_OK);
    CHECK(memcmp(bits, want24, 6) == 0);
    CHECK(nm_candidate_table(4, 8, bits) == NM_OK);
    for (int k = 0; k < 70; ++k) CHECK(__builtin_popcount(bits[k]) == 4);
    for (int k = 1; k < 70; ++k) CHECK(bits[k] != bits[k - 1]);

    /* packed sizes: a 4096 x 4096 bf16 weight at 2:4 keeps half the values and 2 bits each */
    nm_shape sh = {4096, 4096, 2, 4, NM_BF16};
    CHECK(nm_packed_value_elems(&sh) == 4096LL * 2048);
    CHECK(nm_index_words_per_row(&sh) == 4096 / 32);
    CHECK(nm_packed_index_words(&sh) == 4096LL * 128);
    nm_shape sh8 = {3, 8 * 5, 2, 8, NM_F32}; /* 5 groups x 2 fields x 3 bits = 30 bits: 1 word */
    CHECK(nm_index_words_per_row(&sh8) == 1);

    /* validation happens on the host, before any HIP call */
    nm_sample smp = {100.0f, 4.0f, 0, 0};
    void *fake = (void *)(uintptr_t)(1u << 20); /* aligned, never dereferenced */
    nm_shape bad_m = {4, 12, 2, 6, NM_BF16};
    CHECK(nm_mask_forward(&bad_m, &smp, fake, fake, fake, NULL) == NM_EUNSUPPORTED);
    nm_shape bad_cols = {4, 6, 2, 4, NM_BF16};
    CHECK(nm_mask_forward(&bad_cols, &smp, fake, fake, fake, NULL) == NM_EINVAL);
    nm_sample bad_tau = {100.0f, 0.0f, 0, 0};
    CHECK(nm_mask_backward(&sh, &bad_tau, fake, fake, fake, fake, NULL) == NM_EINVAL);
    CHECK(nm_mask_forward(&sh, &smp, fake, fake, NULL, NULL) == NM_EINVAL);
    CHECK(nm_mask_harden_pack(&sh, (void *)((uintptr_t)fake + 4), fake, fake, fake, NULL, NULL) == NM_EALIGN);
    nm_shape empty = {0, 4096, 2, 4, NM_BF16};
    CHECK(nm_unpack(&empty, NULL, NULL, NULL, NULL) == NM_OK); /* nothing to do, nothing launched */

    /* extreme arguments: every size check must answer without overflowing int64 (signed
     * overflow and out-of-range float conversions are what UBSan builds of this file catch) */
    const int64_t big = INT64_MAX - INT64_MAX % 8;
    const nm_shape huge[] = {{big, 8, 2, 4, NM_BF16},   {1, big, 4, 8, NM_F32},        {big, big, 2, 8, NM_BF16},
                             {1 << 20, 1LL << 40, 2, 4, NM_F32}, {INT64_MIN, 4, 2, 4, NM_BF16}, {3, -8, 1, 4, NM_F32}};
    for (size_t i = 0; i < sizeof huge / sizeof huge[0]; ++i) {
        CHECK(nm_packed_value_elems(&huge[i]) == -1);
        CHECK(nm_index_words_per_row(&huge[i]) == -1);
        CHECK(nm_packed_index_words(&huge[i]) == -1);
        CHECK(nm_monitor_workspace_bytes(&huge[i]) == -1);
        CHECK(nm_mask_forward(&huge[i], &smp, fake, fake, fake, NULL) == NM_EINVAL);
        CHECK(nm_mask_backward(&huge[i], &smp, fake, fake, fake, fake, NULL) == NM_EINVAL);
        CHECK(nm_mask_harden_pack(&huge[i], fake, fake, fake, fake, NULL, NULL) == NM_EINVAL);
        CHECK(nm_mask_forward_monitor_static(&huge[i], &smp, fake, fake, fake, NULL, NULL, fake, NULL) == NM_EINVAL);
    }
    /* the largest shapes the checks accept: sizes come out exact */
    const nm_shape widest = {1, (1LL << 31) * 256 * 4 - 1024, 2, 4, NM_BF16}; /* 2^39 - 256 groups */
    CHECK(nm_packed_value_elems(&widest) == widest.cols / 2);
    CHECK(nm_index_words_per_row(&widest) == widest.cols / 32);
    CHECK(nm_monitor_workspace_bytes(&widest) > NM_MONITOR_SCRATCH_BYTES);
    CHECK(nm_mask_forward_monitor_static(&widest, &smp, fake, fake, fake, NULL, NULL, fake, NULL) == NM_ESCRATCH);
    CHECK(nm_mask_forward_monitor(&widest, &smp, fake, fake, fake, NULL, NULL, fake, fake, 64, NULL) == NM_EINVAL);
    /* product: token counts and shapes whose grid or offsets would overflow are refused */
    nm_shape w24 = {4096, 4096, 2, 4, NM_BF16};
    CHECK(nm_sparse_matmul(&w24, fake, fake, fake, INT64_MAX, fake, NM_F32, NULL) == NM_EINVAL);
    CHECK(nm_sparse_matmul(&w24, fake, fake, fake, -1, fake, NM_F32, NULL) == NM_EINVAL);
    CHECK(nm_sparse_matmul(&w24, fake, fake, fake, 1LL << 40, fake, NM_BF16, NULL) == NM_EINVAL);
    nm_shape w24_tall = {(1LL << 31) * 256 * 4 / 64, 64, 2, 4, NM_BF16};
    CHECK(nm_sparse_matmul(&w24_tall, fake, fake, fake, 1LL << 45, fake, NM_F32, NULL) == NM_EINVAL);
    nm_shape w24_odd = {4094, 4096, 2, 4, NM_BF16};
    CHECK(nm_sparse_matmul(&w24_odd, fake, fake, fake, 8, fake, NM_F32, NULL) == NM_EUNSUPPORTED);
    CHECK(nm_sparse_matmul_workspace_bytes(&w24, INT64_MAX) == -1);
    CHECK(nm_sparse_matmul_workspace_bytes(&w24_tall, 1LL << 45) == -1);  /* offsets past int64 */
    CHECK(nm_sparse_matmul_workspace_bytes(&w24_odd, 8) == -1);
    CHECK(nm_sparse_matmul_workspace_bytes(NULL, 8) == -1);
    for (size_t i = 0; i < sizeof huge / sizeof huge[0]; ++i)
        CHECK(nm_sparse_matmul_workspace_bytes(&huge[i], INT64_MAX) == -1);
    CHECK(nm_sparse_matmul_ws(&w24, fake, fake, fake, INT64_MAX, fake, NM_F32, fake, 64, NULL) == NM_EINVAL);
    CHECK(nm_sparse_matmul_ws(&w24_tall, fake, fake, fake, 1LL << 45, fake, NM_F32, fake, 64, NULL) == NM_EINVAL);
    CHECK(nm_sparse_matmul_ws(&w24, fake, fake, fake, 64, fake, NM_F32, NULL, 0, NULL) == NM_EINVAL); /* split, no workspace */
    int32_t tile = 0, parts = 0;
    CHECK(nm_sparse_matmul_plan(&w24, 64, 1, &tile, &parts) == NM_OK && tile == 64 && parts == 4);
    CHECK(nm_sparse_matmul_plan(&w24, 64, 1, NULL, &parts) == NM_EINVAL);
    CHECK(nm_sparse_matmul_plan(&w24_odd, 64, 1, &tile, &parts) == NM_EUNSUPPORTED);
    CHECK(nm_sparse_matmul_plan(&w24, INT64_MAX, 1, &tile, &parts) == NM_EINVAL);
    /* samples whose kappa*log2(e)/tau or 1/tau leave fp32's range, or are not numbers */
    const nm_sample bad_samples[] = {{3.0e38f, 1.0e-3f, 0, 0}, {1.0f, 1.0e-45f, 0, 0}, {1.0f, -1.0f, 0, 0},
                                     {-1.0f, 1.0f, 0, 0},      {INFINITY, 1.0f, 0, 0},   {NAN, 1.0f, 0, 0},
                                     {1.0f, NAN, 0, 0}};
    for (size_t i = 0; i < sizeof bad_samples / sizeof bad_samples[0]; ++i) {
        CHECK(nm_mask_forward(&sh, &bad_samples[i], fake, fake, fake, NULL) == NM_EINVAL);
        CHECK(nm_mask_backward(&sh, &bad_samples[i], fake, fake, fake, fake, NULL) == NM_EINVAL);
    }
    CHECK(nm_mask_backward_wreg(&sh, &smp, 3.0e38f, fake, fake, fake, fake, NULL) == NM_EINVAL); /* 2*lambda */
    CHECK(nm_debug_copy(fake, fake, INT64_MAX - 15, NULL) == NM_EINVAL);
    CHECK(nm_debug_gumbel_log2(fake, fake, INT64_MAX, NULL) == NM_EINVAL);
    CHECK(nm_candidate_table(2, 4, NULL) == NM_EINVAL);
    CHECK(nm_candidate_table(0, 4, bits) == NM_EUNSUPPORTED && nm_candidate_table(9, 8, bits) == NM_EUNSUPPORTED);

    CHECK(strlen(nm_status_str(NM_EALIGN)) > 0);
    CHECK(strlen(nm_status_str(12345)) > 0 && strlen(nm_status_str(-7)) > 0);
    CHECK(strcmp(nm_status_str(NM_OK), nm_status_str(NM_EINVAL)) != 0);

    printf(failures ? "abi host check: %d failure(s)\n" : "abi host check: ok\n", failures);
    return failures ? 1 : 0;
}
