/* A plain C99 caller of the library's C ABI: the header needs no HIP or C++ headers, and the
 * host helpers and argument validation answer without a GPU (no device work is requested:
 * every call below either is a host helper or is rejected before any HIP call).  Prints one
 * line per check and exits non-zero on the first failure. */
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

    CHECK(strlen(nm_status_str(NM_EALIGN)) > 0);
    CHECK(strcmp(nm_status_str(NM_OK), nm_status_str(NM_EINVAL)) != 0);

    printf(failures ? "abi host check: %d failure(s)\n" : "abi host check: ok\n", failures);
    return failures ? 1 : 0;
}
