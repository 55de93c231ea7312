/*
 * A C99 consumer of include/skinny.h.  Built by tests/test_abi_cpu.py with
 * gcc -std=c99 -pedantic -Werror against libskinny.so, it shows that the
 * header is plain C and that a C program links and calls the library with
 * nothing but the header's types.  It makes only host-side calls (argument
 * errors that are reported before any device call, the tactic rules, the
 * table rule), so it runs without a GPU.  Prints "abi ok <checks>" and exits
 * 0, or names the first failed check and exits 1.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "skinny.h"

static int checks;

#define CHECK(cond)                                                               \
    do {                                                                          \
        ++checks;                                                                 \
        if (!(cond)) {                                                            \
            printf("check failed at line %d: %s (last error: %s)\n", __LINE__,    \
                   #cond, skinny_last_error());                                   \
            return 1;                                                             \
        }                                                                         \
    } while (0)

int main(void)
{
    skinny_plan *plan = (skinny_plan *)&checks;   /* must come back NULL on failure */
    skinny_tactic t, bad, table[64];
    skinny_tactic *cand;
    double *times;
    int s, count, i, m;

    /* every status has a distinct text */
    for (s = SKINNY_OK; s <= SKINNY_ERR_HIP; ++s) {
        const char *text = skinny_status_string((skinny_status)s);
        CHECK(text != NULL && text[0] != '\0');
        if (s > SKINNY_OK)
            CHECK(strcmp(text, skinny_status_string((skinny_status)(s - 1))) != 0);
    }

    /* prepare rejects bad arguments before touching a device, clears *plan
       and leaves a reason */
    CHECK(skinny_prepare(NULL, 256, 512, SKINNY_OUT_BF16, &plan) == SKINNY_ERR_INVALID_ARG);
    CHECK(plan == NULL);
    CHECK(skinny_last_error()[0] != '\0');
    CHECK(skinny_prepare((const void *)0x1000, 256, 513, SKINNY_OUT_BF16, &plan) == SKINNY_ERR_SHAPE);
    CHECK(skinny_prepare((const void *)0x1001, 256, 512, SKINNY_OUT_F32, &plan) == SKINNY_ERR_ALIGN);
    CHECK(skinny_prepare_ex((const void *)0x1000, 256, 512, 504, SKINNY_IN_BF16, SKINNY_OUT_BF16, &plan) ==
          SKINNY_ERR_SHAPE);
    CHECK(skinny_prepare_ex((const void *)0x1000, 256, 512, 512, (skinny_in_dtype)5, SKINNY_OUT_BF16, &plan) ==
          SKINNY_ERR_INVALID_ARG);

    /* run and describe on a NULL plan */
    CHECK(skinny_run(NULL, (const void *)0x1000, (void *)0x1000, 1, NULL) == SKINNY_ERR_INVALID_ARG);
    CHECK(skinny_supports(NULL, 1) == 0);
    skinny_destroy(NULL);

    /* tactic rules: a legal MFMAW tactic and an illegal one */
    t.path = SKINNY_PATH_MFMAW;
    t.mt = 32;
    t.rows = 64;
    t.waves = 4;
    t.unroll = 3;
    t.split = 2;
    CHECK(skinny_tactic_check(&t, 6288, 7168) == SKINNY_OK);
    bad = t;
    bad.path = SKINNY_PATH_DOT2X;   /* retired */
    CHECK(skinny_tactic_check(&bad, 6288, 7168) == SKINNY_ERR_INVALID_ARG);
    bad = t;
    bad.mt = 3;
    CHECK(skinny_tactic_check(&bad, 6288, 7168) == SKINNY_ERR_INVALID_ARG);

    /* the candidate list of a 256-CU chip: every entry legal, the
       count-only call agrees */
    count = skinny_enumerate_tactics_ex(6288, 7168, 256, NULL, 0);
    CHECK(count > 100);
    cand = (skinny_tactic *)malloc(sizeof(skinny_tactic) * (size_t)count);
    times = (double *)malloc(sizeof(double) * (size_t)count);
    CHECK(cand != NULL && times != NULL);
    CHECK(skinny_enumerate_tactics_ex(6288, 7168, 256, cand, count) == count);
    for (i = 0; i < count; ++i)
        CHECK(skinny_tactic_check(&cand[i], 6288, 7168) == SKINNY_OK);

    /* the table rule: with every candidate timed equal, each M gets a
       candidate whose tile serves it, and the smallest such tile */
    for (i = 0; i < count; ++i)
        times[i] = 10.0;
    CHECK(skinny_select_table(cand, times, count, table) == SKINNY_OK);
    for (m = 1; m <= 64; ++m) {
        int smallest = 1 << 30;
        for (i = 0; i < count; ++i)
            if (cand[i].mt >= m && cand[i].mt < smallest)
                smallest = cand[i].mt;
        CHECK(table[m - 1].mt == smallest);
    }
    /* no usable candidate for some M: an error, not a table */
    for (i = 0; i < count; ++i)
        times[i] = cand[i].mt >= 64 ? -1.0 : 10.0;
    CHECK(skinny_select_table(cand, times, count, table) == SKINNY_ERR_INVALID_ARG);
    free(cand);
    free(times);

    CHECK(skinny_probe_read_blocks() > 0);
    printf("abi ok %d\n", checks);
    return 0;
}
