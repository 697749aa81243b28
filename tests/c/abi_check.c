/*
 * abi_check.c -- the C ABI used from plain C (C11, no C++): every header compiles as C,
 * and the host-side entry points (launch policy, status strings, version, argument
 * validation) behave as declared. Built and run by tests/test_c_abi.py; no GPU call is
 * made (every call below fails validation or is pure host).
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kvbt.h"
#include "kvbt_attn.h"
#include "kvbt_bench.h"
#include "kvbt_index.h"

static int failures = 0;

#define CHECK(cond)                                                           \
    do {                                                                      \
        if (!(cond)) {                                                        \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            ++failures;                                                       \
        }                                                                     \
    } while (0)

int main(void)
{
    void* fake = (void*)(uintptr_t)0x10000;   /* never dereferenced */
    kvbt_policy p;
    int32_t idx[16];

    CHECK(strlen(kvbt_version()) >= 5);
    CHECK(strcmp(kvbt_status_string(KVBT_OK), "ok") == 0);
    CHECK(strcmp(kvbt_status_string(-99), "unknown status") == 0);

    /* the 128/129 boundary of the launch policy */
    CHECK(kvbt_launch_policy(128, 8192, KVBT_BF16, 256, 2, 16, &p) == KVBT_OK && p.path == 0);
    CHECK(kvbt_launch_policy(129, 8192, KVBT_BF16, 256, 2, 16, &p) == KVBT_OK && p.path == 1);
    CHECK(kvbt_launch_policy(0, 65536, KVBT_F32, 4, 4, 16, &p) == KVBT_OK && p.path == 3);
    CHECK(kvbt_launch_policy(0, 65537, KVBT_F32, 4, 4, 16, &p) == KVBT_OK && p.path == 3 &&
          p.threads_per_block == 512);
    CHECK(kvbt_launch_policy(0, KVBT_MAX_K_TILES, KVBT_BF16, 4, 4, 16, &p) == KVBT_OK &&
          p.path == 3 && p.threads_per_block == 512);
    CHECK(kvbt_launch_policy(0, KVBT_MAX_K_TILES + 1, KVBT_F32, 4, 4, 16, &p) == KVBT_E_RANGE);
    CHECK(kvbt_launch_policy(0, 74, 7, 4, 4, 16, &p) == KVBT_E_DTYPE);
    CHECK(kvbt_launch_policy(0, 74, KVBT_BF16, 4, 4, 16, NULL) == KVBT_E_NULL);
    /* max_block at most max_k_tiles; a dispatch below 2^32 work-items */
    CHECK(kvbt_launch_policy(74, 74, KVBT_BF16, 4, 4, 16, &p) == KVBT_OK && p.path == 0);
    CHECK(kvbt_launch_policy(75, 74, KVBT_BF16, 4, 4, 16, &p) == KVBT_E_RANGE);
    CHECK(kvbt_launch_policy(0, 8192, KVBT_F32, (1 << 26) - 4, 1, 16, &p) == KVBT_OK &&
          p.grid * p.threads_per_block < ((int64_t)1 << 32));
    CHECK(kvbt_launch_policy(0, 8192, KVBT_F32, 1 << 26, 1, 16, &p) == KVBT_E_RANGE);

    /* validation before any HIP call */
    CHECK(kvbt_select_topk_blocks(fake, KVBT_BF16, 4, 2, 74, fake, 65, 1, 2, 0, 0, idx, NULL) ==
          KVBT_E_RANGE);
    CHECK(kvbt_launch_policy(0, 74, KVBT_BF16, 4, 2, 64, &p) == KVBT_OK && p.path == 5);
    CHECK(kvbt_select_topk_blocks(fake, KVBT_BF16, 4, 2, 74, fake, 16, 1, 2, 0, 5, idx, NULL) ==
          KVBT_E_RANGE);
    CHECK(kvbt_select_topk_blocks(fake, KVBT_BF16, 4, 2, 74, fake, 16, 1, 2, 0, -1, idx, NULL) ==
          KVBT_E_RANGE);
    CHECK(kvbt_select_topk_blocks(NULL, KVBT_BF16, 4, 2, 74, fake, 16, 1, 2, 0, 4, idx, NULL) ==
          KVBT_E_NULL);
    CHECK(kvbt_select_topk_blocks(NULL, KVBT_BF16, 0, 2, 74, NULL, 16, 1, 2, 0, 0, NULL, NULL) ==
          KVBT_OK);
    CHECK(kvbt_select_topk_blocks(fake, KVBT_BF16, 4, 2, 74, fake, 16, 1, 2, 75, 0, idx, NULL) ==
          KVBT_E_RANGE);
    CHECK(kvbt_build_sparse_block_table(fake, 6, 1, 16, fake, 4, 74, fake, 4, NULL, NULL, fake,
                                        fake, NULL) == KVBT_E_SHAPE);
    CHECK(kvbt_select_topk_and_build_table(fake, KVBT_F32, 4, 1, 16, fake, 4, 16, fake, 1, NULL,
                                           NULL, 16, 9, 9, 0, 0, fake, fake, fake, NULL) ==
          KVBT_E_RANGE);
    CHECK(kvbt_select_topk_and_build_table(fake, KVBT_F32, 4, 1, 16, fake, 4, 16, fake, 1, NULL,
                                           NULL, 16, 1, 2, 0, 5, fake, fake, fake, NULL) ==
          KVBT_E_RANGE);
    CHECK(kvbt_sparse_attn_decode(fake, 4, 2, 8, 64, fake, fake, 64, fake, 128, fake, 1, 0.088f,
                                  fake, KVBT_F32, 0, NULL) == KVBT_E_RANGE);
    CHECK(kvbt_sparse_attn_decode(fake, 4, 2, 8, 128, fake, fake, 64, fake, 128, fake, 1, 0.088f,
                                  fake, 9, 0, NULL) == KVBT_E_DTYPE);
    CHECK(kvbt_sparse_attn_waves(256, 2, 4) == 4);
    CHECK(kvbt_sparse_attn_waves(256, 2, 1) == 8);
    CHECK(kvbt_sparse_attn_grouped(256, 2, 8, 4) == 0);     /* 128 groups: rows alone */
    CHECK(kvbt_sparse_attn_grouped(512, 2, 8, 4) == 1);     /* 256 groups: together */
    CHECK(kvbt_sparse_attn_grouped(4096, 2, 8, 1) == 0);
    CHECK(kvbt_sparse_attn_grouped(4096, 2, 17, 4) == 0);
    CHECK(kvbt_sparse_attn_splits(16, 2, 0, INT64_MAX) == 4);     /* 32 pairs, 4 each */
    CHECK(kvbt_sparse_attn_splits(16, 2, 0, 0) == 0);             /* no workspace */
    CHECK(kvbt_sparse_attn_splits(256, 2, 0, INT64_MAX) == 0);    /* 512 pairs: no split */
    CHECK(kvbt_sparse_attn_splits(64, 2, 0, INT64_MAX) == 2);     /* 128 pairs, 2 each */
    CHECK(kvbt_sparse_attn_splits(256, 2, 3, INT64_MAX) == 3);
    CHECK(kvbt_sparse_attn_workspace_bytes(16, 2, 0) == 4438 * 256);
    CHECK(kvbt_sparse_attn_workspace_bytes(16, 2, 1) == 0);
    CHECK(kvbt_sparse_attn_decode_ws(fake, 4, 2, 8, 128, fake, fake, 64, fake, 128, fake, 4,
                                     0.088f, fake, KVBT_F32, 0, KVBT_ATTN_MAX_SPLITS + 1, fake,
                                     1 << 20, NULL) == KVBT_E_RANGE);
    CHECK(kvbt_sparse_attn_decode_ws(fake, 4, 2, 8, 128, fake, fake, 64, fake, 128, fake, 4,
                                     0.088f, fake, KVBT_F32, 0, 4, fake, 1024, NULL) ==
          KVBT_E_RANGE);
    CHECK(kvbt_index_decode_scores(fake, 4, 4, 2, 128, fake, KVBT_FP8_E4M3, NULL, 64, fake, 74,
                                   fake, 0.088f, KVBT_REDUCE_LSE, fake, KVBT_F32, 74, NULL) ==
          KVBT_E_NULL);
    CHECK(kvbt_index_decode_scores(fake, 4, 17, 2, 128, fake, KVBT_BF16, NULL, 64, fake, 74,
                                   fake, 0.088f, KVBT_REDUCE_MAX, fake, KVBT_F32, 74, NULL) ==
          KVBT_E_RANGE);
    CHECK(kvbt_bench_read(fake, 100, fake, NULL) != KVBT_OK);

    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("C ABI checks passed\n");
    return 0;
}
