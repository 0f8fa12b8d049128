/* Uses the library's C ABI from plain C99: the header compiles as C, the
 * symbols link, and the host-side contract holds (size queries, config
 * validation, argument errors returned before anything is enqueued).  No
 * call here reaches a kernel launch, so it runs without a GPU. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe_dispatch.h"

static int failures = 0;

#define CHECK(cond)                                                   \
    do {                                                              \
        if (!(cond)) {                                                \
            fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond); \
            failures++;                                               \
        }                                                             \
    } while (0)

int main(void)
{
    moe_config_t c;
    memset(&c, 0, sizeof c);
    c.max_tokens = 8192;
    c.hidden = 7168;
    c.num_experts = 256;
    c.num_topk = 8;
    c.num_ranks = 8;
    c.layout = MOE_LAYOUT_CONTIGUOUS;
    c.align = 128;
    c.capacity = 1;
    c.quant = MOE_QUANT_FP8_UE8M0;
    c.num_cus = 0;

    CHECK(moe_config_check(&c) == MOE_OK);
    CHECK(moe_rows_capacity(&c) == (size_t)8192 * 8 + 256 * 127);
    CHECK(moe_workspace_bytes(&c) > 0);
    CHECK(moe_rank_rows_capacity(&c) == (size_t)8192 * 8);
    CHECK(moe_scale_words(&c) == 14);
    CHECK(strcmp(moe_status_str(MOE_ERR_CAPACITY), "MOE_ERR_CAPACITY") == 0);

    /* invalid configs */
    moe_config_t bad = c;
    bad.num_topk = 33;
    CHECK(moe_config_check(&bad) == MOE_ERR_INVALID_ARG);
    CHECK(moe_rows_capacity(&bad) == 0);
    bad = c;
    bad.hidden = 7168 + 8; /* FP8 needs H % 128 == 0 */
    CHECK(moe_config_check(&bad) == MOE_ERR_INVALID_ARG);
    bad = c;
    bad.num_experts = 4096;
    bad.num_ranks = 1;
    CHECK(moe_config_check(&bad) == MOE_ERR_UNSUPPORTED);
    CHECK(moe_config_check(NULL) == MOE_ERR_INVALID_ARG);

    /* argument errors come back before anything is enqueued */
    int32_t *fake = (int32_t *)(uintptr_t)0x7f0000000000ull; /* never dereferenced */
    moe_handle_t h = {fake, fake, fake, fake, fake, fake, fake};
    CHECK(moe_dispatch_layout(&c, 8193, fake, &h, fake, 1u << 20, NULL) == MOE_ERR_CAPACITY);
    CHECK(moe_dispatch_layout(&c, 16, NULL, &h, fake, 1u << 20, NULL) == MOE_ERR_INVALID_ARG);
    CHECK(moe_dispatch(&c, 16, (const uint16_t *)fake, NULL, &h, fake, NULL, NULL, NULL) ==
          MOE_ERR_INVALID_ARG); /* FP8 needs out_scale */
    CHECK(moe_combine(&c, 16, NULL, NULL, &h, NULL, NULL) == MOE_ERR_INVALID_ARG);
    CHECK(moe_combine(&c, 0, NULL, NULL, &h, NULL, NULL) == MOE_OK); /* zero tokens: nothing to do */
    moe_handle_t hb = h;
    hb.status = NULL;
    CHECK(moe_combine(&c, 16, (const uint16_t *)fake, (const float *)fake, &hb, (uint16_t *)fake, NULL) ==
          MOE_ERR_INVALID_ARG);

    /* status names: every code, and any other int */
    CHECK(strcmp(moe_status_str(MOE_OK), "MOE_OK") == 0);
    CHECK(strcmp(moe_status_str(MOE_ERR_HIP), "MOE_ERR_HIP") == 0);
    CHECK(strcmp(moe_status_str((moe_status_t)-1), "MOE_ERR_UNKNOWN") == 0);
    CHECK(strcmp(moe_status_str((moe_status_t)100000), "MOE_ERR_UNKNOWN") == 0);

    /* the remaining entry points: host-side errors and empty calls */
    moe_config_t m = c;
    m.layout = MOE_LAYOUT_MASKED;
    m.capacity = 256;
    m.align = 1;
    moe_config_t bf = c;
    bf.quant = MOE_QUANT_NONE;
    moe_rank_handle_t rh = {fake, fake, fake, fake};
    CHECK(moe_dispatch_layout_noalloc(&c, 8193, fake, &h, NULL) == MOE_ERR_CAPACITY);
    CHECK(moe_dispatch_layout_noalloc(&c, 16, NULL, &h, NULL) == MOE_ERR_INVALID_ARG);
    CHECK(moe_dispatch_layout_noalloc(&c, 16, (const int32_t *)((const char *)fake + 1), &h, NULL) ==
          MOE_ERR_INVALID_ARG); /* misaligned ids */
    CHECK(moe_dispatch_layout_noalloc(&c, 16, fake, NULL, NULL) == MOE_ERR_INVALID_ARG);
    CHECK(moe_dispatch_layout_noalloc(NULL, 16, fake, &h, NULL) == MOE_ERR_INVALID_ARG);
    CHECK(moe_dispatch_fused(&c, 8193, fake, (const uint16_t *)fake, NULL, &h, fake, 1u << 20, fake, fake, NULL,
                             NULL) == MOE_ERR_CAPACITY);
    CHECK(moe_dispatch_fused(&c, 16, NULL, (const uint16_t *)fake, NULL, &h, fake, 1u << 20, fake, fake, NULL,
                             NULL) == MOE_ERR_INVALID_ARG);
    CHECK(moe_rank_layout(&c, 16, fake, NULL, NULL) == MOE_ERR_INVALID_ARG);
    CHECK(moe_rank_layout(&c, 16, NULL, &rh, NULL) == MOE_ERR_INVALID_ARG);
    CHECK(moe_rank_layout(&c, 8193, fake, &rh, NULL) == MOE_ERR_CAPACITY);
    CHECK(moe_dispatch_dedup(&c, 16, NULL, &rh, fake, fake, NULL) == MOE_ERR_INVALID_ARG);
    CHECK(moe_dispatch_dedup(&c, 16, (const uint16_t *)fake, &rh, fake, NULL, NULL) ==
          MOE_ERR_INVALID_ARG); /* FP8 needs send_scale */
    CHECK(moe_expand(&c, 16, fake, fake, fake, &rh, &h, NULL, fake, NULL) == MOE_ERR_INVALID_ARG);
    CHECK(moe_combine_partial(&c, 16, fake, (const uint16_t *)fake, (const float *)fake, &h, &rh, NULL, NULL) ==
          MOE_ERR_INVALID_ARG);
    CHECK(moe_combine_reduce(&c, 16, NULL, &rh, (uint16_t *)fake, NULL) == MOE_ERR_INVALID_ARG);
    CHECK(moe_combine_reduce(&c, 0, NULL, &rh, NULL, NULL) == MOE_OK);
    CHECK(moe_row_expert(&c, &h, NULL, NULL) == MOE_ERR_INVALID_ARG);
    CHECK(moe_row_expert(&c, NULL, fake, NULL) == MOE_ERR_INVALID_ARG);
    CHECK(moe_repack_rows_capacity(&m, 128) == (size_t)256 * 256 + 256 * 127);
    CHECK(moe_repack_rows_capacity(&m, 0) == 0);
    CHECK(moe_repack_rows_capacity(&c, 128) == 0); /* needs a masked config */
    CHECK(moe_repack_masked_to_contiguous(&c, 128, &h, fake, fake, fake, fake, fake, fake, NULL) ==
          MOE_ERR_INVALID_ARG);
    CHECK(moe_repack_masked_to_contiguous(&m, 128, &h, NULL, fake, fake, fake, fake, fake, NULL) ==
          MOE_ERR_INVALID_ARG);
    CHECK(moe_repack_masked_to_contiguous(&m, 0, &h, fake, fake, fake, fake, fake, fake, NULL) ==
          MOE_ERR_INVALID_ARG);
    CHECK(moe_repack_contiguous_to_masked(&c, &h, fake, (const uint16_t *)fake, (uint16_t *)fake, NULL) ==
          MOE_ERR_INVALID_ARG);
    CHECK(moe_repack_contiguous_to_masked(&m, &h, NULL, (const uint16_t *)fake, (uint16_t *)fake, NULL) ==
          MOE_ERR_INVALID_ARG);
    CHECK(moe_scale_words(&bf) == 0);
    CHECK(moe_scales_mn_major(&c, -1, fake, fake, NULL) == MOE_ERR_INVALID_ARG);
    CHECK(moe_scales_mn_major(&bf, 16, fake, fake, NULL) == MOE_ERR_INVALID_ARG);
    CHECK(moe_scales_mn_major(&c, 16, NULL, fake, NULL) == MOE_ERR_INVALID_ARG);
    CHECK(moe_scales_mn_major(&c, 0, fake, fake, NULL) == MOE_OK);
    moe_config_t many = c;
    many.num_ranks = 64; /* the per-rank exchange takes at most 32 ranks */
    CHECK(moe_rank_rows_capacity(&many) == 0);
    CHECK(moe_rank_layout(&many, 16, fake, &rh, NULL) == MOE_ERR_UNSUPPORTED);

    if (failures == 0)
        printf("C ABI checks passed\n");
    return failures == 0 ? 0 : 1;
}
