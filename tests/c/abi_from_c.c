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

    if (failures == 0)
        printf("C ABI checks passed\n");
    return failures == 0 ? 0 : 1;
}
