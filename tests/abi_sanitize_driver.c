/*
 * Calls the C ABI's host-side paths -- context create/destroy, workspace
 * sizing and every entry point's argument checks -- for a build of the
 * host code with AddressSanitizer and UndefinedBehaviorSanitizer.  No call
 * here gets past its checks, so nothing reaches a GPU.  Device addresses are
 * stand-ins that are never dereferenced.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "moe_mxfp4.h"

#define FAKE ((void*)(uintptr_t)(1u << 20))
#define CHECK(expr, want)                                                              \
    do {                                                                               \
        const int got_ = (int)(expr);                                                  \
        if (got_ != (int)(want)) {                                                     \
            fprintf(stderr, "%s:%d: %s gave %d, expected %d\n", __FILE__, __LINE__, #expr, \
                    got_, (int)(want));                                                \
            exit(1);                                                                   \
        }                                                                              \
    } while (0)

static moe_mxfp4_config cfg(int E, int d, int f, int k, int T, int act) {
    moe_mxfp4_config c;
    c.struct_size = sizeof c;
    c.num_experts = E; c.d_model = d; c.d_ff = f; c.top_k = k; c.max_tokens = T;
    c.act_mode = act; c.out_dtype = MOE_OUT_BF16; c.flags = 0;
    return c;
}

int main(void) {
    moe_mxfp4_weights w = {FAKE, FAKE, FAKE, FAKE, FAKE, FAKE};
    moe_mxfp4_ctx* ctx = NULL;
    moe_mxfp4_config c = cfg(8, 512, 256, 2, 8, MOE_ACT_BF16);

    /* create: bad configs, then a good one */
    moe_mxfp4_config bad = c;
    bad.struct_size = 4;
    CHECK(moe_mxfp4_create(&bad, &w, &ctx), MOE_ERR_INVALID_ARG);
    bad = c; bad.top_k = 9;
    CHECK(moe_mxfp4_create(&bad, &w, &ctx), MOE_ERR_UNSUPPORTED_SHAPE);
    bad = c; bad.d_model = 300;
    CHECK(moe_mxfp4_create(&bad, &w, &ctx), MOE_ERR_UNSUPPORTED_SHAPE);
    bad = c; bad.flags = 1;
    CHECK(moe_mxfp4_create(&bad, &w, &ctx), MOE_ERR_INVALID_ARG);
    CHECK(moe_mxfp4_create(NULL, &w, &ctx), MOE_ERR_INVALID_ARG);
    CHECK(moe_mxfp4_create(&c, NULL, &ctx), MOE_ERR_INVALID_ARG);
    moe_mxfp4_weights wa = w;
    wa.w_up = (const uint8_t*)((uintptr_t)FAKE + 4);
    CHECK(moe_mxfp4_create(&c, &wa, &ctx), MOE_ERR_ALIGNMENT);
    CHECK(moe_mxfp4_create(&c, &w, &ctx), MOE_OK);

    /* workspace sizing and forward checks (all fail before a launch) */
    const size_t need = moe_mxfp4_workspace_bytes(ctx, 8);
    CHECK(need > 0, 1);
    CHECK(moe_mxfp4_workspace_bytes(ctx, 0) == 0, 1);
    CHECK(moe_mxfp4_forward(ctx, FAKE, FAKE, 9, FAKE, FAKE, need, NULL, NULL), MOE_ERR_CAPACITY);
    CHECK(moe_mxfp4_forward(ctx, FAKE, NULL, 8, FAKE, FAKE, need, NULL, NULL), MOE_ERR_INVALID_ARG);
    CHECK(moe_mxfp4_forward(ctx, FAKE, FAKE, 8, FAKE, FAKE, need - 1, NULL, NULL), MOE_ERR_WORKSPACE);
    CHECK(moe_mxfp4_forward(ctx, (void*)((uintptr_t)FAKE + 2), FAKE, 8, FAKE, FAKE, need, NULL, NULL),
          MOE_ERR_ALIGNMENT);
    CHECK(moe_mxfp4_forward(ctx, NULL, NULL, 0, NULL, NULL, 0, NULL, NULL), MOE_OK);
    CHECK(moe_mxfp4_forward_hidden(ctx, FAKE, NULL, 8, FAKE, FAKE, need, NULL, NULL), MOE_ERR_INVALID_ARG);
    CHECK(moe_mxfp4_router_logits(ctx, FAKE, FAKE, 9, FAKE, NULL), MOE_ERR_CAPACITY);
    CHECK(moe_mxfp4_debug_dequant(ctx, 8, 0, 0, 1, FAKE, NULL), MOE_ERR_INVALID_ARG);
    CHECK(moe_mxfp4_stage_times(ctx, NULL, NULL), MOE_ERR_INVALID_ARG);
    CHECK(moe_mxfp4_stage_timing(ctx, -1), MOE_ERR_INVALID_ARG);
    CHECK(moe_mxfp4_destroy(ctx), MOE_OK);
    CHECK(moe_mxfp4_destroy(NULL), MOE_OK);

    /* MXFP8 mode limits */
    moe_mxfp4_config m8 = cfg(8, 512, 512, 2, 8, MOE_ACT_MXFP8_E4M3);
    CHECK(moe_mxfp4_create(&m8, &w, &ctx), MOE_OK);
    CHECK(moe_mxfp4_workspace_bytes(ctx, 8) > 0, 1);
    CHECK(moe_mxfp4_destroy(ctx), MOE_OK);

    /* weight preparation and export checks */
    CHECK(moe_mxfp4_quantize_weights(FAKE, 4, 48, FAKE, FAKE, NULL), MOE_ERR_INVALID_ARG);
    CHECK(moe_mxfp4_quantize_act_mxfp8(FAKE, 4, 0, FAKE, FAKE, NULL), MOE_ERR_INVALID_ARG);
    CHECK(moe_mxfp4_tiled_scale_bytes(16, 100) == 0, 1);
    CHECK(moe_mxfp4_tile_weights(FAKE, FAKE, 15, 128, FAKE, FAKE, NULL), MOE_ERR_INVALID_ARG);

    /* acceptance pass and probes */
    const size_t wb = moe_mxfp4_dflash_workspace_bytes(32, 152064);
    CHECK(wb > 0, 1);
    CHECK(moe_mxfp4_dflash_workspace_bytes(-1, 5) == 0, 1);
    CHECK(moe_mxfp4_dflash_accept(32, 65, 100, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, wb, NULL),
          MOE_ERR_INVALID_ARG);
    CHECK(moe_mxfp4_dflash_accept(32, 8, 152064, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, wb - 1, NULL),
          MOE_ERR_WORKSPACE);
    CHECK(moe_mxfp4_dflash_accept(0, 8, 100, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL), MOE_OK);
    double work = 0;
    CHECK(moe_mxfp4_probe(7, FAKE, 16, 1, FAKE, &work, NULL), MOE_ERR_INVALID_ARG);
    CHECK(moe_mxfp4_probe(6, NULL, 0, 0, FAKE, &work, NULL), MOE_ERR_INVALID_ARG);
    CHECK(moe_mxfp4_probe(0, FAKE, 24, 1, FAKE, &work, NULL), MOE_ERR_INVALID_ARG);

    for (int s = 0; s <= 7; ++s)
        if (!moe_mxfp4_status_string((moe_status)s)) return 1;
    puts("abi sanitizer run: ok");
    return 0;
}
