/* Sanitizer run of the library's host-side logic (the library built with
 * address and undefined-behaviour sanitizers on its host code only, by
 * tests/test_sanitizers.py): workspace sizing and layout over a grid of
 * shapes in every mode, the error strings, and every argument check of the
 * entry points with arguments that are refused before anything touches a
 * device (no GPU is needed or used).  Test infrastructure only. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe_fused.h"

static int bad = 0;
#define EXPECT(cond)                                                   \
    do {                                                               \
        if (!(cond)) {                                                 \
            fprintf(stderr, "check failed line %d: %s\n", __LINE__, #cond); \
            bad = 1;                                                   \
        }                                                              \
    } while (0)

int main(void) {
    const int toks[] = {0, 1, 64, 1000, 8192, 100000};
    const int experts[] = {1, 8, 32, 256};
    const int ks[] = {1, 2, 8};
    const int dims_h[] = {128, 2048, 7168};
    char fake_store[4096];
    void* p = (void*)(((uintptr_t)fake_store + 255) & ~(uintptr_t)255); /* aligned, never dereferenced */
    void* mis = (char*)p + 4;
    int code, mode, a, b, c, d;
    for (code = -1; code < 8; ++code) EXPECT(moe_error_string(code) != NULL && strlen(moe_error_string(code)) > 0);
    EXPECT(moe_block_m() == 16);
    for (mode = 0; mode <= 4; ++mode)
        for (a = 0; a < 6; ++a)
            for (b = 0; b < 4; ++b)
                for (c = 0; c < 3; ++c)
                    for (d = 0; d < 3; ++d) {
                        moe_dims dm = {mode, toks[a], experts[b], ks[c], dims_h[d], dims_h[(d + 1) % 3], 0, 0};
                        moe_ws_layout L;
                        size_t n = moe_workspace_bytes(&dm);
                        EXPECT(n > 0);
                        EXPECT(moe_workspace_layout(&dm, &L) == MOE_OK && L.total == n);
                        EXPECT(L.y < L.total && L.h < L.y && L.stats % 256 == 0);
                    }
    {
        int64_t npc = 0, tc = 0;
        EXPECT(moe_route_caps(1000, 2, 32, &npc, &tc) == MOE_OK && npc == 2000 + 32 * 15 && tc == npc / 16);
        EXPECT(moe_route_caps(-1, 2, 32, &npc, &tc) == MOE_ERR_INVALID_ARG);
        EXPECT(moe_route_caps(10, 2, 32, NULL, &tc) == MOE_ERR_INVALID_ARG);
    }
    {
        moe_dims dm = {MOE_MODE_FP8, 1024, 32, 2, 7168, 2048, 0, 0};
        moe_scales sc = {p, p, p};
        size_t ws = moe_workspace_bytes(&dm);
        EXPECT(moe_fused_forward(NULL, p, p, p, p, p, &sc, p, p, ws, NULL) == MOE_ERR_INVALID_ARG);
        EXPECT(moe_fused_forward(&dm, NULL, p, p, p, p, &sc, p, p, ws, NULL) == MOE_ERR_INVALID_ARG);
        EXPECT(moe_fused_forward(&dm, mis, p, p, p, p, &sc, p, p, ws, NULL) == MOE_ERR_INVALID_ARG);
        EXPECT(moe_fused_forward(&dm, p, p, p, p, p, NULL, p, p, ws, NULL) == MOE_ERR_INVALID_ARG);
        EXPECT(moe_fused_forward(&dm, p, p, p, p, p, &sc, p, p, ws - 1, NULL) == MOE_ERR_WORKSPACE);
        EXPECT(moe_fused_forward(&dm, p, p, p, p, p, &sc, p, NULL, ws, NULL) == MOE_ERR_WORKSPACE);
        EXPECT(moe_fused_forward(&dm, p, p, p, p, p, &sc, p, (char*)p + 16, ws, NULL) == MOE_ERR_WORKSPACE);
        dm.d_hidden = 100;
        EXPECT(moe_fused_forward(&dm, p, p, p, p, p, &sc, p, p, ws, NULL) == MOE_ERR_UNSUPPORTED);
        dm.d_hidden = 7168;
        dm.mode = 9;
        EXPECT(moe_fused_forward(&dm, p, p, p, p, p, &sc, p, p, ws, NULL) == MOE_ERR_INVALID_ARG);
        dm.mode = MOE_MODE_INT8;
        {
            moe_scales s8 = {(char*)p + 2, NULL, NULL}; /* not 4-byte aligned */
            EXPECT(moe_fused_forward(&dm, p, p, p, p, p, &s8, p, p, (size_t)1 << 40, NULL) == MOE_ERR_INVALID_ARG);
        }
        dm.mode = MOE_MODE_FP8;
        dm.num_tokens = 8192;
        EXPECT(moe_fused_forward_noalloc(&dm, p, p, p, p, p, &sc, p, NULL) == MOE_ERR_SCRATCH);
        EXPECT(moe_fused_forward_noalloc(NULL, p, p, p, p, p, &sc, p, NULL) == MOE_ERR_INVALID_ARG);
        dm.num_tokens = 0;
        EXPECT(moe_fused_forward(&dm, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == MOE_OK);
        /* overlapping pack buffers */
        dm.num_tokens = 16;
        EXPECT(moe_pack_weights(&dm, p, (char*)p + 1024, p, (char*)p + 2048, NULL) == MOE_ERR_INVALID_ARG);
        EXPECT(moe_pack_weights(NULL, p, p, p, p, NULL) == MOE_ERR_INVALID_ARG);
    }
    {
        moe_dims bd = {MOE_MODE_BF16, 100, 8, 2, 256, 128, 0, 0};
        size_t bw = moe_backward_workspace_bytes(&bd);
        EXPECT(bw > 0);
        bd.mode = MOE_MODE_FP8;
        EXPECT(moe_backward_workspace_bytes(&bd) == 0);
        EXPECT(moe_fused_backward(&bd, p, p, p, p, p, p, p, p, p, p, p, bw, NULL) == MOE_ERR_UNSUPPORTED);
        bd.mode = MOE_MODE_BF16;
        EXPECT(moe_fused_backward(&bd, p, p, p, p, p, p, p, p, p, p, p, bw - 1, NULL) == MOE_ERR_WORKSPACE);
        EXPECT(moe_fused_backward(&bd, p, p, p, p, p, NULL, p, p, p, p, p, bw, NULL) == MOE_ERR_INVALID_ARG);
        EXPECT(moe_fused_backward(&bd, p, p, p, p, p, p, mis, p, p, p, p, bw, NULL) == MOE_ERR_INVALID_ARG);
        EXPECT(moe_fused_backward(NULL, p, p, p, p, p, p, p, p, p, p, p, bw, NULL) == MOE_ERR_INVALID_ARG);
    }
    {
        moe_route_out ro;
        memset(&ro, 0, sizeof(ro));
        EXPECT(moe_route(10, 2, 4, p, &ro, NULL) == MOE_ERR_INVALID_ARG);
        EXPECT(moe_route(10, 9, 4, p, &ro, NULL) == MOE_ERR_INVALID_ARG);
        EXPECT(moe_route(10, 2, 300, p, &ro, NULL) == MOE_ERR_INVALID_ARG);
        EXPECT(moe_route(10, 2, 4, p, NULL, NULL) == MOE_ERR_INVALID_ARG);
    }
    printf(bad ? "abi sanitizer run: FAILED\n" : "abi sanitizer run: ok\n");
    return bad;
}
