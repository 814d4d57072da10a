/* A plain C program against include/moe.h and libmoe_amd.so, with no Python in between: the
 * host-only entry points (route boundary, workspace sizes, expert stride, the cache policy) and
 * the argument checks of the device entry points, which reject bad arguments before touching
 * a device. Prints one line per check; exits non-zero on the first failure. */
#include <stdio.h>
#include <stdlib.h>

#include "moe.h"

static int fails = 0;
#define CHECK(cond, what)                                  \
    do {                                                   \
        if (cond) printf("ok   %s\n", what);               \
        else { printf("FAIL %s\n", what); ++fails; }       \
    } while (0)

int main(void) {
    const moe_shape s = {2048, 256, 8, 512, 512, 4, 64};
    const moe_shape bad = {2048, 256, 8, 512, 512, 5, 64};

    CHECK(moe_layer_path(&s, 1, 0) == MOE_PATH_DECODE, "T=1 takes the decode path");
    CHECK(moe_layer_path(&s, MOE_DEFAULT_CROSSOVER, 0) == MOE_PATH_DECODE &&
              moe_layer_path(&s, MOE_DEFAULT_CROSSOVER + 1, 0) == MOE_PATH_BATCHED,
          "the default crossover splits the two paths");
    CHECK(moe_layer_path(&s, 8, 8) == MOE_PATH_DECODE, "a crossover of 8 sends T=8 to the decode path");
    CHECK(moe_layer_path(&s, 9, 0) == MOE_PATH_BATCHED, "T=9 takes the batched path");
    CHECK(moe_layer_path(&s, 4, 2) == MOE_PATH_BATCHED, "a crossover of 2 sends T=4 to the batched path");
    CHECK(moe_layer_path(&s, 0, 0) == -1 && moe_layer_path(&bad, 1, 0) == -1, "invalid T or shape: -1");

    CHECK(moe_workspace_bytes(&s, 1, 40, MOE_WS_STACK) > moe_workspace_bytes(&s, 1, 1, MOE_WS_STACK),
          "a 40-layer stack needs more workspace than one layer");
    CHECK(moe_workspace_bytes(&bad, 1, 1, MOE_WS_DECODE) == 0, "no workspace size for an invalid shape");
    CHECK(moe_expert_stride(&s) == 1769472, "35B 4-bit expert block: 1,769,472 bytes");

    /* the cache policy on its own: capacity 2, keys 0 0 0 1 2 3 0 */
    const int32_t keys[7] = {0, 0, 0, 1, 2, 3, 0};
    int32_t hit[7], slot[7], ev[7];
    const int32_t want_hit[7] = {0, 1, 1, 0, 0, 0, 1}, want_ev[7] = {-1, -1, -1, -1, 1, 2, -1};
    int same = moe_cache_policy_run(2, 4, keys, 7, hit, slot, ev) == MOE_OK;
    for (int i = 0; i < 7; ++i) same = same && hit[i] == want_hit[i] && ev[i] == want_ev[i];
    CHECK(same, "LFU + recency keeps the thrice-used key over newcomers");

    /* device entry points refuse bad arguments before any device work */
    float y[4];
    CHECK(moe_layer_decode(&s, NULL, NULL, 1, y, NULL, NULL, NULL, NULL, 0, NULL) == MOE_ERR_INVALID_ARG,
          "decode without a layer is refused");
    CHECK(moe_layer_batched(&bad, NULL, NULL, 1, y, NULL, NULL, NULL, NULL, 0, NULL) != MOE_OK,
          "batched with an invalid shape is refused");
    moe_cache *c = NULL;
    CHECK(moe_cache_create(&s, 1, NULL, 0, NULL, 0, 0, NULL, 0, NULL, 0, NULL, &c) == MOE_ERR_INVALID_ARG && !c,
          "a cache without a container is refused");
    CHECK(moe_status_string(MOE_ERR_WORKSPACE) != NULL, "status strings");

    printf("%s\n", fails ? "FAILED" : "all C-ABI checks passed");
    return fails ? 1 : 0;
}
