// Host-only driver of the expert-residency policy (moe_cache_policy_run), built with AddressSanitizer
// and UndefinedBehaviorSanitizer by tests/test_sanitize_cpu.py. Every output array is heap-allocated
// to its exact size so that an access past it is reported; the outcomes are replayed against a
// slot -> key map to check that they describe a consistent cache.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "../../include/moe.h"

// The driver links the residency source alone; the container stride is used only by
// moe_cache_create, which it does not call.
extern "C" size_t moe_expert_stride(const moe_shape *) { return 0; }

static uint64_t mix(uint64_t &s) {  // splitmix64 step
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static int run(int slots, int n_keys, int64_t n, uint64_t seed, bool skewed) {
    int32_t *keys = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n ? n : 1));
    int32_t *hit = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n ? n : 1));
    int32_t *slot = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n ? n : 1));
    int32_t *ev = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n ? n : 1));
    for (int64_t i = 0; i < n; ++i) {
        uint64_t r = mix(seed) % (uint64_t)n_keys;
        if (skewed) r = r * r % (uint64_t)n_keys % (1 + (uint64_t)n_keys / 4);  // a few hot keys
        keys[i] = (int32_t)r;
    }
    int bad = 0;
    if (moe_cache_policy_run(slots, n_keys, keys, n, hit, slot, ev) != MOE_OK) {
        printf("policy refused slots=%d keys=%d n=%lld\n", slots, n_keys, (long long)n);
        bad = 1;
    }
    std::vector<int> occ(slots > 0 ? slots : 1, -1), where(n_keys, -1);
    for (int64_t i = 0; i < n && !bad; ++i) {
        const int k = keys[i], s = slot[i];
        if (slots == 0) {
            bad = hit[i] != 0 || s != -1 || ev[i] != -1;
        } else if (hit[i]) {
            bad = s < 0 || s >= slots || occ[s] != k || ev[i] != -1;
        } else if (s == -1) {
            bad = ev[i] != -1 || where[k] != -1;
        } else {
            bad = s >= slots || where[k] != -1 || occ[s] != ev[i];
            if (!bad && ev[i] >= 0) where[ev[i]] = -1;
            occ[s] = k;
            where[k] = s;
        }
        if (bad) printf("inconsistent outcome at access %lld (key %d)\n", (long long)i, k);
    }
    free(keys); free(hit); free(slot); free(ev);
    return bad;
}

int main() {
    int bad = 0;
    bad |= run(0, 16, 100, 1, false);
    bad |= run(1, 16, 500, 2, false);
    bad |= run(8, 64, 5000, 3, true);
    bad |= run(37, 512, 20000, 4, false);
    bad |= run(64, 64, 3000, 5, true);  // as many slots as keys
    bad |= run(16, 1, 50, 6, false);    // one key
    bad |= run(4, 8, 0, 7, false);      // no access
    int32_t k = 9, h, s, e;
    bad |= moe_cache_policy_run(4, 8, &k, 1, &h, &s, &e) != MOE_ERR_INVALID_ARG;  // key out of range
    bad |= moe_cache_policy_run(-1, 8, &k, 0, &h, &s, &e) != MOE_ERR_INVALID_ARG;
    if (bad) return 1;
    printf("policy sanitizer checks passed\n");
    return 0;
}
