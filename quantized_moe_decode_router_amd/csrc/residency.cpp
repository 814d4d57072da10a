// Expert residency: a bounded pool of expert slots in HBM in front of a fixed-stride expert
// container, with least-frequently-used eviction and ties broken by least recent use.
//
// Swiftlet (AgentLens project page, "How it works"; xix.ai article, scheduling paragraph; the
// Chinese summary's highlights) keeps the dense weights resident, packs the routed experts into
// fixed-stride blocks so that one read is one fetch, and holds the popular ones in a bounded pool
// with LFU + recency eviction (hit rates of 43-70 % on its machine). Here the container sits in host memory the GPU
// can read (or anywhere in device memory), the pool in HBM, and the decode kernel follows a
// per-(layer, expert) table of block addresses: a resident expert is read from its pool slot, any
// other straight from the container. After each decode call the host feeds that call's routing
// through the policy in order (layer, token, slot), then copies the blocks of newly admitted
// experts into their slots and rewrites the table, all on the caller's stream behind the call.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>

#include <set>
#include <tuple>
#include <unordered_map>
#include <vector>

#include "../../include/moe.h"
#include "moe_internal.hpp"

namespace {

// The eviction policy over keys 0..n_keys-1 and `slots` slots. A resident key has a use count
// (1 at admission, +1 per hit) and the tick of its last use; the victim is the resident key with
// the smallest count, then the oldest last use. Free slots are taken lowest index first.
class LfuRecency {
  public:
    LfuRecency(int slots, int n_keys) : owner_(slots, -1), count_(slots, 0), last_(slots, 0), slot_of_(n_keys, -1) {}

    struct Outcome {
        bool hit;
        int slot;     // slot the key occupies after the access, or -1 (no slots at all)
        int evicted;  // key evicted by this access, or -1
    };

    Outcome access(int key) {
        ++tick_;
        int sl = slot_of_[key];
        if (sl >= 0) {
            order_.erase(std::make_tuple(count_[sl], last_[sl], sl));
            ++count_[sl];
            last_[sl] = tick_;
            order_.insert(std::make_tuple(count_[sl], last_[sl], sl));
            return {true, sl, -1};
        }
        const int slots = (int)owner_.size();
        if (slots == 0) return {false, -1, -1};
        int evicted = -1;
        if (next_free_ < slots) {
            sl = next_free_++;
        } else {
            const auto victim = *order_.begin();
            order_.erase(order_.begin());
            sl = std::get<2>(victim);
            evicted = owner_[sl];
            slot_of_[evicted] = -1;
        }
        owner_[sl] = key;
        count_[sl] = 1;
        last_[sl] = tick_;
        slot_of_[key] = sl;
        order_.insert(std::make_tuple(count_[sl], last_[sl], sl));
        return {false, sl, evicted};
    }
    const std::vector<int> &owners() const { return owner_; }

  private:
    std::vector<int> owner_;
    std::vector<int64_t> count_;
    std::vector<uint64_t> last_;
    std::vector<int> slot_of_;
    std::set<std::tuple<int64_t, uint64_t, int>> order_;  // resident slots by (count, last use)
    uint64_t tick_ = 0;
    int next_free_ = 0;
};

}  // namespace

struct moe_cache {
    int L, E, slots;
    size_t stride;
    const char *container;
    char *pool;
    char *landing = nullptr;  // [L][T][K] blocks (T of the call) written through by the decode, or null
    int max_tokens = 0, K = 0;
    uint64_t *table_dev;
    uint64_t *table_host;  // pinned staging of the whole table (its state after the copies)
    uint64_t *table_mid;   // pinned staging of the table while the copies run
    LfuRecency policy;
    uint64_t hits = 0, misses = 0, bytes_copied = 0;
    bool broken = false;  // an update failed part-way: the pool no longer matches the policy
    moe_cache(int L_, int E_, int slots_) : L(L_), E(E_), slots(slots_), policy(slots_, L_ * E_) {}
};

namespace {
// Feeds n keys through the policy, then queues the admissions' copies and the table rewrite on
// hs (which the caller has synchronised). from_landing: access i was read by the decode call
// whose routing this is, so a block outside the pool during that call is at landing block i.
moe_status apply_keys(moe_cache *c, const int *keys, size_t n, hipStream_t hs, bool from_landing,
                      int32_t *hits_opt, int32_t *misses_opt) {
    const std::vector<int> before = c->policy.owners();
    std::vector<char> was_resident(from_landing ? (size_t)c->L * c->E : 0, 0);
    if (from_landing)
        for (int k : before)
            if (k >= 0) was_resident[k] = 1;
    std::unordered_map<int, size_t> first;  // key -> its first access of this call (the landing block)
    int32_t hits = 0, misses = 0;
    for (size_t i = 0; i < n; ++i) {
        const int key = keys[i];
        first.emplace(key, i);
        const LfuRecency::Outcome o = c->policy.access(key);
        if (o.hit) ++hits;
        else ++misses;
    }
    c->hits += hits;
    c->misses += misses;
    const std::vector<int> &after = c->policy.owners();
    const size_t tbytes = (size_t)c->L * c->E * 8;
    const uint64_t mark = c->landing ? 1u : 0u;
    auto at_container = [&](int key) {
        return reinterpret_cast<uint64_t>(c->container + (size_t)key * c->stride) | mark;
    };
    // an admitted expert that was outside the pool during the call has its block in the landing
    // buffer (written through by the decode); one that was in a pool slot (evicted and re-admitted
    // within this call) is copied from the container
    auto source = [&](int key) -> const char * {
        if (from_landing && !was_resident[key]) {
            return c->landing + first.at(key) * c->stride;  // block [l][t][k] of the call's T
        }
        return c->container + (size_t)key * c->stride;
    };
    // Three steps on the stream, so that the device table never names a slot being rewritten:
    // (1) every expert leaving a slot points at its container block again, (2) the admitted blocks
    // are copied into their slots, (3) the admitted experts point at their slots. If a step fails,
    // the table on the device is (1)'s and the cache refuses further updates.
    for (int sl = 0; sl < c->slots; ++sl)
        if (after[sl] != before[sl] && before[sl] >= 0) c->table_host[before[sl]] = at_container(before[sl]);
    memcpy(c->table_mid, c->table_host, tbytes);
    c->broken = true;
    if (hipMemcpyAsync(c->table_dev, c->table_mid, tbytes, hipMemcpyHostToDevice, hs) != hipSuccess) return MOE_ERR_HIP;
    for (int sl = 0; sl < c->slots; ++sl) {
        if (after[sl] == before[sl]) continue;
        if (hipMemcpyAsync(c->pool + (size_t)sl * c->stride, source(after[sl]), c->stride, hipMemcpyDefault, hs) !=
            hipSuccess)
            return MOE_ERR_HIP;
        c->bytes_copied += c->stride;
    }
    // a key evicted from one slot may have been admitted into another within the same call
    for (int sl = 0; sl < c->slots; ++sl)
        if (after[sl] >= 0) c->table_host[after[sl]] = reinterpret_cast<uint64_t>(c->pool + (size_t)sl * c->stride);
    if (hipMemcpyAsync(c->table_dev, c->table_host, tbytes, hipMemcpyHostToDevice, hs) != hipSuccess)
        return MOE_ERR_HIP;
    c->broken = false;
    if (hits_opt) *hits_opt = hits;
    if (misses_opt) *misses_opt = misses;
    return MOE_OK;
}
}  // namespace


extern "C" {

moe_status moe_cache_create(const moe_shape *s, int32_t n_layers, const void *container, size_t container_bytes,
                            void *pool, size_t pool_bytes, int32_t slots, uint64_t *table, size_t table_bytes,
                            void *landing_opt, size_t landing_bytes, void *stream, moe_cache **out) {
    if (!out) return MOE_ERR_INVALID_ARG;
    *out = nullptr;
    const size_t stride = moe_expert_stride(s);
    if (stride == 0 || n_layers < 1 || n_layers > 4096 || slots < 0) return MOE_ERR_INVALID_ARG;
    const size_t keys = (size_t)n_layers * s->num_experts;
    if (keys > (size_t)INT32_MAX || (size_t)slots > keys) return MOE_ERR_INVALID_ARG;
    if (!container || (reinterpret_cast<uintptr_t>(container) & 4095u) || container_bytes < keys * stride)
        return MOE_ERR_INVALID_ARG;
    if (slots > 0 && (!pool || (reinterpret_cast<uintptr_t>(pool) & 4095u) || pool_bytes < (size_t)slots * stride))
        return MOE_ERR_INVALID_ARG;
    if (!table || (reinterpret_cast<uintptr_t>(table) & 15u) || table_bytes < keys * 8) return MOE_ERR_INVALID_ARG;
    const size_t per_token = (size_t)n_layers * s->top_k * stride;  // landing bytes per token of a call
    if (landing_opt && ((reinterpret_cast<uintptr_t>(landing_opt) & 4095u) || landing_bytes < per_token))
        return MOE_ERR_INVALID_ARG;
    // the kernel reads the container at the addresses the table holds: it must be device memory,
    // or pinned host memory mapped at the same address (pageable memory would fault the device)
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, container) != hipSuccess) {
        (void)hipGetLastError();
        return MOE_ERR_INVALID_ARG;
    }
    if (attr.devicePointer != container) return MOE_ERR_INVALID_ARG;
    moe_cache *c = new moe_cache(n_layers, s->num_experts, slots);
    c->stride = stride;
    c->container = static_cast<const char *>(container);
    c->pool = static_cast<char *>(pool);
    c->table_dev = table;
    c->landing = static_cast<char *>(landing_opt);
    c->K = s->top_k;
    c->max_tokens = landing_opt ? (int)std::min<size_t>(landing_bytes / per_token, 65536) : 0;
    c->table_host = c->table_mid = nullptr;
    if (hipHostMalloc(reinterpret_cast<void **>(&c->table_host), keys * 8, hipHostMallocDefault) != hipSuccess ||
        hipHostMalloc(reinterpret_cast<void **>(&c->table_mid), keys * 8, hipHostMallocDefault) != hipSuccess) {
        if (c->table_host) hipHostFree(c->table_host);
        delete c;
        return MOE_ERR_HIP;
    }
    const uint64_t mark = c->landing ? 1u : 0u;  // bit 0: the decode writes the block's rows through
    for (size_t k = 0; k < keys; ++k) c->table_host[k] = reinterpret_cast<uint64_t>(c->container + k * stride) | mark;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(table, c->table_host, keys * 8, hipMemcpyHostToDevice, hs) != hipSuccess ||
        hipStreamSynchronize(hs) != hipSuccess) {
        hipHostFree(c->table_host);
        hipHostFree(c->table_mid);
        delete c;
        return MOE_ERR_HIP;
    }
    *out = c;
    return MOE_OK;
}

moe_status moe_cache_update(moe_cache *c, const int32_t *topk_idx_all, int32_t T, int32_t top_k, void *stream,
                            int32_t *hits_opt, int32_t *misses_opt) {
    if (!c || !topk_idx_all || T < 1 || top_k < 1) return MOE_ERR_INVALID_ARG;
    if (c->broken) return MOE_ERR_HIP;
    if (c->landing && (T > c->max_tokens || top_k != c->K)) return MOE_ERR_INVALID_ARG;
    const size_t n = (size_t)c->L * T * top_k;
    for (size_t i = 0; i < n; ++i)
        if (topk_idx_all[i] < 0 || topk_idx_all[i] >= c->E) return MOE_ERR_INVALID_ARG;
    std::vector<int> keys(n);
    for (size_t i = 0; i < n; ++i) keys[i] = (int)(i / ((size_t)T * top_k)) * c->E + topk_idx_all[i];
    hipStream_t hs = static_cast<hipStream_t>(stream);
    // the staging table and the pool slots may still be read by work queued earlier
    if (hipStreamSynchronize(hs) != hipSuccess) return MOE_ERR_HIP;
    return apply_keys(c, keys.data(), n, hs, c->landing != nullptr, hits_opt, misses_opt);
}

moe_status moe_cache_admit(moe_cache *c, const int32_t *keys, int64_t n, void *stream, int32_t *hits_opt,
                           int32_t *misses_opt) {
    if (!c || n < 0 || (n > 0 && !keys)) return MOE_ERR_INVALID_ARG;
    if (c->broken) return MOE_ERR_HIP;
    for (int64_t i = 0; i < n; ++i)
        if (keys[i] < 0 || keys[i] >= c->L * c->E) return MOE_ERR_INVALID_ARG;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (hipStreamSynchronize(hs) != hipSuccess) return MOE_ERR_HIP;
    return apply_keys(c, keys, (size_t)n, hs, false, hits_opt, misses_opt);
}

moe_status moe_cache_stats(const moe_cache *c, uint64_t *hits, uint64_t *misses, uint64_t *bytes_copied) {
    if (!c) return MOE_ERR_INVALID_ARG;
    if (hits) *hits = c->hits;
    if (misses) *misses = c->misses;
    if (bytes_copied) *bytes_copied = c->bytes_copied;
    return MOE_OK;
}

moe_status moe_cache_owners(const moe_cache *c, int32_t *owner) {
    if (!c || (!owner && c->slots > 0)) return MOE_ERR_INVALID_ARG;
    const std::vector<int> &o = c->policy.owners();
    for (int sl = 0; sl < c->slots; ++sl) owner[sl] = o[sl];
    return MOE_OK;
}

void moe_cache_destroy(moe_cache *c) {
    if (!c) return;
    hipHostFree(c->table_host);
    hipHostFree(c->table_mid);
    delete c;
}

moe_status moe_cache_policy_run(int32_t slots, int32_t n_keys, const int32_t *keys, int64_t n, int32_t *hit,
                                int32_t *slot, int32_t *evicted) {
    if (slots < 0 || n_keys < 1 || n < 0 || (n > 0 && (!keys || !hit || !slot || !evicted)))
        return MOE_ERR_INVALID_ARG;
    for (int64_t i = 0; i < n; ++i)
        if (keys[i] < 0 || keys[i] >= n_keys) return MOE_ERR_INVALID_ARG;
    LfuRecency pol(slots, n_keys);
    for (int64_t i = 0; i < n; ++i) {
        const LfuRecency::Outcome o = pol.access(keys[i]);
        hit[i] = o.hit ? 1 : 0;
        slot[i] = o.slot;
        evicted[i] = o.evicted;
    }
    return MOE_OK;
}

}  // extern "C"
