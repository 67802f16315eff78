// cache.cpp -- HBM expert-slot cache filled from pinned host memory.
//
// Colibri loads a routed expert only when the router selects it and keeps
// recently used experts in an LRU cache ("Guide Complet de Colibri", section
// "Qu'est-ce que Colibri ?"); a lookahead worker prefetches the next layer's
// predicted experts while the current layer computes (same guide, section
// "Router-Lookahead prefetch"; kongchang article, storage-tier section).
// Placement decides speed only, never results (aifrontierpost tutorial,
// "Honest limitations").
//
// Colibri also records which experts a workload routes to and pins the
// hottest ones (aifrontierpost tutorial, introduction and "Step 4 -- Run it";
// kongchang article, storage-tier section): every DEMAND access counts toward
// its key's usage, and moe_cache_pin_hot pins the keys with the highest counts
// in slots that are never evicted.
//
// Here the tiers are pinned host memory -> an HBM slot pool.  Copies run with
// hipMemcpyAsync on the cache's own copy stream.  Each slot has a fill event
// (recorded on the copy stream after its copy) and a release event (recorded
// on the compute stream when the layer that used it is released).  A compute
// stream waits on the fill events of the slots it reads; the copy stream waits
// on a slot's release event before overwriting it, so a slot is never
// refilled while a kernel may still read it.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <unordered_map>
#include <vector>

#include "host_common.h"

using namespace moe;

namespace {

struct Slot {
    int32_t layer = -1, expert = -1;
    int64_t last_use = -1;
    int32_t locked_by = -1;
    int32_t prefetched = 0;
    int32_t pinned = 0;
    bool fill_recorded = false, release_recorded = false;
    hipEvent_t fill_ev = nullptr, release_ev = nullptr;
    uint8_t *mem = nullptr;
};

}  // namespace

struct moe_cache {
    moe_cache_desc d{};
    int n_slots = 0;
    std::vector<Slot> slots;
    std::unordered_map<int64_t, int> where;
    std::vector<int64_t> usage;           // [L*E] DEMAND accesses per key
    int64_t clock = 0;
    moe_cache_stats st{};
    bool log_on = false;
    std::vector<moe_cache_event> log;
    bool fail_next = false;
    hipStream_t copy = nullptr;
    uint8_t *pool = nullptr;              // device pool, or host pool for the host backend
    const void **table_dev = nullptr;     // [L*E] device (HIP backend)
    std::vector<const void *> table_host; // [L*E] (host backend)
    int32_t *ids_pinned = nullptr;        // routing ids copied back from the device
    int ids_cap = 0;
    // copy timing (HIP backend): a ring of (start, stop) event pairs around
    // the host-to-device copies; copies [cp_tail, cp_head) are recorded and
    // not yet added up.  The copy stream runs one copy at a time, so the sum
    // of the durations is the time the copy engine was busy with them.
    static constexpr int CP_RING = 512;
    std::vector<hipEvent_t> cp_ev;        // [CP_RING][2]
    mutable int64_t cp_head = 0, cp_tail = 0;
    mutable double copy_ms = 0.0;
    mutable int64_t copies_timed = 0;
    mutable hipError_t cp_err = hipSuccess;
};

// waits for the recorded copies (all, or down to `keep` outstanding) and adds
// up their durations
static void copy_timing_drain(const moe_cache *c, int64_t keep)
{
    for (; c->cp_head - c->cp_tail > keep; ++c->cp_tail) {
        const size_t i = (size_t)(c->cp_tail % moe_cache::CP_RING) * 2;
        float ms = 0.0f;
        hipError_t e = hipEventSynchronize(c->cp_ev[i + 1]);
        if (e == hipSuccess)
            e = hipEventElapsedTime(&ms, c->cp_ev[i], c->cp_ev[i + 1]);
        if (e != hipSuccess) {
            if (c->cp_err == hipSuccess)
                c->cp_err = e;
            continue;
        }
        c->copy_ms += ms;
        c->copies_timed += 1;
    }
}

static int64_t key_of(const moe_cache *c, int layer, int expert)
{
    return (int64_t)layer * c->d.n_experts + expert;
}

static void emit(moe_cache *c, int kind, int layer, int expert, int slot)
{
    if (c->log_on)
        c->log.push_back(moe_cache_event{kind, layer, expert, slot});
}

static void part_range(const moe_cache *c, int layer, int *lo, int *hi)
{
    if (c->d.policy == MOE_CACHE_PER_LAYER_LRU) {
        *lo = (int)((int64_t)layer * c->n_slots / c->d.n_layers);
        *hi = (int)((int64_t)(layer + 1) * c->n_slots / c->d.n_layers);
    } else {
        *lo = 0;
        *hi = c->n_slots;
    }
}

static int find_victim(const moe_cache *c, int layer)
{
    int lo, hi, best = -1;
    part_range(c, layer, &lo, &hi);
    for (int i = lo; i < hi; ++i) {
        const Slot &s = c->slots[i];
        if (s.locked_by >= 0 || s.pinned)
            continue;
        if (best < 0 || s.last_use < c->slots[best].last_use)
            best = i;
    }
    return best;
}

static bool hip_backend(const moe_cache *c)
{
    return c->d.backend == MOE_CACHE_BACKEND_HIP;
}

// Clears the slot's key (eviction).  The device table entry is cleared by the
// update kernel that the next fill of this slot enqueues.
static void evict(moe_cache *c, int i, int *cleared_key)
{
    Slot &s = c->slots[i];
    *cleared_key = -1;
    if (s.layer < 0)
        return;
    emit(c, 5, s.layer, s.expert, i);
    c->st.evictions++;
    if (s.prefetched)
        c->st.prefetch_wasted++;
    int64_t k = key_of(c, s.layer, s.expert);
    c->where.erase(k);
    *cleared_key = (int)k;
    if (!hip_backend(c))
        c->table_host[k] = nullptr;
    s.layer = s.expert = -1;
    s.prefetched = 0;
}

// Copies key (layer, expert) into slot i.  On failure the slot stays empty.
static moe_status fill(moe_cache *c, int i, int layer, int expert, int cleared_key)
{
    Slot &s = c->slots[i];
    const int64_t k = key_of(c, layer, expert);
    const void *src = c->d.host_blobs[k];
    if (!src)
        return fail(MOE_E_INVAL, "host blob of (layer %d, expert %d) is NULL", layer, expert);
    if (c->fail_next) {
        c->fail_next = false;
        return fail(MOE_E_HIP, "copy of (layer %d, expert %d) failed (injected)", layer, expert);
    }
    if (hip_backend(c)) {
        hipError_t e;
        if (s.release_recorded && (e = hipStreamWaitEvent(c->copy, s.release_ev, 0)) != hipSuccess)
            return hip_fail(e, "hipStreamWaitEvent(release)");
        if (c->cp_head - c->cp_tail >= moe_cache::CP_RING)
            copy_timing_drain(c, moe_cache::CP_RING - 1);
        const size_t ri = (size_t)(c->cp_head % moe_cache::CP_RING) * 2;
        if ((e = hipEventRecord(c->cp_ev[ri], c->copy)) != hipSuccess)
            return hip_fail(e, "hipEventRecord(copy start)");
        if ((e = hipMemcpyAsync(s.mem, src, c->d.blob_bytes, hipMemcpyHostToDevice, c->copy)) !=
            hipSuccess)
            return hip_fail(e, "hipMemcpyAsync(expert)");
        if ((e = hipEventRecord(c->cp_ev[ri + 1], c->copy)) != hipSuccess)
            return hip_fail(e, "hipEventRecord(copy stop)");
        c->cp_head += 1;
        if ((e = launch_table_update(c->table_dev, (int)k, s.mem, cleared_key, c->copy)) !=
            hipSuccess)
            return hip_fail(e, "table update launch");
        if ((e = hipEventRecord(s.fill_ev, c->copy)) != hipSuccess)
            return hip_fail(e, "hipEventRecord(fill)");
        s.fill_recorded = true;
    } else {
        memcpy(s.mem, src, c->d.blob_bytes);
        c->table_host[k] = s.mem;
    }
    s.layer = layer;
    s.expert = expert;
    c->where[k] = i;
    c->st.bytes_copied += (int64_t)c->d.blob_bytes;
    return MOE_OK;
}

static void destroy(moe_cache *c)
{
    if (!c)
        return;
    if (hip_backend(c)) {
        int prev = 0;
        (void)hipGetDevice(&prev);
        (void)hipSetDevice(c->d.device);
        if (c->copy)
            (void)hipStreamSynchronize(c->copy);
        for (hipEvent_t ev : c->cp_ev)
            if (ev)
                (void)hipEventDestroy(ev);
        for (Slot &s : c->slots) {
            if (s.fill_ev)
                (void)hipEventDestroy(s.fill_ev);
            if (s.release_ev)
                (void)hipEventDestroy(s.release_ev);
        }
        if (c->copy)
            (void)hipStreamDestroy(c->copy);
        if (c->pool)
            (void)hipFree(c->pool);
        if (c->table_dev)
            (void)hipFree(c->table_dev);
        if (c->ids_pinned)
            (void)hipHostFree(c->ids_pinned);
        (void)hipSetDevice(prev);
    } else {
        free(c->pool);
    }
    delete c;
}

extern "C" moe_status moe_cache_create(const moe_cache_desc *desc, moe_cache **out)
{
    if (!out || !desc)
        return fail(MOE_E_INVAL, "NULL argument");
    *out = nullptr;
    if (desc->n_layers < 1 || desc->n_experts < 1 || desc->blob_bytes == 0 || !desc->host_blobs)
        return fail(MOE_E_INVAL, "bad cache descriptor");
    if (desc->policy != MOE_CACHE_GLOBAL_LRU && desc->policy != MOE_CACHE_PER_LAYER_LRU)
        return fail(MOE_E_INVAL, "unknown policy %d", desc->policy);
    if (desc->backend != MOE_CACHE_BACKEND_HIP && desc->backend != MOE_CACHE_BACKEND_HOST)
        return fail(MOE_E_INVAL, "unknown backend %d", desc->backend);
    if (desc->blob_bytes % 256)
        return fail(MOE_E_INVAL, "blob_bytes must be a multiple of 256");
    const size_t n = desc->capacity_bytes / desc->blob_bytes;
    if (n < 1 || n > (1u << 24))
        return fail(MOE_E_CAPACITY, "capacity holds %zu slots", n);
    moe_cache *c = new moe_cache();
    c->d = *desc;
    c->n_slots = (int)n;
    c->slots.resize(n);
    const size_t L = desc->n_layers, E = desc->n_experts;
    if (desc->backend == MOE_CACHE_BACKEND_HIP) {
        moe_status st = check_device(desc->device);
        if (st) {
            delete c;
            return st;
        }
        hipError_t e = hipSetDevice(desc->device);
        if (e == hipSuccess)
            e = hipStreamCreateWithFlags(&c->copy, hipStreamNonBlocking);
        if (e == hipSuccess)
            e = hipMalloc(reinterpret_cast<void **>(&c->pool), n * desc->blob_bytes);
        if (e == hipSuccess)
            e = hipMalloc(reinterpret_cast<void **>(&c->table_dev), L * E * sizeof(void *));
        if (e == hipSuccess)
            e = hipMemset(c->table_dev, 0, L * E * sizeof(void *));
        if (e == hipSuccess) {
            c->ids_cap = 1 << 16;
            e = hipHostMalloc(reinterpret_cast<void **>(&c->ids_pinned), c->ids_cap * 4,
                              hipHostMallocDefault);
        }
        c->cp_ev.assign((size_t)2 * moe_cache::CP_RING, nullptr);
        for (size_t i = 0; e == hipSuccess && i < c->cp_ev.size(); ++i)
            e = hipEventCreate(&c->cp_ev[i]);
        for (size_t i = 0; e == hipSuccess && i < n; ++i) {
            e = hipEventCreateWithFlags(&c->slots[i].fill_ev, hipEventDisableTiming);
            if (e == hipSuccess)
                e = hipEventCreateWithFlags(&c->slots[i].release_ev, hipEventDisableTiming);
            c->slots[i].mem = c->pool + i * desc->blob_bytes;
        }
        if (e != hipSuccess) {
            destroy(c);
            return fail(MOE_E_NOMEM, "cache allocation: %s", hipGetErrorString(e));
        }
    } else {
        c->pool = static_cast<uint8_t *>(malloc(n * desc->blob_bytes));
        if (!c->pool) {
            delete c;
            return fail(MOE_E_NOMEM, "host pool of %zu bytes", n * desc->blob_bytes);
        }
        for (size_t i = 0; i < n; ++i)
            c->slots[i].mem = c->pool + i * desc->blob_bytes;
        c->table_host.assign(L * E, nullptr);
    }
    c->usage.assign(L * E, 0);
    c->st.n_slots = (int64_t)n;
    *out = c;
    return MOE_OK;
}

extern "C" void moe_cache_destroy(moe_cache *cache)
{
    destroy(cache);
}

static moe_status stage_demand(moe_cache *c, int layer, const int32_t *ids, int n,
                               hipStream_t compute, const void **out)
{
    // capacity check first: nothing changes when it fails
    int lo, hi, usable = 0;
    part_range(c, layer, &lo, &hi);
    for (int i = lo; i < hi; ++i) {
        const Slot &s = c->slots[i];
        if (s.locked_by < 0 && !s.pinned) {
            ++usable;
        } else if (s.layer == layer) {
            for (int j = 0; j < n; ++j)
                if (ids[j] == s.expert) {
                    ++usable;
                    break;
                }
        }
    }
    if (usable < n)
        return fail(MOE_E_CAPACITY, "layer %d needs %d slots, %d usable", layer, n, usable);
    for (int j = 0; j < n; ++j) {
        const int e = ids[j];
        c->usage[(size_t)key_of(c, layer, e)] += 1;
        auto it = c->where.find(key_of(c, layer, e));
        int i;
        if (it != c->where.end()) {
            i = it->second;
            emit(c, 0, layer, e, i);
            c->st.demand_hits++;
            if (c->slots[i].prefetched) {
                c->st.prefetch_used++;
                c->slots[i].prefetched = 0;
            }
        } else {
            i = find_victim(c, layer);
            if (i < 0)
                return fail(MOE_E_CAPACITY, "no unlocked slot for layer %d", layer);
            int cleared;
            evict(c, i, &cleared);
            moe_status st = fill(c, i, layer, e, cleared);
            if (st) {
                c->slots[i].last_use = -1;
                return st;
            }
            emit(c, 1, layer, e, i);
            c->st.demand_misses++;
        }
        Slot &s = c->slots[i];
        s.last_use = ++c->clock;
        s.locked_by = layer;
        if (hip_backend(c) && s.fill_recorded) {
            hipError_t err = hipStreamWaitEvent(compute, s.fill_ev, 0);
            if (err != hipSuccess)
                return hip_fail(err, "hipStreamWaitEvent(fill)");
        }
        if (out)
            out[j] = s.mem;
    }
    return MOE_OK;
}

static moe_status stage_prefetch(moe_cache *c, int layer, const int32_t *ids, int n)
{
    for (int j = 0; j < n; ++j) {
        const int e = ids[j];
        auto it = c->where.find(key_of(c, layer, e));
        if (it != c->where.end()) {
            int i = it->second;
            emit(c, 3, layer, e, i);
            c->st.prefetch_resident++;
            c->slots[i].last_use = ++c->clock;
            continue;
        }
        int i = find_victim(c, layer);
        if (i < 0) {
            emit(c, 4, layer, e, -1);
            c->st.prefetch_skipped++;
            continue;
        }
        int cleared;
        evict(c, i, &cleared);
        moe_status st = fill(c, i, layer, e, cleared);
        if (st) {
            c->slots[i].last_use = -1;
            return st;
        }
        Slot &s = c->slots[i];
        s.prefetched = 1;
        s.last_use = ++c->clock;
        emit(c, 2, layer, e, i);
        c->st.prefetch_issued++;
    }
    return MOE_OK;
}

extern "C" moe_status moe_cache_pin_hot(moe_cache *c, int32_t n, int32_t reserve)
{
    if (!c || n < 0 || reserve < 1)
        return fail(MOE_E_INVAL, "bad arguments");
    for (const Slot &s : c->slots)
        if (s.locked_by >= 0)
            return fail(MOE_E_INVAL, "layer %d still holds slots: pin between layers",
                        s.locked_by);
    for (Slot &s : c->slots)
        s.pinned = 0;
    c->st.pinned = 0;
    // keys with a nonzero count, count descending, key ascending
    std::vector<int32_t> order;
    for (size_t key = 0; key < c->usage.size(); ++key)
        if (c->usage[key] > 0)
            order.push_back((int32_t)key);
    std::stable_sort(order.begin(), order.end(), [c](int32_t a, int32_t b) {
        return c->usage[(size_t)a] > c->usage[(size_t)b];
    });
    int pinned = 0;
    for (size_t r = 0; r < order.size() && pinned < n; ++r) {
        const int key = order[r];
        const int layer = key / c->d.n_experts, e = key % c->d.n_experts;
        int lo, hi, part_pinned = 0;
        part_range(c, layer, &lo, &hi);
        for (int i = lo; i < hi; ++i)
            part_pinned += c->slots[i].pinned;
        if (part_pinned >= (hi - lo) - reserve)
            continue;                       // its partition is full of pins
        auto it = c->where.find(key);
        int i;
        if (it != c->where.end()) {
            i = it->second;
            emit(c, 7, layer, e, i);
        } else {
            i = find_victim(c, layer);
            if (i < 0)
                return fail(MOE_E_CAPACITY, "no slot left to pin (layer %d, expert %d)", layer, e);
            int cleared;
            evict(c, i, &cleared);
            moe_status st = fill(c, i, layer, e, cleared);
            if (st) {
                c->slots[i].last_use = -1;
                return st;
            }
            c->slots[i].last_use = ++c->clock;
            emit(c, 6, layer, e, i);
            c->st.pin_fills++;
        }
        c->slots[i].pinned = 1;
        c->st.pinned++;
        ++pinned;
    }
    return MOE_OK;
}

extern "C" moe_status moe_cache_usage_get(const moe_cache *c, int64_t *usage_host)
{
    if (!c || !usage_host)
        return fail(MOE_E_INVAL, "NULL argument");
    std::copy(c->usage.begin(), c->usage.end(), usage_host);
    return MOE_OK;
}

extern "C" moe_status moe_cache_usage_set(moe_cache *c, const int64_t *usage_host)
{
    if (!c || !usage_host)
        return fail(MOE_E_INVAL, "NULL argument");
    for (size_t i = 0; i < c->usage.size(); ++i)
        if (usage_host[i] < 0)
            return fail(MOE_E_INVAL, "negative usage count at key %zu", i);
    std::copy(usage_host, usage_host + c->usage.size(), c->usage.begin());
    return MOE_OK;
}

extern "C" moe_status moe_cache_stage(moe_cache *cache, int32_t layer, const int32_t *ids_host,
                                      int32_t n, int32_t mode, void *compute,
                                      const void **dev_ptrs_host_out)
{
    if (!cache || (!ids_host && n > 0) || n < 0)
        return fail(MOE_E_INVAL, "bad arguments");
    if (layer < 0 || layer >= cache->d.n_layers)
        return fail(MOE_E_INVAL, "layer %d out of range", layer);
    for (int j = 0; j < n; ++j) {
        if (ids_host[j] < 0 || ids_host[j] >= cache->d.n_experts)
            return fail(MOE_E_INVAL, "expert id %d out of range", ids_host[j]);
        for (int i = 0; i < j; ++i)
            if (ids_host[i] == ids_host[j])
                return fail(MOE_E_INVAL, "expert id %d repeated", ids_host[j]);
    }
    if (mode == MOE_STAGE_DEMAND)
        return stage_demand(cache, layer, ids_host, n, static_cast<hipStream_t>(compute),
                            dev_ptrs_host_out);
    if (mode == MOE_STAGE_PREFETCH)
        return stage_prefetch(cache, layer, ids_host, n);
    if (mode == MOE_STAGE_PREFETCH_IDLE) {
        if (hip_backend(cache)) {
            const hipError_t q = hipStreamQuery(cache->copy);
            if (q == hipErrorNotReady) {
                // copies still in flight: a prefetch now would queue behind
                // them and delay the next demand copies
                for (int j = 0; j < n; ++j)
                    emit(cache, 8, layer, ids_host[j], -1);
                cache->st.prefetch_skipped += n;
                return MOE_OK;
            }
            if (q != hipSuccess)
                return hip_fail(q, "hipStreamQuery(copy stream)");
        }
        return stage_prefetch(cache, layer, ids_host, n);
    }
    return fail(MOE_E_INVAL, "unknown stage mode %d", mode);
}

extern "C" moe_status moe_cache_release(moe_cache *cache, int32_t layer, void *compute)
{
    if (!cache)
        return fail(MOE_E_INVAL, "cache is NULL");
    for (Slot &s : cache->slots) {
        if (s.locked_by != layer)
            continue;
        s.locked_by = -1;
        if (hip_backend(cache)) {
            hipError_t e = hipEventRecord(s.release_ev, static_cast<hipStream_t>(compute));
            if (e != hipSuccess)
                return hip_fail(e, "hipEventRecord(release)");
            s.release_recorded = true;
        }
    }
    return MOE_OK;
}

extern "C" const void *const *moe_cache_table(moe_cache *cache, int32_t layer)
{
    if (!cache || layer < 0 || layer >= cache->d.n_layers)
        return nullptr;
    const size_t off = (size_t)layer * cache->d.n_experts;
    if (hip_backend(cache))
        return cache->table_dev + off;
    return cache->table_host.data() + off;
}

extern "C" moe_status moe_cache_stats_get(const moe_cache *cache, moe_cache_stats *out)
{
    if (!cache || !out)
        return fail(MOE_E_INVAL, "NULL argument");
    copy_timing_drain(cache, 0);
    *out = cache->st;
    out->copy_busy_ms = cache->copy_ms;
    out->copies_timed = cache->copies_timed;
    if (cache->cp_err != hipSuccess) {
        const hipError_t e = cache->cp_err;
        cache->cp_err = hipSuccess;
        return hip_fail(e, "copy timing events");
    }
    return MOE_OK;
}

extern "C" void moe_cache_reset_stats(moe_cache *cache)
{
    if (!cache)
        return;
    copy_timing_drain(cache, 0);
    cache->copy_ms = 0.0;
    cache->copies_timed = 0;
    cache->cp_err = hipSuccess;
    const int64_t n = cache->st.n_slots, pinned = cache->st.pinned;
    cache->st = moe_cache_stats{};
    cache->st.n_slots = n;
    cache->st.pinned = pinned;
}

extern "C" moe_status moe_cache_log_enable(moe_cache *cache, int32_t on)
{
    if (!cache)
        return fail(MOE_E_INVAL, "cache is NULL");
    cache->log_on = on != 0;
    if (!cache->log_on)
        cache->log.clear();
    return MOE_OK;
}

extern "C" int64_t moe_cache_event_log(const moe_cache *cache, moe_cache_event *out, int64_t cap)
{
    if (!cache || (!out && cap > 0))
        return -1;
    int64_t n = (int64_t)cache->log.size();
    if (n > cap)
        n = cap;
    for (int64_t i = 0; i < n; ++i)
        out[i] = cache->log[(size_t)i];
    return n;
}

extern "C" moe_status moe_cache_debug_fail_next_copy(moe_cache *cache)
{
    if (!cache)
        return fail(MOE_E_INVAL, "cache is NULL");
    cache->fail_next = true;
    return MOE_OK;
}

namespace moe {

// DEMAND stage for moe_layer_forward: the router's T*k ids are copied back to
// the host (this is the call's one host synchronisation), the distinct experts
// are staged in order of first appearance, and the layer's device table is
// returned.
moe_status cache_check_for_layer(const moe_cache *c, const moe_layer_desc &d, int layer, int T)
{
    if (!c)
        return fail(MOE_E_INVAL, "cache is NULL");
    if (c->d.backend != MOE_CACHE_BACKEND_HIP)
        return fail(MOE_E_INVAL, "moe_layer_forward needs a cache with the HIP backend");
    if (layer < 0 || layer >= c->d.n_layers)
        return fail(MOE_E_INVAL, "layer %d out of range [0,%d)", layer, c->d.n_layers);
    if (c->d.n_experts != d.n_experts)
        return fail(MOE_E_INVAL, "cache has %d experts per layer, layer has %d",
                    c->d.n_experts, d.n_experts);
    const size_t blob = blob_layout(d.hidden, d.ffn, d.group, d.wfmt).total;
    if (c->d.blob_bytes != blob)
        return fail(MOE_E_INVAL, "cache blob size %zu != layer blob size %zu", c->d.blob_bytes,
                    blob);
    if ((int64_t)T * d.top_k > c->ids_cap)
        return fail(MOE_E_INVAL, "T*k=%lld exceeds the cache's id buffer (%d)",
                    (long long)T * d.top_k, c->ids_cap);
    return MOE_OK;
}

moe_status cache_demand_for_layer(moe_cache *c, const moe_layer_desc &d, int layer,
                                  const int32_t *idx_dev, int T, hipStream_t compute,
                                  const void *const **table)
{
    moe_status st = cache_check_for_layer(c, d, layer, T);
    if (st)
        return st;
    const int n = T * d.top_k;
    hipError_t e = hipMemcpyAsync(c->ids_pinned, idx_dev, (size_t)n * 4, hipMemcpyDeviceToHost,
                                  compute);
    if (e == hipSuccess)
        e = hipStreamSynchronize(compute);
    if (e != hipSuccess)
        return hip_fail(e, "routing ids to host");
    std::vector<int32_t> uniq;
    std::vector<char> seen((size_t)d.n_experts, 0);
    for (int i = 0; i < n; ++i) {
        int32_t v = c->ids_pinned[i];
        if (v < 0 || v >= d.n_experts)
            return fail(MOE_E_INVAL, "router produced expert id %d", v);
        if (!seen[(size_t)v]) {
            seen[(size_t)v] = 1;
            uniq.push_back(v);
        }
    }
    st = stage_demand(c, layer, uniq.data(), (int)uniq.size(), compute, nullptr);
    if (st)
        return st;
    *table = moe_cache_table(c, layer);
    return MOE_OK;
}

}  // namespace moe
