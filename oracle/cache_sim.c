/*
 * cache_sim.c -- logical replay of the expert cache.
 * TEST INFRASTRUCTURE ONLY (see moe_oracle.h).
 *
 * Colibri keeps routed experts in an LRU cache and loads an expert only when
 * the router selects it ("Guide Complet de Colibri", section "Qu'est-ce que
 * Colibri ?"; openapps.pro listing, "Under The Hood": staging exactly when the
 * router proves the expert is needed).  A lookahead step prefetches the next
 * layer's predicted experts while the current layer computes (same guide,
 * section "Router-Lookahead prefetch").  Placement never changes results
 * (aifrontierpost tutorial, "Honest limitations").
 *
 * The state machine, independent of any timing:
 *  - a pool of slots, each empty or holding one (layer, expert) key;
 *  - DEMAND(layer, ids): ids in rank order; a resident key is a hit and is
 *    touched; a missing key takes the least-recently-used unlocked slot (never
 *    used slots first, ties to the lowest slot) and is resident at once;
 *    every slot the layer uses is locked until RELEASE(layer);
 *  - PREFETCH(next layer, ids): resident keys are touched; a missing key
 *    takes an unlocked LRU slot and is marked prefetched; with no unlocked
 *    slot the prefetch is skipped.  Prefetched slots are not locked;
 *  - a prefetched slot hit by a demand counts as used; evicted before any
 *    demand, as wasted.
 *
 * Learned pinned hot-store (Colibri records which experts a workload routes
 * to and pins the hottest ones: aifrontierpost tutorial, introduction and
 * "Step 4 -- Run it"; kongchang article, storage-tier section; openapps.pro
 * listing, "Under The Hood"):
 *  - every DEMAND access of a key adds one to its usage count (prefetches do
 *    not: they are guesses, not uses);
 *  - PIN(n), between steps (no slot locked): every pinned slot is unpinned
 *    (it stays resident); then the keys with a nonzero count, ranked by count
 *    descending and key (layer*E + expert) ascending, are taken in rank order
 *    until n are pinned: a resident key's slot is pinned as it is; a missing
 *    key takes the LRU unlocked, unpinned slot of its partition (as a demand
 *    miss would), is filled and pinned.  A partition never pins more than its
 *    size minus k slots, so a layer's demand always finds room; a key whose
 *    partition is full of pins is passed over;
 *  - a pinned slot is never a victim (demand, prefetch or pin).
 */
#include "moe_oracle.h"

#include <stdlib.h>

typedef struct {
    int32_t layer, expert;   /* -1 when empty */
    int64_t last_use;        /* -1 when never used */
    int32_t locked_by;       /* layer holding the lock, -1 if none */
    int32_t prefetched;
    int32_t pinned;
} slot_t;

typedef struct {
    slot_t *slot;
    int n_slots, L, E, k, per_layer;
    int64_t clock;
    orc_cache_event *ev;
    int64_t n_ev, ev_cap;
    int overflow;
    orc_cache_stats *st;
    int64_t *usage;          /* [L*E] demand accesses per key */
} sim_t;

static void emit(sim_t *s, int kind, int layer, int expert, int slot)
{
    if (s->n_ev >= s->ev_cap) {
        s->overflow = 1;
        return;
    }
    orc_cache_event *e = &s->ev[s->n_ev++];
    e->kind = kind;
    e->layer = layer;
    e->expert = expert;
    e->slot = slot;
}

static void part_range(const sim_t *s, int layer, int *lo, int *hi)
{
    if (!s->per_layer) {
        *lo = 0;
        *hi = s->n_slots;
    } else {
        *lo = (int)((int64_t)layer * s->n_slots / s->L);
        *hi = (int)((int64_t)(layer + 1) * s->n_slots / s->L);
    }
}

static int find_resident(const sim_t *s, int layer, int expert)
{
    for (int i = 0; i < s->n_slots; ++i)
        if (s->slot[i].layer == layer && s->slot[i].expert == expert)
            return i;
    return -1;
}

static int find_victim(const sim_t *s, int layer)
{
    int lo, hi, best = -1;
    part_range(s, layer, &lo, &hi);
    for (int i = lo; i < hi; ++i) {
        if (s->slot[i].locked_by >= 0 || s->slot[i].pinned)
            continue;
        if (best < 0 || s->slot[i].last_use < s->slot[best].last_use)
            best = i;
    }
    return best;
}

static void evict(sim_t *s, int i)
{
    slot_t *sl = &s->slot[i];
    if (sl->layer < 0)
        return;
    emit(s, ORC_EV_EVICT, sl->layer, sl->expert, i);
    s->st->evictions++;
    if (sl->prefetched)
        s->st->prefetch_wasted++;
    sl->layer = sl->expert = -1;
    sl->prefetched = 0;
}

static int demand(sim_t *s, int layer, const int32_t *ids, int k)
{
    for (int j = 0; j < k; ++j) {
        int e = ids[j];
        s->usage[(size_t)layer * s->E + e] += 1;
        int i = find_resident(s, layer, e);
        if (i >= 0) {
            emit(s, ORC_EV_HIT, layer, e, i);
            s->st->demand_hits++;
            if (s->slot[i].prefetched) {
                s->st->prefetch_used++;
                s->slot[i].prefetched = 0;
            }
        } else {
            i = find_victim(s, layer);
            if (i < 0)
                return -1;
            evict(s, i);
            s->slot[i].layer = layer;
            s->slot[i].expert = e;
            emit(s, ORC_EV_MISS, layer, e, i);
            s->st->demand_misses++;
        }
        s->slot[i].last_use = ++s->clock;
        s->slot[i].locked_by = layer;
    }
    return 0;
}

static void prefetch(sim_t *s, int layer, const int32_t *ids, int k)
{
    for (int j = 0; j < k; ++j) {
        int e = ids[j];
        int i = find_resident(s, layer, e);
        if (i >= 0) {
            emit(s, ORC_EV_PF_HIT, layer, e, i);
            s->st->prefetch_resident++;
            s->slot[i].last_use = ++s->clock;
            continue;
        }
        i = find_victim(s, layer);
        if (i < 0) {
            emit(s, ORC_EV_PF_SKIP, layer, e, -1);
            s->st->prefetch_skipped++;
            continue;
        }
        evict(s, i);
        s->slot[i].layer = layer;
        s->slot[i].expert = e;
        s->slot[i].prefetched = 1;
        s->slot[i].last_use = ++s->clock;
        emit(s, ORC_EV_PF_ISSUE, layer, e, i);
        s->st->prefetch_issued++;
    }
}

static void release(sim_t *s, int layer)
{
    for (int i = 0; i < s->n_slots; ++i)
        if (s->slot[i].locked_by == layer)
            s->slot[i].locked_by = -1;
}

/* PIN(n): unpin everything, then pin the n hottest keys (see the header). */
static void pin_hot(sim_t *s, int n)
{
    const int nk = s->L * s->E;
    for (int i = 0; i < s->n_slots; ++i)
        s->slot[i].pinned = 0;
    s->st->pinned = 0;
    char *taken = (char *)calloc((size_t)nk, 1);
    for (int r = 0; r < n; ++r) {
        /* the next key in rank order: largest count, then lowest key */
        int best = -1;
        for (int key = 0; key < nk; ++key) {
            if (taken[key] || s->usage[key] <= 0)
                continue;
            if (best < 0 || s->usage[key] > s->usage[best])
                best = key;
        }
        if (best < 0)
            break;
        taken[best] = 1;
        const int layer = best / s->E, e = best % s->E;
        int lo, hi, n_part_pinned = 0;
        part_range(s, layer, &lo, &hi);
        for (int i = lo; i < hi; ++i)
            n_part_pinned += s->slot[i].pinned;
        if (n_part_pinned >= (hi - lo) - s->k) {
            --r;                        /* passed over: its partition is full */
            continue;
        }
        int i = find_resident(s, layer, e);
        if (i >= 0) {
            emit(s, ORC_EV_PIN_KEEP, layer, e, i);
        } else {
            i = find_victim(s, layer);
            evict(s, i);
            s->slot[i].layer = layer;
            s->slot[i].expert = e;
            s->slot[i].last_use = ++s->clock;
            emit(s, ORC_EV_PIN_FILL, layer, e, i);
            s->st->pin_fills++;
        }
        s->slot[i].pinned = 1;
        s->st->pinned++;
    }
    free(taken);
}

int64_t orc_cache_sim_hot(int L, int E, int k, int n_slots, int n_steps,
                          const int32_t *dem, const int32_t *pred, int wrap,
                          int per_layer, const int64_t *usage_init,
                          const int32_t *pin_before, orc_cache_event *ev, int64_t ev_cap,
                          orc_cache_stats *st, int64_t *usage_out)
{
    sim_t s;
    s.slot = (slot_t *)malloc(sizeof(slot_t) * (size_t)(n_slots > 0 ? n_slots : 1));
    s.usage = (int64_t *)calloc((size_t)L * (size_t)E, sizeof(int64_t));
    s.n_slots = n_slots;
    s.L = L;
    s.E = E;
    s.k = k;
    s.per_layer = per_layer;
    s.clock = 0;
    s.ev = ev;
    s.n_ev = 0;
    s.ev_cap = ev_cap;
    s.overflow = 0;
    s.st = st;
    st->demand_hits = st->demand_misses = 0;
    st->prefetch_issued = st->prefetch_used = st->prefetch_wasted = 0;
    st->prefetch_skipped = st->prefetch_resident = st->evictions = 0;
    st->pinned = st->pin_fills = 0;
    for (int i = 0; i < n_slots; ++i) {
        s.slot[i].layer = s.slot[i].expert = -1;
        s.slot[i].last_use = -1;
        s.slot[i].locked_by = -1;
        s.slot[i].prefetched = 0;
        s.slot[i].pinned = 0;
    }
    if (usage_init)
        for (int i = 0; i < L * E; ++i)
            s.usage[i] = usage_init[i];
    int64_t rc = 0;
    for (int t = 0; t < n_steps && rc == 0; ++t) {
        if (pin_before && pin_before[t] >= 0)
            pin_hot(&s, pin_before[t]);
        for (int l = 0; l < L; ++l) {
            const int32_t *ids = dem + ((size_t)t * L + l) * k;
            if (demand(&s, l, ids, k) != 0) {
                rc = -1;
                break;
            }
            if (pred) {
                int nl = l + 1;
                int ok = 1;
                if (nl == L) {
                    nl = 0;
                    ok = wrap && (t + 1 < n_steps);
                }
                if (ok)
                    prefetch(&s, nl, pred + ((size_t)t * L + l) * k, k);
            }
            release(&s, l);
        }
    }
    if (usage_out)
        for (int i = 0; i < L * E; ++i)
            usage_out[i] = s.usage[i];
    free(s.slot);
    free(s.usage);
    if (rc != 0 || s.overflow)
        return -1;
    return s.n_ev;
}

int64_t orc_cache_sim(int L, int E, int k, int n_slots, int n_steps,
                      const int32_t *dem, const int32_t *pred, int wrap,
                      int per_layer, orc_cache_event *ev, int64_t ev_cap,
                      orc_cache_stats *st)
{
    return orc_cache_sim_hot(L, E, k, n_slots, n_steps, dem, pred, wrap, per_layer, NULL, NULL,
                             ev, ev_cap, st, NULL);
}
