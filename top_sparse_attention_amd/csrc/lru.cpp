// Tiered KV: the host half of the HBM page cache with LRU eviction over pinned host memory.
//
// GLM5.3 sparse-attention page ("Cơ chế chú ý thưa (Sparse Attention) trên GLM5.3 ...",
// HiSparse paragraph): pages live in host DRAM, HBM holds an LRU cache of them, a top-k
// selection that misses loads from DRAM and evicts the least recently used page, and the
// loads for one layer overlap the computation of the previous one.  The policy details the
// page leaves open are fixed in tsa.h (touch order, lowest free slot first, pins per tag).
//
// The cache unit is one page of the cache pool: a pool with pages of P tokens caches whole
// pages, a pool with pages of one token caches single token rows (the page's HiSparse loads
// tokens; whole pages are the plainer reading of its LRU sentence, both are supported).
//
// Bookkeeping: slot_of[key] (-1 = absent), key_of[slot], last touch time per slot, pin count
// per slot, and the evictable slots (resident, unpinned) in a doubly linked list ordered by
// last touch, oldest first.  A touch moves a slot to the newest end; a release puts the slots
// back in touch order, which for releases in plan order means at the newest end; so touches,
// pins, releases and evictions cost O(1) in the usual order of calls.
#include <algorithm>
#include <cstring>
#include <new>
#include <stdexcept>
#include <unordered_map>
#include <vector>

#include "tsa_internal.h"

using tsa::fail;

struct tsa_lru {
    tsa_kv_pool* cache = nullptr;
    int32_t num_layers = 0, num_req = 0, pages_per_req = 0;
    int64_t num_keys = 0;
    int32_t capacity = 0;
    size_t page_bytes = 0;                 // one page of K (and of V)
    const unsigned char* host_k = nullptr;  // device-visible addresses of the host copy
    const unsigned char* host_v = nullptr;

    // per-slot state in separate arrays: the list links and pin counts that every touch walks
    // stay small (4 bytes a slot) and cache-friendly even with millions of token slots
    std::vector<int32_t> slot_of;          // per key
    std::vector<int64_t> key_of;           // per slot, -1 = free
    std::vector<uint64_t> touched_at;      // per slot
    std::vector<int32_t> pins;             // per slot
    std::vector<int32_t> free_slots;       // popped from the back: lowest slot first
    // evictable slots, oldest touch first: a list threaded through prev / next (-1 = none)
    std::vector<int32_t> prev, next;
    int32_t head = -1, tail = -1;
    int64_t n_evictable = 0;
    std::unordered_map<int64_t, std::vector<int32_t>> held;   // tag -> pinned slots
    // caller events of released tags: the next fetch's copies may reuse those tags' slots, so
    // they wait for these first
    std::vector<hipEvent_t> wait_events;
    uint64_t clock = 0;
    int64_t hits = 0, misses = 0, evictions = 0, h2d_bytes = 0;

    std::vector<int64_t> pending_key;      // per slot: key whose copy is still to be fetched, -1 none
    std::vector<int32_t> pending_slots;    // slots with a pending copy, in placement order
    // the last plan's table entries (flat index r * pages_per_req + page, slot): what a fetch
    // writes into the device table
    std::vector<int64_t> plan_index;
    std::vector<int32_t> plan_slot;

    // pinned staging for the device transfers, two sets used alternately
    struct Stage {
        void* buf = nullptr;
        size_t bytes = 0;
        hipEvent_t done = nullptr;
        bool used = false;
    } stage[2];
    int next_stage = 0;

    ~tsa_lru() {
        for (auto& st : stage) {
            if (st.done) {
                if (st.used) (void)hipEventSynchronize(st.done);
                (void)hipEventDestroy(st.done);
            }
            if (st.buf) (void)hipHostFree(st.buf);
        }
    }

    void unlink(int32_t slot) {
        const int32_t p = prev[size_t(slot)], n = next[size_t(slot)];
        if (p >= 0) next[size_t(p)] = n; else head = n;
        if (n >= 0) prev[size_t(n)] = p; else tail = p;
        prev[size_t(slot)] = next[size_t(slot)] = -1;
        --n_evictable;
    }
    // insert by touch time, searching from the newest end (O(1) when it is the newest)
    void link(int32_t slot) {
        int32_t after = tail;
        while (after >= 0 && touched_at[size_t(after)] > touched_at[size_t(slot)]) after = prev[size_t(after)];
        const int32_t before = after >= 0 ? next[size_t(after)] : head;
        prev[size_t(slot)] = after;
        next[size_t(slot)] = before;
        if (after >= 0) next[size_t(after)] = slot; else head = slot;
        if (before >= 0) prev[size_t(before)] = slot; else tail = slot;
        ++n_evictable;
    }
    void make_recent(int32_t slot) {
        if (pins[slot] == 0) unlink(slot);
        touched_at[slot] = ++clock;
        if (pins[slot] == 0) link(slot);
    }
    void pin(int32_t slot) {
        if (pins[slot]++ == 0) unlink(slot);
    }
    // a plan's touch of a resident slot: most recent and pinned, in one list operation
    void touch_pin(int32_t slot) {
        if (pins[slot]++ == 0) unlink(slot);
        touched_at[slot] = ++clock;
    }
    void unpin(int32_t slot) {
        if (--pins[slot] == 0) link(slot);
    }
    // a slot for `key`, which is absent; queues its copy.  With `pinned` the slot starts pinned
    // (once) instead of evictable.
    int32_t place(int64_t key, bool count, bool pinned = false) {
        int32_t slot;
        if (!free_slots.empty()) {
            slot = free_slots.back();
            free_slots.pop_back();
        } else {
            if (head < 0) throw std::logic_error("no slot to evict");
            slot = head;
            unlink(slot);
            slot_of[size_t(key_of[slot])] = -1;
            if (count) ++evictions;
        }
        key_of[slot] = key;
        slot_of[size_t(key)] = slot;
        touched_at[slot] = ++clock;
        if (pinned) pins[slot] = 1;
        else link(slot);
        if (pending_key[size_t(slot)] < 0) pending_slots.push_back(slot);
        pending_key[size_t(slot)] = key;      // a later placement in the same slot replaces it
        return slot;
    }
};

namespace tsa {

hipError_t launch_lru_copy(const tsa_lru& lru, const int64_t* keys_dev, const int32_t* slots_dev,
                           int64_t n, const int64_t* tab_index_dev, const int32_t* tab_slot_dev,
                           int64_t n_tab, int32_t* table_dev, hipStream_t s);

const unsigned char* lru_host_k(const tsa_lru& l) { return l.host_k; }
const unsigned char* lru_host_v(const tsa_lru& l) { return l.host_v; }
size_t lru_page_bytes(const tsa_lru& l) { return l.page_bytes; }
const tsa_kv_pool& lru_cache(const tsa_lru& l) { return *l.cache; }

}  // namespace tsa

#define TSA_GUARD_BEGIN try {
#define TSA_GUARD_END                                                   \
    }                                                                   \
    catch (const std::bad_alloc&) {                                     \
        return fail(TSA_ERR_CAPACITY, "host allocation failed");        \
    }                                                                   \
    catch (...) {                                                       \
        return fail(TSA_ERR_INVALID, "unexpected host exception");      \
    }

namespace {

// Bytes of the device workspace: the keys (int64) and slots (int32) of up to `cap` copies, then
// the flat indices (int64) and slots (int32) of up to `cap` table entries (a plan pins distinct
// slots, so it sets at most `cap` entries); 256-byte aligned parts.
size_t ws_keys_bytes(int64_t cap) { return tsa::align_up(size_t(cap) * 8, 256); }
size_t ws_slots_bytes(int64_t cap) { return tsa::align_up(size_t(cap) * 4, 256); }
size_t ws_bytes_total(int64_t cap) { return 2 * (ws_keys_bytes(cap) + ws_slots_bytes(cap)); }

}  // namespace

extern "C" {

tsa_status tsa_lru_create(tsa_kv_pool* cache, int32_t num_layers, int32_t num_req,
                          int32_t pages_per_req, const void* host_k, const void* host_v,
                          tsa_lru** out) {
    TSA_GUARD_BEGIN
    if (!cache || !out) return fail(TSA_ERR_INVALID, "null argument");
    *out = nullptr;
    const tsa_pool_desc& d = cache->d;
    // a metadata-only cache pool (no device regions) gives a bookkeeping-only tier: plans,
    // releases and counters work, fetches are refused
    const bool meta = !cache->k && !cache->v;
    if (d.v_from_k || d.index_dim != 0 || d.num_layers != 1 || (!meta && (!cache->k || !cache->v)))
        return fail(TSA_ERR_INVALID, "the cache must be a one-layer pool with K and V regions and no indexer");
    if (!meta && (!host_k || !host_v)) return fail(TSA_ERR_INVALID, "null host copy");
    if (num_layers <= 0 || num_req <= 0 || pages_per_req <= 0)
        return fail(TSA_ERR_INVALID, "num_layers, num_req and pages_per_req must be positive");
    const int64_t keys = int64_t(num_layers) * num_req * pages_per_req;
    if (keys >= (int64_t(1) << 40)) return fail(TSA_ERR_INVALID, "too many logical pages");
    if (d.head_dim_k != d.head_dim_v)
        return fail(TSA_ERR_UNSUPPORTED, "the tier copies K and V pages of the same size");
    auto l = new tsa_lru();
    l->cache = cache;
    l->num_layers = num_layers;
    l->num_req = num_req;
    l->pages_per_req = pages_per_req;
    l->num_keys = keys;
    l->capacity = d.num_pages;
    l->page_bytes = size_t(d.page_size) * d.num_kv_heads * d.head_dim_k * 2;
    void* dk = nullptr;
    void* dv = nullptr;
    hipError_t e = hipSuccess;
    if (!meta) e = hipHostGetDevicePointer(&dk, const_cast<void*>(host_k), 0);
    if (!meta && e == hipSuccess) e = hipHostGetDevicePointer(&dv, const_cast<void*>(host_v), 0);
    if (e != hipSuccess) {
        delete l;
        return fail(TSA_ERR_INVALID, std::string("host_k / host_v must be pinned host memory mapped for the "
                                                 "device: ") + hipGetErrorString(e));
    }
    l->host_k = static_cast<const unsigned char*>(dk);
    l->host_v = static_cast<const unsigned char*>(dv);
    l->slot_of.assign(size_t(keys), -1);
    l->key_of.assign(size_t(l->capacity), -1);
    l->touched_at.assign(size_t(l->capacity), 0);
    l->pins.assign(size_t(l->capacity), 0);
    l->pending_key.assign(size_t(l->capacity), -1);
    l->prev.assign(size_t(l->capacity), -1);
    l->next.assign(size_t(l->capacity), -1);
    l->free_slots.resize(size_t(l->capacity));
    for (int32_t i = 0; i < l->capacity; ++i) l->free_slots[size_t(i)] = l->capacity - 1 - i;
    *out = l;
    return TSA_OK;
    TSA_GUARD_END
}

tsa_status tsa_lru_destroy(tsa_lru* lru) {
    delete lru;
    return TSA_OK;
}

tsa_status tsa_lru_preload(tsa_lru* l, int64_t n, const int64_t* keys) {
    TSA_GUARD_BEGIN
    if (!l || (n > 0 && !keys) || n < 0) return fail(TSA_ERR_INVALID, "bad arguments");
    int64_t fresh = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (keys[i] < 0 || keys[i] >= l->num_keys) return fail(TSA_ERR_INVALID, "key out of range");
        if (l->slot_of[size_t(keys[i])] < 0) ++fresh;
    }
    if (fresh > int64_t(l->free_slots.size()) + l->n_evictable)
        return fail(TSA_ERR_CAPACITY, "preload exceeds the cache");
    for (int64_t i = 0; i < n; ++i) {
        const int64_t key = keys[i];
        const int32_t slot = l->slot_of[size_t(key)];
        if (slot >= 0) l->make_recent(slot);
        else l->place(key, false);
    }
    return TSA_OK;
    TSA_GUARD_END
}

tsa_status tsa_lru_plan(tsa_lru* l, int32_t layer, int64_t tag, int32_t n_req,
                        const int32_t* positions, int32_t k, int32_t* slot_table,
                        int64_t* n_fetch) {
    TSA_GUARD_BEGIN
    if (!l || (n_req > 0 && k > 0 && !positions)) return fail(TSA_ERR_INVALID, "null argument");
    if (layer < 0 || layer >= l->num_layers) return fail(TSA_ERR_INVALID, "layer out of range");
    if (n_req < 0 || n_req > l->num_req || k < 0) return fail(TSA_ERR_INVALID, "bad n_req or k");
    if (l->held.count(tag)) return fail(TSA_ERR_INVALID, "tag still held");
    const int32_t P = l->cache->d.page_size;
    const int32_t npr = l->pages_per_req;
    // distinct pages per request, ascending (touch order); positions that come sorted (a top-k
    // list is) skip the sort
    std::vector<int32_t> pages;
    pages.reserve(size_t(n_req) * size_t(k));
    std::vector<int32_t> first(size_t(n_req) + 1, 0);
    for (int32_t r = 0; r < n_req; ++r) {
        const int32_t* pos = positions + size_t(r) * k;
        const size_t start = pages.size();
        bool ordered = true;    // strictly increasing pages so far: already distinct and sorted
        for (int32_t j = 0; j < k; ++j) {
            const int32_t t = pos[j];
            if (t < 0 || t / P >= npr) continue;
            const int32_t pg = t / P;
            if (pages.size() > start) {
                if (pg == pages.back()) continue;      // same page as the last: one touch
                if (pg < pages.back()) ordered = false;
            }
            pages.push_back(pg);
        }
        if (!ordered) {
            std::sort(pages.begin() + std::ptrdiff_t(start), pages.end());
            pages.erase(std::unique(pages.begin() + std::ptrdiff_t(start), pages.end()), pages.end());
        }
        first[size_t(r) + 1] = int32_t(pages.size());
    }
    auto key_at = [&](int32_t r, int32_t page) {
        return (int64_t(layer) * l->num_req + r) * npr + page;
    };
    // capacity check before any change: misses must fit in free slots plus pages that are
    // evictable now and not touched (touching pins them).  Misses plus touched evictable pages
    // never exceed the touches, so when the free and evictable slots cover every touch the
    // count is not needed.
    const int64_t room = int64_t(l->free_slots.size()) + l->n_evictable;
    if (room < int64_t(pages.size())) {
        int64_t miss = 0, touched_evictable = 0;
        for (int32_t r = 0; r < n_req; ++r)
            for (int32_t i = first[size_t(r)]; i < first[size_t(r) + 1]; ++i) {
                const int32_t slot = l->slot_of[size_t(key_at(r, pages[size_t(i)]))];
                if (slot < 0) ++miss;
                else if (l->pins[size_t(slot)] == 0) ++touched_evictable;
            }
        if (miss > room - touched_evictable)
            return fail(TSA_ERR_CAPACITY, "the plan's misses exceed the free and unpinned slots");
    }

    if (slot_table) std::fill(slot_table, slot_table + size_t(n_req) * npr, -1);
    std::vector<int32_t>& hold = l->held[tag];
    hold.reserve(pages.size());
    l->plan_index.clear();
    l->plan_slot.clear();
    l->plan_index.reserve(pages.size());
    l->plan_slot.reserve(pages.size());
    // The touches walk a table of millions of keys and slots in random order, so each one would
    // wait on several cache misses in turn; the loop prefetches the key's slot a few touches
    // ahead, and that slot's recency and link entries a little later.
    std::vector<int64_t> tkey(pages.size());
    for (int32_t r = 0; r < n_req; ++r)
        for (int32_t i = first[size_t(r)]; i < first[size_t(r) + 1]; ++i)
            tkey[size_t(i)] = key_at(r, pages[size_t(i)]);
    constexpr size_t kAheadKey = 16, kAheadSlot = 8;
    const size_t n_touch = tkey.size();
    for (int32_t r = 0; r < n_req; ++r)
        for (int32_t i = first[size_t(r)]; i < first[size_t(r) + 1]; ++i) {
            const size_t q = size_t(i);
            if (q + kAheadKey < n_touch) __builtin_prefetch(&l->slot_of[size_t(tkey[q + kAheadKey])]);
            if (q + kAheadSlot < n_touch) {
                const int32_t s2 = l->slot_of[size_t(tkey[q + kAheadSlot])];
                if (s2 >= 0) {
                    __builtin_prefetch(&l->pins[size_t(s2)], 1);
                    __builtin_prefetch(&l->prev[size_t(s2)], 1);
                    __builtin_prefetch(&l->next[size_t(s2)], 1);
                    __builtin_prefetch(&l->touched_at[size_t(s2)], 1);
                }
            }
            const int32_t page = pages[q];
            const int64_t key = tkey[q];
            int32_t slot = l->slot_of[size_t(key)];
            if (slot >= 0) {
                ++l->hits;
                l->touch_pin(slot);
            } else {
                ++l->misses;
                slot = l->place(key, true, true);
            }
            hold.push_back(slot);
            if (slot_table) slot_table[size_t(r) * npr + page] = slot;
            l->plan_index.push_back(int64_t(r) * npr + page);
            l->plan_slot.push_back(slot);
        }
    if (n_fetch) *n_fetch = int64_t(l->pending_slots.size());
    return TSA_OK;
    TSA_GUARD_END
}

tsa_status tsa_lru_release(tsa_lru* l, int64_t tag) {
    TSA_GUARD_BEGIN
    if (!l) return fail(TSA_ERR_INVALID, "null argument");
    auto it = l->held.find(tag);
    if (it == l->held.end()) return fail(TSA_ERR_INVALID, "tag not held");
    const std::vector<int32_t>& hold = it->second;
    for (size_t i = 0; i < hold.size(); ++i) {
        if (i + 8 < hold.size()) {      // random slots: fetch their entries ahead of the unpin
            const size_t s2 = size_t(hold[i + 8]);
            __builtin_prefetch(&l->pins[s2], 1);
            __builtin_prefetch(&l->prev[s2], 1);
            __builtin_prefetch(&l->next[s2], 1);
            __builtin_prefetch(&l->touched_at[s2], 0);
        }
        l->unpin(hold[i]);
    }
    l->held.erase(it);
    return TSA_OK;
    TSA_GUARD_END
}

tsa_status tsa_lru_release_layer(tsa_lru* l, int64_t tag, void* done_event) {
    TSA_GUARD_BEGIN
    if (!l) return fail(TSA_ERR_INVALID, "null argument");
    if (!l->held.count(tag)) return fail(TSA_ERR_INVALID, "tag not held");
    hipEvent_t ev = static_cast<hipEvent_t>(done_event);
    if (ev && std::find(l->wait_events.begin(), l->wait_events.end(), ev) == l->wait_events.end())
        l->wait_events.push_back(ev);
    return tsa_lru_release(l, tag);
    TSA_GUARD_END
}

tsa_status tsa_lru_workspace_bytes(const tsa_lru* l, int32_t n_req, size_t* bytes) {
    if (!l || !bytes || n_req < 0) return fail(TSA_ERR_INVALID, "bad arguments");
    // a fetch carries at most the cache's capacity of copies and of table entries
    *bytes = ws_bytes_total(l->capacity);
    (void)n_req;
    return TSA_OK;
}

namespace {

// Argument checks of a fetch that do not depend on the plan (no side effects).
tsa_status fetch_args_ok(const tsa_lru* l, int32_t n_req, const int32_t* slot_table_dev,
                         const void* workspace, size_t ws_bytes) {
    if (!l || (n_req > 0 && !slot_table_dev) || n_req < 0 || n_req > l->num_req)
        return fail(TSA_ERR_INVALID, "bad arguments");
    if (!l->host_k) return fail(TSA_ERR_INVALID, "a bookkeeping-only tier cannot fetch");
    if (workspace && ws_bytes < ws_bytes_total(l->capacity)) return fail(TSA_ERR_CAPACITY, "workspace too small");
    return TSA_OK;
}

}  // namespace

tsa_status tsa_lru_fetch(tsa_lru* l, int32_t n_req, const int32_t* slot_table,
                         int32_t* slot_table_dev, void* workspace, size_t ws_bytes, void* stream) {
    TSA_GUARD_BEGIN
    (void)slot_table;   // the entries come from the plan itself
    tsa_status chk = fetch_args_ok(l, n_req, slot_table_dev, workspace, ws_bytes);
    if (chk) return chk;
    const int64_t n = int64_t(l->pending_slots.size());
    const int64_t n_tab = int64_t(l->plan_index.size());
    if ((n > 0 || n_tab > 0) && !workspace) return fail(TSA_ERR_INVALID, "workspace required");
    if (n > l->capacity || n_tab > l->capacity) return fail(TSA_ERR_INVALID, "more pending copies than slots");
    for (int64_t i = 0; i < n_tab; ++i)
        if (l->plan_index[size_t(i)] >= int64_t(n_req) * l->pages_per_req)
            return fail(TSA_ERR_INVALID, "the last plan covered more requests than n_req");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t stage_bytes = size_t(n + n_tab) * 12 + 256;
    tsa_lru::Stage& st = l->stage[l->next_stage];
    l->next_stage ^= 1;
    // the staging set is reused two fetches later; its previous transfer must be done
    if (st.used) {
        tsa_status e = tsa::hip_check(hipEventSynchronize(st.done), "hipEventSynchronize");
        if (e != TSA_OK) return e;
        st.used = false;
    }
    if (st.bytes < stage_bytes) {
        if (st.buf) (void)hipHostFree(st.buf);
        st.buf = nullptr;
        st.bytes = 0;
        tsa_status e = tsa::hip_check(hipHostMalloc(&st.buf, stage_bytes, hipHostMallocDefault),
                                      "hipHostMalloc");
        if (e != TSA_OK) return e;
        st.bytes = stage_bytes;
    }
    if (!st.done) {
        tsa_status e = tsa::hip_check(hipEventCreateWithFlags(&st.done, hipEventDisableTiming),
                                      "hipEventCreate");
        if (e != TSA_OK) return e;
    }
    // staging: copy keys (int64) and table indices (int64), then copy slots and table slots
    // (int32); one host-to-device transfer, then one kernel scatters the table entries and
    // copies the pages
    unsigned char* hb = static_cast<unsigned char*>(st.buf);
    int64_t* hkeys = reinterpret_cast<int64_t*>(hb);
    int64_t* hidx = hkeys + n;
    int32_t* hslots = reinterpret_cast<int32_t*>(hidx + n_tab);
    int32_t* htab = hslots + n;
    for (int64_t i = 0; i < n; ++i) {
        const int32_t slot = l->pending_slots[size_t(i)];
        hkeys[i] = l->pending_key[size_t(slot)];
        hslots[i] = slot;
    }
    if (n_tab) {
        std::memcpy(hidx, l->plan_index.data(), size_t(n_tab) * 8);
        std::memcpy(htab, l->plan_slot.data(), size_t(n_tab) * 4);
    }
    tsa_status e = TSA_OK;
    // copies may land in slots of tags released with an event: wait for those first
    for (hipEvent_t ev : l->wait_events)
        if (e == TSA_OK) e = tsa::hip_check(hipStreamWaitEvent(s, ev, 0), "hipStreamWaitEvent");
    if (e != TSA_OK) return e;
    l->wait_events.clear();
    if (n + n_tab > 0) {
        unsigned char* w = static_cast<unsigned char*>(workspace);
        int64_t* dkeys = reinterpret_cast<int64_t*>(w);
        int64_t* didx = dkeys + n;
        int32_t* dslots = reinterpret_cast<int32_t*>(didx + n_tab);
        int32_t* dtab = dslots + n;
        e = tsa::hip_check(hipMemcpyAsync(w, hb, size_t(n + n_tab) * 12, hipMemcpyHostToDevice, s),
                           "hipMemcpyAsync");
        if (e == TSA_OK)
            e = tsa::hip_check(tsa::launch_lru_copy(*l, dkeys, dslots, n, didx, dtab, n_tab, slot_table_dev, s),
                               "lru copy launch");
    }
    if (e == TSA_OK) e = tsa::hip_check(hipEventRecord(st.done, s), "hipEventRecord");
    if (e != TSA_OK) return e;
    st.used = true;
    l->h2d_bytes += n * int64_t(2 * l->page_bytes);
    for (int32_t slot : l->pending_slots) l->pending_key[size_t(slot)] = -1;
    l->pending_slots.clear();
    l->plan_index.clear();
    l->plan_slot.clear();
    return TSA_OK;
    TSA_GUARD_END
}

tsa_status tsa_lru_prefetch(tsa_lru* l, int32_t layer, int64_t tag, int32_t n_req,
                            const int32_t* positions, int32_t k, int32_t* slot_table_dev,
                            void* workspace, size_t ws_bytes, void* stream, void* fetched_event) {
    TSA_GUARD_BEGIN
    tsa_status st = fetch_args_ok(l, n_req, slot_table_dev, workspace, ws_bytes);
    if (st) return st;
    if (!workspace) return fail(TSA_ERR_INVALID, "workspace required");
    if ((st = tsa_lru_plan(l, layer, tag, n_req, positions, k, nullptr, nullptr))) return st;
    if ((st = tsa_lru_fetch(l, n_req, nullptr, slot_table_dev, workspace, ws_bytes, stream))) return st;
    if (fetched_event)
        return tsa::hip_check(hipEventRecord(static_cast<hipEvent_t>(fetched_event), static_cast<hipStream_t>(stream)),
                              "hipEventRecord");
    return TSA_OK;
    TSA_GUARD_END
}

tsa_status tsa_lru_stats(const tsa_lru* l, int64_t* hits, int64_t* misses, int64_t* evictions,
                         int64_t* h2d_bytes) {
    if (!l) return fail(TSA_ERR_INVALID, "null argument");
    if (hits) *hits = l->hits;
    if (misses) *misses = l->misses;
    if (evictions) *evictions = l->evictions;
    if (h2d_bytes) *h2d_bytes = l->h2d_bytes;
    return TSA_OK;
}

}  // extern "C"
