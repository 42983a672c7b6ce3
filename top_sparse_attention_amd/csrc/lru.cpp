// Tiered KV: the host half of the HBM page cache with LRU eviction over pinned host memory.
//
// GLM5.3 sparse-attention page ("Cơ chế chú ý thưa (Sparse Attention) trên GLM5.3 ...",
// HiSparse paragraph): pages live in host DRAM, HBM holds an LRU cache of them, a top-k
// selection that misses loads from DRAM and evicts the least recently used page, and the
// loads for one layer overlap the computation of the previous one.  The policy details the
// page leaves open are fixed in tsa.h (touch order, lowest free slot first, pins per tag).
//
// Bookkeeping: slot_of[key] (-1 = absent), key_of[slot], last touch time per slot, pin count
// per slot, and the evictable slots (resident, unpinned) ordered by last touch in a balanced
// tree, so that each touch, pin, release and eviction costs O(log slots).
#include <algorithm>
#include <cstring>
#include <new>
#include <set>
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

    std::vector<int32_t> slot_of;          // per key
    std::vector<int64_t> key_of;           // per slot, -1 = free
    std::vector<uint64_t> touched_at;      // per slot
    std::vector<int32_t> pins;             // per slot
    std::vector<int32_t> free_slots;       // popped from the back: lowest slot first
    std::set<std::pair<uint64_t, int32_t>> evictable;
    std::unordered_map<int64_t, std::vector<int32_t>> held;   // tag -> pinned slots
    uint64_t clock = 0;
    int64_t hits = 0, misses = 0, evictions = 0, h2d_bytes = 0;

    std::vector<int64_t> pending_key;      // per slot: key whose copy is still to be fetched, -1 none
    std::vector<int32_t> pending_slots;    // slots with a pending copy, in placement order

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

    void make_recent(int32_t slot) {
        if (pins[slot] == 0) evictable.erase({touched_at[slot], slot});
        touched_at[slot] = ++clock;
        if (pins[slot] == 0) evictable.insert({touched_at[slot], slot});
    }
    void pin(int32_t slot) {
        if (pins[slot]++ == 0) evictable.erase({touched_at[slot], slot});
    }
    void unpin(int32_t slot) {
        if (--pins[slot] == 0) evictable.insert({touched_at[slot], slot});
    }
    // a slot for `key`, which is absent; queues its copy
    int32_t place(int64_t key, bool count) {
        int32_t slot;
        if (!free_slots.empty()) {
            slot = free_slots.back();
            free_slots.pop_back();
        } else {
            if (evictable.empty()) throw std::logic_error("no slot to evict");
            const auto victim = *evictable.begin();
            evictable.erase(evictable.begin());
            slot = victim.second;
            slot_of[size_t(key_of[slot])] = -1;
            if (count) ++evictions;
        }
        key_of[slot] = key;
        slot_of[size_t(key)] = slot;
        touched_at[slot] = ++clock;
        evictable.insert({touched_at[slot], slot});   // unpinned until the caller pins it
        if (pending_key[size_t(slot)] < 0) pending_slots.push_back(slot);
        pending_key[size_t(slot)] = key;      // a later placement in the same slot replaces it
        return slot;
    }
};

namespace tsa {

hipError_t launch_lru_copy(const tsa_lru& lru, const int64_t* keys_dev, const int32_t* slots_dev,
                           int64_t n, hipStream_t s);

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

// Bytes of the device workspace: the keys (int64) and slots (int32) of up to max_copies
// copies, 256-byte aligned parts.
size_t ws_keys_bytes(int64_t max_copies) { return tsa::align_up(size_t(max_copies) * 8, 256); }
size_t ws_slots_bytes(int64_t max_copies) { return tsa::align_up(size_t(max_copies) * 4, 256); }

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
    if (fresh > int64_t(l->free_slots.size()) + int64_t(l->evictable.size()))
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
    if (!l || !slot_table || (n_req > 0 && k > 0 && !positions))
        return fail(TSA_ERR_INVALID, "null argument");
    if (layer < 0 || layer >= l->num_layers) return fail(TSA_ERR_INVALID, "layer out of range");
    if (n_req < 0 || n_req > l->num_req || k < 0) return fail(TSA_ERR_INVALID, "bad n_req or k");
    if (l->held.count(tag)) return fail(TSA_ERR_INVALID, "tag still held");
    const int32_t P = l->cache->d.page_size;
    const int32_t npr = l->pages_per_req;
    // distinct pages per request, ascending (touch order)
    std::vector<int32_t> pages;
    std::vector<int32_t> first(size_t(n_req) + 1, 0);
    std::vector<int32_t> tmp;
    for (int32_t r = 0; r < n_req; ++r) {
        tmp.clear();
        for (int32_t j = 0; j < k; ++j) {
            const int32_t t = positions[size_t(r) * k + j];
            if (t >= 0 && t / P < npr) tmp.push_back(t / P);
        }
        std::sort(tmp.begin(), tmp.end());
        tmp.erase(std::unique(tmp.begin(), tmp.end()), tmp.end());
        pages.insert(pages.end(), tmp.begin(), tmp.end());
        first[size_t(r) + 1] = int32_t(pages.size());
    }
    auto key_at = [&](int32_t r, int32_t page) {
        return (int64_t(layer) * l->num_req + r) * npr + page;
    };
    // capacity check before any change: misses must fit in free slots plus pages that are
    // evictable now and not touched (touching pins them)
    int64_t miss = 0, touched_evictable = 0;
    for (int32_t r = 0; r < n_req; ++r)
        for (int32_t i = first[size_t(r)]; i < first[size_t(r) + 1]; ++i) {
            const int32_t slot = l->slot_of[size_t(key_at(r, pages[size_t(i)]))];
            if (slot < 0) ++miss;
            else if (l->pins[size_t(slot)] == 0) ++touched_evictable;
        }
    if (miss > int64_t(l->free_slots.size()) + int64_t(l->evictable.size()) - touched_evictable)
        return fail(TSA_ERR_CAPACITY, "the plan's misses exceed the free and unpinned slots");

    std::fill(slot_table, slot_table + size_t(n_req) * npr, -1);
    std::vector<int32_t>& hold = l->held[tag];
    for (int32_t r = 0; r < n_req; ++r)
        for (int32_t i = first[size_t(r)]; i < first[size_t(r) + 1]; ++i) {
            const int32_t page = pages[size_t(i)];
            const int64_t key = key_at(r, page);
            int32_t slot = l->slot_of[size_t(key)];
            if (slot >= 0) {
                ++l->hits;
                l->make_recent(slot);
            } else {
                ++l->misses;
                slot = l->place(key, true);
            }
            l->pin(slot);
            hold.push_back(slot);
            slot_table[size_t(r) * npr + page] = slot;
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
    for (int32_t slot : it->second) l->unpin(slot);
    l->held.erase(it);
    return TSA_OK;
    TSA_GUARD_END
}

tsa_status tsa_lru_workspace_bytes(const tsa_lru* l, int32_t n_req, size_t* bytes) {
    if (!l || !bytes || n_req < 0) return fail(TSA_ERR_INVALID, "bad arguments");
    // a fetch carries at most the cache's capacity of copies
    const int64_t m = l->capacity;
    *bytes = ws_keys_bytes(m) + ws_slots_bytes(m);
    (void)n_req;
    return TSA_OK;
}

tsa_status tsa_lru_fetch(tsa_lru* l, int32_t n_req, const int32_t* slot_table,
                         int32_t* slot_table_dev, void* workspace, size_t ws_bytes, void* stream) {
    TSA_GUARD_BEGIN
    if (!l || (n_req > 0 && (!slot_table || !slot_table_dev)) || n_req < 0 || n_req > l->num_req)
        return fail(TSA_ERR_INVALID, "bad arguments");
    if (!l->host_k) return fail(TSA_ERR_INVALID, "a bookkeeping-only tier cannot fetch");
    const int64_t n = int64_t(l->pending_slots.size());
    if (n > 0 && !workspace) return fail(TSA_ERR_INVALID, "workspace required");
    if (n > l->capacity) return fail(TSA_ERR_INVALID, "more pending copies than slots");
    const size_t need = ws_keys_bytes(l->capacity) + ws_slots_bytes(l->capacity);
    if (n > 0 && ws_bytes < need) return fail(TSA_ERR_CAPACITY, "workspace too small");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t table_bytes = size_t(n_req) * l->pages_per_req * sizeof(int32_t);
    const size_t stage_bytes = tsa::align_up(table_bytes, 256) + size_t(n) * 12;
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
    unsigned char* hb = static_cast<unsigned char*>(st.buf);
    if (table_bytes) std::memcpy(hb, slot_table, table_bytes);
    int64_t* hkeys = reinterpret_cast<int64_t*>(hb + tsa::align_up(table_bytes, 256));
    int32_t* hslots = reinterpret_cast<int32_t*>(hkeys + n);
    for (int64_t i = 0; i < n; ++i) {
        const int32_t slot = l->pending_slots[size_t(i)];
        hkeys[i] = l->pending_key[size_t(slot)];
        hslots[i] = slot;
    }
    tsa_status e = TSA_OK;
    if (table_bytes)
        e = tsa::hip_check(hipMemcpyAsync(slot_table_dev, hb, table_bytes, hipMemcpyHostToDevice, s),
                           "hipMemcpyAsync");
    if (e == TSA_OK && n) {
        unsigned char* w = static_cast<unsigned char*>(workspace);
        int64_t* dkeys = reinterpret_cast<int64_t*>(w);
        int32_t* dslots = reinterpret_cast<int32_t*>(w + ws_keys_bytes(l->capacity));
        e = tsa::hip_check(hipMemcpyAsync(dkeys, hkeys, size_t(n) * 8, hipMemcpyHostToDevice, s),
                           "hipMemcpyAsync");
        if (e == TSA_OK)
            e = tsa::hip_check(hipMemcpyAsync(dslots, hslots, size_t(n) * 4, hipMemcpyHostToDevice, s),
                               "hipMemcpyAsync");
        if (e == TSA_OK) e = tsa::hip_check(tsa::launch_lru_copy(*l, dkeys, dslots, n, s), "lru copy launch");
    }
    if (e == TSA_OK) e = tsa::hip_check(hipEventRecord(st.done, s), "hipEventRecord");
    if (e != TSA_OK) return e;
    st.used = true;
    l->h2d_bytes += n * int64_t(2 * l->page_bytes);
    for (int32_t slot : l->pending_slots) l->pending_key[size_t(slot)] = -1;
    l->pending_slots.clear();
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
