// KV pool, page tables and appends: the host half of libtsa.
//
// Paging follows the paged-KV page ("KV cache phân trang, hay vì sao đặt trước theo độ dài
// tối đa là hoang phí"): section "Phân trang" (pages = ceil(length / page_size), per-request
// page tables, pages need not be adjacent) and section "Chia sẻ trang" (requests with a
// common prefix map the same full pages; saved = (n - 1) * floor(prefix / page_size)).
// The allocation order is this library's own policy, stated in tsa.h.
#include <algorithm>
#include <cstring>
#include <new>
#include <unordered_map>

#include "tsa_internal.h"

namespace {
thread_local std::string g_last_error;
}

namespace tsa {

tsa_status fail(tsa_status st, const std::string& msg) {
    g_last_error = msg;
    return st;
}

tsa_status ok() { return TSA_OK; }

tsa_status hip_check(hipError_t e, const char* what) {
    if (e == hipSuccess) return TSA_OK;
    return fail(TSA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

}  // namespace tsa

using tsa::fail;

void tsa_kv_pool::compact_free() {
    if (free_head > 0 && free_head * 2 > free_list.size()) {
        free_list.erase(free_list.begin(), free_list.begin() + free_head);
        free_head = 0;
    }
}

#define TSA_GUARD_BEGIN try {
#define TSA_GUARD_END                                                   \
    }                                                                   \
    catch (const std::bad_alloc&) {                                     \
        return fail(TSA_ERR_CAPACITY, "host allocation failed");        \
    }                                                                   \
    catch (...) {                                                       \
        return fail(TSA_ERR_INVALID, "unexpected host exception");      \
    }

extern "C" {

const char* tsa_last_error(void) { return g_last_error.c_str(); }

int32_t tsa_abi_version(void) { return 1; }

static tsa_status check_desc(const tsa_pool_desc* d) {
    if (!d) return fail(TSA_ERR_INVALID, "desc is NULL");
    if (d->num_pages <= 0 || d->page_size <= 0 || d->num_layers <= 0 || d->num_kv_heads <= 0)
        return fail(TSA_ERR_INVALID, "num_pages, page_size, num_layers, num_kv_heads must be > 0");
    if (d->head_dim_k <= 0 || d->head_dim_k % 8 || d->head_dim_k > 1024)
        return fail(TSA_ERR_INVALID, "head_dim_k must be a positive multiple of 8, <= 1024");
    if (d->head_dim_v <= 0 || d->head_dim_v % 8 || d->head_dim_v > 1024)
        return fail(TSA_ERR_INVALID, "head_dim_v must be a positive multiple of 8, <= 1024");
    if (d->v_from_k != 0 && d->v_from_k != 1) return fail(TSA_ERR_INVALID, "v_from_k must be 0 or 1");
    if (d->v_from_k && d->head_dim_v > d->head_dim_k)
        return fail(TSA_ERR_INVALID, "v_from_k needs head_dim_v <= head_dim_k");
    if (d->index_dim < 0 || d->index_dim % 8 || d->index_dim > 1024)
        return fail(TSA_ERR_INVALID, "index_dim must be 0 or a multiple of 8, <= 1024");
    int64_t slots = int64_t(d->num_pages) * d->page_size;
    if (slots > (int64_t(1) << 40)) return fail(TSA_ERR_INVALID, "pool too large");
    return TSA_OK;
}

tsa_status tsa_kv_pool_bytes(const tsa_pool_desc* d, size_t* kb, size_t* vb, size_t* ib) {
    TSA_GUARD_BEGIN
    tsa_status st = check_desc(d);
    if (st) return st;
    if (!kb || !vb || !ib) return fail(TSA_ERR_INVALID, "output pointer is NULL");
    size_t rows = size_t(d->num_layers) * size_t(d->num_pages) * size_t(d->page_size);
    *kb = rows * d->num_kv_heads * d->head_dim_k * 2;
    *vb = d->v_from_k ? 0 : rows * d->num_kv_heads * d->head_dim_v * 2;
    *ib = rows * size_t(d->index_dim) * 2;
    return TSA_OK;
    TSA_GUARD_END
}

tsa_status tsa_kv_pool_create(const tsa_pool_desc* d, void* k_dev, void* v_dev, void* idx_dev,
                              const int32_t* free_order, tsa_kv_pool** out) {
    TSA_GUARD_BEGIN
    tsa_status st = check_desc(d);
    if (st) return st;
    if (!out) return fail(TSA_ERR_INVALID, "out is NULL");
    *out = nullptr;
    bool any = k_dev || v_dev || idx_dev;
    if (any) {
        if (!k_dev) return fail(TSA_ERR_INVALID, "k_dev is NULL");
        if (!d->v_from_k && !v_dev) return fail(TSA_ERR_INVALID, "v_dev is NULL without v_from_k");
        if (d->v_from_k && v_dev) return fail(TSA_ERR_INVALID, "v_dev must be NULL with v_from_k");
        if (d->index_dim && !idx_dev) return fail(TSA_ERR_INVALID, "idx_dev is NULL with index_dim > 0");
        if (!d->index_dim && idx_dev) return fail(TSA_ERR_INVALID, "idx_dev given with index_dim 0");
    }
    auto* p = new tsa_kv_pool();
    p->d = *d;
    p->k = k_dev;
    p->v = v_dev;
    p->idx = idx_dev;
    p->free_list.resize(d->num_pages);
    p->refcount.assign(d->num_pages, 0);
    if (free_order) {
        std::vector<uint8_t> seen(d->num_pages, 0);
        for (int32_t i = 0; i < d->num_pages; ++i) {
            int32_t x = free_order[i];
            if (x < 0 || x >= d->num_pages || seen[x]) {
                delete p;
                return fail(TSA_ERR_INVALID, "free_order is not a permutation of 0..num_pages-1");
            }
            seen[x] = 1;
            p->free_list[i] = x;
        }
    } else {
        for (int32_t i = 0; i < d->num_pages; ++i) p->free_list[i] = i;
    }
    *out = p;
    return TSA_OK;
    TSA_GUARD_END
}

tsa_status tsa_kv_pool_destroy(tsa_kv_pool* pool) {
    delete pool;
    return TSA_OK;
}

tsa_status tsa_kv_pool_usage(const tsa_kv_pool* pool, int32_t* free_pages, int32_t* used_pages) {
    if (!pool) return fail(TSA_ERR_INVALID, "pool is NULL");
    int32_t used = 0;
    for (int32_t c : pool->refcount) used += c > 0;
    if (free_pages) *free_pages = pool->free_count();
    if (used_pages) *used_pages = used;
    return TSA_OK;
}

tsa_status tsa_kv_pool_refcount(const tsa_kv_pool* pool, int32_t page, int32_t* refcount) {
    if (!pool || !refcount) return fail(TSA_ERR_INVALID, "NULL argument");
    if (page < 0 || page >= pool->d.num_pages) return fail(TSA_ERR_INVALID, "page out of range");
    *refcount = pool->refcount[page];
    return TSA_OK;
}

tsa_status tsa_page_table_build(tsa_kv_pool* pool, int32_t n_req, const int32_t* lens,
                                const int32_t* prefix_group, const int32_t* prefix_len_of_group,
                                int32_t n_groups, int32_t max_pages, int32_t* page_table,
                                int32_t* num_pages, int64_t* saved_pages) {
    TSA_GUARD_BEGIN
    if (!pool) return fail(TSA_ERR_INVALID, "pool is NULL");
    if (n_req < 0 || max_pages < 0) return fail(TSA_ERR_INVALID, "negative size");
    if (n_req > 0 && (!lens || !page_table || !num_pages)) return fail(TSA_ERR_INVALID, "NULL array");
    if (prefix_group && (!prefix_len_of_group || n_groups <= 0))
        return fail(TSA_ERR_INVALID, "prefix_group needs prefix_len_of_group and n_groups > 0");
    const int64_t P = pool->d.page_size;
    // validate everything before touching the pool
    std::vector<int32_t> need(n_req);
    std::vector<int32_t> shared(std::max(n_groups, 0), 0);
    std::vector<int32_t> members(std::max(n_groups, 0), 0);
    int64_t total_new = 0;
    for (int32_t i = 0; i < n_req; ++i) {
        if (lens[i] < 0) return fail(TSA_ERR_INVALID, "negative length");
        int64_t n = tsa::ceil_div(lens[i], P);
        if (n > max_pages) return fail(TSA_ERR_INVALID, "a request needs more than max_pages pages");
        need[i] = int32_t(n);
        int32_t g = prefix_group ? prefix_group[i] : -1;
        if (g >= n_groups || g < -1) return fail(TSA_ERR_INVALID, "prefix group id out of range");
        if (g >= 0) {
            int32_t pl = prefix_len_of_group[g];
            if (pl < 0 || pl > lens[i]) return fail(TSA_ERR_INVALID, "a request is shorter than its prefix");
            shared[g] = int32_t(pl / P);
            total_new += (members[g] == 0 ? need[i] : need[i] - shared[g]);
            members[g]++;
        } else {
            total_new += need[i];
        }
    }
    if (total_new > pool->free_count())
        return fail(TSA_ERR_OUT_OF_PAGES, "pool has " + std::to_string(pool->free_count()) +
                                              " free pages, tables need " + std::to_string(total_new));
    // allocate
    std::vector<std::vector<int32_t>> group_pages(std::max(n_groups, 0));
    for (int32_t i = 0; i < n_req; ++i) {
        int32_t* row = page_table + int64_t(i) * max_pages;
        int32_t g = prefix_group ? prefix_group[i] : -1;
        for (int32_t j = 0; j < need[i]; ++j) {
            int32_t pid;
            if (g >= 0 && j < shared[g]) {
                auto& gp = group_pages[g];
                if (j < int32_t(gp.size())) {
                    pid = gp[j];
                } else {
                    pid = pool->pop();
                    gp.push_back(pid);
                }
            } else {
                pid = pool->pop();
            }
            row[j] = pid;
            pool->refcount[pid]++;
        }
        for (int32_t j = need[i]; j < max_pages; ++j) row[j] = -1;
        num_pages[i] = need[i];
    }
    pool->compact_free();
    if (saved_pages) {
        int64_t s = 0;
        for (int32_t g = 0; g < n_groups; ++g)
            if (members[g] > 0) s += int64_t(members[g] - 1) * shared[g];
        *saved_pages = s;
    }
    return TSA_OK;
    TSA_GUARD_END
}

tsa_status tsa_page_table_grow(tsa_kv_pool* pool, int32_t n_req, const int32_t* new_lens,
                               int32_t max_pages, int32_t* page_table, int32_t* num_pages) {
    TSA_GUARD_BEGIN
    if (!pool) return fail(TSA_ERR_INVALID, "pool is NULL");
    if (n_req < 0 || max_pages < 0) return fail(TSA_ERR_INVALID, "negative size");
    if (n_req > 0 && (!new_lens || !page_table || !num_pages)) return fail(TSA_ERR_INVALID, "NULL array");
    const int64_t P = pool->d.page_size;
    int64_t total = 0;
    for (int32_t i = 0; i < n_req; ++i) {
        if (new_lens[i] < 0) return fail(TSA_ERR_INVALID, "negative length");
        int64_t n = tsa::ceil_div(new_lens[i], P);
        if (num_pages[i] < 0 || num_pages[i] > max_pages) return fail(TSA_ERR_INVALID, "num_pages out of range");
        if (n < num_pages[i]) return fail(TSA_ERR_INVALID, "a length shrank");
        if (n > max_pages) return fail(TSA_ERR_INVALID, "a request needs more than max_pages pages");
        total += n - num_pages[i];
    }
    if (total > pool->free_count()) return fail(TSA_ERR_OUT_OF_PAGES, "pool out of pages");
    for (int32_t i = 0; i < n_req; ++i) {
        int32_t* row = page_table + int64_t(i) * max_pages;
        int32_t n = int32_t(tsa::ceil_div(new_lens[i], P));
        for (int32_t j = num_pages[i]; j < n; ++j) {
            int32_t pid = pool->pop();
            row[j] = pid;
            pool->refcount[pid]++;
        }
        num_pages[i] = n;
    }
    pool->compact_free();
    return TSA_OK;
    TSA_GUARD_END
}

tsa_status tsa_page_table_release(tsa_kv_pool* pool, int32_t n_req, const int32_t* page_table,
                                  const int32_t* num_pages, int32_t max_pages) {
    TSA_GUARD_BEGIN
    if (!pool) return fail(TSA_ERR_INVALID, "pool is NULL");
    if (n_req < 0 || max_pages < 0) return fail(TSA_ERR_INVALID, "negative size");
    if (n_req > 0 && (!page_table || !num_pages)) return fail(TSA_ERR_INVALID, "NULL array");
    // validate: every referenced page exists and the drops do not go below zero
    std::unordered_map<int32_t, int32_t> drops;
    for (int32_t i = 0; i < n_req; ++i) {
        if (num_pages[i] < 0 || num_pages[i] > max_pages) return fail(TSA_ERR_INVALID, "num_pages out of range");
        const int32_t* row = page_table + int64_t(i) * max_pages;
        for (int32_t j = 0; j < num_pages[i]; ++j) {
            int32_t pid = row[j];
            if (pid < 0 || pid >= pool->d.num_pages) return fail(TSA_ERR_INVALID, "page id out of range");
            if (++drops[pid] > pool->refcount[pid]) return fail(TSA_ERR_INVALID, "page released more often than mapped");
        }
    }
    for (int32_t i = 0; i < n_req; ++i) {
        const int32_t* row = page_table + int64_t(i) * max_pages;
        for (int32_t j = 0; j < num_pages[i]; ++j) {
            int32_t pid = row[j];
            if (--pool->refcount[pid] == 0) pool->push(pid);
        }
    }
    return TSA_OK;
    TSA_GUARD_END
}

tsa_status tsa_kv_append_check(const tsa_kv_pool* pool, int32_t n_tok, const int32_t* req,
                               const int32_t* pos, int32_t n_req, const int32_t* page_table,
                               const int32_t* num_pages, int32_t max_pages) {
    if (!pool) return fail(TSA_ERR_INVALID, "pool is NULL");
    if (n_tok < 0 || n_req < 0 || max_pages < 0) return fail(TSA_ERR_INVALID, "negative size");
    if (n_tok > 0 && (!req || !pos || !page_table || !num_pages)) return fail(TSA_ERR_INVALID, "NULL array");
    const int32_t P = pool->d.page_size;
    for (int32_t i = 0; i < n_tok; ++i) {
        int32_t r = req[i], t = pos[i];
        if (r < 0 || r >= n_req) return fail(TSA_ERR_INVALID, "request index out of range");
        if (t < 0 || int64_t(t) >= int64_t(num_pages[r]) * P || t / P >= max_pages)
            return fail(TSA_ERR_INVALID, "position outside the request's pages");
        int32_t pid = page_table[int64_t(r) * max_pages + t / P];
        if (pid < 0 || pid >= pool->d.num_pages) return fail(TSA_ERR_INVALID, "page id out of range");
        if (pool->refcount[pid] > 1)
            return fail(TSA_ERR_SHARED_PAGE_WRITE, "position " + std::to_string(t) + " of request " +
                                                       std::to_string(r) + " lies in a shared page");
    }
    return TSA_OK;
}

tsa_status tsa_kv_append(tsa_kv_pool* pool, int32_t layer, int32_t n_tok, const int32_t* req_dev,
                         const int32_t* pos_dev, const int32_t* page_table_dev, int32_t n_req,
                         int32_t max_pages, const void* k_src, const void* v_src,
                         const void* idx_src, int32_t* bad_dev, void* stream) {
    if (!pool) return fail(TSA_ERR_INVALID, "pool is NULL");
    if (!pool->k) return fail(TSA_ERR_INVALID, "pool has no device memory");
    if (layer < 0 || layer >= pool->d.num_layers) return fail(TSA_ERR_INVALID, "layer out of range");
    if (n_tok < 0 || n_req < 0 || max_pages < 0) return fail(TSA_ERR_INVALID, "negative size");
    if (n_tok == 0) return TSA_OK;
    if (!req_dev || !pos_dev || !page_table_dev || !k_src) return fail(TSA_ERR_INVALID, "NULL array");
    if (pool->d.v_from_k ? v_src != nullptr : v_src == nullptr)
        return fail(TSA_ERR_INVALID, "v_src must be NULL exactly when the pool has v_from_k");
    if (idx_src && !pool->d.index_dim) return fail(TSA_ERR_INVALID, "idx_src given for a pool without indexer");
    hipError_t e = tsa::launch_kv_append(*pool, layer, n_tok, req_dev, pos_dev, page_table_dev, n_req,
                                         max_pages, k_src, v_src, idx_src, bad_dev,
                                         static_cast<hipStream_t>(stream));
    return tsa::hip_check(e, "kv_append launch");
}

}  // extern "C"
