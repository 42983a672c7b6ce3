/*
 * tsa.h -- top-k sparse decode attention over a paged KV cache, for AMD MI355X (gfx950).
 *
 * C ABI of libtsa.  Plain pointers and sizes only.  Every device pointer is memory the
 * caller owns (for example a torch tensor's data_ptr()); the library owns only the opaque
 * handles and their host-side metadata (free list, reference counts, LRU state).  It never
 * allocates device memory on its own: sizes are queried up front and passed back in.
 *
 * Pages cited (the operations below restate what they define):
 *   [paged-KV page]  "KV cache phân trang, hay vì sao đặt trước theo độ dài tối đa là hoang
 *                    phí" (interactive-ebooks.coregenaihub.com, llm-moi/sinh-nhanh/kv-phan-trang)
 *   [GLM5.3 page]    "Cơ chế chú ý thưa (Sparse Attention) trên GLM5.3 ảnh hưởng thế nào đến
 *                    bộ nhớ HBM?" (aihot.vn)
 *   [snapshot page]  hert4.github.io ai-infra-notes, "cat-it-di-nho-nhieu-hon"
 *
 * Conventions shared by every call:
 *   - Status: every call returns a tsa_status; on failure tsa_last_error() holds a message
 *     (per thread).  Argument and capacity errors are detected before any side effect: no
 *     partial page allocation, nothing enqueued.  TSA_ERR_HIP reports a failed launch.
 *   - Streams: device work is enqueued on the caller's stream (a hipStream_t passed as
 *     void*; NULL = the default stream).  No call synchronizes the device.
 *   - Handles are not thread-safe; distinct handles may be used from distinct threads.
 *   - bf16 tensors are raw 16-bit bfloat16 values.  Layouts are row-major, innermost last.
 *   - Token positions are logical positions inside one request.  Physical page ids appear
 *     only inside page tables; the library translates (a write through an untranslated id
 *     lands in the wrong slot without any error: [snapshot page], "Ba thứ chặn đường").
 */
#ifndef TSA_H
#define TSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tsa_status {
    TSA_OK = 0,
    TSA_ERR_INVALID = -1,           /* bad pointer, shape, index or state */
    TSA_ERR_OUT_OF_PAGES = -2,      /* the pool's free list cannot cover the request */
    TSA_ERR_SHARED_PAGE_WRITE = -3, /* an append would write a page other tables also map */
    TSA_ERR_HIP = -4,               /* a HIP runtime call or kernel launch failed */
    TSA_ERR_CAPACITY = -5,          /* a caller-sized buffer (workspace, cache) is too small */
    TSA_ERR_UNSUPPORTED = -6        /* a valid shape no kernel of the library handles */
} tsa_status;

/* Message for the last failure on this thread ("" if none).  Valid until the next call. */
const char* tsa_last_error(void);

/* Version of this ABI (incremented on any incompatible change). */
int32_t tsa_abi_version(void);

/* ------------------------------------------------------------------------------------
 * KV pool: fixed-size pages in device memory.
 * [paged-KV page], "Phân trang: bỏ luôn ràng buộc liền mạch": the pool is cut into pages of
 * a fixed size and each request keeps a page table instead of one contiguous block.
 *
 * Device layouts (bf16), slot = page * page_size + position-in-page:
 *   K   [num_layers][num_pages * page_size][num_kv_heads][head_dim_k]
 *   V   [num_layers][num_pages * page_size][num_kv_heads][head_dim_v]   (absent if v_from_k)
 *   IDX [num_layers][num_pages * page_size][index_dim]                   (absent if index_dim 0)
 * With v_from_k = 1 the values are the first head_dim_v dims of each key row, as in the MQA
 * mode of MLA where all query heads read one latent row ([GLM5.3 page], MLA-modes paragraph).
 * ---------------------------------------------------------------------------------- */
typedef struct tsa_pool_desc {
    int32_t num_pages;     /* physical pages; > 0 */
    int32_t page_size;     /* tokens per page; > 0 */
    int32_t num_layers;    /* > 0 */
    int32_t num_kv_heads;  /* > 0 */
    int32_t head_dim_k;    /* multiple of 8, <= 1024 */
    int32_t head_dim_v;    /* multiple of 8, <= head_dim_k when v_from_k */
    int32_t v_from_k;      /* 0 or 1 */
    int32_t index_dim;     /* indexer key width, multiple of 8, or 0 for no indexer */
} tsa_pool_desc;

typedef struct tsa_kv_pool tsa_kv_pool;

/* Bytes the caller must allocate for each region (0 for an absent region).  The sizes are
 * exact and explicit: nothing is over-reserved by a hidden multiple ([snapshot page], "Ba thứ
 * chặn đường": a pool outside memory accounting asking for twice its size killed start-up). */
tsa_status tsa_kv_pool_bytes(const tsa_pool_desc* desc, size_t* k_bytes, size_t* v_bytes,
                             size_t* idx_bytes);

/* Create a pool over caller-owned device memory.  k_dev / v_dev / idx_dev may all be NULL
 * for a metadata-only pool (page tables, accounting; kernels then refuse it).  free_order
 * (host, nullable = ascending ids) is a permutation of 0..num_pages-1: the order in which
 * pages are handed out.  Allocation policy (the pages leave it open): requests are served in
 * index order, each one's logical pages in order, popping from the front of free_order. */
tsa_status tsa_kv_pool_create(const tsa_pool_desc* desc, void* k_dev, void* v_dev, void* idx_dev,
                              const int32_t* free_order, tsa_kv_pool** out);
tsa_status tsa_kv_pool_destroy(tsa_kv_pool* pool);

/* Pages on the free list, and pages referenced by at least one table. */
tsa_status tsa_kv_pool_usage(const tsa_kv_pool* pool, int32_t* free_pages, int32_t* used_pages);

/* Reference count of physical page `page` (number of page-table entries pointing at it). */
tsa_status tsa_kv_pool_refcount(const tsa_kv_pool* pool, int32_t page, int32_t* refcount);

/* ------------------------------------------------------------------------------------
 * Page tables (host arrays).
 * [paged-KV page], "Phân trang": a request of length L holds ceil(L / page_size) pages.
 * [paged-KV page], "Chia sẻ trang": requests sharing a prefix point at the same pages, but
 * only the full pages of the prefix: the page holding the prefix end and the first differing
 * token is private.  Saved pages = (members - 1) * floor(prefix / page_size).
 *
 * page_table: host int32 [n_req * max_pages], entry j of request i = physical page of its
 * logical page j, -1 where unused.  num_pages: host int32 [n_req].
 * ---------------------------------------------------------------------------------- */

/* Allocate tables for n_req requests of lengths lens[i] (>= 0).  prefix_group (nullable):
 * group id per request, -1 = none; prefix_len_of_group[g] (g < n_groups): prefix tokens of
 * group g, <= every member's length.  A group's full prefix pages are taken when its first
 * member (lowest index) is built; later members map the same pages (refcount = members).
 * saved_pages (nullable) receives the pages sharing saved.  On TSA_ERR_OUT_OF_PAGES nothing
 * is allocated. */
tsa_status tsa_page_table_build(tsa_kv_pool* pool, int32_t n_req, const int32_t* lens,
                                const int32_t* prefix_group, const int32_t* prefix_len_of_group,
                                int32_t n_groups, int32_t max_pages, int32_t* page_table,
                                int32_t* num_pages, int64_t* saved_pages);

/* Extend tables so request i covers new_lens[i] tokens (no shrinking), popping new private
 * pages in request order.  page_table / num_pages are updated in place; all-or-nothing. */
tsa_status tsa_page_table_grow(tsa_kv_pool* pool, int32_t n_req, const int32_t* new_lens,
                               int32_t max_pages, int32_t* page_table, int32_t* num_pages);

/* Drop the tables' references; a page whose count reaches 0 returns to the free list
 * (appended in table order).  Entries are not modified. */
tsa_status tsa_page_table_release(tsa_kv_pool* pool, int32_t n_req, const int32_t* page_table,
                                  const int32_t* num_pages, int32_t max_pages);

/* ------------------------------------------------------------------------------------
 * Appending tokens: scatter each new token's K, V and indexer key into the slot its page
 * table assigns ([paged-KV page], "Phân trang": pages need not be contiguous; the table
 * knows where each one is).
 * ---------------------------------------------------------------------------------- */

/* Host check for a planned append: every (req[i], pos[i]) must lie in an allocated page
 * (pos < num_pages[req] * page_size) whose refcount is 1.  Returns TSA_ERR_SHARED_PAGE_WRITE
 * for a shared page (copy-on-write is not provided), TSA_ERR_INVALID otherwise. */
tsa_status tsa_kv_append_check(const tsa_kv_pool* pool, int32_t n_tok, const int32_t* req,
                               const int32_t* pos, int32_t n_req, const int32_t* page_table,
                               const int32_t* num_pages, int32_t max_pages);

/* Device scatter of n_tok rows.  req_dev / pos_dev: device int32 [n_tok];
 * page_table_dev: device int32 [n_req * max_pages].  k_src: bf16 [n_tok][kv_heads][head_dim_k];
 * v_src: bf16 [n_tok][kv_heads][head_dim_v] (NULL iff v_from_k); idx_src: bf16
 * [n_tok][index_dim] (NULL to leave indexer keys untouched).  A token whose request, position
 * or page entry is out of range is skipped and counted in *bad_dev (device int32, nullable;
 * not reset by the call).  Does not check refcounts: use tsa_kv_append_check. */
tsa_status tsa_kv_append(tsa_kv_pool* pool, int32_t layer, int32_t n_tok, const int32_t* req_dev,
                         const int32_t* pos_dev, const int32_t* page_table_dev, int32_t n_req,
                         int32_t max_pages, const void* k_src, const void* v_src,
                         const void* idx_src, int32_t* bad_dev, void* stream);

/* ------------------------------------------------------------------------------------
 * One decode step of one layer: lightning-indexer score for every cached token, top-k
 * selection, scaled dot-product attention over the selected tokens only.
 * [GLM5.3 page], opening paragraph: sparse attention attends to the top-k most relevant
 * tokens, which cuts the bytes SDPA reads, while top-k selection still needs the whole
 * context in HBM.  Lightning-indexer paragraph:
 *     score[t] = sum_h w[h] * max(0, qI[h] . kI[t])      (multi-head query, one-head key)
 * one selection shared by every attention head; a context of at most top_k tokens is kept
 * whole (dense).  Ties (unspecified on the pages) go to the lower position.
 * Attention for query head h (KV head g = h / (num_q_heads / num_kv_heads), consecutive
 * grouping; unspecified on the pages):
 *     o[h] = softmax_j(sm_scale * q[h] . K[t_j, g]) . V[t_j, g]
 * ---------------------------------------------------------------------------------- */
typedef struct tsa_decode_params {
    int32_t batch;        /* requests B */
    int32_t num_q_heads;  /* Hq, a multiple of the pool's num_kv_heads */
    int32_t index_heads;  /* H_I: 1..64 when pages hold >= 16 tokens and index_dim is 32..256
                             (2..64 heads run on the matrix cores), else 1..8; ignored by
                             tsa_sparse_attn_gather.  Others give TSA_ERR_UNSUPPORTED. */
    int32_t top_k;        /* k >= 1 */
    int32_t max_len;      /* >= every seq_len; sizes the score buffer */
    float sm_scale;       /* logit scale, e.g. 1/sqrt(head_dim_k) */
} tsa_decode_params;

/* Workspace bytes the calls below need for these parameters (device memory, caller-owned,
 * 256-byte aligned, contents need not be initialised). */
tsa_status tsa_sparse_decode_workspace(const tsa_kv_pool* pool, const tsa_decode_params* p,
                                       size_t* bytes);

/* Indexer scores only.  qidx_dev: bf16 [B][H_I][index_dim]; widx_dev: fp32 [H_I];
 * seq_lens_dev: int32 [B]; scores_dev: fp32 [B][ld] with ld >= max_len; entries at
 * t >= seq_len are left untouched.  Scores are accumulated in fp32 (exact for integer-valued
 * inputs whose products and sums stay below 2^24). */
tsa_status tsa_indexer_scores(tsa_kv_pool* pool, int32_t layer, const tsa_decode_params* p,
                              const void* qidx_dev, const float* widx_dev,
                              const int32_t* page_table_dev, int32_t max_pages,
                              const int32_t* seq_lens_dev, float* scores_dev, int32_t ld,
                              void* stream);

/* Top-k of precomputed scores: fp32 [B][ld]; topk_dev: int32 [B][top_k], ascending
 * positions, -1 after the min(seq_len, top_k) selected ones.  Scores compare as floats: -0
 * equals +0, equal scores go to the lowest position, and a NaN ranks below every number. */
tsa_status tsa_topk(const tsa_decode_params* p, const float* scores_dev, int32_t ld,
                    const int32_t* seq_lens_dev, int32_t* topk_dev, void* stream);

/* Scores + top-k (the indexer half of the step). */
tsa_status tsa_indexer_topk(tsa_kv_pool* pool, int32_t layer, const tsa_decode_params* p,
                            const void* qidx_dev, const float* widx_dev,
                            const int32_t* page_table_dev, int32_t max_pages,
                            const int32_t* seq_lens_dev, int32_t* topk_dev, void* workspace,
                            size_t ws_bytes, void* stream);

/* Attention over given positions (the SDPA half).  q_dev: bf16 [B][Hq][head_dim_k];
 * topk_dev: int32 [B][top_k] positions (any order; entries < 0 or >= seq_len are ignored);
 * out_dev: fp32 [B][Hq][head_dim_v].  A request with no valid position gets zeros. */
tsa_status tsa_sparse_attn_gather(tsa_kv_pool* pool, int32_t layer, const tsa_decode_params* p,
                                  const void* q_dev, const int32_t* topk_dev,
                                  const int32_t* page_table_dev, int32_t max_pages,
                                  const int32_t* seq_lens_dev, float* out_dev, void* workspace,
                                  size_t ws_bytes, void* stream);

/* The whole step: scores, top-k, attention.  topk_dev (nullable) receives the selection. */
tsa_status tsa_sparse_decode_attn(tsa_kv_pool* pool, int32_t layer, const tsa_decode_params* p,
                                  const void* q_dev, const void* qidx_dev, const float* widx_dev,
                                  const int32_t* page_table_dev, int32_t max_pages,
                                  const int32_t* seq_lens_dev, float* out_dev, int32_t* topk_dev,
                                  void* workspace, size_t ws_bytes, void* stream);

/* The decode step with its own new token: request b's new rows (k_new_dev [B][Hkv][head_dim_k],
 * v_new_dev [B][Hkv][head_dim_v] or NULL exactly when values alias keys, idx_new_dev
 * [B][index_dim], all bf16) are written at position seq_lens[b] - 1 (the token being decoded,
 * already counted in its length) of every request with seq_lens[b] >= 1; then scores, top-k and
 * attention run as in tsa_sparse_decode_attn, the new token included.  Paged-KV page, section
 * "Phân trang": the position's page comes from the page table.  With one indexer head, pages of
 * at least 16 tokens and index_dim 32..256, the writes ride in the scoring launch (the new token
 * is scored from its new row); elsewhere a separate launch writes them first.  A token whose
 * page-table entry is not a page of the pool is not written, scores -inf and is counted in
 * bad_dev (nullable, int32, accumulated).  When max_len <= 1024, min(top_k, max_len) x
 * num_kv_heads <= 128 and tsa_decode_step_fused takes the shapes, the step runs as
 * tsa_decode_step_fused (one launch; the workspace is then unused).
 * Other arguments and errors as tsa_sparse_decode_attn. */
tsa_status tsa_decode_step(tsa_kv_pool* pool, int32_t layer, const tsa_decode_params* p,
                           const void* k_new_dev, const void* v_new_dev, const void* idx_new_dev,
                           int32_t* bad_dev, const void* q_dev, const void* qidx_dev,
                           const float* widx_dev, const int32_t* page_table_dev, int32_t max_pages,
                           const int32_t* seq_lens_dev, float* out_dev, int32_t* topk_dev,
                           void* workspace, size_t ws_bytes, void* stream);

/* tsa_decode_step for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same step, arguments and results,
 * with the workspace taken from a fixed scratch array inside the library instead of a caller
 * buffer.  Each GPU the library runs on holds one 64 MiB array (256-byte aligned) from the time
 * the library's code is loaded on it until the process ends; the call allocates nothing and
 * looks the current device's array up on its first call on that device.  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (on different streams, or from different
 * threads without ordering) race and give wrong results.  The array keeps the last call's
 * contents, which no call depends on.  Returns TSA_ERR_CAPACITY when the step's workspace
 * (tsa_sparse_decode_workspace) exceeds 64 MiB; other errors as tsa_decode_step. */
tsa_status tsa_decode_step_noalloc(tsa_kv_pool* pool, int32_t layer, const tsa_decode_params* p,
                                   const void* k_new_dev, const void* v_new_dev,
                                   const void* idx_new_dev, int32_t* bad_dev, const void* q_dev,
                                   const void* qidx_dev, const float* widx_dev,
                                   const int32_t* page_table_dev, int32_t max_pages,
                                   const int32_t* seq_lens_dev, float* out_dev, int32_t* topk_dev,
                                   void* stream);

/* tsa_decode_step as one launch: workgroup b runs request b's whole step (write its new token,
 * score every cached token, select the top k, attend over them), with the scores and the
 * selection kept on chip.  GLM5.3 page, TileRT paragraph: decode built as one persistent kernel
 * removes the gaps between its stages; paragraph on serving-engine decode (the GLM-5.2 studies):
 * small decode steps are dominated by launch overhead.  Results equal tsa_decode_step's (the
 * same top-k sets; attention within fp32 rounding).  Needs no workspace.  Each request's new
 * position must lie in a page no other request of the batch maps (tsa_kv_append_check verifies
 * this), since other workgroups may read the pages they share while it is written.  Limits:
 * index_dim 8 x a power of two <= 256, index_heads 1..8, head dims multiples of 8, (q heads per
 * KV head) x head_dim_v <= 2048, and the scores of max_len tokens, min(top_k, max_len) selected
 * positions and the attention tiles within 64 KiB of LDS (at top_k 2048, max_len up to about
 * 13,000 tokens);
 * otherwise TSA_ERR_UNSUPPORTED.  Other arguments and errors as tsa_decode_step. */
tsa_status tsa_decode_step_fused(tsa_kv_pool* pool, int32_t layer, const tsa_decode_params* p,
                                 const void* k_new_dev, const void* v_new_dev, const void* idx_new_dev,
                                 int32_t* bad_dev, const void* q_dev, const void* qidx_dev,
                                 const float* widx_dev, const int32_t* page_table_dev,
                                 int32_t max_pages, const int32_t* seq_lens_dev, float* out_dev,
                                 int32_t* topk_dev, void* stream);

/* ------------------------------------------------------------------------------------
 * Captured step.  GLM5.3 page, paragraph on serving-engine prefill and decode (the GLM-5.2
 * studies): running the decode step on a fixed graph-execution path lowered the time per output
 * token; TileRT paragraph: launch overhead is worth removing.  Here the step's launches are
 * recorded once and replayed by one launch.  The
 * step (an optional kv_append, then tsa_sparse_decode_attn) is recorded into a HIP graph over
 * fixed device pointers; each tsa_step_graph_launch replays it on the given stream, reading
 * whatever those buffers hold at that time (new queries, lengths, page tables of the same
 * shape).  Sizes, the pool, the parameters and the pointers are fixed at creation; anything
 * else needs a new graph.  The graph records kernel launches only (no memset or copy nodes).
 * Replays that overlap on one workspace race, as eager calls would.  Errors: the same checks
 * as the eager calls, at creation; TSA_ERR_HIP if capture or instantiation fails.
 * ---------------------------------------------------------------------------------- */
typedef struct tsa_append_args {
    int32_t n_tok;            /* new tokens; 0 records no append */
    const int32_t* req_dev;   /* [n_tok] request of each token */
    const int32_t* pos_dev;   /* [n_tok] its position */
    const void* k_src;        /* as tsa_kv_append */
    const void* v_src;
    const void* idx_src;
    int32_t* bad_dev;         /* nullable rejected-token counter (accumulates over replays) */
} tsa_append_args;

typedef struct tsa_step_graph tsa_step_graph;

/* Record the step.  append may be NULL.  The other arguments are those of
 * tsa_sparse_decode_attn (the append uses the same page table, max_pages and batch). */
tsa_status tsa_step_graph_create(tsa_kv_pool* pool, int32_t layer, const tsa_decode_params* p,
                                 const tsa_append_args* append, const void* q_dev,
                                 const void* qidx_dev, const float* widx_dev,
                                 const int32_t* page_table_dev, int32_t max_pages,
                                 const int32_t* seq_lens_dev, float* out_dev, int32_t* topk_dev,
                                 void* workspace, size_t ws_bytes, tsa_step_graph** graph);
/* Replay on `stream` (NULL = the null stream). */
tsa_status tsa_step_graph_launch(tsa_step_graph* graph, void* stream);
tsa_status tsa_step_graph_destroy(tsa_step_graph* graph);

/* ------------------------------------------------------------------------------------
 * Tiered KV: an HBM page cache with LRU eviction over a host-memory copy of every page.
 * [GLM5.3 page], HiSparse paragraph: the KV cache lives in host DRAM and the HBM part acts as
 * an LRU cache; a top-k selection that misses loads the page from DRAM, the least recently
 * used page is evicted, and the loads for layer N overlap the computation of layer N-1.
 * [snapshot page], "Lợi ích thì đo được rõ": strict LRU falls off a cliff when the working
 * set exceeds the cache (a cyclic scan hits nothing).
 *
 * The cache is an ordinary pool (num_layers 1, num_pages = cache slots, no indexer region);
 * a pool created without device regions gives a bookkeeping-only tier (plan, release, stats;
 * host_k / host_v may then be NULL and fetch is refused);
 * a slot holds one page of any (layer, request).  The cache pool's page size is the unit of
 * caching: pages of P tokens cache whole pages; a pool with page_size 1 and pages_per_req =
 * the request length caches single token rows, which is what the HiSparse paragraph loads on a
 * miss.  The host copy is the same bytes either way.  Logical page keys are
 *     key = (layer * num_req + req) * pages_per_req + page.
 * host_k / host_v: pinned host memory (hipHostMalloc, e.g. torch pin_memory=True), key-major:
 * page `key` occupies bytes [key * page_bytes, (key + 1) * page_bytes) with
 * page_bytes = page_size * num_kv_heads * head_dim * 2 (the pool's K / V page).  The GPU
 * reads missing pages from it directly (mapped pinned memory), so the host copy must stay
 * allocated and unchanged while the cache exists.  The cache owns pinned host staging
 * buffers for its transfer lists; it allocates no device memory.
 *
 * Policy (the pages leave the details open): a plan touches the distinct pages of each
 * request's positions, requests ascending, pages ascending within a request.  A resident page
 * is a hit and becomes most recent; a missing page takes a free slot (lowest first) or evicts
 * the least recently touched page that no unreleased plan holds.  Pages a plan touches stay
 * pinned until that plan's tag is released (the layer being computed and the one being
 * fetched are both in flight).  K/V pages never change once written, so eviction writes
 * nothing back.
 * ---------------------------------------------------------------------------------- */
typedef struct tsa_lru tsa_lru;

/* cache: a pool with v_from_k 0, index_dim 0, num_layers 1, device K and V regions.
 * Initially every slot is free and no page is resident. */
tsa_status tsa_lru_create(tsa_kv_pool* cache, int32_t num_layers, int32_t num_req,
                          int32_t pages_per_req, const void* host_k, const void* host_v,
                          tsa_lru** out);
tsa_status tsa_lru_destroy(tsa_lru* lru);

/* Make `keys` (host int64 [n]) resident, first = least recent, without counting hits or
 * misses; their copies join the next fetch. */
tsa_status tsa_lru_preload(tsa_lru* lru, int64_t n, const int64_t* keys);

/* Host bookkeeping for one layer.  positions: host int32 [n_req][k] token positions (entries
 * < 0 or >= pages_per_req * page_size are ignored).  slot_table (nullable): host int32
 * [n_req][pages_per_req], filled with the slot of every touched page and -1 elsewhere (a page
 * table for tsa_sparse_attn_gather on the cache pool, layer 0); tsa_lru_fetch writes the same
 * entries into the device table whether or not it is given.  The touched pages are pinned
 * under `tag`.  n_fetch (nullable) receives the number of page copies now pending.  Fails
 * with TSA_ERR_CAPACITY, changing nothing, if the misses exceed the free slots plus the
 * unpinned pages the plan does not touch. */
tsa_status tsa_lru_plan(tsa_lru* lru, int32_t layer, int64_t tag, int32_t n_req,
                        const int32_t* positions, int32_t k, int32_t* slot_table,
                        int64_t* n_fetch);

/* Device workspace for tsa_lru_fetch with up to n_req requests per plan. */
tsa_status tsa_lru_workspace_bytes(const tsa_lru* lru, int32_t n_req, size_t* bytes);

/* Enqueue on `stream`: the entries the last plan set (the slots of its touched pages) into
 * slot_table_dev (int32 [n_req][pages_per_req]), and the copies of every pending page from host
 * memory into its slot.  Entries of pages the plan did not touch are left as they were (an
 * attention over the plan's positions reads only touched pages), so a fetch moves 12 bytes
 * per touched page instead of the whole table.  slot_table is not read (the entries come from
 * the plan; it may be NULL).  n_req must cover the last plan's requests.  The caller orders
 * `stream` after every kernel that reads a page a released tag held (eviction reuses those
 * slots) and orders the attention of the layer after this call (e.g. with events). */
tsa_status tsa_lru_fetch(tsa_lru* lru, int32_t n_req, const int32_t* slot_table,
                         int32_t* slot_table_dev, void* workspace, size_t ws_bytes,
                         void* stream);

/* Unpin the pages held under `tag`.  The caller orders any later fetch after every kernel that
 * reads those pages (tsa_lru_release_layer does it for the caller). */
tsa_status tsa_lru_release(tsa_lru* lru, int64_t tag);

/* [GLM5.3 page], HiSparse paragraph: layer N's loads overlap layer N-1's compute, so a slot may be
 * given to a new page while the attention that read its old page is still queued.  This call
 * unpins the pages held under `tag` now (a later plan may evict them) and makes every later fetch
 * (tsa_lru_fetch, tsa_lru_prefetch) wait on its stream for `done_event` before it copies anything:
 * record done_event right after the last kernel that reads the tag's slots (e.g. that layer's
 * attention), on that kernel's stream.  A copy can then never overwrite a slot before that kernel
 * is done ([snapshot page], "Ba thứ chặn đường": a write through a stale slot goes to the wrong
 * place without any error).  done_event (a hipEvent_t, caller-owned, nullable = tsa_lru_release)
 * must stay valid until the next fetch call returns; recording it again later only makes that
 * fetch wait longer. */
tsa_status tsa_lru_release_layer(tsa_lru* lru, int64_t tag, void* done_event);

/* Plan and fetch one layer in one call, ordered for the caller: tsa_lru_plan (no host table),
 * then tsa_lru_fetch on `stream` (after the events of released tags, as above), then
 * fetched_event (a hipEvent_t, caller-owned, nullable) recorded on `stream`: the attention of
 * the layer waits on it (hipStreamWaitEvent) so that it never reads a slot whose copy is still
 * in flight.  Argument errors are reported before the plan changes anything. */
tsa_status tsa_lru_prefetch(tsa_lru* lru, int32_t layer, int64_t tag, int32_t n_req,
                            const int32_t* positions, int32_t k, int32_t* slot_table_dev,
                            void* workspace, size_t ws_bytes, void* stream, void* fetched_event);

/* Counters since creation (preloads excluded): page touches that hit, that missed, evictions,
 * and bytes copied from host memory (preloads included). */
tsa_status tsa_lru_stats(const tsa_lru* lru, int64_t* hits, int64_t* misses,
                         int64_t* evictions, int64_t* h2d_bytes);

#ifdef __cplusplus
}
#endif

#endif /* TSA_H */
