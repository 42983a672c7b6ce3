// Host side of the decode step: argument checks, workspace carve-up, launches on the caller's
// stream.  The step is the GLM5.3 sparse-attention page's DSA decode: lightning-indexer score
// of every cached token, top-k selection, attention over the selected tokens only.
#include <algorithm>
#include <mutex>

#include "tsa_internal.h"

using tsa::fail;

// Scratch memory of tsa_decode_step_noalloc: a workspace that the library owns, for callers that
// cannot allocate.  Each GPU the library runs on holds its own copy of this array from the time the
// library's code is loaded on it until the process ends.  In host code `scratch` names a host-side
// stand-in, not the device array: kernels must receive the address hipGetSymbolAddress reports for
// the current device, which is looked up once per device and kept in scratch_dev.
namespace {
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxScratchDevices = 64;
std::mutex scratch_mu;
void* scratch_dev[kMaxScratchDevices] = {};

// Device address of the current device's scratch array (looked up on the first call per device).
tsa_status current_scratch(void** out) {
    int dev = -1;
    tsa_status st = tsa::hip_check(hipGetDevice(&dev), "hipGetDevice");
    if (st) return st;
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(TSA_ERR_UNSUPPORTED, "device index " + std::to_string(dev) + " above 63");
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_dev[dev]) {
        void* ptr = nullptr;
        st = tsa::hip_check(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
        if (st) return st;
        if (!ptr) return fail(TSA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        scratch_dev[dev] = ptr;
    }
    *out = scratch_dev[dev];
    return TSA_OK;
}
}  // namespace

namespace {

constexpr size_t kAlign = 256;

int scores_ld(int max_len) { return int(tsa::align_up(size_t(std::max(max_len, 1)), 64)); }

struct WsLayout {
    size_t scores = 0, topk = 0, partial = 0, total = 0;
};

WsLayout layout(const tsa_kv_pool& pool, const tsa_decode_params& p, bool with_attn) {
    WsLayout w;
    size_t off = 0;
    w.scores = off;
    off += tsa::align_up(size_t(p.batch) * scores_ld(p.max_len) * sizeof(float), kAlign);
    w.topk = off;
    off += tsa::align_up(size_t(p.batch) * p.top_k * sizeof(int32_t), kAlign);
    w.partial = off;
    if (with_attn) off += tsa::align_up(tsa::plan_attention(pool, p).partial_bytes, kAlign);
    w.total = off;
    return w;
}


tsa_status check_common(const tsa_kv_pool* pool, int32_t layer, const tsa_decode_params* p,
                        const int32_t* page_table, int32_t max_pages, const int32_t* seq_lens) {
    if (!pool) return fail(TSA_ERR_INVALID, "pool is NULL");
    if (!pool->k) return fail(TSA_ERR_INVALID, "pool has no device memory");
    if (!p) return fail(TSA_ERR_INVALID, "params is NULL");
    if (layer < 0 || layer >= pool->d.num_layers) return fail(TSA_ERR_INVALID, "layer out of range");
    if (p->batch < 0 || p->max_len < 0 || p->top_k < 1 || max_pages < 0)
        return fail(TSA_ERR_INVALID, "batch, max_len, max_pages must be >= 0 and top_k >= 1");
    if (p->num_q_heads <= 0 || p->num_q_heads % pool->d.num_kv_heads)
        return fail(TSA_ERR_INVALID, "num_q_heads must be a positive multiple of num_kv_heads");
    if (int64_t(p->max_len) > int64_t(max_pages) * pool->d.page_size)
        return fail(TSA_ERR_INVALID, "max_len exceeds max_pages * page_size");
    if (p->batch > 0 && (!page_table || !seq_lens)) return fail(TSA_ERR_INVALID, "NULL page table or lengths");
    return TSA_OK;
}

tsa_status check_indexer(const tsa_kv_pool* pool, const tsa_decode_params* p, const void* qidx,
                         const float* widx) {
    const int D = pool->d.index_dim;
    if (!D || !pool->idx) return fail(TSA_ERR_INVALID, "pool has no indexer keys");
    std::string why;
    if (!tsa::indexer_supported(*pool, *p, &why)) return fail(TSA_ERR_UNSUPPORTED, why);
    if (p->batch > 0 && (!qidx || !widx)) return fail(TSA_ERR_INVALID, "NULL indexer query or weights");
    return TSA_OK;
}

tsa_status check_topk(const tsa_decode_params* p) {
    if (!tsa::topk_supported(p->max_len)) return fail(TSA_ERR_UNSUPPORTED, "max_len above 65536 tokens");
    return TSA_OK;
}

tsa_status check_attn(const tsa_kv_pool* pool, const tsa_decode_params* p, const void* q, float* out) {
    std::string why;
    if (!tsa::attention_supported(*pool, *p, &why)) return fail(TSA_ERR_UNSUPPORTED, why);
    if (p->batch > 0 && (!q || !out)) return fail(TSA_ERR_INVALID, "NULL query or output");
    return TSA_OK;
}

tsa_status check_ws(void* ws, size_t ws_bytes, size_t need) {
    if (ws_bytes < need) return fail(TSA_ERR_CAPACITY, "workspace of " + std::to_string(ws_bytes) +
                                                           " bytes, need " + std::to_string(need));
    if (need && !ws) return fail(TSA_ERR_INVALID, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(ws) % kAlign) return fail(TSA_ERR_INVALID, "workspace not 256-byte aligned");
    return TSA_OK;
}

char* at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

}  // namespace

extern "C" {

tsa_status tsa_sparse_decode_workspace(const tsa_kv_pool* pool, const tsa_decode_params* p,
                                       size_t* bytes) {
    if (!pool || !p || !bytes) return fail(TSA_ERR_INVALID, "NULL argument");
    if (p->batch < 0 || p->max_len < 0 || p->top_k < 1) return fail(TSA_ERR_INVALID, "bad params");
    if (p->num_q_heads <= 0 || p->num_q_heads % pool->d.num_kv_heads)
        return fail(TSA_ERR_INVALID, "num_q_heads must be a positive multiple of num_kv_heads");
    std::string why;
    const bool attn = tsa::attention_supported(*pool, *p, &why);
    *bytes = layout(*pool, *p, attn).total;
    return TSA_OK;
}

tsa_status tsa_indexer_scores(tsa_kv_pool* pool, int32_t layer, const tsa_decode_params* p,
                              const void* qidx_dev, const float* widx_dev,
                              const int32_t* page_table_dev, int32_t max_pages,
                              const int32_t* seq_lens_dev, float* scores_dev, int32_t ld,
                              void* stream) {
    tsa_status st = check_common(pool, layer, p, page_table_dev, max_pages, seq_lens_dev);
    if (st) return st;
    if ((st = check_indexer(pool, p, qidx_dev, widx_dev))) return st;
    if (ld < p->max_len) return fail(TSA_ERR_INVALID, "ld < max_len");
    if (p->batch == 0 || p->max_len == 0) return TSA_OK;
    if (!scores_dev) return fail(TSA_ERR_INVALID, "scores is NULL");
    hipError_t e = tsa::launch_indexer_scores(*pool, layer, *p, qidx_dev, widx_dev, page_table_dev,
                                              max_pages, seq_lens_dev, scores_dev, ld,
                                              static_cast<hipStream_t>(stream));
    return tsa::hip_check(e, "indexer_score launch");
}

tsa_status tsa_topk(const tsa_decode_params* p, const float* scores_dev, int32_t ld,
                    const int32_t* seq_lens_dev, int32_t* topk_dev, void* stream) {
    if (!p) return fail(TSA_ERR_INVALID, "params is NULL");
    if (p->batch < 0 || p->max_len < 0 || p->top_k < 1) return fail(TSA_ERR_INVALID, "bad params");
    if (ld < p->max_len) return fail(TSA_ERR_INVALID, "ld < max_len");
    tsa_status st = check_topk(p);
    if (st) return st;
    if (p->batch == 0) return TSA_OK;
    if (!scores_dev || !seq_lens_dev || !topk_dev) return fail(TSA_ERR_INVALID, "NULL array");
    hipError_t e = tsa::launch_topk(*p, scores_dev, ld, seq_lens_dev, topk_dev, static_cast<hipStream_t>(stream));
    return tsa::hip_check(e, "topk launch");
}

tsa_status tsa_indexer_topk(tsa_kv_pool* pool, int32_t layer, const tsa_decode_params* p,
                            const void* qidx_dev, const float* widx_dev,
                            const int32_t* page_table_dev, int32_t max_pages,
                            const int32_t* seq_lens_dev, int32_t* topk_dev, void* workspace,
                            size_t ws_bytes, void* stream) {
    tsa_status st = check_common(pool, layer, p, page_table_dev, max_pages, seq_lens_dev);
    if (st) return st;
    if ((st = check_indexer(pool, p, qidx_dev, widx_dev))) return st;
    if ((st = check_topk(p))) return st;
    WsLayout w = layout(*pool, *p, false);
    if ((st = check_ws(workspace, ws_bytes, w.total))) return st;
    if (p->batch == 0) return TSA_OK;
    if (!topk_dev) return fail(TSA_ERR_INVALID, "topk is NULL");
    hipStream_t s = static_cast<hipStream_t>(stream);
    float* scores = reinterpret_cast<float*>(at(workspace, w.scores));
    const int ld = scores_ld(p->max_len);
    hipError_t e = tsa::launch_indexer_scores(*pool, layer, *p, qidx_dev, widx_dev, page_table_dev,
                                              max_pages, seq_lens_dev, scores, ld, s);
    if (e == hipSuccess) e = tsa::launch_topk(*p, scores, ld, seq_lens_dev, topk_dev, s);
    return tsa::hip_check(e, "indexer_topk launch");
}

tsa_status tsa_sparse_attn_gather(tsa_kv_pool* pool, int32_t layer, const tsa_decode_params* p,
                                  const void* q_dev, const int32_t* topk_dev,
                                  const int32_t* page_table_dev, int32_t max_pages,
                                  const int32_t* seq_lens_dev, float* out_dev, void* workspace,
                                  size_t ws_bytes, void* stream) {
    tsa_status st = check_common(pool, layer, p, page_table_dev, max_pages, seq_lens_dev);
    if (st) return st;
    if ((st = check_attn(pool, p, q_dev, out_dev))) return st;
    WsLayout w = layout(*pool, *p, true);
    if ((st = check_ws(workspace, ws_bytes, w.total))) return st;
    if (p->batch == 0) return TSA_OK;
    if (!topk_dev) return fail(TSA_ERR_INVALID, "topk is NULL");
    tsa::AttnPlan plan = tsa::plan_attention(*pool, *p);
    hipError_t e = tsa::launch_attention(*pool, layer, *p, plan, q_dev, topk_dev, page_table_dev,
                                         max_pages, seq_lens_dev, out_dev,
                                         plan.partial_bytes ? at(workspace, w.partial) : nullptr,
                                         static_cast<hipStream_t>(stream));
    return tsa::hip_check(e, "attention launch");
}

tsa_status tsa_sparse_decode_attn(tsa_kv_pool* pool, int32_t layer, const tsa_decode_params* p,
                                  const void* q_dev, const void* qidx_dev, const float* widx_dev,
                                  const int32_t* page_table_dev, int32_t max_pages,
                                  const int32_t* seq_lens_dev, float* out_dev, int32_t* topk_dev,
                                  void* workspace, size_t ws_bytes, void* stream) {
    tsa_status st = check_common(pool, layer, p, page_table_dev, max_pages, seq_lens_dev);
    if (st) return st;
    if ((st = check_indexer(pool, p, qidx_dev, widx_dev))) return st;
    if ((st = check_topk(p))) return st;
    if ((st = check_attn(pool, p, q_dev, out_dev))) return st;
    WsLayout w = layout(*pool, *p, true);
    if ((st = check_ws(workspace, ws_bytes, w.total))) return st;
    if (p->batch == 0) return TSA_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    float* scores = reinterpret_cast<float*>(at(workspace, w.scores));
    int32_t* topk = topk_dev ? topk_dev : reinterpret_cast<int32_t*>(at(workspace, w.topk));
    const int ld = scores_ld(p->max_len);
    tsa::AttnPlan plan = tsa::plan_attention(*pool, *p);
    hipError_t e = tsa::launch_indexer_scores(*pool, layer, *p, qidx_dev, widx_dev, page_table_dev,
                                              max_pages, seq_lens_dev, scores, ld, s);
    if (e == hipSuccess) e = tsa::launch_topk(*p, scores, ld, seq_lens_dev, topk, s);
    if (e == hipSuccess)
        e = tsa::launch_attention(*pool, layer, *p, plan, q_dev, topk, page_table_dev, max_pages,
                                  seq_lens_dev, out_dev,
                                  plan.partial_bytes ? at(workspace, w.partial) : nullptr, s);
    return tsa::hip_check(e, "decode launch");
}

tsa_status tsa_decode_step(tsa_kv_pool* pool, int32_t layer, const tsa_decode_params* p,
                           const void* k_new_dev, const void* v_new_dev, const void* idx_new_dev,
                           int32_t* bad_dev, const void* q_dev, const void* qidx_dev,
                           const float* widx_dev, const int32_t* page_table_dev, int32_t max_pages,
                           const int32_t* seq_lens_dev, float* out_dev, int32_t* topk_dev,
                           void* workspace, size_t ws_bytes, void* stream) {
    tsa_status st = check_common(pool, layer, p, page_table_dev, max_pages, seq_lens_dev);
    if (st) return st;
    if ((st = check_indexer(pool, p, qidx_dev, widx_dev))) return st;
    if ((st = check_topk(p))) return st;
    if ((st = check_attn(pool, p, q_dev, out_dev))) return st;
    if (!pool->k) return fail(TSA_ERR_INVALID, "pool has no device memory");
    if (p->batch > 0 && (!k_new_dev || !idx_new_dev)) return fail(TSA_ERR_INVALID, "NULL new key or indexer rows");
    if (pool->d.v_from_k ? v_new_dev != nullptr : (p->batch > 0 && v_new_dev == nullptr))
        return fail(TSA_ERR_INVALID, "v_new must be NULL exactly when the pool has v_from_k");
    WsLayout w = layout(*pool, *p, true);
    if ((st = check_ws(workspace, ws_bytes, w.total))) return st;
    if (p->batch == 0) return TSA_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    tsa::NewRows rows;
    rows.k = k_new_dev;
    rows.v = v_new_dev;
    rows.idx = idx_new_dev;
    rows.bad = bad_dev;
    if (tsa::fused_step_preferred(*pool, *p))
        return tsa::hip_check(tsa::launch_fused_step(*pool, layer, *p, rows, q_dev, qidx_dev, widx_dev,
                                                     page_table_dev, max_pages, seq_lens_dev, out_dev,
                                                     topk_dev, s),
                              "one-launch step");
    float* scores = reinterpret_cast<float*>(at(workspace, w.scores));
    int32_t* topk = topk_dev ? topk_dev : reinterpret_cast<int32_t*>(at(workspace, w.topk));
    const int ld = scores_ld(p->max_len);
    const bool fused = tsa::indexer_fuses_append(*pool, *p);
    hipError_t e = hipSuccess;
    if (!fused) e = tsa::launch_append_last(*pool, layer, *p, page_table_dev, max_pages, seq_lens_dev, rows, s);
    if (e == hipSuccess)
        e = tsa::launch_indexer_scores(*pool, layer, *p, qidx_dev, widx_dev, page_table_dev, max_pages,
                                       seq_lens_dev, scores, ld, s, fused ? &rows : nullptr);
    tsa::AttnPlan plan = tsa::plan_attention(*pool, *p);
    if (e == hipSuccess) e = tsa::launch_topk(*p, scores, ld, seq_lens_dev, topk, s);
    if (e == hipSuccess)
        e = tsa::launch_attention(*pool, layer, *p, plan, q_dev, topk, page_table_dev, max_pages,
                                  seq_lens_dev, out_dev,
                                  plan.partial_bytes ? at(workspace, w.partial) : nullptr, s);
    return tsa::hip_check(e, "decode step launch");
}

tsa_status tsa_decode_step_noalloc(tsa_kv_pool* pool, int32_t layer, const tsa_decode_params* p,
                                   const void* k_new_dev, const void* v_new_dev, const void* idx_new_dev,
                                   int32_t* bad_dev, const void* q_dev, const void* qidx_dev,
                                   const float* widx_dev, const int32_t* page_table_dev,
                                   int32_t max_pages, const int32_t* seq_lens_dev, float* out_dev,
                                   int32_t* topk_dev, void* stream) {
    if (!pool || !p) return fail(TSA_ERR_INVALID, "NULL argument");
    size_t need = 0;
    tsa_status st = tsa_sparse_decode_workspace(pool, p, &need);
    if (st) return st;
    if (need > kScratchBytes)
        return fail(TSA_ERR_CAPACITY, "the step needs " + std::to_string(need) +
                                          " bytes of workspace; tsa_decode_step_noalloc holds " +
                                          std::to_string(kScratchBytes) + " (use tsa_decode_step)");
    void* ws = nullptr;
    if ((st = current_scratch(&ws))) return st;
    return tsa_decode_step(pool, layer, p, k_new_dev, v_new_dev, idx_new_dev, bad_dev, q_dev, qidx_dev,
                           widx_dev, page_table_dev, max_pages, seq_lens_dev, out_dev, topk_dev, ws,
                           kScratchBytes, stream);
}

tsa_status tsa_decode_step_fused(tsa_kv_pool* pool, int32_t layer, const tsa_decode_params* p,
                                 const void* k_new_dev, const void* v_new_dev, const void* idx_new_dev,
                                 int32_t* bad_dev, const void* q_dev, const void* qidx_dev,
                                 const float* widx_dev, const int32_t* page_table_dev,
                                 int32_t max_pages, const int32_t* seq_lens_dev, float* out_dev,
                                 int32_t* topk_dev, void* stream) {
    tsa_status st = check_common(pool, layer, p, page_table_dev, max_pages, seq_lens_dev);
    if (st) return st;
    if ((st = check_indexer(pool, p, qidx_dev, widx_dev))) return st;
    if ((st = check_attn(pool, p, q_dev, out_dev))) return st;
    std::string why;
    if (!tsa::fused_step_supported(*pool, *p, &why)) return fail(TSA_ERR_UNSUPPORTED, why);
    if (p->batch > 0 && (!k_new_dev || !idx_new_dev)) return fail(TSA_ERR_INVALID, "NULL new key or indexer rows");
    if (pool->d.v_from_k ? v_new_dev != nullptr : (p->batch > 0 && v_new_dev == nullptr))
        return fail(TSA_ERR_INVALID, "v_new must be NULL exactly when the pool has v_from_k");
    if (p->batch == 0) return TSA_OK;
    tsa::NewRows rows;
    rows.k = k_new_dev;
    rows.v = v_new_dev;
    rows.idx = idx_new_dev;
    rows.bad = bad_dev;
    return tsa::hip_check(tsa::launch_fused_step(*pool, layer, *p, rows, q_dev, qidx_dev, widx_dev,
                                                 page_table_dev, max_pages, seq_lens_dev, out_dev,
                                                 topk_dev, static_cast<hipStream_t>(stream)),
                          "one-launch step");
}

}  // extern "C"

// ---- captured step -------------------------------------------------------------------------
// The step's launches are recorded on a private stream with the same entry points an eager
// caller uses (same checks, same plan), so a replay runs exactly the eager kernels.
struct tsa_step_graph {
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
};

extern "C" {

tsa_status tsa_step_graph_create(tsa_kv_pool* pool, int32_t layer, const tsa_decode_params* p,
                                 const tsa_append_args* append, const void* q_dev,
                                 const void* qidx_dev, const float* widx_dev,
                                 const int32_t* page_table_dev, int32_t max_pages,
                                 const int32_t* seq_lens_dev, float* out_dev, int32_t* topk_dev,
                                 void* workspace, size_t ws_bytes, tsa_step_graph** graph) {
    if (!graph) return fail(TSA_ERR_INVALID, "graph is NULL");
    *graph = nullptr;
    if (!pool || !p) return fail(TSA_ERR_INVALID, "NULL argument");
    if (!pool->k) return fail(TSA_ERR_INVALID, "pool has no device memory");
    hipStream_t cs = nullptr;
    tsa_status st = tsa::hip_check(hipStreamCreateWithFlags(&cs, hipStreamNonBlocking), "hipStreamCreate");
    if (st) return st;
    st = tsa::hip_check(hipStreamBeginCapture(cs, hipStreamCaptureModeRelaxed), "hipStreamBeginCapture");
    if (st) {
        (void)hipStreamDestroy(cs);
        return st;
    }
    if (append && append->n_tok > 0)
        st = tsa_kv_append(pool, layer, append->n_tok, append->req_dev, append->pos_dev,
                           page_table_dev, p->batch, max_pages, append->k_src, append->v_src,
                           append->idx_src, append->bad_dev, cs);
    if (st == TSA_OK)
        st = tsa_sparse_decode_attn(pool, layer, p, q_dev, qidx_dev, widx_dev, page_table_dev,
                                    max_pages, seq_lens_dev, out_dev, topk_dev, workspace, ws_bytes, cs);
    const std::string why = st ? std::string(tsa_last_error()) : std::string();
    hipGraph_t g = nullptr;
    const hipError_t ec = hipStreamEndCapture(cs, &g);
    (void)hipStreamDestroy(cs);
    if (st) {
        if (g) (void)hipGraphDestroy(g);
        return fail(st, why);
    }
    if ((st = tsa::hip_check(ec, "hipStreamEndCapture"))) {
        if (g) (void)hipGraphDestroy(g);
        return st;
    }
    hipGraphExec_t exec = nullptr;
    if ((st = tsa::hip_check(hipGraphInstantiate(&exec, g, nullptr, nullptr, 0), "hipGraphInstantiate"))) {
        (void)hipGraphDestroy(g);
        return st;
    }
    *graph = new tsa_step_graph{g, exec};
    return TSA_OK;
}

tsa_status tsa_step_graph_launch(tsa_step_graph* graph, void* stream) {
    if (!graph) return fail(TSA_ERR_INVALID, "graph is NULL");
    return tsa::hip_check(hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream)), "hipGraphLaunch");
}

tsa_status tsa_step_graph_destroy(tsa_step_graph* graph) {
    if (!graph) return TSA_OK;
    tsa_status st = TSA_OK;
    if (graph->exec) st = tsa::hip_check(hipGraphExecDestroy(graph->exec), "hipGraphExecDestroy");
    if (graph->graph) {
        const tsa_status s2 = tsa::hip_check(hipGraphDestroy(graph->graph), "hipGraphDestroy");
        if (st == TSA_OK) st = s2;
    }
    delete graph;
    return st;
}

}  // extern "C"
