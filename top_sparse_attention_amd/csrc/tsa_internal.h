// Internal declarations shared by the host sources and the kernel launchers of libtsa.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <string>
#include <vector>

#include "tsa.h"

struct tsa_kv_pool {
    tsa_pool_desc d;
    void* k = nullptr;
    void* v = nullptr;
    void* idx = nullptr;
    std::vector<int32_t> free_list;  // pages handed out from the front
    size_t free_head = 0;            // free_list[free_head..] are free
    std::vector<int32_t> refcount;   // per physical page

    int64_t slots() const { return int64_t(d.num_pages) * d.page_size; }
    int32_t free_count() const { return int32_t(free_list.size() - free_head); }
    int32_t pop() { return free_list[free_head++]; }
    void push(int32_t p) { free_list.push_back(p); }
    void compact_free();
};

// Cache-policy suffix of the global-to-LDS loads that stream the KV pool.  The pool is read
// once per step, so the loads are marked non-temporal: measured on the 64 x 32k indexer scan,
// that lifts the stream from 5.1 to 5.8 TB/s (the default policy keeps the lines in the
// caches for reuse that never comes).
#ifndef TSA_LOAD_POLICY
#define TSA_LOAD_POLICY " nt"
#endif

namespace tsa {

// Sets the thread's last-error message and returns `st`.
tsa_status fail(tsa_status st, const std::string& msg);
tsa_status ok();
tsa_status hip_check(hipError_t e, const char* what);

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---- kernel launchers (defined in the .hip sources) ----

// One wave per token: copy rows into the pool slot given by the page table.
hipError_t launch_kv_append(const tsa_kv_pool& pool, int layer, int n_tok, const int32_t* req,
                            const int32_t* pos, const int32_t* page_table, int n_req,
                            int max_pages, const void* k_src, const void* v_src,
                            const void* idx_src, int32_t* bad, hipStream_t s);

// Indexer score of every cached token (fp32 [B][ld]).
constexpr int kMaxIndexHeads = 64;
// Whether the indexer kernels take this pool / head count (reason in *why when not).
bool indexer_supported(const tsa_kv_pool& pool, const tsa_decode_params& p, std::string* why);
// The decode step's new token of every request: rows [B][...] for position seq_len - 1.
struct NewRows {
    const void* k = nullptr;
    const void* v = nullptr;      // null when values alias keys
    const void* idx = nullptr;
    int32_t* bad = nullptr;       // nullable count of tokens whose page is not valid
};
// With `fused`, the scoring launch also writes the new rows and scores them from the new indexer
// rows (only where indexer_fuses_append holds).
hipError_t launch_indexer_scores(const tsa_kv_pool& pool, int layer, const tsa_decode_params& p,
                                 const void* qidx, const float* widx, const int32_t* page_table,
                                 int max_pages, const int32_t* seq_lens, float* scores, int ld,
                                 hipStream_t s, const NewRows* fused = nullptr);
bool indexer_fuses_append(const tsa_kv_pool& pool, const tsa_decode_params& p);
// The new rows alone (no scores), for the shapes the fused launch does not take.
hipError_t launch_append_last(const tsa_kv_pool& pool, int layer, const tsa_decode_params& p,
                              const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                              const NewRows& rows, hipStream_t s);

// Whether the top-k kernel handles this maximum length.
bool topk_supported(int max_len);
hipError_t launch_topk(const tsa_decode_params& p, const float* scores, int ld,
                       const int32_t* seq_lens, int32_t* topk, hipStream_t s);

// Attention planning: how the selected tokens are split across workgroups.
struct AttnPlan {
    int kind = 0;         // 0 = VALU grouped-query kernel, 1 = MFMA latent kernel, 2 = MFMA grouped-query
    int splits = 1;       // workgroups per (request, KV head) along the selected tokens
    int chunk = 0;        // selected tokens per split
    size_t partial_bytes = 0;
    bool wg_merge = false;   // grouped-query kernel: the splits of a pair merge inside one workgroup
};
AttnPlan plan_attention(const tsa_kv_pool& pool, const tsa_decode_params& p);
bool attention_supported(const tsa_kv_pool& pool, const tsa_decode_params& p, std::string* why);
// Matrix-core kernel for the latent (MQA-mode MLA) shape.
bool mfma_latent_applicable(const tsa_kv_pool& pool, const tsa_decode_params& p);
int mfma_latent_chunk(const tsa_decode_params& p, int* splits);
hipError_t launch_attention_mfma(const tsa_kv_pool& pool, int layer, const tsa_decode_params& p,
                                 const AttnPlan& plan, const void* q, const int32_t* topk,
                                 const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                                 float* out, float* part_ml, float* part_acc, hipStream_t s);
// Matrix-core kernel for grouped-query shapes (128-dim keys and values, up to 16 q heads per KV head).
bool gqa_mfma_applicable(const tsa_kv_pool& pool, const tsa_decode_params& p);
int gqa_mfma_chunk(const tsa_kv_pool& pool, const tsa_decode_params& p, int* splits);
bool gqa_wg_merge(const tsa_kv_pool& pool, const tsa_decode_params& p);
constexpr int kGqaMergeSplits = 4;
hipError_t launch_attention_gqa(const tsa_kv_pool& pool, int layer, const tsa_decode_params& p,
                                const AttnPlan& plan, const void* q, const int32_t* topk,
                                const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                                float* out, float* part_ml, float* part_acc, hipStream_t s);
// The whole step of each request in one workgroup, one launch (short contexts).
bool fused_step_supported(const tsa_kv_pool& pool, const tsa_decode_params& p, std::string* why);
// tsa_decode_step takes the one-launch step by itself up to this max_len and this many selected
// (row, KV head) pairs per request, min(top_k, max_len) * num_kv_heads.
constexpr int kFusedAutoMaxLen = 1024;
constexpr int kFusedAutoRows = 128;
bool fused_step_preferred(const tsa_kv_pool& pool, const tsa_decode_params& p);
hipError_t launch_fused_step(const tsa_kv_pool& pool, int layer, const tsa_decode_params& p,
                             const NewRows& rows, const void* q, const void* qidx, const float* widx,
                             const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                             float* out, int32_t* topk, hipStream_t s);
hipError_t launch_attention(const tsa_kv_pool& pool, int layer, const tsa_decode_params& p,
                            const AttnPlan& plan, const void* q, const int32_t* topk,
                            const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                            float* out, void* partial, hipStream_t s);

}  // namespace tsa
