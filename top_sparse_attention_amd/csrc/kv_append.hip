// Scatter appended tokens into their pool slots through the page table.
//
// Paged-KV page ("KV cache phân trang, ..."), section "Phân trang": a request's pages need
// not be adjacent; the page table says where each one is.  Logical position t of request r
// lives in physical page table[r][t / page_size], slot t % page_size of that page.
#include "tsa_internal.h"

namespace {

constexpr int kWavesPerBlock = 4;

__device__ inline void copy_row16(uint4* __restrict__ dst, const uint4* __restrict__ src, int n16,
                                  int lane) {
    for (int i = lane; i < n16; i += 64) dst[i] = src[i];
}

__global__ void __launch_bounds__(256) kv_append_kernel(
    int n_tok, const int32_t* __restrict__ req, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ page_table, int n_req, int max_pages, int page_size, int num_pages,
    int64_t layer_slot0, const uint4* __restrict__ k_src, const uint4* __restrict__ v_src,
    const uint4* __restrict__ i_src, uint4* __restrict__ k_pool, uint4* __restrict__ v_pool,
    uint4* __restrict__ i_pool, int k16, int v16, int i16, int32_t* __restrict__ bad) {
    const int w = blockIdx.x * kWavesPerBlock + threadIdx.x / 64;
    const int lane = threadIdx.x & 63;
    if (w >= n_tok) return;
    const int r = req[w];
    const int t = pos[w];
    int page = -1;
    if (r >= 0 && r < n_req && t >= 0 && t / page_size < max_pages)
        page = page_table[int64_t(r) * max_pages + t / page_size];
    if (page < 0 || page >= num_pages) {
        if (lane == 0 && bad) atomicAdd(bad, 1);
        return;
    }
    const int64_t slot = layer_slot0 + int64_t(page) * page_size + t % page_size;
    copy_row16(k_pool + slot * k16, k_src + int64_t(w) * k16, k16, lane);
    if (v_src) copy_row16(v_pool + slot * v16, v_src + int64_t(w) * v16, v16, lane);
    if (i_src) copy_row16(i_pool + slot * i16, i_src + int64_t(w) * i16, i16, lane);
}

}  // namespace

namespace tsa {

hipError_t launch_kv_append(const tsa_kv_pool& pool, int layer, int n_tok, const int32_t* req,
                            const int32_t* pos, const int32_t* page_table, int n_req,
                            int max_pages, const void* k_src, const void* v_src,
                            const void* idx_src, int32_t* bad, hipStream_t s) {
    const tsa_pool_desc& d = pool.d;
    const int k16 = d.num_kv_heads * d.head_dim_k * 2 / 16;
    const int v16 = d.num_kv_heads * d.head_dim_v * 2 / 16;
    const int i16 = d.index_dim * 2 / 16;
    const int64_t layer_slot0 = int64_t(layer) * pool.slots();
    dim3 grid((n_tok + kWavesPerBlock - 1) / kWavesPerBlock);
    hipLaunchKernelGGL(kv_append_kernel, grid, dim3(64 * kWavesPerBlock), 0, s, n_tok, req, pos,
                       page_table, n_req, max_pages, d.page_size, d.num_pages, layer_slot0,
                       static_cast<const uint4*>(k_src), static_cast<const uint4*>(v_src),
                       static_cast<const uint4*>(idx_src), static_cast<uint4*>(pool.k),
                       static_cast<uint4*>(pool.v), static_cast<uint4*>(pool.idx), k16, v16, i16,
                       bad);
    return hipGetLastError();
}

}  // namespace tsa
