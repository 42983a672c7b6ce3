// Tiered KV: copy missed pages from the pinned host copy into their HBM cache slots, and write
// the plan's entries into the device slot table.
//
// GLM5.3 sparse-attention page, HiSparse paragraph: a top-k selection that misses the HBM
// cache loads from host DRAM.  Rather than one DMA call per page (whose per-call cost would
// dominate thousands of misses per layer, and tens of thousands when the unit is a single
// token row), one kernel reads the mapped host memory directly over the host link.  Its
// threads walk the flat list of 16-byte vectors of all missed pages (K page then V page of
// each), with several loads in flight per thread, so small pages and large ones both keep the
// link busy.
#include "tsa_internal.h"

struct tsa_lru;

namespace tsa {
const unsigned char* lru_host_k(const tsa_lru& l);
const unsigned char* lru_host_v(const tsa_lru& l);
size_t lru_page_bytes(const tsa_lru& l);
const tsa_kv_pool& lru_cache(const tsa_lru& l);
}  // namespace tsa

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
// Workgroups of the copy: enough 16-byte loads in flight to fill the host link (64 x 256
// lanes x 8 loads = 2 MiB), few enough that the attention running beside it keeps the CUs.
constexpr int kCopyGroups = 64;

__global__ void __launch_bounds__(kThreads) lru_copy_kernel(const int64_t* __restrict__ keys,
                                                            const int32_t* __restrict__ slots,
                                                            int64_t n, int64_t page_vec,
                                                            const uint4* __restrict__ hk,
                                                            const uint4* __restrict__ hv,
                                                            uint4* __restrict__ ck,
                                                            uint4* __restrict__ cv,
                                                            const int64_t* __restrict__ tab_index,
                                                            const int32_t* __restrict__ tab_slot,
                                                            int64_t n_tab, int32_t* __restrict__ table) {
    const int64_t gid = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    const int64_t gsz = int64_t(gridDim.x) * kThreads;
    for (int64_t i = gid; i < n_tab; i += gsz) table[tab_index[i]] = tab_slot[i];
    // vector e of the list: copy j = e / (2 page_vec), K (first page_vec) or V, vector i
    const int64_t per_copy = 2 * page_vec;
    const int64_t total = n * per_copy;
    for (int64_t e0 = gid; e0 < total; e0 += gsz * kUnroll) {
        uint4 v[kUnroll];
        int64_t dst[kUnroll];
        bool is_v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t e = e0 + int64_t(u) * gsz;
            dst[u] = -1;
            is_v[u] = false;
            if (e < total) {
                const int64_t j = e / per_copy;
                int64_t i = e - j * per_copy;
                is_v[u] = i >= page_vec;
                if (is_v[u]) i -= page_vec;
                v[u] = (is_v[u] ? hv : hk)[keys[j] * page_vec + i];
                dst[u] = int64_t(slots[j]) * page_vec + i;
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            if (dst[u] >= 0) (is_v[u] ? cv : ck)[dst[u]] = v[u];
    }
}

}  // namespace

namespace tsa {

hipError_t launch_lru_copy(const tsa_lru& lru, const int64_t* keys_dev, const int32_t* slots_dev,
                           int64_t n, const int64_t* tab_index_dev, const int32_t* tab_slot_dev,
                           int64_t n_tab, int32_t* table_dev, hipStream_t s) {
    if (n <= 0 && n_tab <= 0) return hipSuccess;
    const tsa_kv_pool& cache = lru_cache(lru);
    const size_t pb = lru_page_bytes(lru);
    if (pb % 16 != 0) return hipErrorInvalidValue;
    const int64_t work = std::max<int64_t>(n * int64_t(pb / 16) * 2, n_tab);
    const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(ceil_div(work, kThreads), kCopyGroups));
    hipLaunchKernelGGL(lru_copy_kernel, dim3(unsigned(grid)), dim3(kThreads), 0, s, keys_dev, slots_dev, n,
                       int64_t(pb / 16), reinterpret_cast<const uint4*>(lru_host_k(lru)),
                       reinterpret_cast<const uint4*>(lru_host_v(lru)), static_cast<uint4*>(cache.k),
                       static_cast<uint4*>(cache.v), tab_index_dev, tab_slot_dev, n_tab, table_dev);
    return hipGetLastError();
}

}  // namespace tsa
