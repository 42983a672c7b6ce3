// Tiered KV: copy missed pages from the pinned host copy into their HBM cache slots.
//
// GLM5.3 sparse-attention page, HiSparse paragraph: a top-k selection that misses the HBM
// cache loads the page from host DRAM.  Rather than one DMA call per 32 KiB page (whose
// per-call cost would dominate thousands of misses per layer), one kernel reads the mapped
// host memory directly over the host link: a few workgroups walk the list of missed pages,
// each lane moving 16-byte vectors, K page then V page, with several loads in flight.
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
                                                            uint4* __restrict__ cv) {
    for (int64_t j = blockIdx.x; j < n; j += gridDim.x) {
        const int64_t key = keys[j];
        const int64_t slot = slots[j];
#pragma unroll
        for (int part = 0; part < 2; ++part) {
            const uint4* src = (part == 0 ? hk : hv) + key * page_vec;
            uint4* dst = (part == 0 ? ck : cv) + slot * page_vec;
            for (int64_t i = threadIdx.x; i < page_vec; i += int64_t(kThreads) * kUnroll) {
                uint4 v[kUnroll];
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    const int64_t e = i + int64_t(u) * kThreads;
                    if (e < page_vec) v[u] = src[e];
                }
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    const int64_t e = i + int64_t(u) * kThreads;
                    if (e < page_vec) dst[e] = v[u];
                }
            }
        }
    }
}

}  // namespace

namespace tsa {

hipError_t launch_lru_copy(const tsa_lru& lru, const int64_t* keys_dev, const int32_t* slots_dev,
                           int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const tsa_kv_pool& cache = lru_cache(lru);
    const size_t pb = lru_page_bytes(lru);
    if (pb % 16 != 0) return hipErrorInvalidValue;
    const int64_t grid = std::min<int64_t>(n, kCopyGroups);
    hipLaunchKernelGGL(lru_copy_kernel, dim3(unsigned(grid)), dim3(kThreads), 0, s, keys_dev, slots_dev, n,
                       int64_t(pb / 16), reinterpret_cast<const uint4*>(lru_host_k(lru)),
                       reinterpret_cast<const uint4*>(lru_host_v(lru)), static_cast<uint4*>(cache.k),
                       static_cast<uint4*>(cache.v));
    return hipGetLastError();
}

}  // namespace tsa
