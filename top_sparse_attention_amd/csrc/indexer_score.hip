// Lightning-indexer score of every cached token, read through the page table.
//
// GLM5.3 sparse-attention page ("Cơ chế chú ý thưa (Sparse Attention) trên GLM5.3 ..."),
// lightning-indexer paragraph: the indexer query has several heads and the indexer key one;
// each head's dot product goes through a ReLU and the token's score is the weighted sum over
// heads.  No values, no softmax:
//     score[b][t] = sum_h w[h] * max(0, qI[b][h] . kI[b][t])
// Opening paragraph: selecting the top k needs every cached token, so this kernel streams the
// whole indexer cache of every request: it is bound by HBM bandwidth (1 FLOP per byte).
//
// Layout: a token's indexer key is index_dim bf16 values (16-byte vectors, 8 values each);
// LPT = index_dim / 8 lanes hold one token, so one wave-wide load covers 64 / LPT whole
// tokens (1 KiB of contiguous rows within a page), and the per-token dot product is reduced
// across those LPT lanes.
#include "tsa_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;     // loads in flight per thread
constexpr int kRounds = 4;     // unrolled rounds per workgroup

__device__ inline float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ inline float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

__device__ inline float dot8(const float (&q)[8], const uint4& k) {
    float s = q[0] * bf16_lo(k.x);
    s = fmaf(q[1], bf16_hi(k.x), s);
    s = fmaf(q[2], bf16_lo(k.y), s);
    s = fmaf(q[3], bf16_hi(k.y), s);
    s = fmaf(q[4], bf16_lo(k.z), s);
    s = fmaf(q[5], bf16_hi(k.z), s);
    s = fmaf(q[6], bf16_lo(k.w), s);
    s = fmaf(q[7], bf16_hi(k.w), s);
    return s;
}

template <int LPT>
__device__ inline float reduce_lanes(float v) {
#pragma unroll
    for (int m = LPT / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, LPT);
    return v;
}

template <int LPT, int MAXH>
__global__ void __launch_bounds__(kThreads) indexer_score_kernel(
    const uint4* __restrict__ qidx, const float* __restrict__ widx, int H,
    const int32_t* __restrict__ page_table, int max_pages, int page_size, int page_shift,
    int num_pages, const int32_t* __restrict__ seq_lens, int max_len,
    const uint4* __restrict__ kpool, float* __restrict__ scores, int ld, int tok_per_block) {
    constexpr int kGroups = kThreads / LPT;  // tokens per block-wide step
    const int b = blockIdx.y;
    int len = seq_lens[b];
    len = len < 0 ? 0 : (len > max_len ? max_len : len);
    const int t0 = blockIdx.x * tok_per_block;
    if (t0 >= len) return;
    const int t1 = min(t0 + tok_per_block, len);
    const int sub = threadIdx.x % LPT;
    const int grp = threadIdx.x / LPT;

    float q[MAXH][8];
    float w[MAXH];
#pragma unroll
    for (int h = 0; h < MAXH; ++h) {
        uint4 v = h < H ? qidx[(int64_t(b) * H + h) * LPT + sub] : make_uint4(0, 0, 0, 0);
        q[h][0] = bf16_lo(v.x); q[h][1] = bf16_hi(v.x);
        q[h][2] = bf16_lo(v.y); q[h][3] = bf16_hi(v.y);
        q[h][4] = bf16_lo(v.z); q[h][5] = bf16_hi(v.z);
        q[h][6] = bf16_lo(v.w); q[h][7] = bf16_hi(v.w);
        w[h] = h < H ? widx[h] : 0.f;
    }
    const int32_t* pt = page_table + int64_t(b) * max_pages;
    float* out = scores + int64_t(b) * ld;

    for (int base = t0 + grp; base < t1; base += kGroups * kUnroll) {
        uint4 kv[kUnroll];
        bool ok[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int t = base + u * kGroups;
            int page = -1, slot = 0;
            if (t < t1) {
                if (page_shift >= 0) {
                    page = pt[t >> page_shift];
                    slot = t & (page_size - 1);
                } else {
                    page = pt[t / page_size];
                    slot = t % page_size;
                }
            }
            ok[u] = page >= 0 && page < num_pages;
            kv[u] = ok[u] ? kpool[(int64_t(page) * page_size + slot) * LPT + sub]
                          : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int t = base + u * kGroups;
            float s = 0.f;
#pragma unroll
            for (int h = 0; h < MAXH; ++h) {
                if (h < H) {
                    float d = reduce_lanes<LPT>(dot8(q[h], kv[u]));
                    s = fmaf(w[h], fmaxf(d, 0.f), s);
                }
            }
            if (t < t1 && sub == 0) out[t] = ok[u] ? s : -INFINITY;
        }
    }
}

template <int LPT>
hipError_t launch_lpt(const tsa_kv_pool& pool, int layer, const tsa_decode_params& p,
                      const void* qidx, const float* widx, const int32_t* page_table,
                      int max_pages, const int32_t* seq_lens, float* scores, int ld,
                      hipStream_t s) {
    const tsa_pool_desc& d = pool.d;
    const int tok_per_block = (kThreads / LPT) * kUnroll * kRounds;
    dim3 grid((p.max_len + tok_per_block - 1) / tok_per_block, p.batch);
    int shift = -1;
    if ((d.page_size & (d.page_size - 1)) == 0) {
        shift = 0;
        while ((1 << shift) < d.page_size) ++shift;
    }
    const uint4* kpool = static_cast<const uint4*>(pool.idx) + int64_t(layer) * pool.slots() * LPT;
    if (p.index_heads == 1) {
        hipLaunchKernelGGL((indexer_score_kernel<LPT, 1>), grid, dim3(kThreads), 0, s,
                           static_cast<const uint4*>(qidx), widx, p.index_heads, page_table,
                           max_pages, d.page_size, shift, d.num_pages, seq_lens, p.max_len,
                           kpool, scores, ld, tok_per_block);
    } else {
        hipLaunchKernelGGL((indexer_score_kernel<LPT, 8>), grid, dim3(kThreads), 0, s,
                           static_cast<const uint4*>(qidx), widx, p.index_heads, page_table,
                           max_pages, d.page_size, shift, d.num_pages, seq_lens, p.max_len,
                           kpool, scores, ld, tok_per_block);
    }
    return hipGetLastError();
}

}  // namespace

namespace tsa {

hipError_t launch_indexer_scores(const tsa_kv_pool& pool, int layer, const tsa_decode_params& p,
                                 const void* qidx, const float* widx, const int32_t* page_table,
                                 int max_pages, const int32_t* seq_lens, float* scores, int ld,
                                 hipStream_t s) {
    switch (pool.d.index_dim / 8) {
        case 1: return launch_lpt<1>(pool, layer, p, qidx, widx, page_table, max_pages, seq_lens, scores, ld, s);
        case 2: return launch_lpt<2>(pool, layer, p, qidx, widx, page_table, max_pages, seq_lens, scores, ld, s);
        case 4: return launch_lpt<4>(pool, layer, p, qidx, widx, page_table, max_pages, seq_lens, scores, ld, s);
        case 8: return launch_lpt<8>(pool, layer, p, qidx, widx, page_table, max_pages, seq_lens, scores, ld, s);
        case 16: return launch_lpt<16>(pool, layer, p, qidx, widx, page_table, max_pages, seq_lens, scores, ld, s);
        case 32: return launch_lpt<32>(pool, layer, p, qidx, widx, page_table, max_pages, seq_lens, scores, ld, s);
        case 64: return launch_lpt<64>(pool, layer, p, qidx, widx, page_table, max_pages, seq_lens, scores, ld, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace tsa
