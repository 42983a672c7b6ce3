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
// A token's indexer key is index_dim bf16 values, stored contiguously, so a page of the indexer
// cache is one contiguous run of page_size rows.  Two kernels:
//  * pages of at least 16 tokens and index_dim 32..256 (every workload here): each wave owns a
//    contiguous run of a request's tokens and streams it, 16 rows at a time, through a private
//    ring of LDS slots with global-to-LDS loads (described where it is defined below).  One
//    head is dotted on the vector ALUs; 2..64 heads make the slot a [heads x dim] . [dim x 16]
//    contraction, which runs on the matrix cores (H FLOP per byte read: at 64 heads the vector
//    ALUs could not keep up with the stream);
//  * smaller pages, up to 8 heads: LPT = index_dim / 8 lanes hold one token in registers
//    (16-byte vectors, 8 values each), so one wave-wide load covers 64 / LPT whole tokens, and
//    each head's dot product is reduced across those LPT lanes.
// Positions whose page-table entry is not a valid page score -inf.
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

// ---------------------------------------------------------------------------------------
// Runs of tokens per wave, the LDS ring of the multi-head kernel and the score stage of both
// streaming kernels.
typedef __attribute__((address_space(3))) unsigned char lds_u8;

constexpr int kRing = 4;              // slots per wave
constexpr int kUnit = 16;             // tokens per slot
constexpr int kMaxTpw = 4096;         // tokens per wave at most
constexpr int kMinPage = 16;          // smallest page size this kernel takes
constexpr int kPagesPerWave = kMaxTpw / kMinPage + 2;
constexpr int kStage = 512;           // scores staged per wave before they are stored

__device__ __forceinline__ void load_lds16(const void* gsrc, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" TSA_LOAD_POLICY
                 :
                 : "v"(gsrc), "s"(lds)
                 : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ float sum4groups(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int D>
struct IdxGeo {
    static constexpr int kRowBytes = 2 * D;
    static constexpr int kCpr = D / 8;                    // 16-byte chunks per row
    static constexpr int kSlotBytes = kUnit * kRowBytes;
    static constexpr int kLoads = kSlotBytes / 1024;      // wave-wide loads per slot
    static constexpr int kPart = D / 4;                   // dims per lane
    static constexpr int kPartChunks = kPart / 8;
    static constexpr int kRowsPer256 = 256 / kRowBytes > 0 ? 256 / kRowBytes : 1;
    static_assert(kSlotBytes % 1024 == 0, "a slot is a whole number of wave loads");
};

// stored chunk position of logical chunk c of slot row r
template <int D>
__device__ __forceinline__ int idx_swz(int r, int c) {
    using G = IdxGeo<D>;
    const int m = G::kCpr < 16 ? G::kCpr - 1 : 15;
    return c ^ ((r / G::kRowsPer256) & m);
}

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

// The decode step's own token: request b's new rows land at position seq_len[b] - 1, through the
// page table like kv_append's.  Fused into the scoring launch, the token's score is taken from its
// new indexer row directly and the scoring workgroups stop one position short, so no workgroup
// reads a row the launch writes.
struct AppendLast {
    const uint4* k_src;        // [B] rows of num_kv_heads * head_dim_k bf16
    const uint4* v_src;        // [B] value rows, or null when values alias keys
    const uint4* i_src;        // [B] indexer rows
    uint4* k_pool;             // layer bases
    uint4* v_pool;
    uint4* i_pool;
    int k16, v16, i16;         // 16-byte vectors per row
    int32_t* bad;              // nullable count of tokens whose page-table entry is not a page
};

__device__ inline float wave_sum_f(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

// one wave per request b (strided over the waves of the caller's grid); with `score`, also
// writes the token's indexer score (-inf when its page is not valid)
__device__ void append_last(const AppendLast& f, int wave_id, int n_waves, int batch,
                            const int32_t* __restrict__ page_table, int max_pages, int page_size,
                            int num_pages, const int32_t* __restrict__ seq_lens, int max_len,
                            bool score, const uint16_t* __restrict__ qidx,
                            const float* __restrict__ widx, int H, int D, float* __restrict__ scores,
                            int ld) {
    const int lane = threadIdx.x & 63;
    for (int b = wave_id; b < batch; b += n_waves) {
        int len = seq_lens[b];
        len = len < 0 ? 0 : (len > max_len ? max_len : len);
        if (len == 0) continue;
        const int t = len - 1;
        const int page = page_table[int64_t(b) * max_pages + t / page_size];
        const bool ok = page >= 0 && page < num_pages;
        if (ok) {
            const int64_t slot = int64_t(page) * page_size + t % page_size;
            for (int i = lane; i < f.k16; i += 64) f.k_pool[slot * f.k16 + i] = f.k_src[int64_t(b) * f.k16 + i];
            if (f.v_src)
                for (int i = lane; i < f.v16; i += 64) f.v_pool[slot * f.v16 + i] = f.v_src[int64_t(b) * f.v16 + i];
            for (int i = lane; i < f.i16; i += 64) f.i_pool[slot * f.i16 + i] = f.i_src[int64_t(b) * f.i16 + i];
        } else if (lane == 0 && f.bad) {
            atomicAdd(f.bad, 1);
        }
        if (!score) continue;
        // lane h dots head h's query with the new key (every lane reads the same key chunks),
        // then the weighted ReLU terms are summed over the lanes
        float term = 0.f;
        if (ok && lane < H) {
            const uint4* kn = f.i_src + int64_t(b) * f.i16;
            const uint4* qh = reinterpret_cast<const uint4*>(qidx + (int64_t(b) * H + lane) * D);
            float d = 0.f;
            for (int c = 0; c < f.i16; ++c) {
                const uint4 x = qh[c], y = kn[c];
                const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ys[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    d = fmaf(__uint_as_float(xs[e] << 16), __uint_as_float(ys[e] << 16), d);
                    d = fmaf(__uint_as_float(xs[e] & 0xffff0000u), __uint_as_float(ys[e] & 0xffff0000u), d);
                }
            }
            term = widx[lane] * fmaxf(d, 0.f);
        }
        const float sc = wave_sum_f(term);
        if (lane == 0) scores[int64_t(b) * ld + t] = ok ? sc : -INFINITY;
    }
}

__global__ void __launch_bounds__(256) append_last_kernel(AppendLast f, int batch,
                                                          const int32_t* __restrict__ page_table,
                                                          int max_pages, int page_size, int num_pages,
                                                          const int32_t* __restrict__ seq_lens,
                                                          int max_len) {
    append_last(f, blockIdx.x * 4 + (threadIdx.x >> 6), gridDim.x * 4, batch, page_table, max_pages,
                page_size, num_pages, seq_lens, max_len, false, nullptr, nullptr, 0, 0, nullptr, 0);
}

// Single-head indexer, register stream.  Wave w owns a run of one request's tokens.  One
// wave-wide load brings 1 KiB = kRowsPerLoad key rows into registers (each row spread over
// D/8 lanes, 16 bytes each, with the non-temporal policy); each lane dots its 8 dims with the
// matching 8 query dims (four v_dot2 on bf16 pairs), and a DPP sum over the row's lanes gives
// the token's dot product.  A batch of kStreamLoads loads is issued before any is used.  Scores
// are staged in LDS and stored kStage at a time with 16-byte stores.  On 64 x 32k tokens this
// streams 545 MB in 82 us against 87 us for the LDS-ring kernel below.  The multi-head indexer
// keeps the LDS ring: its matrix-core version of this stream (query rows of 64 heads held in
// registers, 16-token slots loaded in the MFMA operand order) measured 107-132 us against 94 us,
// since the registers the queries take leave too few waves and loads in flight.
template <int D>
struct StreamGeo {
    static constexpr int kLanesPerRow = D / 8;
    static constexpr int kRowsPerLoad = 64 / kLanesPerRow;
    static_assert(kLanesPerRow >= 4 && kLanesPerRow <= 32, "D in 32 .. 256");
};
constexpr int kStreamLoads = 4;      // wave loads per batch (4 measured faster than 2, 8 or 16, and
                                      // than keeping two batches in flight)
constexpr int kStreamWaves = 4096;    // waves per launch over the whole batch

template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// sum over each aligned group of L lanes (L = 4, 8, 16 or 32), the result in every lane
template <int L>
__device__ __forceinline__ float group_sum(float x) {
    x = dpp_add<0xB1>(x);                         // quad_perm [1, 0, 3, 2]
    x = dpp_add<0x4E>(x);                         // quad_perm [2, 3, 0, 1]
    if constexpr (L >= 8) x = dpp_add<0x141>(x);  // row_half_mirror: the other quad of 8
    if constexpr (L >= 16) x = dpp_add<0x140>(x); // row_mirror: the other half of 16
    if constexpr (L >= 32) {
        const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    }
    return x;
}

template <int D, bool ALIGNED>
__global__ void __launch_bounds__(256) indexer_score_stream_kernel(
    const uint16_t* __restrict__ qidx, const float* __restrict__ widx,
    const int32_t* __restrict__ page_table, int max_pages, int page_size, int page_shift,
    int num_pages, const int32_t* __restrict__ seq_lens, int max_len,
    const uint16_t* __restrict__ kpool, float* __restrict__ scores, int ld, int tok_per_wave,
    int batch, AppendLast fused) {
    using G = StreamGeo<D>;
    constexpr int R = G::kRowsPerLoad, U = kStreamLoads;
    static_assert(kStage % (U * R) == 0, "a stage is a whole number of batches");
    __shared__ int32_t wpages[4][kPagesPerWave];   // page ids of each wave's token run
    __shared__ __align__(16) float stage[4][kStage];
    const bool append = fused.k_src != nullptr;
    if (append && blockIdx.y == 0) {     // the first row of workgroups (dispatched first): the new tokens
        append_last(fused, blockIdx.x * 4 + (threadIdx.x >> 6), gridDim.x * 4, batch, page_table,
                    max_pages, page_size, num_pages, seq_lens, max_len, true, qidx, widx, 1, D, scores, ld);
        return;
    }
    const int b = blockIdx.y - (append ? 1 : 0);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane / G::kLanesPerRow, c = lane % G::kLanesPerRow;
    int len = seq_lens[b];
    len = len < 0 ? 0 : (len > max_len ? max_len : len);
    const int t0 = (blockIdx.x * 4 + wave) * tok_per_wave;
    const int t1 = min(t0 + tok_per_wave, append ? len - 1 : len);   // the new token is scored above
    if (t0 >= t1) return;
    const int32_t* pt = page_table + int64_t(b) * max_pages;
    const int pg0 = ALIGNED ? (t0 >> page_shift) : t0 / page_size;
    const int pg1 = ALIGNED ? ((t1 - 1) >> page_shift) : (t1 - 1) / page_size;
    int32_t* wp = wpages[wave];
    for (int i = lane; i <= pg1 - pg0; i += 64) {
        const int32_t pid = pt[pg0 + i];
        wp[i] = (pid >= 0 && pid < num_pages) ? pid : -1;
    }
    uint32_t q[4];
    {
        const uint4 v = reinterpret_cast<const uint4*>(qidx + int64_t(b) * D)[c];
        q[0] = v.x; q[1] = v.y; q[2] = v.z; q[3] = v.w;
    }
    const float w = widx[0];
    float* srow = scores + int64_t(b) * ld;
    float* st = stage[wave];
    const int n_loads = (t1 - t0 + R - 1) / R;
    auto issue = [&](uint4 (&v)[U], int (&pgs)[U], int i) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // the row this lane loads: token t (clamped into the run, masked below)
            const int t = min(t0 + (i + u) * R + r, t1 - 1);
            pgs[u] = ALIGNED ? wp[(t >> page_shift) - pg0] : wp[t / page_size - pg0];
            const int off = ALIGNED ? (t & (page_size - 1)) : t % page_size;
            const int64_t row = pgs[u] >= 0 ? int64_t(pgs[u]) * page_size + off : 0;
            const uint4* src = reinterpret_cast<const uint4*>(kpool + row * D) + c;
            v[u] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src)));
        }
    };
    auto consume = [&](const uint4 (&v)[U], const int (&pgs)[U], int i) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float d = dot2(q[0], v[u].x, 0.f);
            d = dot2(q[1], v[u].y, d);
            d = dot2(q[2], v[u].z, d);
            d = dot2(q[3], v[u].w, d);
            d = group_sum<G::kLanesPerRow>(d);
            const int rel = (i + u) * R + r;
            if (c == 0 && t0 + rel < t1) st[rel & (kStage - 1)] = pgs[u] >= 0 ? w * fmaxf(d, 0.f) : -INFINITY;
        }
        // Scores leave in bursts of kStage (16-byte stores of a contiguous run) rather than a few
        // bytes per load: stores spread between the key loads cost the stream several percent.
        if (((i + U) * R) % kStage == 0 || i + U >= n_loads) {
            const int s0 = ((i * R) / kStage) * kStage;        // run-relative start of this stage
            const int n = min(kStage, t1 - t0 - s0);
            float* dst = srow + t0 + s0;
            if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0) {     // the workspace's rows always are
                for (int e = 4 * lane; e < n; e += 256) {
                    if (e + 4 <= n)
                        *reinterpret_cast<float4*>(dst + e) = *reinterpret_cast<const float4*>(st + e);
                    else
                        for (int f = e; f < n; ++f) dst[f] = st[f];
                }
            } else {
                for (int e = lane; e < n; e += 64) dst[e] = st[e];
            }
        }
    };
    for (int i = 0; i < n_loads; i += U) {
        uint4 v[U];
        int pgs[U];
        issue(v, pgs, i);
        consume(v, pgs, i);
    }
}

// Multi-head indexer (LDS ring).  Every wave streams its own run of tokens through a private
// ring of LDS slots with global-to-LDS loads.  A slot holds 16 token rows, stored with their
// 16-byte chunks XOR-swizzled so that the 16 rows read in parallel fall on distinct LDS banks.
// ALIGNED: page_size is a power of two and a multiple of the 16-token slot, so every slot lies in
// one page and the page id is the same for the whole wave.
//
// H <= 16 NB heads on the matrix cores.  The heads are the rows and the slot's 16 tokens
// the columns of S = Q K^T, one 16 x 16 x 32 MFMA per (16-head block, 32 dims).  The contraction
// index is free to be relabelled, so MFMA k = 8 g + i of step c stands for dim g * D/4 + 8 c + i:
// lane group g (lanes 16 g .. 16 g + 15) then reads one quarter of its token's row, and the query
// registers follow the same relabelling.  The MFMA leaves heads
// 4 g .. 4 g + 3 of every block with lane group g, so each lane applies ReLU and the weights to
// its heads and the four groups are summed across lanes.  Heads H .. 16 NB - 1 are zero rows
// with weight 0 and add exactly 0.
template <int D, bool ALIGNED, int NB>
__global__ void __launch_bounds__(256) indexer_score_lds_kernel(
    const uint16_t* __restrict__ qidx, const float* __restrict__ widx, int H,
    const int32_t* __restrict__ page_table, int max_pages, int page_size, int page_shift,
    int num_pages, const int32_t* __restrict__ seq_lens, int max_len,
    const uint16_t* __restrict__ kpool, float* __restrict__ scores, int ld, int tok_per_wave,
    int batch, AppendLast fused) {
    using G = IdxGeo<D>;
    static_assert(NB > 0, "one head takes the register stream kernel");
    __shared__ __align__(16) unsigned char ring[4][kRing][G::kSlotBytes];
    __shared__ int32_t wpages[4][kPagesPerWave];   // page ids of each wave's token run
    __shared__ __align__(16) float stage[4][kStage];   // scores of each wave, stored kStage at a time
    const bool append = fused.k_src != nullptr;
    if (append && blockIdx.y == 0) {     // the first row of workgroups (dispatched first): the new tokens
        append_last(fused, blockIdx.x * 4 + (threadIdx.x >> 6), gridDim.x * 4, batch, page_table,
                    max_pages, page_size, num_pages, seq_lens, max_len, true, qidx, widx, H, D,
                    scores, ld);
        return;
    }
    const int b = blockIdx.y - (append ? 1 : 0);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j16 = lane & 15, g16 = lane >> 4;
    int len = seq_lens[b];
    len = len < 0 ? 0 : (len > max_len ? max_len : len);
    const int t0 = (blockIdx.x * 4 + wave) * tok_per_wave;
    const int t1 = min(t0 + tok_per_wave, append ? len - 1 : len);   // the new token is scored above
    if (t0 >= t1) return;
    const int n_units = (t1 - t0 + kUnit - 1) / kUnit;
    const int32_t* pt = page_table + int64_t(b) * max_pages;
    // the run's page ids, staged once so that load addresses do not wait on the page table
    const int pg0 = ALIGNED ? (t0 >> page_shift) : t0 / page_size;
    const int pg1 = ALIGNED ? ((t1 - 1) >> page_shift) : (t1 - 1) / page_size;
    int32_t* wp = wpages[wave];
    for (int i = lane; i <= pg1 - pg0; i += 64) {
        const int32_t pid = pt[pg0 + i];
        wp[i] = (pid >= 0 && pid < num_pages) ? pid : -1;
    }

    // rows of head j16 of every block (the MFMA A operand), and the weights of the heads this
    // lane's accumulator rows hold
    uint4 qm[NB][G::kPartChunks];
    float wm[NB][4];
    {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int h = nb * 16 + j16;
            const uint4* src = reinterpret_cast<const uint4*>(qidx + (int64_t(b) * H + h) * D + g16 * G::kPart);
#pragma unroll
            for (int c = 0; c < G::kPartChunks; ++c) qm[nb][c] = h < H ? src[c] : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int hw = nb * 16 + 4 * g16 + r;
                wm[nb][r] = hw < H ? widx[hw] : 0.f;
            }
        }
    }
    wait_vm<0>();

    const uint32_t ring_base = uint32_t(reinterpret_cast<uintptr_t>((lds_u8*)(&ring[wave][0][0])));
    // load k of a slot fills stored chunks 64 k .. 64 k + 63 (row-major); each lane fetches the
    // logical chunk that belongs at its stored position
    int lrow[G::kLoads], lsrc[G::kLoads];   // lane constants: slot row, element offset in the row
#pragma unroll
    for (int k = 0; k < G::kLoads; ++k) {
        const int pc = k * 64 + lane;
        lrow[k] = pc / G::kCpr;
        lsrc[k] = idx_swz<D>(lrow[k], pc % G::kCpr) * 8;
    }
    auto issue = [&](int u) {
        const uint32_t slot = ring_base + uint32_t((u % kRing) * G::kSlotBytes);
        const int tu = t0 + u * kUnit;
        if (ALIGNED) {
            // one page for the slot; rows past the run re-read the slot's first row
            const int page = __builtin_amdgcn_readfirstlane(wp[(tu >> page_shift) - pg0]);
            const int64_t row0 = int64_t(page < 0 ? 0 : page) * page_size + (tu & (page_size - 1));
#pragma unroll
            for (int k = 0; k < G::kLoads; ++k) {
                const int r = tu + lrow[k] < t1 ? lrow[k] : 0;
                load_lds16(kpool + (row0 + r) * D + lsrc[k],
                           __builtin_amdgcn_readfirstlane(slot + uint32_t(k * 1024)));
            }
        } else {
#pragma unroll
            for (int k = 0; k < G::kLoads; ++k) {
                const int t = tu + lrow[k];
                int page = -1, off = 0;
                if (t < t1) {
                    page = wp[t / page_size - pg0];
                    off = t % page_size;
                }
                const uint16_t* src = kpool + (page >= 0 ? (int64_t(page) * page_size + off) * D + lsrc[k] : 0);
                load_lds16(src, __builtin_amdgcn_readfirstlane(slot + uint32_t(k * 1024)));
            }
        }
    };
    for (int u = 0; u < kRing - 1 && u < n_units; ++u) issue(u);

    const int rd_row = j16 * G::kRowBytes;
    int rd_off[G::kPartChunks];
#pragma unroll
    for (int c = 0; c < G::kPartChunks; ++c) rd_off[c] = rd_row + idx_swz<D>(j16, g16 * G::kPartChunks + c) * 16;

    for (int u = 0; u < n_units; ++u) {
        if (u + kRing - 1 < n_units) {
            issue(u + kRing - 1);
            wait_vm<(kRing - 1) * G::kLoads>();
        } else if (u + 2 < n_units) {
            wait_vm<2 * G::kLoads>();
        } else if (u + 1 < n_units) {
            wait_vm<G::kLoads>();
        } else {
            wait_vm<0>();
        }
        const unsigned char* slot = &ring[wave][u % kRing][0];
        float sc;
        {
            f32x4 acc[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < G::kPartChunks; ++c) {
                const bf16x8 kb = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(slot + rd_off[c]));
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qm[nb][c]),
                                                                      kb, acc[nb], 0, 0, 0);
            }
            float part = 0.f;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
                for (int r = 0; r < 4; ++r) part = fmaf(wm[nb][r], fmaxf(acc[nb][r], 0.f), part);
            }
            sc = sum4groups(part);
        }
        const int t = t0 + u * kUnit + j16;
        if (g16 == 0 && t < t1) {
            const int page = ALIGNED ? wp[(t >> page_shift) - pg0] : wp[t / page_size - pg0];
            stage[wave][(u * kUnit + j16) & (kStage - 1)] = page >= 0 ? sc : -INFINITY;
        }
        // Scores leave in bursts of kStage (16-byte stores of a contiguous run) rather than 64
        // bytes per slot: stores spread between the key loads cost the stream about 5 % more.
        if ((u + 1) % (kStage / kUnit) == 0 || u + 1 == n_units) {
            const int s0 = t0 + (u / (kStage / kUnit)) * kStage;
            const int n = min(kStage, t1 - s0);
            float* dst = scores + int64_t(b) * ld + s0;
            const float* src = stage[wave];
            if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0) {     // the workspace's rows always are
                for (int i = 4 * lane; i < n; i += 256) {
                    if (i + 4 <= n)
                        *reinterpret_cast<float4*>(dst + i) = *reinterpret_cast<const float4*>(src + i);
                    else
                        for (int e = i; e < n; ++e) dst[e] = src[e];
                }
            } else {
                for (int i = lane; i < n; i += 64) dst[i] = src[i];
            }
        }
    }
}

template <int D, int NB>
hipError_t launch_lds(const tsa_kv_pool& pool, int layer, const tsa_decode_params& p,
                      const void* qidx, const float* widx, const int32_t* page_table,
                      int max_pages, const int32_t* seq_lens, float* scores, int ld,
                      hipStream_t s, int shift, const AppendLast& fused) {
    const tsa_pool_desc& d = pool.d;
    // about 4096 waves over the whole batch (16 per CU, eight resident at a time), at least a
    // few slots each: shorter runs even out the end of the launch (measured 92.4 against 93.6 us
    // with 2048 waves on 64 x 32k)
    const int64_t total = int64_t(p.batch) * p.max_len;
    int tpw = int((total + 4095) / 4096);
    tpw = std::max(kUnit * 4, std::min(tpw, kMaxTpw));
    tpw = (tpw + kUnit - 1) / kUnit * kUnit;
    // at least one column of workgroups: a batch whose requests are all empty still launches
    // (every scoring workgroup exits at once; the append row, if any, writes nothing)
    dim3 grid(std::max(1, (p.max_len + 4 * tpw - 1) / (4 * tpw)), p.batch + (fused.k_src ? 1 : 0));
    const uint16_t* kpool = static_cast<const uint16_t*>(pool.idx) + int64_t(layer) * pool.slots() * D;
    const bool aligned = shift >= 0 && d.page_size % kUnit == 0;
    if (aligned)
        hipLaunchKernelGGL((indexer_score_lds_kernel<D, true, NB>), grid, dim3(256), 0, s,
                           static_cast<const uint16_t*>(qidx), widx, p.index_heads, page_table, max_pages,
                           d.page_size, shift, d.num_pages, seq_lens, p.max_len, kpool, scores, ld, tpw,
                           p.batch, fused);
    else
        hipLaunchKernelGGL((indexer_score_lds_kernel<D, false, NB>), grid, dim3(256), 0, s,
                           static_cast<const uint16_t*>(qidx), widx, p.index_heads, page_table, max_pages,
                           d.page_size, shift, d.num_pages, seq_lens, p.max_len, kpool, scores, ld, tpw,
                           p.batch, fused);
    return hipGetLastError();
}

template <int D>
hipError_t launch_stream(const tsa_kv_pool& pool, int layer, const tsa_decode_params& p,
                         const void* qidx, const float* widx, const int32_t* page_table,
                         int max_pages, const int32_t* seq_lens, float* scores, int ld,
                         hipStream_t s, int shift, const AppendLast& fused) {
    const tsa_pool_desc& d = pool.d;
    // about 4096 waves over the whole batch (16 per CU), at least a few loads each
    const int64_t total = int64_t(p.batch) * p.max_len;
    int tpw = int((total + kStreamWaves - 1) / kStreamWaves);
    tpw = std::max(kUnit * 4, std::min(tpw, kMaxTpw));
    tpw = (tpw + kUnit - 1) / kUnit * kUnit;
    dim3 grid(std::max(1, (p.max_len + 4 * tpw - 1) / (4 * tpw)), p.batch + (fused.k_src ? 1 : 0));
    const uint16_t* kpool = static_cast<const uint16_t*>(pool.idx) + int64_t(layer) * pool.slots() * D;
    const bool aligned = shift >= 0 && d.page_size % kUnit == 0;
    if (aligned)
        hipLaunchKernelGGL((indexer_score_stream_kernel<D, true>), grid, dim3(256), 0, s,
                           static_cast<const uint16_t*>(qidx), widx, page_table, max_pages,
                           d.page_size, shift, d.num_pages, seq_lens, p.max_len, kpool, scores, ld, tpw,
                           p.batch, fused);
    else
        hipLaunchKernelGGL((indexer_score_stream_kernel<D, false>), grid, dim3(256), 0, s,
                           static_cast<const uint16_t*>(qidx), widx, page_table, max_pages,
                           d.page_size, shift, d.num_pages, seq_lens, p.max_len, kpool, scores, ld, tpw,
                           p.batch, fused);
    return hipGetLastError();
}

template <int D>
hipError_t launch_lds_heads(const tsa_kv_pool& pool, int layer, const tsa_decode_params& p,
                            const void* qidx, const float* widx, const int32_t* page_table,
                            int max_pages, const int32_t* seq_lens, float* scores, int ld,
                            hipStream_t s, int shift, const AppendLast& f) {
    const int h = p.index_heads;
    if (h == 1) return launch_stream<D>(pool, layer, p, qidx, widx, page_table, max_pages, seq_lens, scores, ld, s, shift, f);
    if (h <= 16) return launch_lds<D, 1>(pool, layer, p, qidx, widx, page_table, max_pages, seq_lens, scores, ld, s, shift, f);
    if (h <= 32) return launch_lds<D, 2>(pool, layer, p, qidx, widx, page_table, max_pages, seq_lens, scores, ld, s, shift, f);
    if (h <= tsa::kMaxIndexHeads) return launch_lds<D, 4>(pool, layer, p, qidx, widx, page_table, max_pages, seq_lens, scores, ld, s, shift, f);
    return hipErrorInvalidValue;
}

template <int LPT>
hipError_t launch_lpt(const tsa_kv_pool& pool, int layer, const tsa_decode_params& p,
                      const void* qidx, const float* widx, const int32_t* page_table,
                      int max_pages, const int32_t* seq_lens, float* scores, int ld,
                      hipStream_t s) {
    const tsa_pool_desc& d = pool.d;
    const int tok_per_block = (kThreads / LPT) * kUnroll * kRounds;
    dim3 grid(std::max(1, (p.max_len + tok_per_block - 1) / tok_per_block), p.batch);
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

static bool lds_kernel_takes(const tsa_kv_pool& pool) {
    const int D = pool.d.index_dim;
    return pool.d.page_size >= kMinPage && (D == 32 || D == 64 || D == 128 || D == 256);
}

bool indexer_supported(const tsa_kv_pool& pool, const tsa_decode_params& p, std::string* why) {
    const int D = pool.d.index_dim;
    if (D < 8 || D % 8 || (D / 8 & (D / 8 - 1)) || D / 8 > 64) {
        *why = "index_dim must be 8 x a power of two, <= 512";
        return false;
    }
    const int hmax = lds_kernel_takes(pool) ? kMaxIndexHeads : 8;
    if (p.index_heads < 1 || p.index_heads > hmax) {
        *why = "index_heads must be in 1.." + std::to_string(hmax) +
               (hmax == 8 ? " (more heads need index_dim 32..256 and pages of >= 16 tokens)" : "");
        return false;
    }
    return true;
}

static AppendLast append_args(const tsa_kv_pool& pool, int layer, const NewRows* rows) {
    AppendLast f{};
    if (!rows) return f;
    const tsa_pool_desc& d = pool.d;
    const int64_t slot0 = int64_t(layer) * pool.slots();
    f.k16 = d.num_kv_heads * d.head_dim_k * 2 / 16;
    f.v16 = d.num_kv_heads * d.head_dim_v * 2 / 16;
    f.i16 = d.index_dim * 2 / 16;
    f.k_src = static_cast<const uint4*>(rows->k);
    f.v_src = static_cast<const uint4*>(rows->v);
    f.i_src = static_cast<const uint4*>(rows->idx);
    f.k_pool = static_cast<uint4*>(pool.k) + slot0 * f.k16;
    f.v_pool = pool.v ? static_cast<uint4*>(pool.v) + slot0 * f.v16 : nullptr;
    f.i_pool = static_cast<uint4*>(pool.idx) + slot0 * f.i16;
    f.bad = rows->bad;
    return f;
}

// The fused writes take one extra row of workgroups, which pushes as many scoring workgroups into
// a second round of the grid; they start once the first new-token workgroups are done.  With one
// head that costs less than the separate launch it replaces (64 x 32k: 162.1 against 165.3 us
// per step); with 64 heads, whose per-token score takes longer, it lost (194 against 175 us).
bool indexer_fuses_append(const tsa_kv_pool& pool, const tsa_decode_params& p) {
    return lds_kernel_takes(pool) && p.index_heads == 1;
}

hipError_t launch_append_last(const tsa_kv_pool& pool, int layer, const tsa_decode_params& p,
                              const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                              const NewRows& rows, hipStream_t s) {
    const AppendLast f = append_args(pool, layer, &rows);
    const int grid = int(std::max<int64_t>(1, ceil_div(p.batch, 4)));
    hipLaunchKernelGGL(append_last_kernel, dim3(grid), dim3(256), 0, s, f, p.batch, page_table,
                       max_pages, pool.d.page_size, pool.d.num_pages, seq_lens, p.max_len);
    return hipGetLastError();
}

hipError_t launch_indexer_scores(const tsa_kv_pool& pool, int layer, const tsa_decode_params& p,
                                 const void* qidx, const float* widx, const int32_t* page_table,
                                 int max_pages, const int32_t* seq_lens, float* scores, int ld,
                                 hipStream_t s, const NewRows* fused) {
    if (fused && !indexer_fuses_append(pool, p)) return hipErrorInvalidValue;
    const AppendLast f = append_args(pool, layer, fused);
    if (lds_kernel_takes(pool)) {
        int shift = -1;
        if ((pool.d.page_size & (pool.d.page_size - 1)) == 0) {
            shift = 0;
            while ((1 << shift) < pool.d.page_size) ++shift;
        }
        switch (pool.d.index_dim) {
            case 32: return launch_lds_heads<32>(pool, layer, p, qidx, widx, page_table, max_pages, seq_lens, scores, ld, s, shift, f);
            case 64: return launch_lds_heads<64>(pool, layer, p, qidx, widx, page_table, max_pages, seq_lens, scores, ld, s, shift, f);
            case 128: return launch_lds_heads<128>(pool, layer, p, qidx, widx, page_table, max_pages, seq_lens, scores, ld, s, shift, f);
            case 256: return launch_lds_heads<256>(pool, layer, p, qidx, widx, page_table, max_pages, seq_lens, scores, ld, s, shift, f);
            default: break;
        }
    }
    if (p.index_heads > 8) return hipErrorInvalidValue;   // the register kernel holds at most 8 heads
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
