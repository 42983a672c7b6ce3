// Sparse gather-attention on the vector ALUs, for grouped-query shapes (a few query heads per
// KV head), plus the split combine shared by every attention kernel.
//
// GLM5.3 sparse-attention page: sparse attention runs SDPA over only the top-k tokens the
// indexer kept (opening paragraph), one selection shared by all heads (lightning-indexer
// paragraph).  For query head h of request b, KV head g = h / (Hq / Hkv):
//     o[b][h] = softmax_j(scale * q[b][h] . K[t_j, g]) . V[t_j, g]
// The selected rows are scattered over the pool; the paged-KV page's limits section notes
// that attention must be written to walk the page table or paging loses what it saved.  Here
// each workgroup gathers whole rows of a tile of selected tokens into LDS (16-byte vectors,
// each row contiguous in HBM), then computes logits, an online softmax and the weighted sum
// from LDS.
//
// Work split: grid (split, KV head, request); a split is a contiguous run of the request's
// selected list.  With one split the kernel writes the normalised output; otherwise it writes
// (running max, running sum, unnormalised accumulator) partials that combine_kernel merges.
#include "tsa_internal.h"

namespace {

constexpr int kThreads = 256;

__device__ inline float bf16_to_f(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }
__device__ inline float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ inline float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

__device__ inline float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
    return v;
}
__device__ inline float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

struct AttnArgs {
    const uint16_t* q;        // [B][Hq][dk]
    const int32_t* topk;      // [B][k]
    const int32_t* page_table;
    const int32_t* seq_lens;
    const uint16_t* kpool;    // layer base; row (slot, g) at (slot * Hkv + g) * dk
    const uint16_t* vpool;    // layer base; row (slot, g) at (slot * Hkv + g) * v_head_stride
    float* out;               // [B][Hq][dv]
    float* part_ml;           // [B][Hq][S][2]
    float* part_acc;          // [B][Hq][S][dv]
    int k, max_pages, page_size, num_pages, max_len;
    int hq, hkv, dk, dv, v_head_stride;
    int splits, chunk;
    float scale;
};

// LDS layout (dynamic): q [G][dk] bf16 | K tile [T][dk + 8] bf16 | V tile [T][dv + 8] bf16
// (absent when values alias keys) | logits [G][T] f32 | m, l, alpha [G] f32 | pos [T] i32
template <int T, int NACC>
__global__ void __launch_bounds__(kThreads) attn_valu_kernel(AttnArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int s_idx = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int G = a.hq / a.hkv;
    const int dk = a.dk, dv = a.dv;
    const int kstride = dk + 8, vstride = dv + 8;  // +16 bytes per row staggers LDS banks
    const bool alias = a.vpool == a.kpool && a.v_head_stride == dk;

    uint16_t* q_s = reinterpret_cast<uint16_t*>(smem);
    uint16_t* k_s = q_s + G * dk;
    uint16_t* v_s = alias ? k_s : k_s + T * kstride;
    const int vs = alias ? kstride : vstride;
    float* lg_s = reinterpret_cast<float*>(alias ? k_s + T * kstride : v_s + T * vstride);
    float* m_s = lg_s + G * T;
    float* l_s = m_s + G;
    float* al_s = l_s + G;
    int64_t* row_s = reinterpret_cast<int64_t*>(al_s + G + (G & 1));  // 8-byte aligned

    int len = a.seq_lens[b];
    len = len < 0 ? 0 : (len > a.max_len ? a.max_len : len);
    const int n_sel = min(len, a.k);
    const int j0 = s_idx * a.chunk;
    const int j1 = min(j0 + a.chunk, n_sel);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // stage the group's queries
    {
        const uint4* src = reinterpret_cast<const uint4*>(a.q + (int64_t(b) * a.hq + g * G) * dk);
        uint4* dst = reinterpret_cast<uint4*>(q_s);
        for (int i = tid; i < G * dk / 8; i += kThreads) dst[i] = src[i];
    }
    for (int h = tid; h < G; h += kThreads) {
        m_s[h] = -INFINITY;
        l_s[h] = 0.f;
    }
    float acc[NACC];
#pragma unroll
    for (int i = 0; i < NACC; ++i) acc[i] = 0.f;
    const int n_out = G * dv;
    const int32_t* sel = a.topk + int64_t(b) * a.k;
    const int32_t* pt = a.page_table + int64_t(b) * a.max_pages;

    for (int jt = j0; jt < j1; jt += T) {
        __syncthreads();
        // resolve the tile's rows: position -> page -> slot (-1 when invalid)
        for (int j = tid; j < T; j += kThreads) {
            int64_t row = -1;
            if (jt + j < j1) {
                const int t = sel[jt + j];
                if (t >= 0 && t < len) {
                    const int page = pt[t / a.page_size];
                    if (page >= 0 && page < a.num_pages)
                        row = (int64_t(page) * a.page_size + t % a.page_size) * a.hkv + g;
                }
            }
            row_s[j] = row;
        }
        __syncthreads();
        // gather K (and V) rows
        {
            const int kv16 = dk / 8;
            for (int i = tid; i < T * kv16; i += kThreads) {
                const int j = i / kv16, c = i % kv16;
                const int64_t row = row_s[j];
                uint4 v = make_uint4(0, 0, 0, 0);
                if (row >= 0) v = reinterpret_cast<const uint4*>(a.kpool + row * dk)[c];
                *reinterpret_cast<uint4*>(k_s + j * kstride + c * 8) = v;
            }
            if (!alias) {
                const int vv16 = dv / 8;
                for (int i = tid; i < T * vv16; i += kThreads) {
                    const int j = i / vv16, c = i % vv16;
                    const int64_t row = row_s[j];
                    uint4 v = make_uint4(0, 0, 0, 0);
                    if (row >= 0) v = reinterpret_cast<const uint4*>(a.vpool + row * a.v_head_stride)[c];
                    *reinterpret_cast<uint4*>(v_s + j * vstride + c * 8) = v;
                }
            }
        }
        __syncthreads();
        // logits
        for (int pidx = tid; pidx < G * T; pidx += kThreads) {
            const int h = pidx / T, j = pidx % T;
            float lg = -INFINITY;
            if (row_s[j] >= 0) {
                const uint4* qv = reinterpret_cast<const uint4*>(q_s + h * dk);
                const uint4* kv = reinterpret_cast<const uint4*>(k_s + j * kstride);
                float d = 0.f;
                for (int c = 0; c < dk / 8; ++c) {
                    uint4 x = qv[c], y = kv[c];
                    d = fmaf(bf16_lo(x.x), bf16_lo(y.x), d);
                    d = fmaf(bf16_hi(x.x), bf16_hi(y.x), d);
                    d = fmaf(bf16_lo(x.y), bf16_lo(y.y), d);
                    d = fmaf(bf16_hi(x.y), bf16_hi(y.y), d);
                    d = fmaf(bf16_lo(x.z), bf16_lo(y.z), d);
                    d = fmaf(bf16_hi(x.z), bf16_hi(y.z), d);
                    d = fmaf(bf16_lo(x.w), bf16_lo(y.w), d);
                    d = fmaf(bf16_hi(x.w), bf16_hi(y.w), d);
                }
                lg = d * a.scale;
            }
            lg_s[h * T + j] = lg;
        }
        __syncthreads();
        // online softmax, one wave per head
        for (int h = wave; h < G; h += kThreads / 64) {
            float x = lane < T ? lg_s[h * T + lane] : -INFINITY;
            if (T > 64) {
                for (int j = lane + 64; j < T; j += 64) x = fmaxf(x, lg_s[h * T + j]);
            }
            const float tmax = wave_max(x);
            const float m_old = m_s[h];
            const float m_new = fmaxf(m_old, tmax);
            float sum = 0.f;
            for (int j = lane; j < T; j += 64) {
                const float l = lg_s[h * T + j];
                const float p = (l == -INFINITY) ? 0.f : __expf(l - m_new);
                lg_s[h * T + j] = p;
                sum += p;
            }
            sum = wave_sum(sum);
            if (lane == 0) {
                const float alpha = (m_old == -INFINITY) ? 0.f : __expf(m_old - m_new);
                al_s[h] = alpha;
                l_s[h] = l_s[h] * alpha + sum;
                m_s[h] = m_new;
            }
        }
        __syncthreads();
        // weighted sum of values
#pragma unroll
        for (int i = 0; i < NACC; ++i) {
            const int o = tid + i * kThreads;
            if (o < n_out) {
                const int h = o / dv, d = o % dv;
                float x = acc[i] * al_s[h];
                const float* p = lg_s + h * T;
                for (int j = 0; j < T; ++j) x = fmaf(p[j], bf16_to_f(v_s[j * vs + d]), x);
                acc[i] = x;
            }
        }
    }
    __syncthreads();
    const int h0 = g * G;
    if (a.splits == 1) {
#pragma unroll
        for (int i = 0; i < NACC; ++i) {
            const int o = tid + i * kThreads;
            if (o < n_out) {
                const int h = o / dv, d = o % dv;
                const float l = l_s[h];
                a.out[(int64_t(b) * a.hq + h0 + h) * dv + d] = l > 0.f ? acc[i] / l : 0.f;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < NACC; ++i) {
            const int o = tid + i * kThreads;
            if (o < n_out) {
                const int h = o / dv, d = o % dv;
                a.part_acc[((int64_t(b) * a.hq + h0 + h) * a.splits + s_idx) * dv + d] = acc[i];
            }
        }
        for (int h = tid; h < G; h += kThreads) {
            float* ml = a.part_ml + ((int64_t(b) * a.hq + h0 + h) * a.splits + s_idx) * 2;
            ml[0] = m_s[h];
            ml[1] = l_s[h];
        }
    }
}

// Merge split partials: o = sum_s acc_s e^(m_s - M) / sum_s l_s e^(m_s - M), M = max_s m_s.
// One workgroup of kCombineThreads per (request, head); a lane owns 4 consecutive value dims
// (16-byte loads, dv % 4 == 0); the split weights are computed once per workgroup.
constexpr int kCombineThreads = 128;
constexpr int kCombineMaxSplits = 64;
__global__ void __launch_bounds__(kCombineThreads) combine_kernel(const float* __restrict__ part_ml,
                                                                  const float* __restrict__ part_acc,
                                                                  int splits, int dv,
                                                                  float* __restrict__ out) {
    __shared__ float wsh[kCombineMaxSplits];
    const int bh = blockIdx.x;  // b * Hq + h
    const float* ml = part_ml + int64_t(bh) * splits * 2;
    if (threadIdx.x < 64) {
        // one wave: M and L by lane reduction over the splits (splits <= 64)
        const int sl = threadIdx.x;
        const float m = sl < splits ? ml[2 * sl] : -INFINITY;
        float M = m;
        for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
        const float e = (m == -INFINITY) ? 0.f : __expf(m - M);
        float L = sl < splits ? ml[2 * sl + 1] * e : 0.f;
        for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o);
        if (sl < splits) wsh[sl] = L > 0.f ? e / L : 0.f;
    }
    __syncthreads();
    const float4* acc = reinterpret_cast<const float4*>(part_acc + int64_t(bh) * splits * dv);
    float4* o = reinterpret_cast<float4*>(out + int64_t(bh) * dv);
    const int dv4 = dv >> 2;
    for (int d = threadIdx.x; d < dv4; d += kCombineThreads) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int sp = 0; sp < splits; ++sp) {
            const float w = wsh[sp];
            const float4 v = acc[int64_t(sp) * dv4 + d];
            x.x = fmaf(v.x, w, x.x);
            x.y = fmaf(v.y, w, x.y);
            x.z = fmaf(v.z, w, x.z);
            x.w = fmaf(v.w, w, x.w);
        }
        o[d] = x;
    }
}

// The same merge for at most kSmallSplits splits, as one pass with no barrier: every thread
// first issues its loads of all the splits' accumulators, then reads the (max, sum) pairs (the
// same few addresses for the whole workgroup) and computes the split weights in registers
// while those loads are in flight.
constexpr int kSmallSplits = 8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4v;

__device__ __forceinline__ float4 load_nt_f4(const float4* p) {
    const f32x4v v = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
}

__global__ void __launch_bounds__(kCombineThreads) combine_small_kernel(const float* __restrict__ part_ml,
                                                                        const float* __restrict__ part_acc,
                                                                        int splits, int dv,
                                                                        float* __restrict__ out) {
    const int bh = blockIdx.x;  // b * Hq + h
    const float4* acc = reinterpret_cast<const float4*>(part_acc + int64_t(bh) * splits * dv);
    float4* o = reinterpret_cast<float4*>(out + int64_t(bh) * dv);
    const int dv4 = dv >> 2;
    const float* ml = part_ml + int64_t(bh) * splits * 2;
    float w[kSmallSplits];
    bool have_w = false;
    for (int d = threadIdx.x; d < dv4; d += kCombineThreads) {
        float4 v[kSmallSplits];
#pragma unroll
        for (int sp = 0; sp < kSmallSplits; ++sp)
            v[sp] = sp < splits ? load_nt_f4(acc + int64_t(sp) * dv4 + d) : make_float4(0.f, 0.f, 0.f, 0.f);
        if (!have_w) {
            float m[kSmallSplits], M = -INFINITY;
#pragma unroll
            for (int sp = 0; sp < kSmallSplits; ++sp) {
                m[sp] = sp < splits ? ml[2 * sp] : -INFINITY;
                M = fmaxf(M, m[sp]);
            }
            float L = 0.f;
#pragma unroll
            for (int sp = 0; sp < kSmallSplits; ++sp) {
                w[sp] = m[sp] == -INFINITY ? 0.f : __expf(m[sp] - M);
                L += sp < splits ? ml[2 * sp + 1] * w[sp] : 0.f;
            }
#pragma unroll
            for (int sp = 0; sp < kSmallSplits; ++sp) w[sp] = L > 0.f ? w[sp] / L : 0.f;
            have_w = true;
        }
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int sp = 0; sp < kSmallSplits; ++sp) {
            x.x = fmaf(v[sp].x, w[sp], x.x);
            x.y = fmaf(v[sp].y, w[sp], x.y);
            x.z = fmaf(v[sp].z, w[sp], x.z);
            x.w = fmaf(v[sp].w, w[sp], x.w);
        }
        o[d] = x;
    }
}

size_t valu_smem_bytes(int T, int G, int dk, int dv, bool alias) {
    size_t s = size_t(G) * dk * 2 + size_t(T) * (dk + 8) * 2;
    if (!alias) s += size_t(T) * (dv + 8) * 2;
    s += size_t(G) * T * 4 + size_t(3 * G + (G & 1)) * 4 + size_t(T) * 8;
    return s;
}

template <int T, int NACC>
hipError_t launch_tn(const AttnArgs& a, dim3 grid, size_t smem, hipStream_t s) {
    auto kern = attn_valu_kernel<T, NACC>;
    if (smem > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), smem, s, a);
    return hipGetLastError();
}

template <int T>
hipError_t launch_t(const AttnArgs& a, int nacc, dim3 grid, size_t smem, hipStream_t s) {
    if (nacc <= 4) return launch_tn<T, 4>(a, grid, smem, s);
    if (nacc <= 8) return launch_tn<T, 8>(a, grid, smem, s);
    if (nacc <= 16) return launch_tn<T, 16>(a, grid, smem, s);
    if (nacc <= 32) return launch_tn<T, 32>(a, grid, smem, s);
    if (nacc <= 64) return launch_tn<T, 64>(a, grid, smem, s);
    if (nacc <= 128) return launch_tn<T, 128>(a, grid, smem, s);
    return hipErrorInvalidValue;
}

constexpr size_t kMaxSmem = 160 * 1024;

int pick_tile(int G, int dk, int dv, bool alias) {
    for (int T : {64, 32, 16}) {
        if (valu_smem_bytes(T, G, dk, dv, alias) <= kMaxSmem) return T;
    }
    return 0;
}

}  // namespace

namespace tsa {

bool attention_supported(const tsa_kv_pool& pool, const tsa_decode_params& p, std::string* why) {
    const tsa_pool_desc& d = pool.d;
    if (p.num_q_heads % d.num_kv_heads) {
        *why = "num_q_heads must be a multiple of num_kv_heads";
        return false;
    }
    if (mfma_latent_applicable(pool, p) || gqa_mfma_applicable(pool, p)) return true;
    const int G = p.num_q_heads / d.num_kv_heads;
    if (ceil_div(int64_t(G) * d.head_dim_v, kThreads) > 128) {
        *why = "query heads per KV head x head_dim_v exceeds 32768";
        return false;
    }
    if (!pick_tile(G, d.head_dim_k, d.head_dim_v, d.v_from_k)) {
        *why = "query group and head dims do not fit LDS";
        return false;
    }
    return true;
}

// Partials: (max, sum) pairs for n rows, padded to 16 bytes, then n accumulator rows of dv.
size_t partial_ml_floats(size_t n) { return (2 * n + 3) / 4 * 4; }
size_t partial_bytes(size_t n, int dv) { return (partial_ml_floats(n) + n * size_t(dv)) * sizeof(float); }

AttnPlan plan_attention(const tsa_kv_pool& pool, const tsa_decode_params& p) {
    AttnPlan plan;
    const tsa_pool_desc& d = pool.d;
    if (mfma_latent_applicable(pool, p)) {
        plan.kind = 1;
        plan.chunk = mfma_latent_chunk(p, &plan.splits);
        plan.partial_bytes = plan.splits > 1 ? partial_bytes(size_t(p.batch) * p.num_q_heads * plan.splits,
                                                             d.head_dim_v)
                                             : 0;
        return plan;
    }
    if (gqa_mfma_applicable(pool, p)) {
        plan.kind = 2;
        if (gqa_wg_merge(pool, p)) {
            const int k_eff = std::max(1, std::min(p.top_k, p.max_len));
            plan.wg_merge = true;
            plan.splits = kGqaMergeSplits;
            plan.chunk = int(ceil_div(ceil_div(k_eff, kGqaMergeSplits), 32)) * 32;
            plan.partial_bytes = 0;
            return plan;
        }
        plan.chunk = gqa_mfma_chunk(pool, p, &plan.splits);
        plan.partial_bytes = plan.splits > 1 ? partial_bytes(size_t(p.batch) * p.num_q_heads * plan.splits,
                                                             d.head_dim_v)
                                             : 0;
        return plan;
    }
    const int G = p.num_q_heads / d.num_kv_heads;
    const int T = pick_tile(G, d.head_dim_k, d.head_dim_v, d.v_from_k);
    const int units = p.batch * d.num_kv_heads;
    const int k_eff = std::max(1, std::min(p.top_k, p.max_len));   // most tokens any request selects
    const int tiles = int(ceil_div(k_eff, T));
    int splits = int(ceil_div(512, units));  // aim for >= 2 workgroups per CU
    splits = std::max(1, std::min({splits, tiles, kCombineMaxSplits}));
    plan.kind = 0;
    plan.chunk = int(ceil_div(tiles, splits)) * T;
    plan.splits = int(ceil_div(k_eff, plan.chunk));
    plan.partial_bytes = plan.splits > 1 ? partial_bytes(size_t(p.batch) * p.num_q_heads * plan.splits,
                                                         d.head_dim_v)
                                         : 0;
    return plan;
}

hipError_t launch_valu(const AttnArgs& a, const tsa_kv_pool& pool, const tsa_decode_params& p,
                       const AttnPlan& plan, hipStream_t s);

hipError_t launch_attention(const tsa_kv_pool& pool, int layer, const tsa_decode_params& p,
                            const AttnPlan& plan, const void* q, const int32_t* topk,
                            const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                            float* out, void* partial, hipStream_t s) {
    const tsa_pool_desc& d = pool.d;
    AttnArgs a;
    const int64_t rows = pool.slots() * d.num_kv_heads;
    a.q = static_cast<const uint16_t*>(q);
    a.topk = topk;
    a.page_table = page_table;
    a.seq_lens = seq_lens;
    a.kpool = static_cast<const uint16_t*>(pool.k) + int64_t(layer) * rows * d.head_dim_k;
    if (d.v_from_k) {
        a.vpool = a.kpool;
        a.v_head_stride = d.head_dim_k;
    } else {
        a.vpool = static_cast<const uint16_t*>(pool.v) + int64_t(layer) * rows * d.head_dim_v;
        a.v_head_stride = d.head_dim_v;
    }
    a.out = out;
    a.k = p.top_k;
    a.max_pages = max_pages;
    a.page_size = d.page_size;
    a.num_pages = d.num_pages;
    a.max_len = p.max_len;
    a.hq = p.num_q_heads;
    a.hkv = d.num_kv_heads;
    a.dk = d.head_dim_k;
    a.dv = d.head_dim_v;
    a.splits = plan.splits;
    a.chunk = plan.chunk;
    a.scale = p.sm_scale;
    const size_t n_part = size_t(p.batch) * p.num_q_heads * plan.splits;
    a.part_ml = static_cast<float*>(partial);
    a.part_acc = a.part_ml ? a.part_ml + partial_ml_floats(n_part) : nullptr;

    hipError_t e;
    if (plan.kind == 1) {
        e = launch_attention_mfma(pool, layer, p, plan, q, topk, page_table, max_pages, seq_lens,
                                  out, a.part_ml, a.part_acc, s);
    } else if (plan.kind == 2) {
        e = launch_attention_gqa(pool, layer, p, plan, q, topk, page_table, max_pages, seq_lens,
                                 out, a.part_ml, a.part_acc, s);
    } else {
        e = launch_valu(a, pool, p, plan, s);
    }
    if (e != hipSuccess || plan.splits == 1 || plan.wg_merge) return e;
    if (plan.splits <= kSmallSplits)
        hipLaunchKernelGGL(combine_small_kernel, dim3(p.batch * p.num_q_heads), dim3(kCombineThreads), 0, s,
                           a.part_ml, a.part_acc, plan.splits, d.head_dim_v, out);
    else
        hipLaunchKernelGGL(combine_kernel, dim3(p.batch * p.num_q_heads), dim3(kCombineThreads), 0, s,
                           a.part_ml, a.part_acc, plan.splits, d.head_dim_v, out);
    return hipGetLastError();
}

hipError_t launch_valu(const AttnArgs& a, const tsa_kv_pool& pool, const tsa_decode_params& p,
                       const AttnPlan& plan, hipStream_t s) {
    const tsa_pool_desc& d = pool.d;
    const int G = p.num_q_heads / d.num_kv_heads;
    const int T = pick_tile(G, d.head_dim_k, d.head_dim_v, d.v_from_k);
    const size_t smem = valu_smem_bytes(T, G, d.head_dim_k, d.head_dim_v, d.v_from_k);
    const int nacc = int(ceil_div(int64_t(G) * d.head_dim_v, kThreads));
    dim3 grid(plan.splits, d.num_kv_heads, p.batch);
    hipError_t e;
    switch (T) {
        case 64: e = launch_t<64>(a, nacc, grid, smem, s); break;
        case 32: e = launch_t<32>(a, nacc, grid, smem, s); break;
        default: e = launch_t<16>(a, nacc, grid, smem, s); break;
    }
    return e;
}

}  // namespace tsa
