// The whole decode step of a request in one workgroup: one launch per step, scores kept in LDS.
//
// GLM5.3 sparse-attention page, TileRT paragraph: decode built as one persistent kernel removes
// the launch and serialisation gaps between its stages; paragraph on serving-engine decode (the
// GLM-5.2 studies): small decode steps are dominated by such overhead.  The step itself is the
// page's DSA decode (opening and lightning-indexer paragraphs): score every cached token,
// keep the top k (lowest position on ties, ascending), attend over those rows only.
//
// For a short context the separate kernels leave most of the chip idle and pay a launch, a
// scores round-trip through HBM and a drain between each stage.  Here workgroup b runs request
// b from start to end:
//   1. writes the request's new token (K, V and indexer rows) at position seq_len - 1 through
//      the page table (paged-KV page, section "Phân trang") and stages the request's queries in
//      LDS; the new token is scored and attended from its source rows, so the kernel never
//      reads back what it writes and needs no fence;
//   2. scores every cached token into LDS as an order-preserving 32-bit key (LPT = index_dim / 8
//      lanes per token, 16 bytes each, reduced across those lanes);
//   3. selects the top k in LDS: four 8-bit radix passes find the k-th largest key; every key
//      above it is kept, and of the keys equal to it the lowest positions fill the rest; a
//      block scan in position order gives each kept position its output slot, so the list comes
//      out ascending;
//   4. turns the selected positions into pool slots once, then, for each KV head, gathers tiles
//      of the selected rows into LDS and runs logits, an online softmax and the weighted sum of
//      values on the vector ALUs, writing the normalised output.
// The score region of LDS is reused for the attention tiles once the selection is made.
#include "tsa_internal.h"

namespace {

// 16 waves: with one workgroup per CU, four waves per SIMD hide the LDS and memory latency of
// the dependent chains below
constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxAcc = 2;          // value outputs per thread: G * head_dim_v <= 2048
constexpr int kMaxIdxHeads = 8;
constexpr int kLoads = 4;           // indexer rows in flight per thread
constexpr size_t kLdsLimit = 64 * 1024;

__device__ inline float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ inline float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ inline float bf16_to_f(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }

__device__ inline uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

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

// Exclusive prefix sum over the workgroup in thread order.  tot_s: kWaves words of LDS.
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* tot_s) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        const uint32_t o = __shfl_up(x, m);
        if (lane >= m) x += o;
    }
    if (lane == 63) tot_s[wave] = x;
    __syncthreads();
    uint32_t base = 0;
    for (int w = 0; w < wave; ++w) base += tot_s[w];
    __syncthreads();
    return base + x - v;
}

struct FusedArgs {
    const uint4* k_new;       // [B][Hkv * dk / 8]
    const uint4* v_new;       // [B][Hkv * dv / 8], null when values alias keys
    const uint4* i_new;       // [B][D / 8]
    int32_t* bad;             // nullable
    uint16_t* kpool;          // layer bases; K row (slot, g) at (slot * Hkv + g) * dk
    uint16_t* vpool;          // V row (slot, g) at (slot * Hkv + g) * v_stride
    uint16_t* ipool;          // indexer row of slot at slot * D
    const uint16_t* q;        // [B][Hq][dk]
    const uint16_t* qidx;     // [B][H][D]
    const float* widx;        // [H]
    const int32_t* page_table;
    const int32_t* seq_lens;
    float* out;               // [B][Hq][dv]
    int32_t* topk;            // [B][k] or null
    int max_pages, page_size, num_pages, max_len, k;
    int hq, hkv, dk, dv, v_stride, H, D, T;
    bool alias;
    float scale;
    // LDS byte offsets (computed by the host from the same sizes)
    int off_sel, off_u, off_qf, off_q, off_pt, off_k, off_v, off_lg, off_m;
};

__global__ void __launch_bounds__(kThreads) fused_step_kernel(FusedArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    uint32_t* hist = reinterpret_cast<uint32_t*>(smem);          // [256]
    uint32_t* tot_s = hist + 256;                                 // [kWaves] scan carries
    int32_t* ctrl = reinterpret_cast<int32_t*>(tot_s + kWaves);   // [4] radix digit, remainder
    int32_t* sel_s = reinterpret_cast<int32_t*>(smem + a.off_sel);

    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int len = a.seq_lens[b];
    len = len < 0 ? 0 : (len > a.max_len ? a.max_len : len);
    const int32_t* pt = a.page_table + int64_t(b) * a.max_pages;
    const int ps = a.page_size;

    // 1. the new token's rows
    if (len > 0) {
        const int t = len - 1;
        const int page = pt[t / ps];
        if (page >= 0 && page < a.num_pages) {
            const int64_t slot = int64_t(page) * ps + t % ps;
            const int k16 = a.hkv * a.dk / 8, i16 = a.D / 8;
            uint4* kd = reinterpret_cast<uint4*>(a.kpool) + slot * k16;
            for (int i = tid; i < k16; i += kThreads) kd[i] = a.k_new[int64_t(b) * k16 + i];
            if (!a.alias) {
                const int v16 = a.hkv * a.dv / 8;
                uint4* vd = reinterpret_cast<uint4*>(a.vpool) + slot * v16;
                for (int i = tid; i < v16; i += kThreads) vd[i] = a.v_new[int64_t(b) * v16 + i];
            }
            uint4* id = reinterpret_cast<uint4*>(a.ipool) + slot * i16;
            for (int i = tid; i < i16; i += kThreads) id[i] = a.i_new[int64_t(b) * i16 + i];
        } else if (tid == 0 && a.bad) {
            atomicAdd(a.bad, 1);
        }
    }
    // every query head of the request (for step 4) and its page-table row, so that steps 2 and
    // 4 look pages up in LDS
    uint16_t* q_s = reinterpret_cast<uint16_t*>(smem + a.off_q);
    {
        const uint4* src = reinterpret_cast<const uint4*>(a.q + int64_t(b) * a.hq * a.dk);
        uint4* dst = reinterpret_cast<uint4*>(q_s);
        for (int i = tid; i < a.hq * a.dk / 8; i += kThreads) dst[i] = src[i];
    }
    int32_t* pt_s = reinterpret_cast<int32_t*>(smem + a.off_pt);
    for (int i = tid; i < (len + ps - 1) / ps; i += kThreads) pt_s[i] = pt[i];

    // 2. scores -> keys in LDS
    uint32_t* key_s = reinterpret_cast<uint32_t*>(smem + a.off_u);
    float* qf_s = reinterpret_cast<float*>(smem + a.off_qf);     // [H][D]
    float* w_s = qf_s + a.H * a.D;
    {
        const uint16_t* qi = a.qidx + int64_t(b) * a.H * a.D;
        for (int i = tid; i < a.H * a.D; i += kThreads) qf_s[i] = bf16_to_f(qi[i]);
        for (int h = tid; h < a.H; h += kThreads) w_s[h] = a.widx[h];
    }
    __syncthreads();
    {
        const int LPT = a.D / 8;               // power of two, <= 32
        const int per = kThreads / LPT;        // tokens per round of loads
        const int sub = tid % LPT, grp = tid / LPT;
        const uint4* ipool = reinterpret_cast<const uint4*>(a.ipool);
        for (int t0 = 0; t0 < len; t0 += per * kLoads) {
            uint4 kv[kLoads];
            bool ok[kLoads];
#pragma unroll
            for (int u = 0; u < kLoads; ++u) {
                const int t = t0 + u * per + grp;
                int page = -1;
                if (t < len) page = pt_s[t / ps];
                ok[u] = page >= 0 && page < a.num_pages;
                const uint4* src = t == len - 1 ? a.i_new + int64_t(b) * LPT
                                                : ipool + (int64_t(page) * ps + t % ps) * LPT;
                kv[u] = ok[u] ? src[sub] : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < kLoads; ++u) {
                const int t = t0 + u * per + grp;
                float s = 0.f;
                for (int h = 0; h < a.H; ++h) {
                    const float4 q0 = *reinterpret_cast<const float4*>(qf_s + h * a.D + sub * 8);
                    const float4 q1 = *reinterpret_cast<const float4*>(qf_s + h * a.D + sub * 8 + 4);
                    float d = q0.x * bf16_lo(kv[u].x);
                    d = fmaf(q0.y, bf16_hi(kv[u].x), d);
                    d = fmaf(q0.z, bf16_lo(kv[u].y), d);
                    d = fmaf(q0.w, bf16_hi(kv[u].y), d);
                    d = fmaf(q1.x, bf16_lo(kv[u].z), d);
                    d = fmaf(q1.y, bf16_hi(kv[u].z), d);
                    d = fmaf(q1.z, bf16_lo(kv[u].w), d);
                    d = fmaf(q1.w, bf16_hi(kv[u].w), d);
                    for (int m = LPT / 2; m >= 1; m >>= 1) d += __shfl_xor(d, m, LPT);
                    s = fmaf(w_s[h], fmaxf(d, 0.f), s);
                }
                if (sub == 0 && t < len) key_s[t] = order_key(ok[u] ? s : -INFINITY);
            }
        }
    }
    __syncthreads();

    // 3. top-k in LDS
    const int n_sel = min(len, a.k);
    if (len <= a.k) {
        for (int j = tid; j < len; j += kThreads) sel_s[j] = j;
    } else {
        uint32_t prefix = 0, mask = 0;
        uint32_t rem = uint32_t(a.k);          // still to take among keys matching the prefix
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            if (tid < 256) hist[tid] = 0;
            __syncthreads();
            for (int t = tid; t < len; t += kThreads) {
                const uint32_t key = key_s[t];
                if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
            }
            __syncthreads();
            if (wave == 0) {
                // lane l owns bins 4l..4l+3; `above` counts the candidates in higher bins
                const uint32_t c0 = hist[4 * lane], c1 = hist[4 * lane + 1];
                const uint32_t c2 = hist[4 * lane + 2], c3 = hist[4 * lane + 3];
                const uint32_t tot = c0 + c1 + c2 + c3;
                uint32_t incl = tot;
#pragma unroll
                for (int m = 1; m < 64; m <<= 1) {
                    const uint32_t o = __shfl_down(incl, m);
                    if (lane + m < 64) incl += o;
                }
                const uint32_t above = incl - tot;
                // the digit of the rem-th largest candidate: more than `gt` above it, rem <= gt + count
                int digit = -1;
                uint32_t gt = 0;
                if (above < rem) {
                    if (above + c3 >= rem) { digit = 4 * lane + 3; gt = above; }
                    else if (above + c3 + c2 >= rem) { digit = 4 * lane + 2; gt = above + c3; }
                    else if (above + c3 + c2 + c1 >= rem) { digit = 4 * lane + 1; gt = above + c3 + c2; }
                    else if (above + tot >= rem) { digit = 4 * lane; gt = above + c3 + c2 + c1; }
                }
                if (digit >= 0) {
                    ctrl[0] = digit;
                    ctrl[1] = int32_t(rem - gt);
                }
            }
            __syncthreads();
            prefix |= uint32_t(ctrl[0]) << shift;
            mask |= 0xffu << shift;
            rem = uint32_t(ctrl[1]);
        }
        // prefix is now the k-th largest key; rem of the keys equal to it are taken
        const int per_t = (len + kThreads - 1) / kThreads;
        const int p0 = min(tid * per_t, len), p1 = min(p0 + per_t, len);
        uint32_t gt = 0, eq = 0;
        for (int t = p0; t < p1; ++t) {
            const uint32_t key = key_s[t];
            gt += key > prefix;
            eq += key == prefix;
        }
        const uint32_t eq_base = block_exclusive_scan(eq, tot_s);
        const uint32_t take_eq = eq_base >= rem ? 0u : min(eq, rem - eq_base);
        uint32_t o = block_exclusive_scan(gt + take_eq, tot_s);
        uint32_t er = eq_base;
        for (int t = p0; t < p1; ++t) {
            const uint32_t key = key_s[t];
            bool take = key > prefix;
            if (key == prefix) take = er++ < rem;
            if (take) sel_s[o++] = t;
        }
    }
    __syncthreads();
    if (a.topk) {
        int32_t* dst = a.topk + int64_t(b) * a.k;
        for (int j = tid; j < a.k; j += kThreads) dst[j] = j < n_sel ? sel_s[j] : -1;
    }

    // 4. attention over the selected rows, one KV head at a time.  The selection becomes pool
    // slots: -1 for a position whose page is not valid, -2 for the new token (read from its
    // source rows).
    __syncthreads();
    for (int j = tid; j < n_sel; j += kThreads) {
        const int t = sel_s[j];
        const int page = pt_s[t / ps];
        int slot = -1;
        if (page >= 0 && page < a.num_pages) slot = t == len - 1 ? -2 : page * ps + t % ps;
        sel_s[j] = slot;
    }
    const int G = a.hq / a.hkv, dk = a.dk, dv = a.dv, T = a.T;
    const int kstride = dk + 8, vstride = a.alias ? kstride : dv + 8;
    uint16_t* k_s = reinterpret_cast<uint16_t*>(smem + a.off_k);
    uint16_t* v_s = a.alias ? k_s : reinterpret_cast<uint16_t*>(smem + a.off_v);
    float* lg_s = reinterpret_cast<float*>(smem + a.off_lg);
    float* m_s = reinterpret_cast<float*>(smem + a.off_m);
    float* l_s = m_s + G;
    float* al_s = l_s + G;
    const int n_out = G * dv;
    const uint16_t* k_new = reinterpret_cast<const uint16_t*>(a.k_new) + int64_t(b) * a.hkv * dk;
    const uint16_t* v_new = a.alias ? k_new : reinterpret_cast<const uint16_t*>(a.v_new) + int64_t(b) * a.hkv * dv;
    const int v_new_stride = a.alias ? dk : dv;
    for (int g = 0; g < a.hkv; ++g) {
        const uint16_t* qg_s = q_s + g * G * dk;
        __syncthreads();
        for (int h = tid; h < G; h += kThreads) {
            m_s[h] = -INFINITY;
            l_s[h] = 0.f;
        }
        float acc[kMaxAcc];
#pragma unroll
        for (int i = 0; i < kMaxAcc; ++i) acc[i] = 0.f;

        for (int jt = 0; jt < n_sel; jt += T) {
            __syncthreads();
            for (int i = tid; i < T * (dk / 8); i += kThreads) {
                const int j = i / (dk / 8), c = i % (dk / 8);
                const int slot = jt + j < n_sel ? sel_s[jt + j] : -1;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (slot >= 0) v = reinterpret_cast<const uint4*>(a.kpool + (int64_t(slot) * a.hkv + g) * dk)[c];
                else if (slot == -2) v = reinterpret_cast<const uint4*>(k_new + g * dk)[c];
                *reinterpret_cast<uint4*>(k_s + j * kstride + c * 8) = v;
            }
            if (!a.alias) {
                for (int i = tid; i < T * (dv / 8); i += kThreads) {
                    const int j = i / (dv / 8), c = i % (dv / 8);
                    const int slot = jt + j < n_sel ? sel_s[jt + j] : -1;
                    uint4 v = make_uint4(0, 0, 0, 0);
                    if (slot >= 0)
                        v = reinterpret_cast<const uint4*>(a.vpool + (int64_t(slot) * a.hkv + g) * a.v_stride)[c];
                    else if (slot == -2)
                        v = reinterpret_cast<const uint4*>(v_new + g * v_new_stride)[c];
                    *reinterpret_cast<uint4*>(v_s + j * vstride + c * 8) = v;
                }
            }
            __syncthreads();
            for (int pidx = tid; pidx < G * T; pidx += kThreads) {
                const int h = pidx / T, j = pidx % T;
                float lg = -INFINITY;
                if (jt + j < n_sel && sel_s[jt + j] != -1) {
                    const uint4* qv = reinterpret_cast<const uint4*>(qg_s + h * dk);
                    const uint4* kv = reinterpret_cast<const uint4*>(k_s + j * kstride);
                    // two independent chains over the 16-byte chunks (dk / 8 is even or one)
                    float d0 = 0.f, d1 = 0.f;
                    int c = 0;
                    for (; c + 1 < dk / 8; c += 2) {
                        const uint4 x0 = qv[c], y0 = kv[c], x1 = qv[c + 1], y1 = kv[c + 1];
                        d0 = fmaf(bf16_lo(x0.x), bf16_lo(y0.x), d0);
                        d1 = fmaf(bf16_lo(x1.x), bf16_lo(y1.x), d1);
                        d0 = fmaf(bf16_hi(x0.x), bf16_hi(y0.x), d0);
                        d1 = fmaf(bf16_hi(x1.x), bf16_hi(y1.x), d1);
                        d0 = fmaf(bf16_lo(x0.y), bf16_lo(y0.y), d0);
                        d1 = fmaf(bf16_lo(x1.y), bf16_lo(y1.y), d1);
                        d0 = fmaf(bf16_hi(x0.y), bf16_hi(y0.y), d0);
                        d1 = fmaf(bf16_hi(x1.y), bf16_hi(y1.y), d1);
                        d0 = fmaf(bf16_lo(x0.z), bf16_lo(y0.z), d0);
                        d1 = fmaf(bf16_lo(x1.z), bf16_lo(y1.z), d1);
                        d0 = fmaf(bf16_hi(x0.z), bf16_hi(y0.z), d0);
                        d1 = fmaf(bf16_hi(x1.z), bf16_hi(y1.z), d1);
                        d0 = fmaf(bf16_lo(x0.w), bf16_lo(y0.w), d0);
                        d1 = fmaf(bf16_lo(x1.w), bf16_lo(y1.w), d1);
                        d0 = fmaf(bf16_hi(x0.w), bf16_hi(y0.w), d0);
                        d1 = fmaf(bf16_hi(x1.w), bf16_hi(y1.w), d1);
                    }
                    if (c < dk / 8) {
                        const uint4 x = qv[c], y = kv[c];
                        d0 = fmaf(bf16_lo(x.x), bf16_lo(y.x), d0);
                        d0 = fmaf(bf16_hi(x.x), bf16_hi(y.x), d0);
                        d0 = fmaf(bf16_lo(x.y), bf16_lo(y.y), d0);
                        d0 = fmaf(bf16_hi(x.y), bf16_hi(y.y), d0);
                        d0 = fmaf(bf16_lo(x.z), bf16_lo(y.z), d0);
                        d0 = fmaf(bf16_hi(x.z), bf16_hi(y.z), d0);
                        d0 = fmaf(bf16_lo(x.w), bf16_lo(y.w), d0);
                        d0 = fmaf(bf16_hi(x.w), bf16_hi(y.w), d0);
                    }
                    lg = (d0 + d1) * a.scale;
                }
                lg_s[h * T + j] = lg;
            }
            __syncthreads();
            for (int h = wave; h < G; h += kWaves) {
                float x = -INFINITY;
                for (int j = lane; j < T; j += 64) x = fmaxf(x, lg_s[h * T + j]);
                const float m_old = m_s[h];
                const float m_new = fmaxf(m_old, wave_max(x));
                float sum = 0.f;
                for (int j = lane; j < T; j += 64) {
                    const float l = lg_s[h * T + j];
                    const float p = l == -INFINITY ? 0.f : __expf(l - m_new);
                    lg_s[h * T + j] = p;
                    sum += p;
                }
                sum = wave_sum(sum);
                if (lane == 0) {
                    const float alpha = m_old == -INFINITY ? 0.f : __expf(m_old - m_new);
                    al_s[h] = alpha;
                    l_s[h] = l_s[h] * alpha + sum;
                    m_s[h] = m_new;
                }
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < kMaxAcc; ++i) {
                const int o = tid + i * kThreads;
                if (o < n_out) {
                    const int h = o / dv, d = o % dv;
                    const float* p = lg_s + h * T;
                    const uint16_t* vcol = v_s + d;
                    // four rows per step: independent LDS reads, two chains (T is a multiple of 16)
                    float x0 = acc[i] * al_s[h], x1 = 0.f;
                    for (int j = 0; j < T; j += 4) {
                        const float4 pp = *reinterpret_cast<const float4*>(p + j);
                        const float v0 = bf16_to_f(vcol[(j + 0) * vstride]);
                        const float v1 = bf16_to_f(vcol[(j + 1) * vstride]);
                        const float v2 = bf16_to_f(vcol[(j + 2) * vstride]);
                        const float v3 = bf16_to_f(vcol[(j + 3) * vstride]);
                        x0 = fmaf(pp.x, v0, x0);
                        x1 = fmaf(pp.y, v1, x1);
                        x0 = fmaf(pp.z, v2, x0);
                        x1 = fmaf(pp.w, v3, x1);
                    }
                    acc[i] = x0 + x1;
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kMaxAcc; ++i) {
            const int o = tid + i * kThreads;
            if (o < n_out) {
                const int h = o / dv, d = o % dv;
                const float l = l_s[h];
                a.out[(int64_t(b) * a.hq + g * G + h) * dv + d] = l > 0.f ? acc[i] / l : 0.f;
            }
        }
    }
}

// LDS plan for a tile of T selected rows; 0 when it does not fit.
struct FusedLds {
    int T = 0;
    int off_sel = 0, off_u = 0, off_qf = 0, off_q = 0, off_pt = 0, off_k = 0, off_v = 0, off_lg = 0,
        off_m = 0;
    size_t total = 0;
};

size_t up16(size_t x) { return (x + 15) / 16 * 16; }

FusedLds plan_lds(const tsa_kv_pool& pool, const tsa_decode_params& p, int T) {
    const tsa_pool_desc& d = pool.d;
    const int G = p.num_q_heads / d.num_kv_heads;
    FusedLds L;
    L.T = T;
    size_t off = up16((256 + kWaves + 4) * sizeof(uint32_t));  // histogram, scan carries, control
    L.off_sel = int(off);
    off += up16(size_t(std::max(1, std::min(p.top_k, p.max_len))) * sizeof(int32_t));
    L.off_q = int(off);
    off += up16(size_t(p.num_q_heads) * d.head_dim_k * 2);
    L.off_pt = int(off);
    off += up16(size_t(std::max<int64_t>(1, (int64_t(p.max_len) + d.page_size - 1) / d.page_size)) * sizeof(int32_t));
    L.off_u = int(off);
    // scoring phase: keys, then the indexer query as floats and the head weights
    size_t u = up16(size_t(std::max(p.max_len, 1)) * sizeof(uint32_t));
    L.off_qf = int(off + u);
    u += up16(size_t(p.index_heads) * (d.index_dim + 1) * sizeof(float));
    // attention phase, over the same bytes
    size_t v = 0;
    L.off_k = int(off + v);
    v += up16(size_t(T) * (d.head_dim_k + 8) * 2);
    L.off_v = int(off + v);
    if (!d.v_from_k) v += up16(size_t(T) * (d.head_dim_v + 8) * 2);
    L.off_lg = int(off + v);
    v += up16(size_t(G) * T * sizeof(float));
    L.off_m = int(off + v);
    v += up16(size_t(3) * G * sizeof(float));
    L.total = off + std::max(u, v);
    return L;
}

FusedLds pick_lds(const tsa_kv_pool& pool, const tsa_decode_params& p) {
    for (int T : {64, 32, 16}) {
        FusedLds L = plan_lds(pool, p, T);
        if (L.total <= kLdsLimit) return L;
    }
    return FusedLds{};
}

}  // namespace

namespace tsa {

bool fused_step_supported(const tsa_kv_pool& pool, const tsa_decode_params& p, std::string* why) {
    const tsa_pool_desc& d = pool.d;
    const int D = d.index_dim;
    if (D < 8 || D > 256 || D % 8 || (D / 8 & (D / 8 - 1))) {
        *why = "one-launch step: index_dim must be 8 x a power of two, <= 256";
        return false;
    }
    if (p.index_heads < 1 || p.index_heads > kMaxIdxHeads) {
        *why = "one-launch step: index_heads must be in 1.." + std::to_string(kMaxIdxHeads);
        return false;
    }
    if (d.head_dim_k % 8 || d.head_dim_v % 8) {
        *why = "one-launch step: head dims must be multiples of 8";
        return false;
    }
    const int G = p.num_q_heads / d.num_kv_heads;
    if (int64_t(G) * d.head_dim_v > int64_t(kThreads) * kMaxAcc) {
        *why = "one-launch step: (q heads per KV head) x head_dim_v above " + std::to_string(kThreads * kMaxAcc);
        return false;
    }
    if (pool.slots() >= (int64_t(1) << 31)) {
        *why = "one-launch step: pool of 2^31 or more token slots";
        return false;
    }
    if (!pick_lds(pool, p).T) {
        *why = "one-launch step: scores, selection and tiles exceed 64 KiB of LDS (max_len, top_k or heads too large)";
        return false;
    }
    return true;
}

// The one-launch step wins while a request's whole step is short work for one CU.  Measured on
// MI355X (kernel time per step): the five-request worked example takes 15 us in one launch
// against 24 us for the separate kernels; 32 requests of 1024 tokens, top-64 over 4 KV heads,
// take 36 us against 19 us, as one workgroup per request walks its 4 x 64 rows alone.
bool fused_step_preferred(const tsa_kv_pool& pool, const tsa_decode_params& p) {
    std::string why;
    const int64_t rows = int64_t(std::min(p.top_k, p.max_len)) * pool.d.num_kv_heads;
    return p.max_len <= kFusedAutoMaxLen && rows <= kFusedAutoRows && fused_step_supported(pool, p, &why);
}

hipError_t launch_fused_step(const tsa_kv_pool& pool, int layer, const tsa_decode_params& p,
                             const NewRows& rows, const void* q, const void* qidx, const float* widx,
                             const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                             float* out, int32_t* topk, hipStream_t s) {
    const tsa_pool_desc& d = pool.d;
    const FusedLds L = pick_lds(pool, p);
    if (!L.T) return hipErrorInvalidValue;
    const int64_t slots = pool.slots();
    FusedArgs a{};
    a.k_new = static_cast<const uint4*>(rows.k);
    a.v_new = static_cast<const uint4*>(rows.v);
    a.i_new = static_cast<const uint4*>(rows.idx);
    a.bad = rows.bad;
    a.kpool = static_cast<uint16_t*>(pool.k) + int64_t(layer) * slots * d.num_kv_heads * d.head_dim_k;
    a.alias = d.v_from_k != 0;
    if (a.alias) {
        a.vpool = a.kpool;
        a.v_stride = d.head_dim_k;
    } else {
        a.vpool = static_cast<uint16_t*>(pool.v) + int64_t(layer) * slots * d.num_kv_heads * d.head_dim_v;
        a.v_stride = d.head_dim_v;
    }
    a.ipool = static_cast<uint16_t*>(pool.idx) + int64_t(layer) * slots * d.index_dim;
    a.q = static_cast<const uint16_t*>(q);
    a.qidx = static_cast<const uint16_t*>(qidx);
    a.widx = widx;
    a.page_table = page_table;
    a.seq_lens = seq_lens;
    a.out = out;
    a.topk = topk;
    a.max_pages = max_pages;
    a.page_size = d.page_size;
    a.num_pages = d.num_pages;
    a.max_len = p.max_len;
    a.k = p.top_k;
    a.hq = p.num_q_heads;
    a.hkv = d.num_kv_heads;
    a.dk = d.head_dim_k;
    a.dv = d.head_dim_v;
    a.H = p.index_heads;
    a.D = d.index_dim;
    a.T = L.T;
    a.scale = p.sm_scale;
    a.off_sel = L.off_sel;
    a.off_u = L.off_u;
    a.off_qf = L.off_qf;
    a.off_q = L.off_q;
    a.off_pt = L.off_pt;
    a.off_k = L.off_k;
    a.off_v = L.off_v;
    a.off_lg = L.off_lg;
    a.off_m = L.off_m;
    hipLaunchKernelGGL(fused_step_kernel, dim3(p.batch), dim3(kThreads), L.total, s, a);
    return hipGetLastError();
}

}  // namespace tsa
