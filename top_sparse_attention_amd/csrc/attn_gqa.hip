// Sparse gather-attention on the matrix cores for grouped-query shapes: up to 16 query heads per
// KV head, keys and values stored apart, head dims (keys, values) of (64, 64), (128, 128),
// (192, 128) or (256, 256).
//
// GLM5.3 sparse-attention page: SDPA runs over only the tokens the indexer kept (opening
// paragraph), one selection for every head (lightning-indexer paragraph).  For query head h of
// request b and KV head g = h / G (G = Hq / Hkv):
//     o[b][h] = softmax_j(scale * q[b][h] . K[t_j, g]) . V[t_j, g]
//
// One wave owns one unit (request, KV head, split of the selected list) and works alone, with no
// workgroup barrier.  It writes the unit's physical rows to LDS, then streams 32-row tiles of K
// and V through a private ring of LDS slots with global-to-LDS loads (all but one slot in flight
// while the oldest is consumed).  Per tile:
//   S^T = K_tile Q^T   2 row blocks x DK/32 k-steps of mfma_f32_16x16x32_bf16; tokens are rows, the
//                      G heads are columns padded to 16 (zero queries, never written out);
//   softmax            online, per head: running max (log2 units) and sum, with the accumulator
//                      rescaled when the max moves;
//   O^T += V^T P^T     DV/16 output blocks of 16 dims, each with P split into bf16 hi + lo (two
//                      MFMAs, fp32-like accuracy).  V^T comes straight from the tile through the
//                      LDS transpose read; the contraction index k = 8 g + i of lane group g
//                      stands for token (i < 4 ? 4 g + i : 16 + 4 g + i - 4), which is exactly
//                      where the S^T accumulator left that lane's probabilities, so P needs no
//                      shuffle.
// Rows are stored with their 16-byte chunks XOR-swizzled by row, so the rows an MFMA operand read
// touches fall on distinct LDS banks (on 16 bank groups; 64-dim rows, 8 chunks wide, pair up).
//
// With few (request, KV head) pairs (at most 256: one workgroup per CU), the splits of a pair run
// as the waves of one workgroup instead (kMergeWaves of them), each exactly as above, and merge
// their running max, sum and accumulator through LDS at the end: the split partials never reach
// memory and the step needs no combine launch.
#include "tsa_internal.h"
#include "mfma_lds.h"

namespace {

constexpr int kMaxG = 16;                        // query heads per KV head (one MFMA column block)
constexpr int kTileG = 32;                       // rows per tile
// Two tiles per wave and one wave per workgroup (36 KiB of LDS at 128 dims, so four waves share
// a CU, and a CU picks up a new unit as soon as any of its waves finishes).  Measured on the
// 128-request shared-prefix workload: 60 us, against 70-98 us for 3-4 tiles per wave or 2-4
// units per workgroup (fewer waves per CU, or units that hold their CU until the slowest of the
// group is done).
constexpr int kRingG = 2;                        // tiles per wave in LDS (the loop assumes 2)
constexpr int kUnitsPerWg = 1;                   // waves (units) per workgroup
constexpr int kRowsMaxG = 1024;                  // selected rows per unit (its LDS row list)
constexpr int kMergeWaves = 4;                   // splits merged inside one workgroup
constexpr float kLog2eG = 1.4426950408889634f;

template <int DK, int DV>
struct GqaGeo {
    static constexpr int kChunksK = DK / 8, kChunksV = DV / 8;        // 16-byte chunks per row
    static constexpr int kRowBytesK = DK * 2, kRowBytesV = DV * 2;
    static constexpr int kHalfK = kTileG * kRowBytesK, kHalfV = kTileG * kRowBytesV;
    static constexpr int kTileBytes = kHalfK + kHalfV;
    static constexpr int kLoadsK = kHalfK / 1024, kLoadsV = kHalfV / 1024;   // wave-wide 1 KiB loads
    static constexpr int kLoadsTile = kLoadsK + kLoadsV;
    static constexpr int kWaveLds = kRingG * kTileBytes + kRowsMaxG * 4;
    static_assert(kHalfK % 1024 == 0 && kHalfV % 1024 == 0, "whole wave loads per tile half");
    static_assert(kLoadsTile < 64, "vmcnt range");
    static_assert(DK % 32 == 0 && DV % 16 == 0, "MFMA k-steps and output blocks");
};

// stored chunk position of logical chunk c in a tile row r of C chunks (an involution on c):
// full groups of 16 chunks XOR the low 4 bits of the row, a trailing group of 8 the low 3
template <int C>
__device__ __forceinline__ int swz(int r, int c) {
    if constexpr (C % 16 == 0) return c ^ (r & 15);
    else if constexpr (C == 8) return c ^ (r & 7);
    else return c < (C & ~15) ? (c ^ (r & 15)) : (c ^ (r & 7));
}

struct GqaArgs {
    const uint16_t* q;          // [B][Hq][DK]
    const int32_t* topk;        // [B][k]
    const int32_t* page_table;
    const int32_t* seq_lens;
    const uint16_t* kpool;      // layer bases; row (slot, g) at (slot * hkv + g) * DK (V: * DV)
    const uint16_t* vpool;
    float* out;                 // [B][Hq][DV]
    float* part_ml;             // [B][Hq][S][2]
    float* part_acc;            // [B][Hq][S][DV]
    int k, max_pages, page_size, num_pages, max_len, hq, hkv, splits, chunk, n_units;
    float scale_log2;           // sm_scale * log2(e)
};

// W = 1: one independent unit per workgroup; W = kMergeWaves: workgroup = (request, KV head), wave
// = split, merged in LDS at the end.
template <int DK, int DV, int W>
__global__ void __launch_bounds__(64 * W) attn_gqa_kernel(GqaArgs a) {
    using Geo = GqaGeo<DK, DV>;
    constexpr int CK = Geo::kChunksK, CV = Geo::kChunksV;
    extern __shared__ __align__(16) unsigned char smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int unit = W == 1 ? int(blockIdx.x) * kUnitsPerWg + wave : int(blockIdx.x) * W + wave;
    if (unit >= a.n_units) return;                      // uniform (W > 1: every wave of the group)
    unsigned char* ring = smem + wave * Geo::kWaveLds;
    int32_t* rows = reinterpret_cast<int32_t*>(ring + kRingG * Geo::kTileBytes);
    const int s_idx = unit % a.splits;
    const int g = (unit / a.splits) % a.hkv;
    const int b = unit / (a.splits * a.hkv);
    const int G = a.hq / a.hkv;
    const int j16 = lane & 15, g16 = lane >> 4;

    int len = a.seq_lens[b];
    len = len < 0 ? 0 : (len > a.max_len ? a.max_len : len);
    const int n_sel = min(len, a.k);
    const int j0 = s_idx * a.chunk;
    const int n = max(min(j0 + a.chunk, n_sel) - j0, 0);
    const int n_tiles = (n + kTileG - 1) / kTileG;

    // queries, the B operand of S^T = K Q^T: lane (j16, g16) holds dims 32 ks + 8 g16 .. of
    // head h0 + j16
    const int h0 = g * G;
    uint4 qreg[DK / 32];
    {
        const bool hv = j16 < G;
        const uint4* src = reinterpret_cast<const uint4*>(a.q + (int64_t(b) * a.hq + h0 + (hv ? j16 : 0)) * DK);
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks) qreg[ks] = hv ? src[4 * ks + g16] : make_uint4(0, 0, 0, 0);
    }
    // physical rows (slot * hkv + g) of the unit's positions, -1 when absent (fetched from row 0
    // like any other and masked out of the softmax); all position loads, then all page loads
    {
        constexpr int kPer = kRowsMaxG / 64;
        const int32_t* sel = a.topk + int64_t(b) * a.k;
        const int32_t* pt = a.page_table + int64_t(b) * a.max_pages;
        int tpos[kPer], page[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int j = lane + 64 * i;
            const int t = j < n ? sel[j0 + j] : -1;
            tpos[i] = (t >= 0 && t < len) ? t : -1;
        }
#pragma unroll
        for (int i = 0; i < kPer; ++i) page[i] = tpos[i] >= 0 ? pt[tpos[i] / a.page_size] : -1;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int j = lane + 64 * i;
            if (j < n_tiles * kTileG) {
                const bool ok = page[i] >= 0 && page[i] < a.num_pages;
                rows[j] = ok ? (page[i] * a.page_size + tpos[i] % a.page_size) * a.hkv + g : -1;
            }
        }
    }
    __builtin_amdgcn_wave_barrier();

    const uint32_t ring_base = lds_addr(ring);
    // tile t into slot t % kRingG: load i of a half fills its 1 KiB at 1024 i, lane l the 16 bytes
    // at chunk position 64 i + l of the row-major stored layout, so each lane fetches the logical
    // chunk that belongs there
    auto issue_tile = [&](int t) {
        const uint32_t slot = ring_base + uint32_t((t % kRingG) * Geo::kTileBytes);
#pragma unroll
        for (int i = 0; i < Geo::kLoadsK; ++i) {
            const int pc = 64 * i + lane, r = pc / CK;
            const int32_t row = rows[t * kTileG + r];
            load_lds16(a.kpool + int64_t(row < 0 ? 0 : row) * DK + swz<CK>(r, pc % CK) * 8,
                       __builtin_amdgcn_readfirstlane(slot + uint32_t(i * 1024)));
        }
#pragma unroll
        for (int i = 0; i < Geo::kLoadsV; ++i) {
            const int pc = 64 * i + lane, r = pc / CV;
            const int32_t row = rows[t * kTileG + r];
            load_lds16(a.vpool + int64_t(row < 0 ? 0 : row) * DV + swz<CV>(r, pc % CV) * 8,
                       __builtin_amdgcn_readfirstlane(slot + uint32_t(Geo::kHalfK + i * 1024)));
        }
    };
    // lane-constant byte offsets in a tile: K operand of row j16 (+16 rows for the second
    // block), chunk 4 ks + g16; V^T transpose reads of rows r0 and r0 + 16, dims 16 db + e0 ..
    int koff[DK / 32], voff[DV / 16];
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) koff[ks] = j16 * Geo::kRowBytesK + swz<CK>(j16, 4 * ks + g16) * 16;
    {
        const int r0 = 4 * g16 + (j16 >> 2), e0 = 4 * (j16 & 3);
#pragma unroll
        for (int db = 0; db < DV / 16; ++db)
            voff[db] = Geo::kHalfK + r0 * Geo::kRowBytesV + swz<CV>(r0, 2 * db + (e0 >> 3)) * 16 + (e0 & 7) * 2;
    }

    for (int t = 0; t < kRingG - 1 && t < n_tiles; ++t) issue_tile(t);
    float m_run = -INFINITY;     // head j16: running max of the scaled logits (log2 units)
    float l_run = 0.f;           // this lane's share of head j16's running sum
    f32x4 acc[DV / 16];          // O^T[16 db + 4 g16 + r][head j16], unnormalised
#pragma unroll
    for (int db = 0; db < DV / 16; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int t = 0; t < n_tiles; ++t) {
        // the slot tile t + 1 takes held tile t - 1, read (and consumed) in the previous iteration
        if (t + 1 < n_tiles) {
            issue_tile(t + 1);
            wait_vm<Geo::kLoadsTile>();      // tile t landed, tile t + 1 in flight
        } else {
            wait_vm<0>();
        }
        const unsigned char* tile = ring + (t % kRingG) * Geo::kTileBytes;
        // tokens of the tile that are present
        const uint32_t live = uint32_t(__ballot(lane < kTileG && t * kTileG + lane < n &&
                                                rows[t * kTileG + (lane & (kTileG - 1))] >= 0));
        f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks) {
            const uint4 k0 = *reinterpret_cast<const uint4*>(tile + koff[ks]);
            const uint4 k1 = *reinterpret_cast<const uint4*>(tile + koff[ks] + 16 * Geo::kRowBytesK);
            const bf16x8 qb = as_bf16x8(qreg[ks]);
            s[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(k0), qb, s[0], 0, 0, 0);
            s[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(k1), qb, s[1], 0, 0, 0);
        }
        // online softmax; this lane holds head j16's tokens (i >> 2) * 16 + 4 g16 + (i & 3)
        float x[8];
        float tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int tok = (i >> 2) * 16 + 4 * g16 + (i & 3);
            x[i] = ((live >> tok) & 1u) ? s[i >> 2][i & 3] * a.scale_log2 : -INFINITY;
            tmax = fmaxf(tmax, x[i]);
        }
        tmax = max4groups(tmax);
        const float m_new = fmaxf(m_run, tmax);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;   // no token yet: any finite value
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_new;
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x[i] = __builtin_amdgcn_exp2f(x[i] - m_use);
            psum += x[i];
        }
        l_run = l_run * alpha + psum;
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t hb = pack_bf16(x[2 * e], x[2 * e + 1]);
            hw[e] = hb;
            lw[e] = pack_bf16(x[2 * e] - __uint_as_float(hb << 16),
                              x[2 * e + 1] - __uint_as_float(hb & 0xffff0000u));
        }
        const bf16x8 phi = as_bf16x8(make_uint4(hw[0], hw[1], hw[2], hw[3]));
        const bf16x8 plo = as_bf16x8(make_uint4(lw[0], lw[1], lw[2], lw[3]));
#pragma unroll
        for (int db = 0; db < DV / 16; ++db) {
            const unsigned char* p0 = tile + voff[db];
            const uint2 w0 = lds_read_tr16(p0);
            const uint2 w1 = lds_read_tr16(p0 + 16 * Geo::kRowBytesV);
            const bf16x8 va = as_bf16x8(make_uint4(w0.x, w0.y, w1.x, w1.y));
            acc[db] = acc[db] * alpha;
            acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, phi, acc[db], 0, 0, 0);
            acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, plo, acc[db], 0, 0, 0);
        }
    }

    const float l_tot = sum4groups(l_run);
    if constexpr (W > 1) {
        // each wave leaves (max, sum) of its lanes' heads and its O^T blocks in its own ring, which
        // only it has used; after the barrier wave w writes output blocks w, w + W, ...
        float* mine = reinterpret_cast<float*>(ring);
        f32x4* macc = reinterpret_cast<f32x4*>(ring + 512);
        mine[lane] = m_run;
        mine[64 + lane] = l_tot;
#pragma unroll
        for (int db = 0; db < DV / 16; ++db) macc[db * 64 + lane] = acc[db];
        __syncthreads();
        float wt[W];
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            wt[w] = reinterpret_cast<const float*>(smem + w * Geo::kWaveLds)[lane];
            M = fmaxf(M, wt[w]);
        }
        float L = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            // a split without tokens has max -inf, sum 0 and a zero accumulator
            wt[w] = wt[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(wt[w] - M);
            L += wt[w] * reinterpret_cast<const float*>(smem + w * Geo::kWaveLds)[64 + lane];
        }
        if (j16 >= G) return;
        const float inv = L > 0.f ? 1.f / L : 0.f;
        float* o = a.out + (int64_t(b) * a.hq + h0 + j16) * DV;
        for (int db = wave; db < DV / 16; db += W) {
            f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < W; ++w)
                x += wt[w] * reinterpret_cast<const f32x4*>(smem + w * Geo::kWaveLds + 512)[db * 64 + lane];
            *reinterpret_cast<float4*>(o + db * 16 + 4 * g16) = make_float4(x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv);
        }
        return;
    }
    if (j16 >= G) return;
    const int h = h0 + j16;
    if (a.splits == 1) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        float* o = a.out + (int64_t(b) * a.hq + h) * DV;
#pragma unroll
        for (int db = 0; db < DV / 16; ++db)
            *reinterpret_cast<float4*>(o + db * 16 + 4 * g16) =
                make_float4(acc[db][0] * inv, acc[db][1] * inv, acc[db][2] * inv, acc[db][3] * inv);
    } else {
        const int64_t pidx = (int64_t(b) * a.hq + h) * a.splits + s_idx;
        float* o = a.part_acc + pidx * DV;
#pragma unroll
        for (int db = 0; db < DV / 16; ++db)
            *reinterpret_cast<float4*>(o + db * 16 + 4 * g16) =
                make_float4(acc[db][0], acc[db][1], acc[db][2], acc[db][3]);
        if (g16 == 0) {
            // natural-log units, as the combine expects
            a.part_ml[pidx * 2] = m_run == -INFINITY ? -INFINITY : m_run * 0.6931471805599453f;
            a.part_ml[pidx * 2 + 1] = l_tot;
        }
    }
}

}  // namespace

namespace {

// LDS bytes of one wave for a shape the kernel takes, 0 for others
size_t gqa_wave_lds(int dk, int dv) {
    if (dk == 64 && dv == 64) return GqaGeo<64, 64>::kWaveLds;
    if (dk == 128 && dv == 128) return GqaGeo<128, 128>::kWaveLds;
    if (dk == 192 && dv == 128) return GqaGeo<192, 128>::kWaveLds;
    if (dk == 256 && dv == 256) return GqaGeo<256, 256>::kWaveLds;
    return 0;
}

template <int DK, int DV, int W>
hipError_t launch_gqa_w(const GqaArgs& a, hipStream_t s) {
    auto kern = attn_gqa_kernel<DK, DV, W>;
    const int per_wg = W == 1 ? kUnitsPerWg : W;
    const size_t smem = size_t(per_wg) * GqaGeo<DK, DV>::kWaveLds;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
    if (e != hipSuccess) return e;
    const int wgs = (a.n_units + per_wg - 1) / per_wg;
    hipLaunchKernelGGL(kern, dim3(wgs), dim3(64 * per_wg), smem, s, a);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_gqa(const GqaArgs& a, bool merge, hipStream_t s) {
    if constexpr (kMergeWaves * GqaGeo<DK, DV>::kWaveLds <= 160 * 1024) {
        if (merge) return launch_gqa_w<DK, DV, kMergeWaves>(a, s);
    } else {
        if (merge) return hipErrorInvalidValue;
    }
    return launch_gqa_w<DK, DV, 1>(a, s);
}

}  // namespace

namespace tsa {

bool gqa_mfma_applicable(const tsa_kv_pool& pool, const tsa_decode_params& p) {
    const tsa_pool_desc& d = pool.d;
    if (d.v_from_k || !gqa_wave_lds(d.head_dim_k, d.head_dim_v)) return false;
    if (p.num_q_heads % d.num_kv_heads || p.num_q_heads / d.num_kv_heads > kMaxG) return false;
    if (pool.slots() * int64_t(d.num_kv_heads) >= (int64_t(1) << 31)) return false;   // int32 rows
    int splits = 0;
    return gqa_mfma_chunk(pool, p, &splits) <= kRowsMaxG;
}

// Rows per unit.  Enough splits that the units fill every CU's workgroup slots, then the split
// count whose workgroups come closest to whole rounds over the CUs (equal units finish together,
// so a partial last round leaves CUs idle), preferring fewer splits.
int gqa_mfma_chunk(const tsa_kv_pool& pool, const tsa_decode_params& p, int* splits) {
    const int k_eff = std::max(1, std::min(p.top_k, p.max_len));
    const int tiles = int(ceil_div(k_eff, kTileG));
    const int64_t base = std::max<int64_t>(1, int64_t(p.batch) * pool.d.num_kv_heads);
    const size_t wave_lds = std::max<size_t>(1, gqa_wave_lds(pool.d.head_dim_k, pool.d.head_dim_v));
    const int wg_per_cu = std::max<int>(1, int((160 * 1024) / (kUnitsPerWg * wave_lds)));   // LDS-bound
    const int64_t wg_slots = int64_t(256) * wg_per_cu;
    const int64_t slots = wg_slots * kUnitsPerWg;
    int s_min = int(std::max<int64_t>(1, ceil_div(slots, base)));
    s_min = std::max(s_min, int(ceil_div(tiles, kRowsMaxG / kTileG)));
    s_min = std::min({s_min, tiles, 64});
    int best_s = s_min;
    double best_fill = -1.0;
    for (int s = s_min; s <= std::min({2 * s_min + 1, tiles, 64}); ++s) {
        const int chunk_t = int(ceil_div(tiles, s));
        const int sp = int(ceil_div(tiles, chunk_t));
        const int64_t wgs = ceil_div(base * sp, kUnitsPerWg);
        const double fill = double(wgs) / double(ceil_div(wgs, wg_slots) * wg_slots);
        if (fill > best_fill + 0.02) {
            best_fill = fill;
            best_s = s;
        }
    }
    const int chunk = int(ceil_div(tiles, best_s)) * kTileG;
    *splits = int(ceil_div(k_eff, chunk));
    return chunk;
}

// Splits merged inside the workgroup: for 64 to 256 (request, KV head) pairs (one workgroup of
// kMergeWaves waves per CU at most, and at least a quarter of the CUs busy), selections of at
// least one tile per wave, and head dims whose kMergeWaves rings fit in LDS.
bool gqa_wg_merge(const tsa_kv_pool& pool, const tsa_decode_params& p) {
    const int64_t base = int64_t(p.batch) * pool.d.num_kv_heads;
    const int k_eff = std::max(1, std::min(p.top_k, p.max_len));
    const size_t lds = gqa_wave_lds(pool.d.head_dim_k, pool.d.head_dim_v);
    return base >= 64 && base <= 256 && k_eff >= kMergeWaves * kTileG && lds > 0 &&
           kMergeWaves * lds <= 160 * 1024 && ceil_div(k_eff, kMergeWaves) <= kRowsMaxG;
}

hipError_t launch_attention_gqa(const tsa_kv_pool& pool, int layer, const tsa_decode_params& p,
                                const AttnPlan& plan, const void* q, const int32_t* topk,
                                const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                                float* out, float* part_ml, float* part_acc, hipStream_t s) {
    const tsa_pool_desc& d = pool.d;
    GqaArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.topk = topk;
    a.page_table = page_table;
    a.seq_lens = seq_lens;
    const int64_t layer_rows = pool.slots() * d.num_kv_heads;
    a.kpool = static_cast<const uint16_t*>(pool.k) + int64_t(layer) * layer_rows * d.head_dim_k;
    a.vpool = static_cast<const uint16_t*>(pool.v) + int64_t(layer) * layer_rows * d.head_dim_v;
    a.out = out;
    a.part_ml = part_ml;
    a.part_acc = part_acc;
    a.k = p.top_k;
    a.max_pages = max_pages;
    a.page_size = d.page_size;
    a.num_pages = d.num_pages;
    a.max_len = p.max_len;
    a.hq = p.num_q_heads;
    a.hkv = d.num_kv_heads;
    a.splits = plan.splits;
    a.chunk = plan.chunk;
    a.n_units = p.batch * d.num_kv_heads * plan.splits;
    a.scale_log2 = p.sm_scale * kLog2eG;
    if (plan.wg_merge && plan.splits != kMergeWaves) return hipErrorInvalidValue;
    if (d.head_dim_k == 64) return launch_gqa<64, 64>(a, plan.wg_merge, s);
    if (d.head_dim_k == 128) return launch_gqa<128, 128>(a, plan.wg_merge, s);
    if (d.head_dim_k == 192) return launch_gqa<192, 128>(a, plan.wg_merge, s);
    if (d.head_dim_k == 256) return launch_gqa<256, 256>(a, plan.wg_merge, s);
    return hipErrorInvalidValue;
}

}  // namespace tsa
