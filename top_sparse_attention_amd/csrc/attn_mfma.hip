// Sparse gather-attention on the matrix cores, for the MQA mode of MLA: many query heads over
// one latent KV head whose first head_dim_v dims are the values.
//
// GLM5.3 sparse-attention page: DSA runs MLA in MQA mode (MLA-modes paragraph) over the top-k
// tokens the indexer kept; with H = 64 query heads every latent row is reused by 64 heads, so
// QK^T and PV are dense contractions (roofline paragraph: about 120 FLOP per byte at the GLM-5
// shape, far above what the vector ALUs sustain per byte of HBM bandwidth).
//
// Formulation per workgroup (one request, one split of its selected tokens; four waves, each
// owning 16 query heads):
//   S^T [tokens x heads] = K_tile [tokens x dk] . Q^T [dk x heads]      (MFMA 16x16x32 bf16)
//       A operand: K rows read from LDS (token-major, 16 bytes per lane)
//       B operand: the wave's queries, held in registers for the whole kernel
//   online softmax over the token axis, per head (a lane always holds one head's column)
//   O^T [dv x heads] += V^T [dv x tokens] . P^T [tokens x heads]        (MFMA 16x16x32 bf16)
//       A operand: the same LDS tile read with the LDS transpose load, which hands each lane
//                  4 consecutive tokens of one value dim, so no transposed copy is stored
//       B operand: P taken straight from the S^T accumulators (the contraction runs over the
//                  tokens in a permuted order; A and B use the same permutation)
// P is split into bf16 hi + lo parts (two PV MFMAs) so the probabilities keep ~16 bits.
// Tiles of 64 selected rows are gathered from the page table straight into LDS (global-to-LDS
// loads, no staging registers), double-buffered: the next tile streams in while the current one
// is computed.
#include "tsa_internal.h"

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 64;                 // selected rows per tile
constexpr float kLog2e = 1.4426950408889634f;

template <int DK>
struct Geo {
    static constexpr int kChunks = DK / 8;                // 16-byte chunks of a row
    static constexpr int kRowChunks = kChunks + 1;        // +1 padding chunk staggers LDS banks
    static constexpr int kRowBytes = kRowChunks * 16;
    static constexpr int kTileBytes = kTile * kRowBytes;
    // one wave-wide direct load fills 64 consecutive 16-byte LDS chunks; a tile of 64 padded
    // rows is therefore exactly kRowChunks such loads
    static constexpr int kLoads = kRowChunks;
};

__device__ inline bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef __attribute__((address_space(3))) unsigned char lds_u8;

// Wave-wide global-to-LDS load: lane i's 16 bytes land at lds + 16 * i.
__device__ inline void load_lds16(const void* gsrc, unsigned char* lds) {
    __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void*)((lds_u8*)(lds)),
                                     16, 0, 0);
}

// LDS transpose load of 4 x 16-bit (see the formulation above for the lane mapping).
__device__ inline uint2 lds_read_tr16(const unsigned char* p) {
    lds_i16x4* lp = (lds_i16x4*)((lds_u8*)(p));
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(lp));
}

struct MfmaArgs {
    const uint16_t* q;         // [B][Hq][DK]
    const int32_t* topk;       // [B][k]
    const int32_t* page_table;
    const int32_t* seq_lens;
    const uint16_t* kpool;     // layer base; row of slot s at s * DK (one latent head)
    float* out;                // [B][Hq][DV]
    float* part_ml;            // [B][Hq][S][2]
    float* part_acc;           // [B][Hq][S][DV]
    int k, max_pages, page_size, num_pages, max_len, hq, splits, chunk;
    float scale_log2;          // sm_scale * log2(e)
};

template <int DK, int DV>
__global__ void __launch_bounds__(kThreads, 1) attn_mfma_kernel(MfmaArgs a) {
    using G = Geo<DK>;
    constexpr int KS = DK / 32;   // QK k-steps
    constexpr int DB = DV / 16;   // output dim blocks per wave
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char* tiles = smem;                                              // 2 x [kTile][kRowBytes]
    int32_t* rows = reinterpret_cast<int32_t*>(smem + 2 * G::kTileBytes);   // [chunk] slot or -1

    const int s_idx = blockIdx.x, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g16 = lane >> 4, j16 = lane & 15;
    const int h0 = blockIdx.y * (kWaves * 16) + wave * 16;   // this wave's first head

    int len = a.seq_lens[b];
    len = len < 0 ? 0 : (len > a.max_len ? a.max_len : len);
    const int n_sel = min(len, a.k);
    const int j0 = s_idx * a.chunk;
    const int j1 = min(j0 + a.chunk, n_sel);
    const int n = max(j1 - j0, 0);

    // resolve this split's selected positions to physical rows; zero both tile buffers so rows
    // that are never loaded (past the selection) hold finite values
    {
        const int32_t* sel = a.topk + int64_t(b) * a.k;
        const int32_t* pt = a.page_table + int64_t(b) * a.max_pages;
        for (int j = tid; j < a.chunk; j += kThreads) {
            int32_t row = -1;
            if (j < n) {
                const int t = sel[j0 + j];
                if (t >= 0 && t < len) {
                    const int page = pt[t / a.page_size];
                    if (page >= 0 && page < a.num_pages) row = page * a.page_size + t % a.page_size;
                }
            }
            rows[j] = row;
        }
        for (int i = tid; i < 2 * G::kTileBytes / 16; i += kThreads)
            reinterpret_cast<uint4*>(tiles)[i] = make_uint4(0, 0, 0, 0);
    }

    // queries of this wave's 16 heads, as the B operand of S^T = K Q^T
    uint4 qreg[KS];
    {
        const uint4* qsrc = reinterpret_cast<const uint4*>(a.q + (int64_t(b) * a.hq + h0 + j16) * DK);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qreg[ks] = qsrc[ks * 4 + g16];
    }

    f32x4 acc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;   // running max (log2 units) of head h0 + j16
    float l_run = 0.f;         // this lane's share of the running sum

    __syncthreads();
    const int n_tiles = (n + kTile - 1) / kTile;

    // issue the direct loads of tile t into buffer t & 1: load i of the tile covers padded
    // chunks 64 i .. 64 i + 63; waves take loads round-robin; padding and absent rows are skipped
    auto issue_tile = [&](int t) {
        unsigned char* buf = tiles + (t & 1) * G::kTileBytes;
        for (int i = wave; i < G::kLoads; i += kWaves) {
            const int c = i * 64 + lane;
            const int r = c / G::kRowChunks, col = c - r * G::kRowChunks;
            const int j = t * kTile + r;
            const int32_t row = (col < G::kChunks && j < n) ? rows[j] : -1;
            if (row >= 0) load_lds16(a.kpool + int64_t(row) * DK + col * 8, buf + i * 1024);
        }
    };
    if (n_tiles > 0) issue_tile(0);

    for (int t = 0; t < n_tiles; ++t) {
        __builtin_amdgcn_s_waitcnt(0);   // this wave's loads of tile t have landed
        __syncthreads();                 // everyone's have, and tile t-1 is no longer read
        if (t + 1 < n_tiles) issue_tile(t + 1);
        const unsigned char* tile = tiles + (t & 1) * G::kTileBytes;

        // ---- S^T = K Q^T : four 16-token blocks x 16 heads
        f32x4 s[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) s[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 qb = as_bf16x8(qreg[ks]);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const uint4 kv = *reinterpret_cast<const uint4*>(
                    tile + (tb * 16 + j16) * G::kRowBytes + (ks * 32 + g16 * 8) * 2);
                s[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kv), qb, s[tb], 0, 0, 0);
            }
        }
        // lane holds S^T[token tb*16 + 4*g16 + r][head h0 + j16]
        const int valid = min(kTile, n - t * kTile);
        float tmax = -INFINITY;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tok = tb * 16 + g16 * 4 + r;
                float x = s[tb][r] * a.scale_log2;
                x = tok < valid ? x : -INFINITY;
                s[tb][r] = x;
                tmax = fmaxf(tmax, x);
            }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = (m_run == -INFINITY) ? 1.f : exp2f(m_run - m_new);
        float psum = 0.f;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = (s[tb][r] == -INFINITY) ? 0.f : exp2f(s[tb][r] - m_new);
                s[tb][r] = p;
                psum += p;
            }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int i = 0; i < DB; ++i) acc[i] *= alpha;

        // ---- O^T += V^T P^T over two 32-token k-steps
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            // B operand: P^T[kappa][head], kappa = 8*g16 + i  <->  token kk*32 + (i < 4 ? 4*g16 + i
            //            : 16 + 4*g16 + i - 4), i.e. blocks 2kk and 2kk+1 of the S^T accumulators
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p0 = (e < 2) ? s[2 * kk][2 * e] : s[2 * kk + 1][2 * e - 4];
                const float p1 = (e < 2) ? s[2 * kk][2 * e + 1] : s[2 * kk + 1][2 * e - 3];
                const uint32_t u0 = __float_as_uint(p0) & 0xffff0000u;
                const uint32_t u1 = __float_as_uint(p1) & 0xffff0000u;
                const float r0 = p0 - __uint_as_float(u0), r1 = p1 - __uint_as_float(u1);
                // remainders rounded to nearest bf16
                const uint32_t v0 = __float_as_uint(r0), v1 = __float_as_uint(r1);
                const uint32_t w0 = (v0 + 0x7fffu + ((v0 >> 16) & 1u)) >> 16;
                const uint32_t w1 = (v1 + 0x7fffu + ((v1 >> 16) & 1u)) >> 16;
                hi[e] = (u0 >> 16) | u1;
                lo[e] = w0 | (w1 << 16);
            }
            const bf16x8 phi = as_bf16x8(make_uint4(hi[0], hi[1], hi[2], hi[3]));
            const bf16x8 plo = as_bf16x8(make_uint4(lo[0], lo[1], lo[2], lo[3]));
            // A operand: V^T[d][kappa] via the transpose load.  In each 16-lane group, lane i
            // points at row k0 + i/4, dims n0 + 4*(i%4); lane j receives rows k0..k0+3 of dim n0+j.
            const int rbase0 = kk * 32 + 4 * g16 + (j16 >> 2);
            const int rbase1 = rbase0 + 16;
            const int cofs = 4 * (j16 & 3);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int col = db * 16 + cofs;
                const uint2 w0 = lds_read_tr16(tile + rbase0 * G::kRowBytes + col * 2);
                const uint2 w1 = lds_read_tr16(tile + rbase1 * G::kRowBytes + col * 2);
                const bf16x8 va = as_bf16x8(make_uint4(w0.x, w0.y, w1.x, w1.y));
                acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, phi, acc[db], 0, 0, 0);
                acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, plo, acc[db], 0, 0, 0);
            }
        }
    }

    // full row sum of head h0 + j16 across the four lane groups
    float l_tot = l_run;
    l_tot += __shfl_xor(l_tot, 16);
    l_tot += __shfl_xor(l_tot, 32);
    const int h = h0 + j16;
    // lane holds O^T[d = db*16 + 4*g16 + r][head h]
    if (a.splits == 1) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        float* o = a.out + (int64_t(b) * a.hq + h) * DV;
#pragma unroll
        for (int db = 0; db < DB; ++db)
            *reinterpret_cast<float4*>(o + db * 16 + g16 * 4) =
                make_float4(acc[db][0] * inv, acc[db][1] * inv, acc[db][2] * inv, acc[db][3] * inv);
    } else {
        const int64_t pidx = (int64_t(b) * a.hq + h) * a.splits + s_idx;
        float* o = a.part_acc + pidx * DV;
#pragma unroll
        for (int db = 0; db < DB; ++db)
            *reinterpret_cast<float4*>(o + db * 16 + g16 * 4) =
                make_float4(acc[db][0], acc[db][1], acc[db][2], acc[db][3]);
        if (g16 == 0) {
            // natural-log units, as the combine expects
            a.part_ml[pidx * 2] = m_run == -INFINITY ? -INFINITY : m_run * 0.6931471805599453f;
            a.part_ml[pidx * 2 + 1] = l_tot;
        }
    }
}

template <int DK, int DV>
size_t mfma_smem(int chunk) {
    return 2 * size_t(Geo<DK>::kTileBytes) + size_t(chunk) * sizeof(int32_t);
}

}  // namespace

namespace tsa {

// Shapes the latent kernel handles: values alias the keys, 64 query heads per KV head group,
// the 576 / 512 latent widths.
bool mfma_latent_applicable(const tsa_kv_pool& pool, const tsa_decode_params& p) {
    const tsa_pool_desc& d = pool.d;
    if (!d.v_from_k || d.head_dim_k != 576 || d.head_dim_v != 512) return false;
    if (p.num_q_heads % d.num_kv_heads) return false;
    if (pool.slots() >= (int64_t(1) << 31)) return false;   // slots kept as 32-bit in LDS
    if (mfma_smem<576, 512>(int(ceil_div(p.top_k, kTile)) * kTile) > 160 * 1024) return false;
    return p.num_q_heads / d.num_kv_heads == 64 && d.num_kv_heads == 1;
}

int mfma_latent_chunk(const tsa_decode_params& p, int* splits) {
    const int tiles = int(ceil_div(p.top_k, kTile));
    int s = int(ceil_div(256, std::max(p.batch, 1)));   // one workgroup per CU
    s = std::max(1, std::min(s, tiles));
    const int chunk = int(ceil_div(tiles, s)) * kTile;
    *splits = int(ceil_div(p.top_k, chunk));
    return chunk;
}

hipError_t launch_attention_mfma(const tsa_kv_pool& pool, int layer, const tsa_decode_params& p,
                                 const AttnPlan& plan, const void* q, const int32_t* topk,
                                 const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                                 float* out, float* part_ml, float* part_acc, hipStream_t s) {
    const tsa_pool_desc& d = pool.d;
    MfmaArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.topk = topk;
    a.page_table = page_table;
    a.seq_lens = seq_lens;
    a.kpool = static_cast<const uint16_t*>(pool.k) + int64_t(layer) * pool.slots() * d.head_dim_k;
    a.out = out;
    a.part_ml = part_ml;
    a.part_acc = part_acc;
    a.k = p.top_k;
    a.max_pages = max_pages;
    a.page_size = d.page_size;
    a.num_pages = d.num_pages;
    a.max_len = p.max_len;
    a.hq = p.num_q_heads;
    a.splits = plan.splits;
    a.chunk = plan.chunk;
    a.scale_log2 = p.sm_scale * kLog2e;
    auto kern = attn_mfma_kernel<576, 512>;
    const size_t smem = mfma_smem<576, 512>(plan.chunk);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
    if (e != hipSuccess) return e;
    dim3 grid(plan.splits, p.num_q_heads / (kWaves * 16), p.batch);
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), smem, s, a);
    return hipGetLastError();
}

}  // namespace tsa
