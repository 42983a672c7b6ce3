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
//
// Data movement: tiles of 32 selected rows are gathered from the page table straight into LDS
// with global-to-LDS loads (no staging registers), into a ring of 4 buffers so that 3 tiles
// stream in while one is computed.  The loads are issued from inline assembly and waited for
// with explicit vector-memory counts: the compiler would otherwise wait for every outstanding
// LDS-bound load before the first LDS read, which serialises the ring.  A tile is stored as two
// regions: the first DV dims of each row (value dims, DV/8 16-byte chunks, one wave-wide load
// per row) and the remaining DK-DV dims (8 chunks per row, one load per 8 rows).  Within each
// region the chunk index is XOR-swizzled with the row so that row-parallel operand reads spread
// over the LDS banks.
#include "tsa_internal.h"

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 32;                 // selected rows per tile
#ifndef TSA_RING
#define TSA_RING 4
#endif
constexpr int kRing = TSA_RING;           // tile buffers in LDS
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kQkAhead = 4;               // QK k-steps whose LDS operands are read ahead
constexpr float kHeadroom = 32.f;         // log2 headroom of the fixed softmax reference

template <int DK, int DV>
struct Geo {
    static constexpr int kChunksA = DV / 8;                 // value-dim chunks of a row
    static constexpr int kChunksB = (DK - DV) / 8;          // remaining chunks of a row
    static constexpr int kRowBytesA = DV * 2;
    static constexpr int kRowBytesB = (DK - DV) * 2;
    static constexpr int kBytesA = kTile * kRowBytesA;
    static constexpr int kTileBytes = kTile * (kRowBytesA + kRowBytesB);
    static constexpr int kRowsPerWaveA = kTile / kWaves;    // one load per row of region A
    static_assert(kChunksA == 64, "region A rows are one wave-wide load each");
    static_assert(kChunksB == 8, "region B holds 8 chunks of 8 rows per load");
    static_assert(kTile / 8 == kWaves, "one region-B load per wave");
};
constexpr int kLoadsPerWave = kTile / kWaves + 1;

// stored chunk position of logical chunk c of tile row r, region A (groups of 16 chunks) and
// region B (8 chunks per row); both are involutions on c
__device__ __forceinline__ int swz_a(int r, int c) { return c ^ (r & 15); }
__device__ __forceinline__ int swz_b(int r, int c) { return c ^ (((r >> 1) ^ (r << 2)) & 7); }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t lds_addr(const unsigned char* p) {
    return uint32_t(reinterpret_cast<uintptr_t>((lds_u8*)(p)));
}

// Wave-wide global-to-LDS load: lane i's 16 bytes land at (uniform) lds + 16 * i.
__device__ __forceinline__ void load_lds16(const void* gsrc, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" TSA_LOAD_POLICY
                 :
                 : "v"(gsrc), "s"(lds)
                 : "memory", "m0");
}

// The same with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane byte offset.
__device__ __forceinline__ void load_lds16_s(const void* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" TSA_LOAD_POLICY
                 :
                 : "v"(voff), "s"(sbase), "s"(lds)
                 : "memory", "m0");
}

// Wait until at most N vector-memory instructions of this wave are outstanding.  Emitted as a
// real s_waitcnt (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt left at their
// maxima) so that the compiler's own wait tracking sees it too.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// max over lanes l, l^16, l^32, l^48 (the four 16-lane groups), with the cross-half swaps
__device__ __forceinline__ float max4groups(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum4groups(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// two floats rounded to nearest-even bf16, packed (first in the low half)
__device__ __forceinline__ uint32_t pack_bf16(float x, float y) {
    typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
    const bf16x2 v = {(__bf16)x, (__bf16)y};
    return __builtin_bit_cast(uint32_t, v);
}

// LDS transpose load of 4 x 16-bit.  In each 16-lane group, lane i supplies the address of 4
// consecutive elements; lane j receives element j%4 of the data addressed by lanes
// j/4, 4 + j/4, 8 + j/4, 12 + j/4.
__device__ __forceinline__ uint2 lds_read_tr16(const unsigned char* p) {
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
    using G = Geo<DK, DV>;
    constexpr int KS = DK / 32;   // QK k-steps (the first KSA read region A, the rest region B)
    constexpr int KSA = DV / 32;
    constexpr int DB = DV / 16;   // output dim blocks per wave
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char* ring = smem;                                                // kRing tiles
    int32_t* flag = reinterpret_cast<int32_t*>(smem + kRing * G::kTileBytes);  // rescan request
    int32_t* rows = flag + 4;                                                   // [chunk]

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
    const int n_tiles = (n + kTile - 1) / kTile;

    // resolve this split's selected positions to physical rows (-1 = absent: such rows are
    // fetched from slot 0 like any other row and masked out of the softmax)
    {
        const int32_t* sel = a.topk + int64_t(b) * a.k;
        const int32_t* pt = a.page_table + int64_t(b) * a.max_pages;
        for (int j = tid; j < n_tiles * kTile; j += kThreads) {
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
    float m_ref = -INFINITY;   // reference max (log2 units) of head h0 + j16
    float l_run = 0.f;         // this lane's share of the running sum

    // lane-constant byte offsets inside a tile:
    //  QK, region A: row j16 (+16 for the second block), chunk ks*4 + g16 = 16*(ks/4) +
    //      (4*(ks%4) + g16); the swizzle XORs the low 4 bits with the row's low 4 bits (j16)
    //  QK, region B: chunk 4*(ks-KSA) + g16 of row j16 (+16), swizzled within the row's 8
    //  PV: rows r0 = 4*g16 + j16/4 and r0 + 16, dims db*16 + 4*(j16%4): chunk 2*db + b0 =
    //      16*(db/8) + (2*(db%8) + b0), byte (e0 % 8) * 2 inside it
    int qk_off[4], qkb_off[KS - KSA], pv_off[8];
#pragma unroll
    for (int u = 0; u < 4; ++u) qk_off[u] = j16 * G::kRowBytesA + swz_a(j16, 4 * u + g16) * 16;
#pragma unroll
    for (int u = 0; u < KS - KSA; ++u)
        qkb_off[u] = G::kBytesA + j16 * G::kRowBytesB + swz_b(j16, 4 * u + g16) * 16;
    {
        const int r0 = 4 * g16 + (j16 >> 2);
        const int e0 = 4 * (j16 & 3);
#pragma unroll
        for (int u = 0; u < 8; ++u)
            pv_off[u] = r0 * G::kRowBytesA + swz_a(r0, 2 * u + (e0 >> 3)) * 16 + (e0 & 7) * 2;
    }
    // loads: region A row r = wave*8 + m is one wave-wide load (lane = stored chunk position);
    // region B rows wave*8 .. wave*8+7 are one load (lane = 8 * row-in-group + stored chunk)
    const int a_src_chunk = lane;                      // XORed with the row's swizzle per load
    const int b_row = wave * 8 + (lane >> 3);
    const int b_src_el = DV + swz_b(b_row, lane & 7) * 8;

    wait_vm<0>();              // query registers loaded
    if (tid == 0) *flag = 0;
    __syncthreads();           // rows[] and the flag visible

    const uint32_t ring_base = lds_addr(ring);
    // Load m of this wave's share of tile t: m < 8 is region A of row wave*8 + m (one
    // wave-wide load), m == 8 region B of rows wave*8 .. +7.  my8 holds those rows in lanes
    // 0..7 and rowb the row of this lane's region-B chunk.
    auto issue_part = [&](int t, int m, int32_t my8, int32_t rowb) {
        const uint32_t buf = ring_base + uint32_t((t % kRing) * G::kTileBytes);
        if (m < G::kRowsPerWaveA) {
            const int r = wave * 8 + m;
            const int32_t row = __builtin_amdgcn_readlane(my8, m);
            const uint16_t* src = a.kpool + int64_t(row < 0 ? 0 : row) * DK;   // uniform
            load_lds16_s(src, uint32_t(swz_a(r, a_src_chunk) * 16),
                         __builtin_amdgcn_readfirstlane(buf + uint32_t(r * G::kRowBytesA)));
        } else {
            const uint16_t* srcb = a.kpool + int64_t(rowb < 0 ? 0 : rowb) * DK + b_src_el;
            load_lds16(srcb, __builtin_amdgcn_readfirstlane(buf + uint32_t(G::kBytesA + wave * 1024)));
        }
    };
    auto tile_rows = [&](int t, int32_t& my8, int32_t& rowb) {
        my8 = rows[t * kTile + wave * 8 + (lane & 7)];
        rowb = rows[t * kTile + b_row];
    };
    auto issue_tile = [&](int t) {
        int32_t my8, rowb;
        tile_rows(t, my8, rowb);
#pragma unroll
        for (int m = 0; m < kLoadsPerWave; ++m) issue_part(t, m, my8, rowb);
    };
    // A tile issued inside the loop is spread over the iteration: loads kQkLoads[..] after
    // the QK k-steps listed, the rest after PV output groups, so that the load queue drains
    // steadily instead of stalling the wave on a burst.
    int32_t pend_t = -1, pend_my8 = 0, pend_rowb = 0;   // the tile being issued (uniform)

    // Softmax reference: the probabilities are exp2(logit - m_ref) with m_ref fixed at the first
    // tile where the head has a valid token, never rescaled.  Any reference gives the same
    // softmax as long as exp2 cannot overflow, so a tile whose max exceeds m_ref by more than
    // kHeadroom (2^32) switches the whole workgroup to a scan that only tracks the true max;
    // the split is then computed again with m_ref = that max.  Inputs whose logits stay within
    // 2^32 of the first tile's max take one pass.
    float m_seen = -INFINITY;  // max logit (log2 units) over the tiles scanned so far

    // Softmax of one tile as a sequence of small stages, so that they can be slotted between
    // the QK MFMAs of the next tile: the matrix cores work while the vector ALUs run these.
    // State of the tile being normalised:
    float sx[8];                 // scaled logits, then probabilities
    float stmax = -INFINITY, spsum = 0.f;
    bool sviol = false;
    float m_use = 0.f;           // m_ref, or 0 while it is unset
    uint32_t phi_w[4], plo_w[4];
    bool scan = false;           // uniform; the workgroup is only tracking the max
    auto soft_stage = [&](int st, const f32x4 (&sc)[2], uint64_t live) {
        if (st == 0 || st == 1) {
            if (uint32_t(live) == 0xffffffffu) {   // uniform: every token of the tile present
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float x = sc[st][r] * a.scale_log2;
                    sx[4 * st + r] = x;
                    stmax = fmaxf(stmax, x);
                }
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tok = st * 16 + g16 * 4 + r;
                    const float x = ((live >> tok) & 1) ? sc[st][r] * a.scale_log2 : -INFINITY;
                    sx[4 * st + r] = x;
                    stmax = fmaxf(stmax, x);
                }
            }
        } else if (st == 2) {
            stmax = max4groups(stmax);
            m_seen = fmaxf(m_seen, stmax);
            if (m_ref == -INFINITY) m_ref = stmax;   // first tile with a valid token for the head
            sviol = stmax > m_ref + kHeadroom;
            // exp2(-inf - m) = 0 for any finite m; before the head has a reference every
            // logit of the tile is -inf and any finite m does
            m_use = m_ref == -INFINITY ? 0.f : m_ref;
        } else if (st == 3) {
            if (!scan && __ballot(sviol)) *flag = 1;
        } else if (st >= 4 && st < 8) {
            const int i = 2 * (st - 4);
            sx[i] = __builtin_amdgcn_exp2f(sx[i] - m_use);
            sx[i + 1] = __builtin_amdgcn_exp2f(sx[i + 1] - m_use);
            spsum += sx[i] + sx[i + 1];
        } else if (st >= 8 && st < 12) {
            // B operand of PV: P^T[kappa][head], kappa = 8*g16 + i <-> token (i < 4 ? 4*g16 + i :
            // 16 + 4*g16 + i - 4), i.e. sx[i] in order; split into bf16 hi + lo
            const int e = st - 8;
            const uint32_t h = pack_bf16(sx[2 * e], sx[2 * e + 1]);
            phi_w[e] = h;
            plo_w[e] = pack_bf16(sx[2 * e] - __uint_as_float(h << 16),
                                 sx[2 * e + 1] - __uint_as_float(h & 0xffff0000u));
        }
    };
    constexpr int kStages = 12;
    auto soft_reset = [&]() {
        stmax = -INFINITY;
        spsum = 0.f;
        sviol = false;
    };

    // S^T = K Q^T for one tile: two 16-token blocks x 16 heads.  Operand reads run kQkAhead
    // k-steps ahead of the MFMAs (a register ring).  When `prev` is set, softmax stage ks of the
    // previous tile runs after the MFMAs of k-step ks.  The scheduling fences keep the compiler
    // from regrouping the pieces.
    auto qk_tile = [&](const unsigned char* tile, f32x4 (&s)[2], bool with_soft,
                       const f32x4 (&sc)[2], uint64_t live) {
        s[0] = s[1] = f32x4{0.f, 0.f, 0.f, 0.f};
        uint4 kv[kQkAhead][2];
        auto qk_read = [&](int ks, uint4 (&dst)[2]) {
            const unsigned char* base = ks < KSA ? tile + qk_off[ks & 3] + (ks >> 2) * 256
                                                 : tile + qkb_off[ks - KSA];
            const int second = ks < KSA ? 16 * G::kRowBytesA : 16 * G::kRowBytesB;
            dst[0] = *reinterpret_cast<const uint4*>(base);
            dst[1] = *reinterpret_cast<const uint4*>(base + second);
        };
#pragma unroll
        for (int ks = 0; ks < kQkAhead; ++ks) qk_read(ks, kv[ks]);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            __builtin_amdgcn_sched_barrier(0);
            const bf16x8 qb = as_bf16x8(qreg[ks]);
            s[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kv[ks % kQkAhead][0]), qb, s[0], 0, 0, 0);
            s[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kv[ks % kQkAhead][1]), qb, s[1], 0, 0, 0);
            if (with_soft && ks < kStages) soft_stage(ks, sc, live);
            if ((ks & 3) == 1 && pend_t >= 0) issue_part(pend_t, ks >> 2, pend_my8, pend_rowb);
            __builtin_amdgcn_sched_barrier(0);
            if (ks + kQkAhead < KS) qk_read(ks + kQkAhead, kv[ks % kQkAhead]);
        }
    };

    // O^T += V^T P^T over one tile's 32 tokens.  A operand: V^T[d][kappa] via the transpose
    // load (in each 16-lane group, lane i points at row k0 + i/4, dims n0 + 4*(i%4) .. +3; lane j
    // receives rows k0..k0+3 of dim n0 + j).  Groups of 4 output blocks: group g+1 is read while
    // group g's MFMAs issue (fenced so the compiler keeps the two-stage ring).
    auto pv_tile = [&](const unsigned char* tile, const bf16x8& phi, const bf16x8& plo) {
        bf16x8 va[2][4];
        auto pv_read = [&](int db0, bf16x8 (&dst)[4]) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int db = db0 + u;
                const unsigned char* p0 = tile + pv_off[db & 7] + (db >> 3) * 256;
                const uint2 w0 = lds_read_tr16(p0);
                const uint2 w1 = lds_read_tr16(p0 + 16 * G::kRowBytesA);
                dst[u] = as_bf16x8(make_uint4(w0.x, w0.y, w1.x, w1.y));
            }
        };
        pv_read(0, va[0]);
#pragma unroll
        for (int g = 0; g < DB / 4; ++g) {
            __builtin_amdgcn_sched_barrier(0);
            if (g + 1 < DB / 4) pv_read(4 * (g + 1), va[(g + 1) & 1]);
            if ((g & 1) == 1 && pend_t >= 0) issue_part(pend_t, 5 + (g >> 1), pend_my8, pend_rowb);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < 4; ++u)
                acc[4 * g + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[g & 1][u], phi, acc[4 * g + u], 0, 0, 0);
#pragma unroll
            for (int u = 0; u < 4; ++u)
                acc[4 * g + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[g & 1][u], plo, acc[4 * g + u], 0, 0, 0);
        }
    };

    // Softmax reference: the probabilities are exp2(logit - m_ref) with m_ref fixed at the first
    // tile where the head has a valid token, never rescaled.  Any reference gives the same
    // softmax as long as exp2 cannot overflow, so a tile whose max exceeds m_ref by more than
    // kHeadroom (2^32) switches the whole workgroup to a scan that only tracks the true max;
    // the split is then computed again with m_ref = that max.  Inputs whose logits stay within
    // 2^32 of the first tile's max take one pass.
    //
    // Loop body for tile t: QK of tile t+1 (with tile t's softmax stages in its shadow), then PV
    // of tile t.
    for (int pass = 0; pass < 2; ++pass) {
        scan = false;
        f32x4 s_cur[2], s_next[2];
        uint64_t live_cur = 0, live_next = 0;
        auto live_mask = [&](int t) {
            return __ballot(lane < kTile && t * kTile + lane < n &&
                            rows[t * kTile + (lane & (kTile - 1))] >= 0);
        };
        for (int t = 0; t < kRing - 1 && t < n_tiles; ++t) issue_tile(t);
        if (n_tiles > 0) {
            // tile 0 has landed once at most the later prologue tiles are outstanding
            const int later = min(kRing - 2, n_tiles - 1);
            if (later >= 2) wait_vm<2 * kLoadsPerWave>();
            else if (later == 1) wait_vm<kLoadsPerWave>();
            else wait_vm<0>();
            __syncthreads();
            live_cur = live_mask(0);
            qk_tile(ring, s_cur, false, s_cur, 0);
        }
        for (int t = 0; t < n_tiles; ++t) {
            soft_reset();
            if (t + 1 < n_tiles) {
                // tile t+1 has landed once at most the tiles issued after it are outstanding
                const int later = min(t + kRing - 2, n_tiles - 1) - (t + 1);
                if (later >= 1) wait_vm<kLoadsPerWave>();
                else wait_vm<0>();
                __syncthreads();   // every wave's part landed; tile t-1's buffer is free again
                scan = *flag != 0;
                pend_t = -1;
                if (t + kRing - 1 < n_tiles) {
                    pend_t = t + kRing - 1;
                    tile_rows(pend_t, pend_my8, pend_rowb);
                }
                live_next = live_mask(t + 1);
                qk_tile(ring + ((t + 1) % kRing) * G::kTileBytes, s_next, true, s_cur, live_cur);
            } else {
#pragma unroll
                for (int st = 0; st < kStages; ++st) soft_stage(st, s_cur, live_cur);
            }
            // In scan mode the products are discarded (the split is computed again), but PV
            // still runs: skipping it conditionally costs the accumulators their registers.
            l_run += spsum;
            pv_tile(ring + (t % kRing) * G::kTileBytes,
                    as_bf16x8(make_uint4(phi_w[0], phi_w[1], phi_w[2], phi_w[3])),
                    as_bf16x8(make_uint4(plo_w[0], plo_w[1], plo_w[2], plo_w[3])));
            s_cur[0] = s_next[0];
            s_cur[1] = s_next[1];
            live_cur = live_next;
        }
        wait_vm<0>();
        __syncthreads();                 // a flag raised on the last tile is visible
        if (*flag == 0) break;           // uniform
        // second pass with the true max as the reference
        m_ref = m_seen;
        l_run = 0.f;
#pragma unroll
        for (int i = 0; i < DB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        __syncthreads();                 // everyone has read the flag
        if (tid == 0) *flag = 0;
        __syncthreads();
    }

    // full row sum of head h0 + j16 across the four lane groups
    const float l_tot = sum4groups(l_run);
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
            a.part_ml[pidx * 2] = m_ref == -INFINITY ? -INFINITY : m_ref * 0.6931471805599453f;
            a.part_ml[pidx * 2 + 1] = l_tot;
        }
    }
}

template <int DK, int DV>
size_t mfma_smem(int chunk) {
    return size_t(kRing) * Geo<DK, DV>::kTileBytes + size_t(chunk + 4) * sizeof(int32_t);
}

}  // namespace

namespace tsa {

// Shapes the latent kernel handles: values alias the keys, 64 query heads over one latent KV
// head of 576 dims whose first 512 are the values.
bool mfma_latent_applicable(const tsa_kv_pool& pool, const tsa_decode_params& p) {
    const tsa_pool_desc& d = pool.d;
    if (!d.v_from_k || d.head_dim_k != 576 || d.head_dim_v != 512 || d.num_kv_heads != 1) return false;
    if (p.num_q_heads != 64) return false;
    if (pool.slots() >= (int64_t(1) << 31)) return false;   // slots kept as 32-bit in LDS
    return mfma_smem<576, 512>(int(ceil_div(p.top_k, kTile)) * kTile) <= 160 * 1024;
}

int mfma_latent_chunk(const tsa_decode_params& p, int* splits) {
    const int tiles = int(ceil_div(p.top_k, kTile));
    int s = int(ceil_div(256, std::max(p.batch, 1)));   // one workgroup per CU
    s = std::max(1, std::min({s, tiles, 64}));   // the combine takes at most 64 splits
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
