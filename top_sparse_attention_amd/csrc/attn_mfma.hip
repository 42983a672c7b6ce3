// Sparse gather-attention on the matrix cores, for the MQA mode of MLA: many query heads over
// one latent KV head whose first head_dim_v dims are the values.
//
// GLM5.3 sparse-attention page: DSA runs MLA in MQA mode (MLA-modes paragraph) over the top-k
// tokens the indexer kept; with H = 64 query heads every latent row is reused by 64 heads, so
// QK^T and PV are dense contractions (roofline paragraph: about 120 FLOP per byte at the GLM-5
// shape, far above what the vector ALUs sustain per byte of HBM bandwidth).
//
// Formulation per workgroup (one request, one split of its selected tokens), for each group of
// 16 query heads:
//   S^T [tokens x heads] = K_tile [tokens x dk] . Q^T [dk x heads]      (MFMA 16x16x32 bf16)
//       A operand: K rows read from LDS (token-major, 16 bytes per lane)
//       B operand: the group's queries, held in registers for the whole kernel
//   softmax over the token axis, per head (a lane always holds one head's column)
//   O^T [dv x heads] += V^T [dv x tokens] . P^T [tokens x heads]        (MFMA 16x16x32 bf16)
//       A operand: the same LDS tile read with the LDS transpose load, which hands each lane
//                  4 consecutive tokens of one value dim, so no transposed copy is stored
//       B operand: P in the layout of the S^T accumulators (the contraction runs over the
//                  tokens in a permuted order; A and B use the same permutation)
// P is split into bf16 hi + lo parts (two PV MFMAs) so the probabilities keep ~16 bits.
//
// Warp specialisation: each head group has two waves on the same SIMD.  The QK wave holds the
// queries and computes S and the softmax of tile t+1; the PV wave holds the O^T accumulators
// and multiplies tile t by P(t), which it reads from LDS.  Queries (72 registers) and
// accumulators (128) then live in different waves, so two waves fit per SIMD and one wave's
// matrix work overlaps the other's LDS reads, softmax and load issue.  (With one wave per SIMD
// doing both, those phases ran back to back.)
//
// Data movement: tiles of 32 selected rows are gathered from the page table straight into LDS
// with global-to-LDS loads (no staging registers), into a ring of 4 buffers so that two tiles
// stream in while two are computed.  The loads are issued from inline assembly and waited for
// with explicit vector-memory counts: the compiler would otherwise wait for every outstanding
// LDS-bound load before the first LDS read, which serialises the ring.  A tile is stored as two
// regions: the first DV dims of each row (value dims, DV/8 16-byte chunks, one wave-wide load
// per row) and the remaining DK-DV dims (8 chunks per row, one load per 8 rows).  Within each
// region the chunk index is XOR-swizzled with the row so that row-parallel operand reads spread
// over the LDS banks.  An LDS-bound load blocks its wave at issue for a long time, so each
// wave's share of a tile is spread over its matrix work: the QK waves load 6 value rows each,
// the PV waves 2 value rows and 8 rows of the rope dims.
#include "tsa_internal.h"
#include "mfma_lds.h"

namespace {

constexpr int kGroups = 4;                // head groups of 16 query heads
constexpr int kWaves = 2 * kGroups;       // per group: a QK + softmax wave and a PV wave
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 32;                 // selected rows per tile
constexpr int kRing = 4;                  // tile buffers in LDS
constexpr int kRowsQ = 6;                 // value-region rows each QK wave loads per tile
constexpr int kRowsP = (kTile - kGroups * kRowsQ) / kGroups;   // ... each PV wave (2)
constexpr int kLoadsQK = kRowsQ;          // loads per tile of a QK wave
constexpr int kLoadsPV = kRowsP + 1;      // ... of a PV wave: its rows + 8 rows of region B
constexpr int kPBytes = 64 * 32;          // P of one group: 64 lanes x (hi 16 B, lo 16 B)
constexpr int kMaxChunk = 1024;           // selected tokens per workgroup (LDS row list)
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kQkAhead = 4;               // QK k-steps whose LDS operands are read ahead
constexpr float kHeadroom = 32.f;         // log2 headroom of the fixed softmax reference
static_assert(kGroups * (kRowsQ + kRowsP) == kTile, "every value row loaded once");

template <int DK, int DV>
struct Geo {
    static constexpr int kChunksA = DV / 8;                 // value-dim chunks of a row
    static constexpr int kChunksB = (DK - DV) / 8;          // remaining chunks of a row
    static constexpr int kRowBytesA = DV * 2;
    static constexpr int kRowBytesB = (DK - DV) * 2;
    static constexpr int kBytesA = kTile * kRowBytesA;
    static constexpr int kTileBytes = kTile * (kRowBytesA + kRowBytesB);
    static_assert(kChunksA == 64, "region A rows are one wave-wide load each");
    static_assert(kChunksB == 8, "region B holds 8 chunks of 8 rows per load");
    static_assert(kTile / 8 == kGroups, "one region-B load per PV wave");
};

// stored chunk position of logical chunk c of tile row r, region A (groups of 16 chunks) and
// region B (8 chunks per row); both are involutions on c
__device__ __forceinline__ int swz_a(int r, int c) { return c ^ (r & 15); }
__device__ __forceinline__ int swz_b(int r, int c) { return c ^ (((r >> 1) ^ (r << 2)) & 7); }

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
    constexpr int DB = DV / 16;   // output dim blocks of a PV wave
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char* ring = smem;                                     // kRing tiles
    unsigned char* pbuf = smem + kRing * G::kTileBytes;             // [group][hi 1 KiB, lo 1 KiB]
    float* lbuf = reinterpret_cast<float*>(pbuf + kGroups * kPBytes);   // [head][m, l]
    int32_t* flag = reinterpret_cast<int32_t*>(lbuf + 2 * kGroups * 16);  // rescan request
    int32_t* pv_seen = flag + 4;                                    // [group] P reads done
    int32_t* rows = pv_seen + kGroups;                              // [chunk]

    // Unit of this workgroup: (request b, split s_idx, head block hblk of 64 query heads).
    // Workgroups reach the 8 XCDs round-robin by linear id, so the ids are renumbered to give
    // each XCD consecutive units, head blocks fastest: the head blocks of one split then read the
    // same rows through one L2, and a request's splits share its queries there.
    int s_idx, hblk, b;
    {
        const int S = gridDim.x, Y = gridDim.y;
        const int units = S * Y * int(gridDim.z);
        const int lin = int(blockIdx.x) + S * (int(blockIdx.y) + Y * int(blockIdx.z));
        const int u = (units % 8 == 0) ? (lin % 8) * (units / 8) + lin / 8 : lin;
        hblk = u % Y;
        s_idx = (u / Y) % S;
        b = u / (Y * S);
    }
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool is_qk = wave < kGroups;          // uniform
    const int grp = wave & (kGroups - 1);
    const int g16 = lane >> 4, j16 = lane & 15;
    const int h0 = hblk * (kGroups * 16) + grp * 16;   // the group's first head
    // Head counts that are not a multiple of 64 leave the last block's upper groups without
    // heads: they compute on zero queries (their loads still fill the shared tiles) and store
    // nothing.
    const bool active = h0 < a.hq;              // uniform

    int len = a.seq_lens[b];
    len = len < 0 ? 0 : (len > a.max_len ? a.max_len : len);
    const int n_sel = min(len, a.k);
    const int j0 = s_idx * a.chunk;
    const int j1 = min(j0 + a.chunk, n_sel);
    const int n = max(j1 - j0, 0);
    const int n_tiles = (n + kTile - 1) / kTile;

    // physical rows of this split's selected positions (-1 = absent: fetched from slot 0 like
    // any other row and masked out of the softmax)
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

    uint4 qreg[KS];            // QK waves: the group's queries, B operand of S^T = K Q^T
    float m_ref = -INFINITY;   // QK waves: reference max (log2 units) of head h0 + j16
    float m_seen = -INFINITY;  // QK waves: max logit seen
    float l_run = 0.f;         // QK waves: this lane's share of the running sum

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
    // loads: QK wave q fetches region A of rows q*kRowsQ .. (one wave-wide load per row, lane
    // = stored chunk position); PV wave p region A of rows kGroups*kRowsQ + p*kRowsP .. and
    // region B of rows 8p .. 8p+7 (lane = 8 * row-in-group + stored chunk position)
    const int a_src_chunk = lane;
    const int my_rows = is_qk ? kRowsQ : kRowsP;
    const int row_base = is_qk ? grp * kRowsQ : kGroups * kRowsQ + grp * kRowsP;
    const int my_loads = is_qk ? kLoadsQK : kLoadsPV;
    const int b_row = (grp * 8 + (lane >> 3)) & (kTile - 1);
    const int b_src_el = DV + swz_b(b_row, lane & 7) * 8;

    if (tid == 0) *flag = 0;
    if (tid < kGroups) pv_seen[tid] = 0;
    __syncthreads();           // rows[], the flag and the counts visible

    const uint32_t ring_base = lds_addr(ring);
    // Load m of this wave's share of tile t: m < my_rows is region A of row row_base + m, the
    // next (PV waves) region B.  my4 holds the wave's rows in lanes 0.. and rowb the row of
    // this lane's region-B chunk.
    auto issue_part = [&](int t, int m, int32_t my4, int32_t rowb) {
        const uint32_t buf = ring_base + uint32_t((t % kRing) * G::kTileBytes);
        if (m < my_rows) {
            const int r = row_base + m;
            const int32_t row = __builtin_amdgcn_readlane(my4, m);
            const uint16_t* src = a.kpool + int64_t(row < 0 ? 0 : row) * DK;   // uniform
            load_lds16_s(src, uint32_t(swz_a(r, a_src_chunk) * 16),
                         __builtin_amdgcn_readfirstlane(buf + uint32_t(r * G::kRowBytesA)));
        } else {
            const uint16_t* srcb = a.kpool + int64_t(rowb < 0 ? 0 : rowb) * DK + b_src_el;
            load_lds16(srcb, __builtin_amdgcn_readfirstlane(buf + uint32_t(G::kBytesA + grp * 1024)));
        }
    };
    auto tile_rows = [&](int t, int32_t& my4, int32_t& rowb) {
        my4 = rows[t * kTile + row_base + (lane & 7) % my_rows];
        rowb = is_qk ? 0 : rows[t * kTile + b_row];
    };
    auto issue_tile = [&](int t) {
        int32_t my4, rowb;
        tile_rows(t, my4, rowb);
        for (int m = 0; m < my_loads; ++m) issue_part(t, m, my4, rowb);
    };
    // wait until this wave's loads of a tile have landed, `later` tiles having been issued
    // after it
    auto wait_tile = [&](int later) {
        if (is_qk) {
            if (later >= 2) wait_vm<2 * kLoadsQK>();
            else if (later == 1) wait_vm<kLoadsQK>();
            else wait_vm<0>();
        } else {
            if (later >= 2) wait_vm<2 * kLoadsPV>();
            else if (later == 1) wait_vm<kLoadsPV>();
            else wait_vm<0>();
        }
    };

    bool scan = false;           // uniform; the workgroup is only tracking the max

    // S^T = K Q^T for one tile: two 16-token blocks x 16 heads.  Operand reads run kQkAhead
    // k-steps ahead of the MFMAs; this wave's loads of tile pend_t go after k-steps 1, 5, 9, 13.
    auto qk_tile = [&](const unsigned char* tile, f32x4 (&s)[2], int pend_t, int32_t my4, int32_t rowb) {
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
            if ((ks & 1) == 1 && (ks >> 1) < kLoadsQK && pend_t >= 0) issue_part(pend_t, ks >> 1, my4, rowb);
            __builtin_amdgcn_sched_barrier(0);
            if (ks + kQkAhead < KS) qk_read(ks + kQkAhead, kv[ks % kQkAhead]);
        }
    };

    // Softmax of one tile against the fixed reference (first tile with a valid token; a tile
    // more than kHeadroom above it requests a rescan with the true max).  Produces P^T as the
    // PV B operand, split into bf16 hi + lo: kappa = 8*g16 + i <-> token (i < 4 ? 4*g16 + i :
    // 16 + 4*g16 + i - 4).
    auto softmax = [&](const f32x4 (&sc)[2], uint64_t live, uint4& ph, uint4& pl) {
        float x[8];
        float tmax = -INFINITY;
        if (uint32_t(live) == 0xffffffffu) {   // uniform: every token of the tile present
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                x[i] = sc[i >> 2][i & 3] * a.scale_log2;
                tmax = fmaxf(tmax, x[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int tok = (i >> 2) * 16 + g16 * 4 + (i & 3);
                x[i] = ((live >> tok) & 1) ? sc[i >> 2][i & 3] * a.scale_log2 : -INFINITY;
                tmax = fmaxf(tmax, x[i]);
            }
        }
        tmax = max4groups(tmax);
        m_seen = fmaxf(m_seen, tmax);
        if (m_ref == -INFINITY) m_ref = tmax;
        const bool viol = tmax > m_ref + kHeadroom;
        if (!scan && __ballot(viol)) *flag = 1;
        // exp2(-inf - m) = 0 for any finite m; before the head has a reference every logit of
        // the tile is -inf and any finite m does
        const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x[i] = __builtin_amdgcn_exp2f(x[i] - m_use);
            psum += x[i];
        }
        l_run += psum;
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t h = pack_bf16(x[2 * e], x[2 * e + 1]);
            hw[e] = h;
            lw[e] = pack_bf16(x[2 * e] - __uint_as_float(h << 16),
                              x[2 * e + 1] - __uint_as_float(h & 0xffff0000u));
        }
        ph = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        pl = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    };
    uint4* pb_hi = reinterpret_cast<uint4*>(__builtin_assume_aligned(pbuf + grp * kPBytes, 16)) + lane;
    uint4* pb_lo = pb_hi + 64;
    // Bounded wait for the group's PV wave to have read `count` P tiles.  The PV wave reads
    // P(t) right after the barrier that opens iteration t, without waiting on anything else,
    // so the wait normally passes at once; the bound only guarantees that the wave cannot
    // hang, and running out of it poisons the head's sum so the output shows NaN.
    auto wait_seen = [&](int count) {
        for (int spin = 0; spin < (1 << 22); ++spin) {
            if (__hip_atomic_load(&pv_seen[grp], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= count)
                return;
            __builtin_amdgcn_s_sleep(1);
        }
        l_run = __builtin_nanf("");
    };

    // O^T += V^T P^T over one tile's 32 tokens (LDS transpose reads, groups of 4 output blocks
    // read one group ahead); this wave's loads of tile pend_t go after output groups 1 .. 5.
    auto pv_tile = [&](f32x4 (&acc)[DB], const unsigned char* tile, const bf16x8& phi, const bf16x8& plo, int pend_t,
                       int32_t my4, int32_t rowb) {
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
            if (g >= 1 && g <= kLoadsPV && pend_t >= 0) issue_part(pend_t, g - 1, my4, rowb);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < 4; ++u)
                acc[4 * g + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[g & 1][u], phi, acc[4 * g + u], 0, 0, 0);
#pragma unroll
            for (int u = 0; u < 4; ++u)
                acc[4 * g + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[g & 1][u], plo, acc[4 * g + u], 0, 0, 0);
        }
    };
    auto live_mask = [&](int t) {
        return __ballot(lane < kTile && t * kTile + lane < n && rows[t * kTile + (lane & (kTile - 1))] >= 0);
    };

    // Pipeline, per tile t: QK waves compute S and P of tile t+1 while PV waves accumulate tile
    // t with P(t).  The barrier that opens iteration t means: tile t+1 landed, P(t) written,
    // PV(t-1) done (so tile t-1's buffer takes tile t+3).  A per-group count in LDS tells the
    // QK wave when its PV wave has read P(t), after which P(t+1) replaces it.  The two roles run separate
    // copies of the loop with the same sequence of barriers, so that the queries (QK) and the
    // accumulators (PV) never need registers in the same wave.
    const int h = h0 + j16;
    if (is_qk) {
        if (active) {
            const uint4* qsrc = reinterpret_cast<const uint4*>(a.q + (int64_t(b) * a.hq + h) * DK);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qreg[ks] = qsrc[ks * 4 + g16];
        } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qreg[ks] = make_uint4(0, 0, 0, 0);
        }
        wait_vm<0>();
        for (int pass = 0; pass < 2; ++pass) {
            scan = false;
            for (int t = 0; t < kRing - 1 && t < n_tiles; ++t) issue_tile(t);
            uint4 ph = make_uint4(0, 0, 0, 0), pl = ph;
            if (n_tiles > 0) {
                wait_tile(min(kRing - 2, n_tiles - 1));
                __syncthreads();
                f32x4 s[2];
                qk_tile(ring, s, -1, 0, 0);
                softmax(s, live_mask(0), ph, pl);
                *pb_hi = ph;
                *pb_lo = pl;
            }
            for (int t = 0; t < n_tiles; ++t) {
                if (t + 1 < n_tiles) wait_tile(min(t + 2, n_tiles - 1) - (t + 1));
                __syncthreads();                                       // B_t
                scan = *flag != 0;
                int pend_t = -1;
                int32_t my4 = 0, rowb = 0;
                if (t + kRing - 1 < n_tiles) {
                    pend_t = t + kRing - 1;
                    tile_rows(pend_t, my4, rowb);
                }
                if (t + 1 < n_tiles) {
                    const uint64_t live = live_mask(t + 1);
                    f32x4 s[2];
                    qk_tile(ring + ((t + 1) % kRing) * G::kTileBytes, s, pend_t, my4, rowb);
                    softmax(s, live, ph, pl);
                    // P(t) must have been read by the group's PV wave before it is replaced
                    wait_seen(pass * n_tiles + t + 1);
                    *pb_hi = ph;
                    *pb_lo = pl;
                }
            }
            wait_vm<0>();
            __syncthreads();                 // a flag raised on the last tile is visible
            if (*flag == 0) break;           // uniform
            // second pass with the true max as the reference
            m_ref = m_seen;
            l_run = 0.f;
            __syncthreads();                 // everyone has read the flag
            if (tid == 0) *flag = 0;
            __syncthreads();
        }
        // full row sum of head h across the four lane groups
        const float l_tot = sum4groups(l_run);
        if (g16 == 0) {
            lbuf[(grp * 16 + j16) * 2] = m_ref;
            lbuf[(grp * 16 + j16) * 2 + 1] = l_tot;
            if (a.splits > 1 && active) {
                const int64_t pidx = (int64_t(b) * a.hq + h) * a.splits + s_idx;
                // natural-log units, as the combine expects
                a.part_ml[pidx * 2] = m_ref == -INFINITY ? -INFINITY : m_ref * 0.6931471805599453f;
                a.part_ml[pidx * 2 + 1] = l_tot;
            }
        }
        __syncthreads();
    } else {
        f32x4 acc[DB];
        for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
            for (int i = 0; i < DB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int t = 0; t < kRing - 1 && t < n_tiles; ++t) issue_tile(t);
            if (n_tiles > 0) {
                wait_tile(min(kRing - 2, n_tiles - 1));
                __syncthreads();
            }
            for (int t = 0; t < n_tiles; ++t) {
                if (t + 1 < n_tiles) wait_tile(min(t + 2, n_tiles - 1) - (t + 1));
                __syncthreads();                                       // B_t
                int pend_t = -1;
                int32_t my4 = 0, rowb = 0;
                if (t + kRing - 1 < n_tiles) {
                    pend_t = t + kRing - 1;
                    tile_rows(pend_t, my4, rowb);
                }
                const uint4 rh = *pb_hi, rl = *pb_lo;
                // both reads have returned before the count tells the QK wave
                __hip_atomic_store(&pv_seen[grp], pass * n_tiles + t + 1, __ATOMIC_RELEASE,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
                pv_tile(acc, ring + (t % kRing) * G::kTileBytes, as_bf16x8(rh), as_bf16x8(rl), pend_t, my4, rowb);
            }
            wait_vm<0>();
            __syncthreads();
            if (*flag == 0) break;
            __syncthreads();
            __syncthreads();
        }
        __syncthreads();                     // lbuf written
        // lane holds O^T[d = db*16 + 4*g16 + r][head h]
        if (!active) {
        } else if (a.splits == 1) {
            const float l_tot = lbuf[(grp * 16 + j16) * 2 + 1];
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
        }
    }
}

template <int DK, int DV>
size_t mfma_smem(int chunk) {
    return size_t(kRing) * Geo<DK, DV>::kTileBytes + size_t(kGroups) * kPBytes +
           size_t(2 * kGroups * 16) * sizeof(float) + size_t(chunk + 4 + kGroups) * sizeof(int32_t);
}

}  // namespace

namespace tsa {

// Shapes the latent kernel handles: values alias the keys, one latent KV head of 576 dims whose
// first 512 are the values, and a multiple of 16 query heads (blocks of 64; GLM-5's 64 heads
// make one block, DeepSeek V3.2's 128 two; 16, 32 or 48 heads fill one block in part).
bool mfma_latent_applicable(const tsa_kv_pool& pool, const tsa_decode_params& p) {
    const tsa_pool_desc& d = pool.d;
    if (!d.v_from_k || d.head_dim_k != 576 || d.head_dim_v != 512 || d.num_kv_heads != 1) return false;
    if (p.num_q_heads < 16 || p.num_q_heads % 16 || p.num_q_heads > 1024) return false;
    if (pool.slots() >= (int64_t(1) << 31)) return false;   // slots kept as 32-bit in LDS
    int splits = 0;
    const int chunk = mfma_latent_chunk(p, &splits);
    // the split combine merges at most 64 splits: a longer selection (more than 64 row lists
    // of kMaxChunk) goes to the vector-ALU kernel, whose chunks are not bounded by LDS
    return splits <= 64 && chunk <= kMaxChunk && mfma_smem<576, 512>(chunk) <= 160 * 1024;
}

int mfma_latent_chunk(const tsa_decode_params& p, int* splits) {
    // no request selects more than min(top_k, max_len) tokens: split that, not top_k
    const int k_eff = std::max(1, std::min(p.top_k, p.max_len));
    const int tiles = int(ceil_div(k_eff, kTile));
    const int hblocks = int(ceil_div(p.num_q_heads, kGroups * 16));
    int s = int(ceil_div(256, std::max(p.batch, 1) * hblocks));   // one workgroup per CU
    s = std::max(1, std::min({s, tiles, 64}));   // the combine takes at most 64 splits
    s = std::max(s, int(ceil_div(tiles, kMaxChunk / kTile)));   // the row list fits in LDS
    const int chunk = int(ceil_div(tiles, s)) * kTile;
    *splits = int(ceil_div(k_eff, chunk));
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
    dim3 grid(plan.splits, int(ceil_div(p.num_q_heads, kGroups * 16)), p.batch);
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), smem, s, a);
    return hipGetLastError();
}

}  // namespace tsa
