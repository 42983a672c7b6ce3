// Top-k selection of indexer scores: one workgroup per request.
//
// GLM5.3 sparse-attention page, lightning-indexer paragraph: the score selects the top K
// tokens; a query with fewer than K tokens stays dense.  Equal scores are ordered by position
// (lowest first), so the selected set is unique; it is written as ascending positions.
//
// Scores map to order-preserving 32-bit keys (equal scores to equal keys, NaN lowest), 1 to 64
// per thread in registers.  One workgroup
// holds a whole request, so what the kernel costs is the instruction count of each wave between
// barriers: it makes one cheap pass over all elements and does the exact selection on a short list.
//  1. Sample: one key per thread (1,024 regularly spaced positions).  A histogram of the sample's
//     12-bit first digits (sign, exponent, top three mantissa bits) gives a bound t_lo: the lower
//     edge of the bin holding the sample's r-th largest key, with r the sample's expected share
//     of the k kept elements plus four standard deviations.  The k largest keys of the request are
//     then almost surely all >= t_lo.
//  2. One pass in position order compacts every element with key >= t_lo (key and position) into
//     an LDS list, its place given by a prefix count: a wave scan per load group plus one block
//     scan of the wave totals.  Each wave owns a contiguous block of positions and reads it with
//     wave-contiguous 16-byte loads (one 1 KiB run per instruction).  The same pass takes the
//     request's largest key.
//  3. If the list holds at least k and at most 8,192 elements, the selection runs on it alone,
//     up to 8 per thread in list order (which is position order).  The k-th largest key lies in
//     [t_lo, largest key]; each pass splits that interval into 4,096 equal bins of keys and keeps
//     the bin holding the k-th largest, until the bin is one key or is kept whole (at most three
//     passes).  A bin of dozens of entries is first checked for being one repeated key, which
//     ends the search on integer-valued scores.  A prefix count in list order of the packed pair
//     (above the bin, inside it) then gives the tie ranks and the output offsets at once, so the
//     output comes out ascending with no sort.
//  4. Otherwise (an unlucky sample, heavy ties, a crowded range), and for selections of at most
//     8 scores per thread, where steps 1-3 cost more than they save, the same selection runs over
//     every element in registers with 8-bit digits from the top.
// Histograms are LDS atomics (the 8-bit passes on interleaved copies, so that lanes hitting one
// bin spread over banks); consecutive passes double-buffer their histograms and scan areas by
// parity to save barriers, and wave scans and min / max use DPP lane moves.
#include "tsa_internal.h"

namespace {

constexpr int kMaxThreads = 1024;
constexpr int kCopies = 16;               // histogram copies of the 8-bit passes
constexpr int kBins1 = 4096;              // 12-bit digit: key bits 31..20
constexpr int kShift1 = 20;
constexpr int kListCap = 8192;            // list entries (keys, then positions, in `big`)
constexpr int kTied = 32;                 // a list bin this full is checked for a single key first
// Up to 8 scores per thread (8,192 per request), the register passes of step 4 alone are faster
// than sample + compaction + list: 5.3 against 8.3 us for five requests of 403 scores, 8.0
// against 9.8 us for 32 x 8,192 integer-valued scores (0.2 us slower on 32 x 8,192 floats).
constexpr int kListMinIpt = 12;
static_assert(kBins1 == 256 * kCopies, "a 12-bit histogram fills one 8-bit pass buffer");
static_assert(kBins1 <= 2 * kListCap, "the sample histogram fits where the list goes");

// Shape of a launch: NT threads, each holding up to IPT scores; the list gives each thread
// kListCap / NT entries, and each thread scans kBins1 / NT bins of a 12-bit histogram.
template <int NT>
struct Shape {
    static constexpr int kWaves = NT / 64;
    static constexpr int kPer = kListCap / NT;
    static constexpr int kBinsPer = kBins1 / NT;
    static_assert(NT % 64 == 0 && NT >= 256 && NT <= kMaxThreads, "whole waves, at least one per 8-bit bin group");
    static_assert(kBins1 % NT == 0 && kListCap % NT == 0, "bins and list entries divide evenly");
};

// Order-preserving key of a score under ordinary float comparison: -0 and +0 are equal scores
// and get one key (x + 0 turns -0 into +0 and leaves every other value as it is), and a NaN ranks
// below every number, with key 0.  No number has key 0 (-inf's is 0x007fffff); positions past
// len get 0 as well, so the list path never keeps either, and the general path, which checks
// positions, orders NaNs last by position.
__device__ inline uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f + 0.0f);
    const uint32_t key = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return f != f ? 0u : key;
}

// DPP lane move: lanes whose source falls outside the pattern (or a disabled row) read 0.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ uint32_t dpp0(uint32_t x) {
    return uint32_t(__builtin_amdgcn_update_dpp(0, int(x), CTRL, ROWS, 0xf, false));
}

// Inclusive prefix sum over the wave in lane order (modulo 2^32): shifts within each row of
// 16 lanes, then the last lane of row 0 and of row 1 carried into the rows above.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t x) {
    x += dpp0<0x111>(x);          // row_shr:1
    x += dpp0<0x112>(x);          // row_shr:2
    x += dpp0<0x114>(x);          // row_shr:4
    x += dpp0<0x118>(x);          // row_shr:8
    x += dpp0<0x142, 0xa>(x);     // row_bcast:15 into rows 1 and 3
    x += dpp0<0x143, 0xc>(x);     // row_bcast:31 into rows 2 and 3
    return x;
}

// min / max over the wave (every lane gets the result): rotations within each row of 16
// lanes, then the cross-row lane swaps
__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
    x = min(x, uint32_t(__builtin_amdgcn_mov_dpp(int(x), 0x128, 0xf, 0xf, false)));
    x = min(x, uint32_t(__builtin_amdgcn_mov_dpp(int(x), 0x124, 0xf, 0xf, false)));
    x = min(x, uint32_t(__builtin_amdgcn_mov_dpp(int(x), 0x122, 0xf, 0xf, false)));
    x = min(x, uint32_t(__builtin_amdgcn_mov_dpp(int(x), 0x121, 0xf, 0xf, false)));
    const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = min(a[0], a[1]);
    const auto c = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return min(c[0], c[1]);
}
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
    x = max(x, uint32_t(__builtin_amdgcn_mov_dpp(int(x), 0x128, 0xf, 0xf, false)));
    x = max(x, uint32_t(__builtin_amdgcn_mov_dpp(int(x), 0x124, 0xf, 0xf, false)));
    x = max(x, uint32_t(__builtin_amdgcn_mov_dpp(int(x), 0x122, 0xf, 0xf, false)));
    x = max(x, uint32_t(__builtin_amdgcn_mov_dpp(int(x), 0x121, 0xf, 0xf, false)));
    const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = max(a[0], a[1]);
    const auto c = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return max(c[0], c[1]);
}

// Exclusive scan over the block in thread order; returns this thread's prefix, total in *total.
// sh_waves holds 2 * kWaves + 1 ints; callers alternate between two such areas so that one
// call's reads never race the next call's writes.
template <int kWaves>
__device__ inline int block_exclusive_scan(int v, int* sh_waves, int* total) {
    // sums wrap modulo 2^32 (unsigned arithmetic): packed counts rely on it
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t x = wave_inclusive_sum(uint32_t(v));
    if (lane == 63) sh_waves[wave] = int(x);
    __syncthreads();
    if (threadIdx.x < 64) {
        const uint32_t w = threadIdx.x < kWaves ? uint32_t(sh_waves[threadIdx.x]) : 0u;
        const uint32_t s = wave_inclusive_sum(w);
        if (threadIdx.x < kWaves) sh_waves[kWaves + threadIdx.x] = int(s - w);
        if (threadIdx.x == kWaves - 1) sh_waves[2 * kWaves] = int(s);
    }
    __syncthreads();
    *total = sh_waves[2 * kWaves];
    return int(uint32_t(sh_waves[kWaves + wave]) + x - uint32_t(v));
}

template <int IPT, int NT>
__global__ void __launch_bounds__(NT) topk_radix_kernel(const float* __restrict__ scores,
                                                              int ld,
                                                              const int32_t* __restrict__ seq_lens,
                                                              int max_len, int k,
                                                              int32_t* __restrict__ out) {
    // the sample histogram, then the list: (key, position) pairs
    __shared__ __align__(16) uint32_t big[2 * kListCap];
    uint2* list = reinterpret_cast<uint2*>(big);
    // per pass parity: the general path's 8-bit histograms (kCopies copies of 256 bins) or one
    // 12-bit histogram of the list (kBins1 bins)
    __shared__ uint32_t hist[2][256 * kCopies];
    using Sh = Shape<NT>;
    constexpr int kThreads = NT;
    constexpr int kWaves = Sh::kWaves;
    constexpr int kPer = Sh::kPer;
    constexpr int kBinsPer = Sh::kBinsPer;
    __shared__ int sh_scan[2][2 * kWaves + 1];
    __shared__ int sh_sel[2][4];
    // candidate key ranges: the general path's, per pass parity; the list passes', per pass
    __shared__ uint32_t sh_mm[4];
    __shared__ uint32_t sh_kmax;                   // largest key of the request
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    int len = seq_lens[b];
    len = len < 0 ? 0 : (len > max_len ? max_len : len);
    int32_t* o = out + int64_t(b) * k;
    if (len <= k) {  // dense: every position, then padding
        for (int i = tid; i < k; i += kThreads) o[i] = i < len ? i : -1;
        return;
    }
    const float* s = scores + int64_t(b) * ld;
    // Wave w owns the contiguous positions [w * 64 * IPT, (w + 1) * 64 * IPT).  Inside it, element
    // (g, e) of lane l (g < G groups of E values) sits at 64 E g + E l + e: every load instruction
    // of the wave then covers one contiguous run of 64 E values (1 KiB when E = 4), and position
    // order within the wave is (g, lane, e).  Positions at or past len get key 0.
    constexpr int E = IPT < 4 ? IPT : 4;
    constexpr int G = IPT / E;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wbase = wave * 64 * IPT + E * lane;   // position of element (0, 0)
    uint32_t key[IPT];
    if (E == 4 && (ld & 3) == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int p0 = wbase + 64 * E * g;
            if (p0 + 3 < len) {
                const float4 v = *reinterpret_cast<const float4*>(s + p0);
                key[4 * g + 0] = order_key(v.x);
                key[4 * g + 1] = order_key(v.y);
                key[4 * g + 2] = order_key(v.z);
                key[4 * g + 3] = order_key(v.w);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) key[4 * g + e] = p0 + e < len ? order_key(s[p0 + e]) : 0u;
            }
        }
    } else {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int p = wbase + 64 * E * g + e;
                key[E * g + e] = p < len ? order_key(s[p]) : 0u;
            }
    }
    auto valid = [&](int i) { return wbase + 64 * E * (i / E) + (i % E) < len; };

    if constexpr (IPT >= kListMinIpt) {
    // ---- 1. sample: element 0 of every thread; t_lo from its 12-bit digit histogram ----
    for (int i = tid; i < kBins1; i += kThreads) big[i] = 0;
    for (int i = tid; i < 256 * kCopies; i += kThreads) {
        hist[0][i] = 0;
        hist[1][i] = 0;
    }
    if (tid == 0) {
        sh_kmax = 0u;
        for (int i = 0; i < 4; i += 2) {
            sh_mm[i] = 0xffffffffu;
            sh_mm[i + 1] = 0u;
        }
    }
    __syncthreads();
    if (valid(0)) atomicAdd(&big[key[0] >> kShift1], 1u);
    __syncthreads();
    {
        uint32_t c[kBinsPer];
        int t = 0;
#pragma unroll
        for (int e = 0; e < kBinsPer; ++e) {
            c[e] = big[kBins1 - 1 - kBinsPer * tid - e];
            t += int(c[e]);
        }
        int n_s;
        int above = block_exclusive_scan<kWaves>(t, sh_scan[1], &n_s);
        // the sample's expected count of kept elements, plus four standard deviations and a floor
        const float expect = float(k) * float(n_s) / float(len);
        const int r = min(n_s, int(ceilf(expect + 4.f * sqrtf(expect))) + 16);
#pragma unroll
        for (int e = 0; e < kBinsPer; ++e) {
            if (above < r && above + int(c[e]) >= r) sh_sel[1][0] = kBins1 - 1 - kBinsPer * tid - e;
            above += int(c[e]);
        }
    }
    __syncthreads();
    // at least 1, so that the key 0 of positions past len is never kept (a valid element whose
    // key is 0 is then missing from the list only when fewer than k keys are >= 1, and the
    // count check below sends that case to the general path)
    const uint32_t t_lo = max(uint32_t(sh_sel[1][0]) << kShift1, 1u);

    // ---- 2. compact the elements with key >= t_lo, in position order ----
    // An element's place: earlier waves (one block scan of the wave totals), then earlier groups
    // of its wave (their totals), then earlier lanes of its group (a wave scan per group).
    uint32_t n_keep;
    {
        uint32_t cnt[G], pre[G];
        uint32_t run = 0, kmx = 0;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            uint32_t c = 0;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                c += key[E * g + e] >= t_lo ? 1u : 0u;
                kmx = max(kmx, key[E * g + e]);
            }
            cnt[g] = c;
        }
        kmx = wave_max(kmx);
        if (lane == 0) atomicMax(&sh_kmax, kmx);    // read after the scan's barriers
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const uint32_t x = wave_inclusive_sum(cnt[g]);
            pre[g] = run + x - cnt[g];
            run += uint32_t(__builtin_amdgcn_readlane(int(x), 63));
        }
        int total;
        const uint32_t wave_pre = uint32_t(block_exclusive_scan<kWaves>(lane == 63 ? int(run) : 0, sh_scan[0], &total));
        n_keep = uint32_t(total);
        // the sample histogram (aliased by the list) was last read before the scan's barriers
        if (n_keep >= uint32_t(k) && n_keep <= uint32_t(kListCap)) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                uint32_t idx = wave_pre + pre[g];
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    if (key[E * g + e] >= t_lo) {
                        list[idx] = make_uint2(key[E * g + e], uint32_t(wbase + 64 * E * g + e));
                        ++idx;
                    }
                }
            }
        }
    }
    const bool use_list = n_keep >= uint32_t(k) && n_keep <= uint32_t(kListCap);   // uniform
    __syncthreads();

    if (use_list) {
        // ---- 3. select on the list: thread t holds entries per t .. per t + per - 1 ----
        const int per = (int(n_keep) + kThreads - 1) / kThreads;   // at most kPer
        uint32_t lk[kPer];
        int32_t lp[kPer];
        bool lv[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int idx = per * tid + j;
            lv[j] = j < per && idx < int(n_keep);
            const uint2 v = lv[j] ? list[idx] : make_uint2(0u, 0u);
            lk[j] = v.x;
            lp[j] = int32_t(v.y);
        }
        // The k-th largest key lies in [lo_k, hi_k], initially [t_lo, kmax] (every list key).  A
        // pass splits the interval into 4,096 bins of 2^sh keys, (key - lo_k) >> sh, so the bins
        // cover it evenly whatever the float exponents, and keeps the bin that holds the k-th
        // largest: sh drops by 12 a pass until the bin is a single key, or the bin is kept whole.
        uint32_t lo_k = t_lo, hi_k = sh_kmax;
        int remaining = k;               // how many of the entries in [lo_k, hi_k] to keep
        int pass = 0;
        if (hi_k != lo_k) {              // uniform (equal: every entry has the same key)
            int sh = max(0, 32 - __builtin_clz(hi_k - lo_k) - 12);
            for (bool done = false; !done; ++pass) {         // uniform; at most 3 passes
                uint32_t* h = hist[pass & 1];
                // the other buffer was last read before the previous pass's selection barrier
                if (pass >= 1)
                    for (int i = tid; i < kBins1; i += kThreads) hist[(pass + 1) & 1][i] = 0;
#pragma unroll
                for (int j = 0; j < kPer; ++j)
                    if (lv[j] && lk[j] >= lo_k && lk[j] <= hi_k) atomicAdd(&h[(lk[j] - lo_k) >> sh], 1u);
                __syncthreads();
                uint32_t c[kBinsPer];
                int t = 0;
#pragma unroll
                for (int e = 0; e < kBinsPer; ++e) {
                    c[e] = h[kBins1 - 1 - kBinsPer * tid - e];
                    t += int(c[e]);
                }
                int total;
                int above = block_exclusive_scan<kWaves>(t, sh_scan[pass & 1], &total);
#pragma unroll
                for (int e = 0; e < kBinsPer; ++e) {
                    if (above < remaining && above + int(c[e]) >= remaining) {
                        sh_sel[pass & 1][0] = kBins1 - 1 - kBinsPer * tid - e;
                        sh_sel[pass & 1][1] = remaining - above;
                        sh_sel[pass & 1][2] = int(c[e]);
                    }
                    above += int(c[e]);
                }
                __syncthreads();
                lo_k += uint32_t(sh_sel[pass & 1][0]) << sh;
                hi_k = uint32_t(min(uint64_t(hi_k), uint64_t(lo_k) + ((uint64_t(1) << sh) - 1)));
                remaining = sh_sel[pass & 1][1];
                const int in_bin = sh_sel[pass & 1][2];
                // the whole bin is kept, or the bin is one key
                done = in_bin == remaining || sh == 0;
                if (!done && in_bin >= kTied) {          // uniform
                    // A bin of dozens of entries is often one key repeated (integer-valued scores,
                    // ties): its range decides that in one reduction, where a histogram pass would
                    // queue the entries on one LDS address.
                    uint32_t blo = 0xffffffffu, bhi = 0u;
#pragma unroll
                    for (int j = 0; j < kPer; ++j) {
                        if (lv[j] && lk[j] >= lo_k && lk[j] <= hi_k) {
                            blo = min(blo, lk[j]);
                            bhi = max(bhi, lk[j]);
                        }
                    }
                    blo = wave_min(blo);
                    bhi = wave_max(bhi);
                    uint32_t* mm = sh_mm + 2 * pass;   // each pass's slots are used once
                    if (lane == 0) {
                        atomicMin(&mm[0], blo);
                        atomicMax(&mm[1], bhi);
                    }
                    __syncthreads();
                    if (mm[0] == mm[1]) {                               // uniform
                        lo_k = hi_k = mm[0];
                        done = true;
                    }
                }
                sh = sh >= 12 ? sh - 12 : 0;
            }
        }
        // kept entries in list order: above hi_k, or in [lo_k, hi_k] and among the first
        // `remaining` there; packed (above << 16 | in) counts, both below 2^16 here
        uint32_t cc = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            cc += (lv[j] && lk[j] > hi_k) ? 0x10000u : 0u;
            cc += (lv[j] && lk[j] >= lo_k && lk[j] <= hi_k) ? 1u : 0u;
        }
        int total;
        const uint32_t cpre = uint32_t(block_exclusive_scan<kWaves>(int(cc), sh_scan[pass & 1], &total));
        int gt = int(cpre >> 16), eq = int(cpre & 0xffffu);
        int off = gt + min(eq, remaining);
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            bool take = lv[j] && lk[j] > hi_k;
            if (lv[j] && lk[j] >= lo_k && lk[j] <= hi_k) take = eq++ < remaining;
            if (take && off < k) o[off++] = lp[j];
        }
        return;
    }
    }   // IPT >= kListMinIpt

    // ---- 4. general path: 8-bit radix passes over every element, then the selection ----
    uint32_t prefix = 0, mask = 0;
    int remaining = k;  // how many of the elements matching `prefix` under `mask` to keep
    for (int i = tid; i < 256 * kCopies; i += kThreads) hist[0][i] = 0;
    if (tid == 0) {
        sh_mm[0] = 0xffffffffu;
        sh_mm[1] = 0u;
    }
    __syncthreads();
    int pass = 0;
    for (int shift = 24; shift >= 0; shift -= 8, ++pass) {
        uint32_t* h = hist[pass & 1];
        // the other buffer was last read before the previous pass's selection barrier
        for (int i = tid; i < 256 * kCopies; i += kThreads) hist[(pass + 1) & 1][i] = 0;
        const int copy = tid & (kCopies - 1);
        uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
        for (int i = 0; i < IPT; ++i) {
            if (valid(i) && (key[i] & mask) == prefix) {
                atomicAdd(&h[((key[i] >> shift) & 255u) * kCopies + copy], 1u);
                kmin = min(kmin, key[i]);
                kmax = max(kmax, key[i]);
            }
        }
        // candidates' key range: once they are all equal, the k-th key is known exactly
        kmin = wave_min(kmin);
        kmax = wave_max(kmax);
        if ((tid & 63) == 0) {
            atomicMin(&sh_mm[2 * (pass & 1)], kmin);
            atomicMax(&sh_mm[2 * (pass & 1) + 1], kmax);
        }
        // the next pass's range slots start empty (last read before this pass began)
        if (tid == 0) {
            sh_mm[2 * ((pass + 1) & 1)] = 0xffffffffu;
            sh_mm[2 * ((pass + 1) & 1) + 1] = 0u;
        }
        __syncthreads();
        if (sh_mm[2 * (pass & 1)] == sh_mm[2 * (pass & 1) + 1]) {      // uniform
            prefix = sh_mm[2 * (pass & 1)];
            mask = 0xffffffffu;
            break;
        }
        // bins in descending digit order: thread j < 256 owns digit 255 - j
        int c = 0;
        if (tid < 256) {
            const int dgt = 255 - tid;
#pragma unroll
            for (int j = 0; j < kCopies; ++j) c += h[dgt * kCopies + ((j + tid) & (kCopies - 1))];
        }
        int total;
        const int above = block_exclusive_scan<kWaves>(c, sh_scan[pass & 1], &total);  // count with a larger digit
        if (tid < 256 && above < remaining && above + c >= remaining) {
            sh_sel[0][0] = 255 - tid;
            sh_sel[0][1] = remaining - above;
            sh_sel[0][2] = c;
        }
        __syncthreads();
        const uint32_t dgt = sh_sel[0][0];
        remaining = sh_sel[0][1];
        const int in_bin = sh_sel[0][2];
        __syncthreads();
        prefix |= dgt << shift;
        mask |= 255u << shift;
        if (in_bin == remaining) break;  // the whole bin is kept: no finer digit matters
    }

    // final selection: above the threshold, or equal to it and among the first `remaining` in
    // position order.  Counts are packed (above << 16 | equal): an exclusive prefix of either
    // count stays below 2^16 (at most 64 * kThreads elements, fewer than k above the threshold),
    // so the low field never carries into the high one.  The prefix of an element in position
    // order is: earlier waves (one block scan of the wave totals), then earlier groups of its
    // wave (their wave totals), then earlier lanes of its group (a wave scan per group).
    uint32_t cnt[G], pre[G];
    uint32_t run = 0;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        uint32_t c = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int i = E * g + e;
            const bool v = valid(i);
            const uint32_t m = key[i] & mask;
            c += (v && m > prefix) ? 0x10000u : 0u;
            c += (v && m == prefix) ? 1u : 0u;
        }
        cnt[g] = c;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const uint32_t x = wave_inclusive_sum(cnt[g]);
        pre[g] = run + x - cnt[g];
        run += uint32_t(__builtin_amdgcn_readlane(int(x), 63));
    }
    int total;
    const uint32_t wave_pre = uint32_t(block_exclusive_scan<kWaves>(lane == 63 ? int(run) : 0, sh_scan[pass & 1], &total));
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const uint32_t packed = wave_pre + pre[g];
        const int gt_before = int(packed >> 16), eq_before = int(packed & 0xffffu);
        // output offset: every earlier element above, plus the earlier equal ones that are kept
        int off = gt_before + min(eq_before, remaining);
        int eq_rank = eq_before;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int i = E * g + e;
            const bool v = valid(i);
            const uint32_t m = key[i] & mask;
            bool take = v && m > prefix;
            if (v && m == prefix) take = eq_rank++ < remaining;
            if (take && off < k) o[off++] = wbase + 64 * E * g + e;
        }
    }
}

template <int IPT, int NT>
void launch_shape(const tsa_decode_params& p, const float* scores, int ld, const int32_t* seq_lens,
                  int32_t* topk, hipStream_t s) {
    hipLaunchKernelGGL((topk_radix_kernel<IPT, NT>), dim3(p.batch), dim3(NT), 0, s, scores, ld,
                       seq_lens, p.max_len, p.top_k, topk);
}

}  // namespace

namespace tsa {

bool topk_supported(int max_len) { return max_len <= 64 * kMaxThreads; }

hipError_t launch_topk(const tsa_decode_params& p, const float* scores, int ld,
                       const int32_t* seq_lens, int32_t* topk, hipStream_t s) {
    // 1,024 threads from 2,049 scores up: the phases are latency-bound, and sixteen waves hide one
    // another's latency better than fewer waves with more elements each (256 or 512 threads
    // measured 10 to 70 % slower there).  Up to 2,048 scores, 512 threads with 1, 2 or 4 scores
    // each are 0.4-0.7 us faster than 1,024 with 1 or 2 (half the waves go through each barrier)
    // and 256 threads are slower again.  The scores per thread follow the length closely, since
    // every pass walks all of them (24 instead of 32 per thread took a 20k-token selection from
    // 13.2 to 12.6 us).
    if (p.max_len <= 2048) {
        const int ipt = (p.max_len + 511) / 512;
        if (ipt <= 1) launch_shape<1, 512>(p, scores, ld, seq_lens, topk, s);
        else if (ipt <= 2) launch_shape<2, 512>(p, scores, ld, seq_lens, topk, s);
        else launch_shape<4, 512>(p, scores, ld, seq_lens, topk, s);
        return hipGetLastError();
    }
    const int ipt = (p.max_len + kMaxThreads - 1) / kMaxThreads;
    if (ipt <= 4) launch_shape<4, 1024>(p, scores, ld, seq_lens, topk, s);
    else if (ipt <= 8) launch_shape<8, 1024>(p, scores, ld, seq_lens, topk, s);
    else if (ipt <= 12) launch_shape<12, 1024>(p, scores, ld, seq_lens, topk, s);
    else if (ipt <= 16) launch_shape<16, 1024>(p, scores, ld, seq_lens, topk, s);
    else if (ipt <= 24) launch_shape<24, 1024>(p, scores, ld, seq_lens, topk, s);
    else if (ipt <= 32) launch_shape<32, 1024>(p, scores, ld, seq_lens, topk, s);
    else if (ipt <= 48) launch_shape<48, 1024>(p, scores, ld, seq_lens, topk, s);
    else if (ipt <= 64) launch_shape<64, 1024>(p, scores, ld, seq_lens, topk, s);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace tsa
