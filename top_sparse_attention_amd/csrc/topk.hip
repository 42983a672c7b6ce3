// Top-k selection of indexer scores: one workgroup per request.
//
// GLM5.3 sparse-attention page, lightning-indexer paragraph: the score selects the top K
// tokens; a query with fewer than K tokens stays dense.  Equal scores are ordered by position
// (lowest first), so the selected set is unique; it is written as ascending positions.
//
// Scores map to order-preserving 32-bit keys, 32 to 64 per thread in registers.  One workgroup
// holds a whole request, so what the kernel costs is the vector-ALU work per element: it makes one
// cheap pass over all elements and does the exact selection on a short list.
//  1. Sample: one key per thread (1,024 regularly spaced positions).  A histogram of the sample's
//     12-bit first digits (sign, exponent, top three mantissa bits) gives a bound t_lo: the lower
//     edge of the bin holding the sample's r-th largest key, with r the sample's expected share
//     of the k kept elements plus four standard deviations.  The k largest keys of the request are
//     then almost surely all >= t_lo.
//  2. One pass in position order compacts every element with key >= t_lo (key and position) into
//     an LDS list, its place given by a prefix count: a wave scan per load group plus one block
//     scan of the wave totals.  Each wave owns a contiguous block of positions and reads it with
//     wave-contiguous 16-byte loads (one 1 KiB run per instruction).
//  3. If the list holds at least k and at most 8,192 elements, the selection runs on it alone,
//     8 per thread in list order (which is position order): radix passes narrow the key of the
//     k-th largest (a 12-bit digit, then 8, 8 and 4 bits; a pass stops the search once the
//     remaining candidates are equal or their bin is kept whole), then a prefix count in list
//     order of the packed pair (above the threshold, equal to it) gives the tie ranks and the
//     output offsets at once, so the output comes out ascending with no sort.
//  4. Otherwise (an unlucky sample, heavy ties, a crowded range) the same selection runs over
//     every element in registers with 8-bit digits from the top.
// Radix-pass histograms are LDS atomics on interleaved copies, so that lanes hitting one bin
// spread over banks; consecutive passes double-buffer their histograms and key-range slots by
// parity to save barriers, and wave scans and min / max use DPP lane moves.
#include "tsa_internal.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kCopies = 16;               // histogram copies of the 8-bit passes
constexpr int kBins1 = 4096;              // 12-bit digit: key bits 31..20
constexpr int kShift1 = 20;
constexpr int kCopies12 = 2;              // histogram copies of the list's 12-bit pass
constexpr int kListCap = 8192;            // list entries (keys, then positions, in `big`)
constexpr int kPer = kListCap / kThreads; // list entries per thread
static_assert(kBins1 * kCopies12 <= 2 * kListCap, "the 12-bit histogram fits where the list was");

__device__ inline uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
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

template <int IPT>
__global__ void __launch_bounds__(kThreads) topk_radix_kernel(const float* __restrict__ scores,
                                                              int ld,
                                                              const int32_t* __restrict__ seq_lens,
                                                              int max_len, int k,
                                                              int32_t* __restrict__ out) {
    // the sample histogram, then the list (keys | positions), then the list's 12-bit histogram
    __shared__ uint32_t big[2 * kListCap];
    __shared__ uint32_t hist[2][256 * kCopies];    // 8-bit passes, one buffer per pass parity
    __shared__ int sh_scan[2][2 * kWaves + 1];
    __shared__ int sh_sel[4];
    __shared__ uint32_t sh_mm[4];                  // candidate key range, per pass parity
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
    // order within the wave is (g, lane, e).
    constexpr int E = IPT < 4 ? IPT : 4;
    constexpr int G = IPT / E;
    const int lane = tid & 63;
    const int wbase = (tid >> 6) * 64 * IPT + E * lane;   // position of element (0, 0)
    uint32_t key[IPT];
    if (E == 4 && (ld & 3) == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int p0 = wbase + 64 * E * g;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (p0 + 3 < len) {
                v = *reinterpret_cast<const float4*>(s + p0);
            } else {
                if (p0 < len) v.x = s[p0];
                if (p0 + 1 < len) v.y = s[p0 + 1];
                if (p0 + 2 < len) v.z = s[p0 + 2];
            }
            key[4 * g + 0] = order_key(v.x);
            key[4 * g + 1] = order_key(v.y);
            key[4 * g + 2] = order_key(v.z);
            key[4 * g + 3] = order_key(v.w);
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


    // ---- 1. sample: element 0 of every thread; t_lo from its 12-bit digit histogram ----
    for (int i = tid; i < kBins1; i += kThreads) big[i] = 0;
    for (int i = tid; i < 256 * kCopies; i += kThreads) hist[0][i] = 0;
    if (tid == 0) {
        sh_mm[0] = 0xffffffffu;
        sh_mm[1] = 0u;
    }
    __syncthreads();
    if (valid(0)) atomicAdd(&big[key[0] >> kShift1], 1u);
    __syncthreads();
    {
        uint32_t c[4];
        int t = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            c[e] = big[kBins1 - 1 - 4 * tid - e];
            t += int(c[e]);
        }
        int n_s;
        int above = block_exclusive_scan(t, sh_scan[1], &n_s);
        // the sample's expected count of kept elements, plus four standard deviations and a floor
        const float expect = float(k) * float(n_s) / float(len);
        const int r = min(n_s, int(ceilf(expect + 4.f * sqrtf(expect))) + 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (above < r && above + int(c[e]) >= r) sh_sel[0] = kBins1 - 1 - 4 * tid - e;
            above += int(c[e]);
        }
    }
    __syncthreads();
    const uint32_t t_lo = uint32_t(sh_sel[0]) << kShift1;

    // ---- 2. compact the elements with key >= t_lo, in position order ----
    int n_keep;
    {
        uint32_t cnt[G], pre[G];
        uint32_t run = 0;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            uint32_t c = 0;
#pragma unroll
            for (int e = 0; e < E; ++e) c += (valid(E * g + e) && key[E * g + e] >= t_lo) ? 1u : 0u;
            cnt[g] = c;
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const uint32_t x = wave_inclusive_sum(cnt[g]);
            pre[g] = run + x - cnt[g];
            run += uint32_t(__builtin_amdgcn_readlane(int(x), 63));
        }
        const uint32_t wave_pre = uint32_t(block_exclusive_scan(lane == 63 ? int(run) : 0, sh_scan[0], &n_keep));
        // the sample histogram (aliased by the list) was last read before the scan's barriers
        if (n_keep >= k && n_keep <= kListCap) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                int idx = int(wave_pre + pre[g]);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int i = E * g + e;
                    if (valid(i) && key[i] >= t_lo) {
                        if (idx < kListCap) {
                            big[idx] = key[i];
                            big[kListCap + idx] = uint32_t(wbase + 64 * E * g + e);
                        }
                        ++idx;
                    }
                }
            }
        }
    }
    __syncthreads();

    if (n_keep >= k && n_keep <= kListCap) {     // uniform
        // ---- 3. select on the list: thread t holds entries kPer t .. kPer t + kPer - 1 ----
        uint32_t lk[kPer];
        int32_t lp[kPer];
        bool lv[kPer];
        uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int idx = kPer * tid + j;
            lv[j] = idx < n_keep;
            lk[j] = lv[j] ? big[idx] : 0u;
            lp[j] = lv[j] ? int32_t(big[kListCap + idx]) : 0;
            if (lv[j]) {
                kmin = min(kmin, lk[j]);
                kmax = max(kmax, lk[j]);
            }
        }
        kmin = wave_min(kmin);
        kmax = wave_max(kmax);
        if (lane == 0) {
            atomicMin(&sh_mm[0], kmin);
            atomicMax(&sh_mm[1], kmax);
        }
        __syncthreads();                 // the list is in registers; `big` is free again
        uint32_t prefix = 0, mask = 0;
        int remaining = k;               // how many of the entries matching `prefix` under `mask` to keep
        int pass = 0;
        bool done = false;
        if (sh_mm[0] == sh_mm[1]) {      // uniform: every entry has the same key
            prefix = sh_mm[0];
            mask = 0xffffffffu;
            done = true;
        } else {
            // 12-bit first digit
            uint32_t* h12 = big;
            for (int i = tid; i < kBins1 * kCopies12; i += kThreads) h12[i] = 0;
            if (tid == 0) {
                sh_mm[2] = 0xffffffffu;
                sh_mm[3] = 0u;
            }
            __syncthreads();
            const int copy = tid & (kCopies12 - 1);
#pragma unroll
            for (int j = 0; j < kPer; ++j)
                if (lv[j]) atomicAdd(&h12[(lk[j] >> kShift1) * kCopies12 + copy], 1u);
            __syncthreads();
            uint32_t c[4];
            int t = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int dgt = kBins1 - 1 - 4 * tid - e;
                c[e] = 0;
#pragma unroll
                for (int j = 0; j < kCopies12; ++j) c[e] += h12[dgt * kCopies12 + j];
                t += int(c[e]);
            }
            int total;
            int above = block_exclusive_scan(t, sh_scan[1], &total);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (above < remaining && above + int(c[e]) >= remaining) {
                    sh_sel[0] = kBins1 - 1 - 4 * tid - e;
                    sh_sel[1] = remaining - above;
                    sh_sel[2] = int(c[e]);
                }
                above += int(c[e]);
            }
            __syncthreads();
            prefix = uint32_t(sh_sel[0]) << kShift1;
            mask = 0xfff00000u;
            remaining = sh_sel[1];
            done = sh_sel[2] == remaining;       // the whole bin is kept
            __syncthreads();
        }
        // 8, 8 and 4 more bits over the entries still matching
        for (int shift = 12; !done && shift >= -4; shift -= 8, ++pass) {
            const int sh = shift > 0 ? shift : 0;
            const uint32_t width_mask = shift > 0 ? 255u : 15u;
            uint32_t* h = hist[pass & 1];
            // the other buffer was last read before the previous pass's selection barrier
            for (int i = tid; i < 256 * kCopies; i += kThreads) hist[(pass + 1) & 1][i] = 0;
            const int copy = tid & (kCopies - 1);
            uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                if (lv[j] && (lk[j] & mask) == prefix) {
                    atomicAdd(&h[((lk[j] >> sh) & width_mask) * kCopies + copy], 1u);
                    lo = min(lo, lk[j]);
                    hi = max(hi, lk[j]);
                }
            }
            lo = wave_min(lo);
            hi = wave_max(hi);
            const int slot = 2 * ((pass + 1) & 1);   // sh_mm[0..1] held the whole list's range
            if (lane == 0) {
                atomicMin(&sh_mm[slot], lo);
                atomicMax(&sh_mm[slot + 1], hi);
            }
            if (tid == 0) {
                sh_mm[2 * (pass & 1)] = 0xffffffffu;
                sh_mm[2 * (pass & 1) + 1] = 0u;
            }
            __syncthreads();
            if (sh_mm[slot] == sh_mm[slot + 1]) {      // uniform
                prefix = sh_mm[slot];
                mask = 0xffffffffu;
                break;
            }
            int cb = 0;
            if (tid < 256) {
                const int dgt = 255 - tid;
#pragma unroll
                for (int j = 0; j < kCopies; ++j) cb += h[dgt * kCopies + ((j + tid) & (kCopies - 1))];
            }
            int total;
            const int above = block_exclusive_scan(cb, sh_scan[pass & 1], &total);
            if (tid < 256 && above < remaining && above + cb >= remaining) {
                sh_sel[0] = 255 - tid;
                sh_sel[1] = remaining - above;
                sh_sel[2] = cb;
            }
            __syncthreads();
            const uint32_t dgt = uint32_t(sh_sel[0]);
            remaining = sh_sel[1];
            const int bin_count = sh_sel[2];
            __syncthreads();
            prefix |= dgt << sh;
            mask |= width_mask << sh;
            if (bin_count == remaining) break;
        }
        // kept entries in list order: above the threshold, or equal to it and among the first
        // `remaining` equal ones; packed (above << 16 | equal) counts, both below 2^16 here
        uint32_t cc = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const uint32_t m = lk[j] & mask;
            cc += (lv[j] && m > prefix) ? 0x10000u : 0u;
            cc += (lv[j] && m == prefix) ? 1u : 0u;
        }
        int total;
        const uint32_t cpre = uint32_t(block_exclusive_scan(int(cc), sh_scan[pass & 1], &total));
        int gt = int(cpre >> 16), eq = int(cpre & 0xffffu);
        int off = gt + min(eq, remaining);
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const uint32_t m = lk[j] & mask;
            bool take = lv[j] && m > prefix;
            if (lv[j] && m == prefix) take = eq++ < remaining;
            if (take && off < k) o[off++] = lp[j];
        }
        return;
    }

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
        const int above = block_exclusive_scan(c, sh_scan[pass & 1], &total);  // count with a larger digit
        if (tid < 256 && above < remaining && above + c >= remaining) {
            sh_sel[0] = 255 - tid;
            sh_sel[1] = remaining - above;
            sh_sel[2] = c;
        }
        __syncthreads();
        const uint32_t dgt = sh_sel[0];
        remaining = sh_sel[1];
        const int in_bin = sh_sel[2];
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
    const uint32_t wave_pre = uint32_t(block_exclusive_scan(lane == 63 ? int(run) : 0, sh_scan[pass & 1], &total));
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

template <int IPT>
void launch_ipt(const tsa_decode_params& p, const float* scores, int ld, const int32_t* seq_lens,
                int32_t* topk, hipStream_t s) {
    hipLaunchKernelGGL((topk_radix_kernel<IPT>), dim3(p.batch), dim3(kThreads), 0, s, scores, ld,
                       seq_lens, p.max_len, p.top_k, topk);
}

}  // namespace

namespace tsa {

bool topk_supported(int max_len) { return max_len <= 64 * kThreads; }

hipError_t launch_topk(const tsa_decode_params& p, const float* scores, int ld,
                       const int32_t* seq_lens, int32_t* topk, hipStream_t s) {
    const int ipt = (p.max_len + kThreads - 1) / kThreads;
    if (ipt <= 1) launch_ipt<1>(p, scores, ld, seq_lens, topk, s);
    else if (ipt <= 2) launch_ipt<2>(p, scores, ld, seq_lens, topk, s);
    else if (ipt <= 4) launch_ipt<4>(p, scores, ld, seq_lens, topk, s);
    else if (ipt <= 8) launch_ipt<8>(p, scores, ld, seq_lens, topk, s);
    else if (ipt <= 16) launch_ipt<16>(p, scores, ld, seq_lens, topk, s);
    else if (ipt <= 32) launch_ipt<32>(p, scores, ld, seq_lens, topk, s);
    else if (ipt <= 64) launch_ipt<64>(p, scores, ld, seq_lens, topk, s);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace tsa
