// Top-k selection of indexer scores: one workgroup per request, radix select in LDS.
//
// GLM5.3 sparse-attention page, lightning-indexer paragraph: the score selects the top K
// tokens; a query with fewer than K tokens stays dense.  Equal scores are ordered by position
// (lowest first), so the selected set is unique; it is written as ascending positions.
//
// Method: scores map to order-preserving 32-bit keys.  Four 8-bit radix passes narrow the key
// of the k-th largest element (a histogram of the candidate digits per pass, kept in LDS as 16
// interleaved copies so that lanes hitting the same bin spread over distinct addresses).  A pass
// also finds the smallest and largest candidate key; when they are equal the threshold key is
// known and the remaining passes are skipped (ties at the threshold are common for
// integer-valued scores).  After the passes, every element whose key exceeds the threshold is
// kept, and of the elements equal to it the lowest positions fill the rest; one block-wide
// scan over positions (each thread owns a contiguous run) of the packed counts (above,
// equal) yields both the tie ranks and the output offsets, so the output comes out ascending
// with no sort.
#include "tsa_internal.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kCopies = 16;

__device__ inline uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive scan over the block in thread order; returns this thread's prefix, total in *total.
__device__ inline int block_exclusive_scan(int v, int* sh_waves, int* total) {
    // sums wrap modulo 2^32 (unsigned arithmetic): packed counts rely on it
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = uint32_t(v);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = uint32_t(__shfl_up(int(x), o));
        if (lane >= o) x += y;
    }
    if (lane == 63) sh_waves[wave] = int(x);
    __syncthreads();
    if (threadIdx.x < 64) {
        const uint32_t w = threadIdx.x < kWaves ? uint32_t(sh_waves[threadIdx.x]) : 0u;
        uint32_t s = w;
#pragma unroll
        for (int o = 1; o < kWaves; o <<= 1) {
            const uint32_t y = uint32_t(__shfl_up(int(s), o));
            if ((int)threadIdx.x >= o) s += y;
        }
        if (threadIdx.x < kWaves) sh_waves[kWaves + threadIdx.x] = int(s - w);
        if (threadIdx.x == kWaves - 1) sh_waves[2 * kWaves] = int(s);
    }
    __syncthreads();
    const int r = int(uint32_t(sh_waves[kWaves + wave]) + x - uint32_t(v));
    *total = sh_waves[2 * kWaves];
    __syncthreads();
    return r;
}

template <int IPT>
__global__ void __launch_bounds__(kThreads) topk_radix_kernel(const float* __restrict__ scores,
                                                              int ld,
                                                              const int32_t* __restrict__ seq_lens,
                                                              int max_len, int k,
                                                              int32_t* __restrict__ out) {
    __shared__ uint32_t hist[256 * kCopies];
    __shared__ int sh_scan[2 * kWaves + 1];
    __shared__ int sh_sel[4];
    __shared__ uint32_t sh_mm[2];

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
    const int base = tid * IPT;
    uint32_t key[IPT];
    if (IPT >= 4 && (ld & 3) == 0) {
#pragma unroll
        for (int i = 0; i < IPT; i += 4) {
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (base + i + 3 < len) {
                v = *reinterpret_cast<const float4*>(s + base + i);
            } else {
                if (base + i < len) v.x = s[base + i];
                if (base + i + 1 < len) v.y = s[base + i + 1];
                if (base + i + 2 < len) v.z = s[base + i + 2];
            }
            key[i] = order_key(v.x);
            key[i + 1] = order_key(v.y);
            key[i + 2] = order_key(v.z);
            key[i + 3] = order_key(v.w);
        }
    } else {
#pragma unroll
        for (int i = 0; i < IPT; ++i) key[i] = (base + i < len) ? order_key(s[base + i]) : 0u;
    }

    uint32_t prefix = 0, mask = 0;
    int remaining = k;  // how many of the elements matching `prefix` under `mask` to keep
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256 * kCopies; i += kThreads) hist[i] = 0;
        if (tid == 0) {
            sh_mm[0] = 0xffffffffu;
            sh_mm[1] = 0u;
        }
        __syncthreads();
        const int copy = tid & (kCopies - 1);
        uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
        for (int i = 0; i < IPT; ++i) {
            if (base + i < len && (key[i] & mask) == prefix) {
                atomicAdd(&hist[((key[i] >> shift) & 255u) * kCopies + copy], 1u);
                kmin = min(kmin, key[i]);
                kmax = max(kmax, key[i]);
            }
        }
        // candidates' key range: once they are all equal, the k-th key is known exactly
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
            kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
        }
        if ((tid & 63) == 0) {
            atomicMin(&sh_mm[0], kmin);
            atomicMax(&sh_mm[1], kmax);
        }
        __syncthreads();
        if (sh_mm[0] == sh_mm[1]) {      // uniform
            prefix = sh_mm[0];
            mask = 0xffffffffu;
            __syncthreads();
            break;
        }
        // bins in descending digit order: thread j < 256 owns digit 255 - j
        int c = 0;
        if (tid < 256) {
            const int dgt = 255 - tid;
#pragma unroll
            for (int j = 0; j < kCopies; ++j) c += hist[dgt * kCopies + ((j + tid) & (kCopies - 1))];
        }
        int total;
        const int above = block_exclusive_scan(c, sh_scan, &total);  // count with a larger digit
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

    // final selection: above the threshold, or equal to it and among the first `remaining`;
    // one scan of the packed counts (above << 16 | equal): an exclusive prefix of either count
    // stays below 2^16 (at most 64 * kThreads elements, fewer than k above the threshold), so
    // the low field never carries into the high one
    int gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        const bool v = base + i < len;
        const uint32_t m = key[i] & mask;
        gt += (v && m > prefix);
        eq += (v && m == prefix);
    }
    int total;
    const uint32_t packed = uint32_t(block_exclusive_scan(int((uint32_t(gt) << 16) | uint32_t(eq)), sh_scan, &total));
    const int gt_before = int(packed >> 16), eq_before = int(packed & 0xffffu);
    // output offset: every earlier element above, plus the earlier equal ones that are kept
    int off = gt_before + min(eq_before, remaining);
    int eq_rank = eq_before;
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        const bool v = base + i < len;
        const uint32_t m = key[i] & mask;
        bool take = v && m > prefix;
        if (v && m == prefix) take = eq_rank++ < remaining;
        if (take && off < k) o[off++] = base + i;
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
