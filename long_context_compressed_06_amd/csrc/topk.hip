// Per-query top-k over the indexer scores (DeepSeek-V4 overview page,
// section 2.2 step 2: keep only the top-k most relevant compressed entries).
//
// Order: score descending, then entry index ascending, so the kept set is
// unique even with equal scores.  Output: kept indices ascending, -1 padded.
//
// Method: exact radix select on order-preserving 32-bit keys, one 1024-thread
// workgroup per query.  Three histogram passes (11, 11 and 10 bits, LDS
// atomics) narrow the k-th key down to a single value T; one ordered pass
// then keeps every key above T and the lowest-indexed keys equal to T, using
// wave ballots and a block scan to place the kept indices in ascending order.
// Rows that fit (n_visible <= LDS_KEYS) are staged once in LDS; longer rows are
// re-read from the score buffer (L2) on each pass.
#include "kernels.h"

namespace csa {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;

__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;  // -0 ranks with +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// exclusive prefix over the workgroup of one flag per thread; returns the
// prefix and writes the total to *total (all threads).
__device__ __forceinline__ int block_scan_flag(bool f, int *wave_tot, int *total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const uint64_t bal = __ballot(f);
    const int in_wave = __popcll(bal & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
    if (lane == 0) wave_tot[wv] = __popcll(bal);
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kTopkWaves; ++i) {
        const int v = wave_tot[i];
        before += i < wv ? v : 0;
        tot += v;
    }
    __syncthreads();
    *total = tot;
    return before + in_wave;
}

template <bool IN_LDS>
__global__ __launch_bounds__(kTopkThreads) void k_topk(int Tq, int N, int m, int k, int64_t q_pos0,
                                                        const float *__restrict__ scores, int32_t *__restrict__ out) {
    extern __shared__ uint32_t lds_keys[];
    __shared__ uint32_t hist[2048];
    __shared__ int wave_tot[kTopkWaves];
    __shared__ uint32_t sh_digit;
    __shared__ int sh_above, sh_at;

    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t nv = n_visible(q_pos0 + row % Tq, m, N);
    int32_t *orow = out + row * k;
    if (nv <= k) {
        for (int i = tid; i < k; i += kTopkThreads) orow[i] = i < nv ? i : -1;
        return;
    }
    const float *srow = scores + row * (int64_t)N;
    if (IN_LDS) {
        for (int64_t j = tid; j < nv; j += kTopkThreads) lds_keys[j] = order_key(srow[j]);
        __syncthreads();
    }
    auto key_at = [&](int64_t j) -> uint32_t { return IN_LDS ? lds_keys[j] : order_key(srow[j]); };

    uint32_t prefix = 0, mask = 0;
    int rem = k;  // how many keys equal to the current prefix still have to be kept
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const int nbins = pass == 2 ? 1024 : 2048;
        for (int i = tid; i < 2048; i += kTopkThreads) hist[i] = 0;
        __syncthreads();
        for (int64_t j = tid; j < nv; j += kTopkThreads) {
            const uint32_t key = key_at(j);
            if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & (nbins - 1)], 1u);
        }
        __syncthreads();
        // Find digit D with  count(digit > D) < rem <= count(digit >= D).
        // Thread i owns bins [2i, 2i+2); a descending inclusive scan over
        // owners gives the count of keys in bins >= 2i.
        const int per = nbins / kTopkThreads;  // 2 or 1
        int own = 0;
        for (int q = 0; q < per; ++q) own += (int)hist[tid * per + q];
        // suffix sum over threads: count in bins owned by threads > tid
        // (two-level: within wave via shuffles, across waves via LDS)
        const int lane = tid & 63, wv = tid >> 6;
        int suf = own;
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_down(suf, o);
            if (lane + o < 64) suf += v;
        }
        if (lane == 0) wave_tot[wv] = suf;  // total of the wave
        __syncthreads();
        int after_waves = 0;
        for (int i = wv + 1; i < kTopkWaves; ++i) after_waves += wave_tot[i];
        const int incl = suf + after_waves;  // keys in bins >= tid*per
        const int excl = incl - own;         // keys in bins >= (tid+1)*per
        if (excl < rem && incl >= rem) {
            // the digit is in this thread's bins: walk them from the top
            int above = excl;
            for (int q = per - 1; q >= 0; --q) {
                const int h = (int)hist[tid * per + q];
                if (above + h >= rem) {
                    sh_digit = (uint32_t)(tid * per + q);
                    sh_above = above;
                    sh_at = h;
                    break;
                }
                above += h;
            }
        }
        __syncthreads();
        const uint32_t digit = sh_digit;
        rem -= sh_above;
        prefix |= digit << shift;
        mask |= (uint32_t)(nbins - 1) << shift;
        const bool all_equal_kept = (sh_at == rem);
        __syncthreads();
        if (all_equal_kept) break;
    }

    // ordered compaction: keys above the prefix, then the first `rem` equal ones
    int out_base = 0, eq_base = 0;
    for (int64_t c0 = 0; c0 < nv; c0 += kTopkThreads) {
        const int64_t j = c0 + tid;
        bool gt = false, eq = false;
        if (j < nv) {
            const uint32_t km = key_at(j) & mask;
            gt = km > prefix;
            eq = km == prefix;
        }
        int eq_tot, sel_tot;
        const int eq_before = eq_base + block_scan_flag(eq, wave_tot, &eq_tot);
        const bool sel = gt || (eq && eq_before < rem);
        const int pos = out_base + block_scan_flag(sel, wave_tot, &sel_tot);
        if (sel && pos < k) orow[pos] = (int32_t)j;
        eq_base += eq_tot;
        out_base += sel_tot;
    }
}

hipError_t launch_topk(int B, int Tq, int N, int m, int k, int64_t q_pos0, const float *scores, int32_t *out,
                       hipStream_t st) {
    const int64_t rows = (int64_t)B * Tq;
    if (N <= kTopkLdsKeys) {
        const size_t lds = (size_t)(N > 0 ? N : 1) * sizeof(uint32_t);
        static const hipError_t attr = hipFuncSetAttribute(
            (const void *)k_topk<true>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)(kTopkLdsKeys * sizeof(uint32_t)));
        if (attr != hipSuccess) return attr;
        hipLaunchKernelGGL(k_topk<true>, dim3((unsigned)rows), dim3(kTopkThreads), lds, st, Tq, N, m, k, q_pos0,
                           scores, out);
    } else {
        hipLaunchKernelGGL(k_topk<false>, dim3((unsigned)rows), dim3(kTopkThreads), 0, st, Tq, N, m, k, q_pos0,
                           scores, out);
    }
    return hipGetLastError();
}

}  // namespace csa
