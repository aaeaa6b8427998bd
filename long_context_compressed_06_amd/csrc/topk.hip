// Per-query top-k over the indexer scores (DeepSeek-V4 overview page,
// section 2.2 step 2: keep only the top-k most relevant compressed entries).
//
// Order: score descending, then entry index ascending, so the kept set is
// unique even with equal scores.  Output: kept indices ascending, -1 padded.
//
// Method: exact radix select on order-preserving 32-bit keys.  The first
// digit (top 11 bits) is counted by the indexer epilogue into a per-query
// histogram, so no workgroup here rescans a row for it.  From the histogram
// the digit D holding the k-th key follows; keys with a higher digit are kept,
// keys with digit D are the candidates, resolved by two more digits (11 and
// 10 bits, LDS histograms) and, for keys that are fully equal, by index.
//
// Few queries (decode): one query's row is cut into chunks of
// kTopkFilterChunk scores; a filter workgroup per chunk writes the kept and
// the candidate indices of its chunk, in index order, to a segment of the
// workspace, and one final workgroup per query selects among the candidates
// in LDS and merges both sorted lists.  Many queries (prefill): one
// workgroup per query with the row staged in LDS.  Either way the kept set
// leaves in ascending index order through block scans, never a sort.
#include "kernels.h"

namespace csa {

// ------------------------------------------------------------------ helpers
// exclusive prefix of v over the workgroup (NT threads); *total gets the sum
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int *sh, int *total) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) sh[wv] = x;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int s = sh[i];
        before += i < wv ? s : 0;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return before + x - v;
}

struct Digit {
    uint32_t digit;
    int above;  // keys in higher bins
    int at;     // keys in the digit's bin
};

// Find D with count(bin > D) < rem <= count(bin >= D) over nbins bins.
template <int NT>
__device__ Digit find_digit(const uint32_t *hist, int nbins, int rem, int *sh, Digit *shd) {
    const int per = nbins / NT;
    const int tid = threadIdx.x;
    int own = 0;
    for (int q = 0; q < per; ++q) own += (int)hist[tid * per + q];
    int total;
    const int before = block_excl_scan<NT>(own, sh, &total);
    const int incl = total - before;  // keys in bins >= tid*per
    const int excl = incl - own;      // keys in bins >= (tid+1)*per
    if (excl < rem && incl >= rem) {
        int above = excl;
        for (int q = per - 1; q >= 0; --q) {
            const int h = (int)hist[tid * per + q];
            if (above + h >= rem) {
                shd->digit = (uint32_t)(tid * per + q);
                shd->above = above;
                shd->at = h;
                break;
            }
            above += h;
        }
    }
    __syncthreads();
    const Digit d = *shd;
    __syncthreads();
    return d;
}

// Narrow the selection among keys matching (prefix, mask) down to one full
// key value with radix digits at bits [20:10] and [9:0].  On return, keys
// with (key & mask) > prefix are kept, and `rem` of those equal to prefix.
template <int NT, class KeyAt>
__device__ void refine(KeyAt key_at, int64_t n, uint32_t &prefix, uint32_t &mask, int &rem, uint32_t *hist, int *sh,
                       Digit *shd) {
    for (int pass = 1; pass < 3; ++pass) {
        const int shift = pass == 1 ? 10 : 0;
        const int nbins = pass == 1 ? 2048 : 1024;
        for (int i = threadIdx.x; i < 2048; i += NT) hist[i] = 0;
        __syncthreads();
        for (int64_t j = threadIdx.x; j < n; j += NT) {
            const uint32_t key = key_at(j);
            if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & (nbins - 1)], 1u);
        }
        __syncthreads();
        const Digit d = find_digit<NT>(hist, nbins, rem, sh, shd);
        rem -= d.above;
        prefix |= d.digit << shift;
        mask |= (uint32_t)(nbins - 1) << shift;
        if (d.at == rem) break;  // every key equal to the prefix is kept
    }
}

// Walk n items in index order; keep those above the prefix and the first
// `rem` equal to it; emit(pos, i) for the kept ones, pos ascending.
template <int NT, class KeyAt, class Emit>
__device__ void ordered_keep(KeyAt key_at, int64_t n, uint32_t prefix, uint32_t mask, int rem, int *sh, Emit emit) {
    int out_base = 0, eq_base = 0;
    for (int64_t c0 = 0; c0 < n; c0 += NT) {
        const int64_t i = c0 + threadIdx.x;
        int gt = 0, eq = 0;
        if (i < n) {
            const uint32_t km = key_at(i) & mask;
            gt = km > prefix;
            eq = km == prefix;
        }
        int eq_tot, sel_tot;
        const int eq_before = eq_base + block_excl_scan<NT>(eq, sh, &eq_tot);
        const int sel = gt || (eq && eq_before < rem);
        const int pos = out_base + block_excl_scan<NT>(sel, sh, &sel_tot);
        if (sel) emit(pos, i);
        eq_base += eq_tot;
        out_base += sel_tot;
    }
}

__device__ __forceinline__ int lower_bound(const int32_t *a, int n, int32_t x) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (a[mid] < x) lo = mid + 1; else hi = mid;
    }
    return lo;
}

constexpr int kNT = 1024;   // threads of the per-query workgroups
constexpr int kFT = 256;    // threads of a filter workgroup
constexpr int kFPT = kTopkFilterChunk / kFT;  // scores per filter thread

__global__ void k_fill_u32(uint32_t *p, int64_t n, uint32_t v) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

__device__ __forceinline__ bool trivial_row(int64_t nv, int k, int32_t *orow) {
    if (nv > k) return false;
    for (int i = threadIdx.x; i < k; i += blockDim.x) orow[i] = i < nv ? i : -1;
    return true;
}

// --------------------------------------------------- one workgroup per query
template <bool IN_LDS>
__global__ __launch_bounds__(kNT) void k_topk_rows(int Tq, int N, int m, int k, int64_t q_pos0,
                                                   const float *__restrict__ scores,
                                                   const uint32_t *__restrict__ ghist, int32_t *__restrict__ out) {
    extern __shared__ uint32_t lds_keys[];
    __shared__ uint32_t hist[2048];
    __shared__ int sh[kNT / 64];
    __shared__ Digit shd;
    const int64_t row = blockIdx.x;
    const int64_t nv = n_visible(q_pos0 + row % Tq, m, N);
    int32_t *orow = out + row * k;
    if (trivial_row(nv, k, orow)) return;
    const float *srow = scores + row * (int64_t)N;
    if (IN_LDS) {
        for (int64_t j = threadIdx.x; j < nv; j += kNT) lds_keys[j] = order_key(srow[j]);
    }
    auto key_at = [&](int64_t j) -> uint32_t { return IN_LDS ? lds_keys[j] : order_key(srow[j]); };
    const Digit d = find_digit<kNT>(ghist + row * kTopkBins, kTopkBins, k, sh, &shd);
    uint32_t prefix = d.digit << (32 - kTopkBinBits), mask = ~0u << (32 - kTopkBinBits);
    int rem = k - d.above;
    if (d.at != rem) refine<kNT>(key_at, nv, prefix, mask, rem, hist, sh, &shd);
    ordered_keep<kNT>(key_at, nv, prefix, mask, rem, sh, [&](int pos, int64_t j) {
        if (pos < k) orow[pos] = (int32_t)j;
    });
}

// ----------------------------------------------------- decode: filter + final
__global__ __launch_bounds__(kFT) void k_topk_filter(int Tq, int N, int m, int k, int64_t q_pos0, int nblk,
                                                     const float *__restrict__ scores,
                                                     const uint32_t *__restrict__ ghist, int32_t *__restrict__ seg,
                                                     int32_t *__restrict__ counts) {
    __shared__ int sh[kFT / 64];
    __shared__ Digit shd;
    const int64_t row = blockIdx.x / nblk;
    const int blk = blockIdx.x % nblk;
    const int64_t nv = n_visible(q_pos0 + row % Tq, m, N);
    if (nv <= k) return;
    const Digit d = find_digit<kFT>(ghist + row * kTopkBins, kTopkBins, k, sh, &shd);
    const float *srow = scores + row * (int64_t)N;
    const int64_t j0 = (int64_t)blk * kTopkFilterChunk + threadIdx.x * kFPT;
    uint32_t sure_bits = 0, cand_bits = 0;
#pragma unroll
    for (int u = 0; u < kFPT; ++u) {
        const int64_t j = j0 + u;
        if (j < nv) {
            const uint32_t dg = order_key(srow[j]) >> (32 - kTopkBinBits);
            sure_bits |= (uint32_t)(dg > d.digit) << u;
            cand_bits |= (uint32_t)(dg == d.digit) << u;
        }
    }
    // one scan of both counts: kept in the high half, candidates in the low half
    int total;
    const int pre = block_excl_scan<kFT>((int)((__popc(sure_bits) << 16) | __popc(cand_bits)), sh, &total);
    int ps = pre >> 16, pc = pre & 0xffff;
    int32_t *sg = seg + (row * nblk + blk) * (int64_t)kTopkFilterChunk;
#pragma unroll
    for (int u = 0; u < kFPT; ++u) {
        if ((sure_bits >> u) & 1) sg[ps++] = (int32_t)(j0 + u);
        if ((cand_bits >> u) & 1) sg[kTopkFilterChunk - 1 - pc++] = (int32_t)(j0 + u);
    }
    if (threadIdx.x == 0) {
        counts[(row * nblk + blk) * 2 + 0] = total >> 16;
        counts[(row * nblk + blk) * 2 + 1] = total & 0xffff;
    }
}

__global__ __launch_bounds__(kNT) void k_topk_final(int Tq, int N, int m, int k, int64_t q_pos0, int nblk,
                                                    const float *__restrict__ scores,
                                                    const uint32_t *__restrict__ ghist,
                                                    const int32_t *__restrict__ seg,
                                                    const int32_t *__restrict__ counts, int32_t *__restrict__ out) {
    extern __shared__ int32_t dyn[];
    __shared__ uint32_t hist[2048];
    __shared__ int sh[kNT / 64];
    __shared__ Digit shd;
    __shared__ int tot_s, tot_c;
    const int64_t row = blockIdx.x;
    const int64_t nv = n_visible(q_pos0 + row % Tq, m, N);
    int32_t *orow = out + row * k;
    if (trivial_row(nv, k, orow)) return;
    const float *srow = scores + row * (int64_t)N;
    const Digit d = find_digit<kNT>(ghist + row * kTopkBins, kTopkBins, k, sh, &shd);
    const uint32_t prefix0 = d.digit << (32 - kTopkBinBits), mask0 = ~0u << (32 - kTopkBinBits);
    const int rem0 = k - d.above;  // candidates to keep

    // prefix sums of the per-chunk kept / candidate counts (nblk <= kNT)
    int32_t *ps = dyn;                 // [nblk + 1]
    int32_t *pc = ps + (nblk + 1);     // [nblk + 1]
    int32_t *sidx = pc + (nblk + 1);   // [k]  kept indices
    int32_t *sel = sidx + k;           // [k]  chosen candidates
    int32_t *cidx = sel + k;           // [kTopkFinalCand]
    uint32_t *ckey = (uint32_t *)(cidx + kTopkFinalCand);
    {
        const int i = threadIdx.x;
        const int cs = i < nblk ? counts[(row * nblk + i) * 2 + 0] : 0;
        const int cc = i < nblk ? counts[(row * nblk + i) * 2 + 1] : 0;
        int ts, tc;
        const int xs = block_excl_scan<kNT>(cs, sh, &ts);
        const int xc = block_excl_scan<kNT>(cc, sh, &tc);
        if (i <= nblk) {
            ps[i] = xs;
            pc[i] = xc;
        }
        if (i == 0) {
            tot_s = ts;
            tot_c = tc;
        }
        __syncthreads();
    }
    const int S = tot_s, C = tot_c;
    const int32_t *segr = seg + row * nblk * (int64_t)kTopkFilterChunk;
    if (C > kTopkFinalCand || S != d.above) {
        // too many candidates for LDS: exact select straight over the row
        uint32_t prefix = prefix0, mask = mask0;
        int rem = rem0;
        auto key_at = [&](int64_t j) -> uint32_t { return order_key(srow[j]); };
        if (d.at != rem) refine<kNT>(key_at, nv, prefix, mask, rem, hist, sh, &shd);
        ordered_keep<kNT>(key_at, nv, prefix, mask, rem, sh, [&](int pos, int64_t j) {
            if (pos < k) orow[pos] = (int32_t)j;
        });
        return;
    }
    // candidates (index order) and kept indices (index order) into LDS
    for (int i = threadIdx.x; i < C; i += kNT) {
        const int b = lower_bound(pc, nblk + 1, i + 1) - 1;  // last chunk with pc[b] <= i
        const int32_t j = segr[b * (int64_t)kTopkFilterChunk + kTopkFilterChunk - 1 - (i - pc[b])];
        cidx[i] = j;
        ckey[i] = order_key(srow[j]);
    }
    for (int i = threadIdx.x; i < S; i += kNT) {
        const int b = lower_bound(ps, nblk + 1, i + 1) - 1;
        sidx[i] = segr[b * (int64_t)kTopkFilterChunk + (i - ps[b])];
    }
    __syncthreads();
    uint32_t prefix = prefix0, mask = mask0;
    int rem = rem0;
    auto ckey_at = [&](int64_t i) -> uint32_t { return ckey[i]; };
    if (d.at != rem) refine<kNT>(ckey_at, C, prefix, mask, rem, hist, sh, &shd);
    ordered_keep<kNT>(ckey_at, C, prefix, mask, rem, sh, [&](int pos, int64_t i) {
        if (pos < k) sel[pos] = cidx[i];
    });
    __syncthreads();
    // merge the two ascending lists
    for (int i = threadIdx.x; i < S; i += kNT) {
        const int pos = i + lower_bound(sel, rem0, sidx[i]);
        if (pos < k) orow[pos] = sidx[i];
    }
    for (int i = threadIdx.x; i < rem0; i += kNT) {
        const int pos = i + lower_bound(sidx, S, sel[i]);
        if (pos < k) orow[pos] = sel[i];
    }
}

// ------------------------------------------------------------------ host side
TopkPlan topk_plan(int64_t rows, int64_t N) {
    TopkPlan p;
    p.filter = rows < 256 || N > kTopkLdsKeys;
    p.nblk = (N + kTopkFilterChunk - 1) / kTopkFilterChunk;
    if (p.nblk < 1) p.nblk = 1;
    return p;
}

size_t topk_scratch_bytes(int64_t rows, int64_t N) {
    const TopkPlan p = topk_plan(rows, N);
    size_t bytes = (size_t)rows * kTopkBins * 4;
    if (p.filter) bytes += (size_t)rows * p.nblk * (kTopkFilterChunk + 2) * 4;
    return bytes;
}

hipError_t launch_fill_u32(uint32_t *p, int64_t n, uint32_t v, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)blocks), dim3(256), 0, st, p, n, v);
    return hipGetLastError();
}

hipError_t launch_topk(int B, int Tq, int N, int m, int k, int64_t q_pos0, const float *scores, void *scratch,
                       int32_t *out, hipStream_t st) {
    const int64_t rows = (int64_t)B * Tq;
    const TopkPlan p = topk_plan(rows, N);
    uint32_t *hist = (uint32_t *)scratch;
    if (!p.filter) {
        static const hipError_t attr = hipFuncSetAttribute(
            (const void *)k_topk_rows<true>, hipFuncAttributeMaxDynamicSharedMemorySize, kTopkLdsKeys * 4);
        if (attr != hipSuccess) return attr;
        const size_t lds = (size_t)(N > 0 ? N : 1) * sizeof(uint32_t);
        hipLaunchKernelGGL(k_topk_rows<true>, dim3((unsigned)rows), dim3(kNT), lds, st, Tq, N, m, k, q_pos0, scores,
                           hist, out);
        return hipGetLastError();
    }
    int32_t *seg = (int32_t *)(hist + rows * kTopkBins);
    int32_t *counts = seg + rows * p.nblk * kTopkFilterChunk;
    if (N > 0) {
        hipLaunchKernelGGL(k_topk_filter, dim3((unsigned)(rows * p.nblk)), dim3(kFT), 0, st, Tq, N, m, k, q_pos0,
                           (int)p.nblk, scores, hist, seg, counts);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const size_t lds = (size_t)(2 * (p.nblk + 1) + 2 * k + 2 * kTopkFinalCand) * 4;
    static const hipError_t attr =
        hipFuncSetAttribute((const void *)k_topk_final, hipFuncAttributeMaxDynamicSharedMemorySize, 144 * 1024);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(k_topk_final, dim3((unsigned)rows), dim3(kNT), lds, st, Tq, N, m, k, q_pos0, (int)p.nblk,
                       scores, hist, seg, counts, out);
    return hipGetLastError();
}

}  // namespace csa
