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
// Many queries with rows of up to kTopkCompactMax scores (prefill chunks):
// one workgroup per query holds its row in registers, packs the pairs of digit
// >= D into LDS and resolves them there.  Few queries (decode) or long rows
// (1M context): the row is
// cut into chunks of kTopkFilterChunk scores; a workgroup per chunk writes
// the (index, key) pairs of its chunk whose digit is >= D, in index order, to
// a segment of the workspace; then one workgroup per query gathers all
// segments into LDS and resolves them.  Either way the kept set leaves in
// ascending index order through one exchange of per-wavefront totals and
// in-wave ballots, never a sort.
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

// popcount of the bits of m below this lane
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Walk n items in index order; keep those above the prefix and the first
// `rem` equal to it; emit(pos, i) for the kept ones.  Wavefront w owns one
// contiguous run of the items: a first pass counts its kept and tied items,
// one exchange of the per-wave totals gives each run its starting position,
// and a second pass places the items with ballots.  sh: 2*NT/64 ints.
template <int NT, class KeyAt, class Emit>
__device__ void ordered_keep(KeyAt key_at, int64_t n, uint32_t prefix, uint32_t mask, int rem, int *sh, Emit emit) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t per = ((n + NW - 1) / NW + 63) / 64 * 64;
    const int64_t s0 = min(n, (int64_t)wv * per), s1 = min(n, s0 + per);
    int gt = 0, eq = 0;
    for (int64_t c = s0; c < s1; c += 64) {
        const int64_t i = c + lane;
        const uint32_t km = i < s1 ? key_at(i) & mask : 0u;
        gt += __popcll(__ballot(i < s1 && km > prefix));
        eq += __popcll(__ballot(i < s1 && km == prefix));
    }
    if (lane == 0) {
        sh[wv] = gt;
        sh[NW + wv] = eq;
    }
    __syncthreads();
    int gt_b = 0, eq_b = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        gt_b += i < wv ? sh[i] : 0;
        eq_b += i < wv ? sh[NW + i] : 0;
    }
    __syncthreads();
    int pos = gt_b + min(eq_b, rem);
    for (int64_t c = s0; c < s1; c += 64) {
        const int64_t i = c + lane;
        const uint32_t km = i < s1 ? key_at(i) & mask : 0u;
        const bool e = i < s1 && km == prefix;
        const uint64_t em = __ballot(e);
        const bool sel = (i < s1 && km > prefix) || (e && eq_b + lanes_below(em) < rem);
        const uint64_t sm = __ballot(sel);
        if (sel) emit(pos + lanes_below(sm), i);
        pos += __popcll(sm);
        eq_b += __popcll(em);
    }
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

struct IdxKey {
    int32_t j;
    uint32_t key;
};

// Exact select straight over a score row in global memory (used only when
// the pairs of digit >= D do not fit in LDS).
__device__ void select_row_global(const float *srow, int64_t nv, int k, Digit d, int32_t *orow, uint32_t *hist,
                                  int *sh, Digit *shd) {
    uint32_t prefix = d.digit << (32 - kTopkBinBits), mask = ~0u << (32 - kTopkBinBits);
    int rem = k - d.above;
    auto key_at = [&](int64_t j) -> uint32_t { return order_key(srow[j]); };
    if (d.at != rem) refine<kNT>(key_at, nv, prefix, mask, rem, hist, sh, shd);
    ordered_keep<kNT>(key_at, nv, prefix, mask, rem, sh, [&](int pos, int64_t j) {
        if (pos < k) orow[pos] = (int32_t)j;
    });
}

// The M pairs of digit >= D sit in LDS in index order: resolve digit D with
// the lower digits and write the kept indices, ascending.
__device__ void select_items(const IdxKey *items, int M, int k, Digit d, int32_t *orow, uint32_t *hist, int *sh,
                             Digit *shd) {
    uint32_t prefix = d.digit << (32 - kTopkBinBits), mask = ~0u << (32 - kTopkBinBits);
    int rem = k - d.above;  // keys of digit D to keep
    auto key_at = [&](int64_t i) -> uint32_t { return items[i].key; };
    if (d.at != rem) refine<kNT>(key_at, M, prefix, mask, rem, hist, sh, shd);
    ordered_keep<kNT>(key_at, M, prefix, mask, rem, sh, [&](int pos, int64_t i) {
        if (pos < k) orow[pos] = items[i].j;
    });
}

// ------------------------------------- rows of up to kNT*KPL scores: one pass
// One workgroup per query.  Wavefront w owns a contiguous run of the row and
// loads it into registers (KPL scores per lane, as 16-byte vectors of four
// consecutive scores) while the digit D is found from the histogram; the
// pairs of digit >= D are then packed into LDS in index order (run offsets
// from one exchange of per-wave counts, in-run offsets from ballots) and
// resolved there.
template <int KPL>
__global__ __launch_bounds__(kNT) void k_topk_compact(int Tq, int N, int m, int k, QPos q_pos0,
                                                      const float *__restrict__ scores,
                                                      const uint32_t *__restrict__ ghist, int32_t *__restrict__ out) {
    extern __shared__ IdxKey items[];  // [kTopkFinalItems]
    __shared__ uint32_t hist[2048];
    __shared__ int sh[2 * kNT / 64];
    __shared__ Digit shd;
    constexpr int NW = kNT / 64;
    constexpr int F4 = KPL / 4;        // 16-byte vectors per lane
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t row = blockIdx.x;
    const int64_t nv = n_visible(q_pos0.at(row / Tq, row % Tq), m, N);
    int32_t *orow = out + row * k;
    if (trivial_row(nv, k, orow)) return;
    const int stride = (int)topk_score_stride(N);
    const float *srow = scores + row * stride;
    const int per = (int)((nv + NW * 256 - 1) / (NW * 256)) * 256;  // run length, <= 64*KPL
    const int s0 = wv * per;
    const int s1 = (int)min((int64_t)s0 + per, nv);
    // unconditional loads (vectors past the row's end reread its last one) so
    // that all F4 are in flight together; positions >= s1 are masked below
    float4 sc[F4];
#pragma unroll
    for (int c = 0; c < F4; ++c) sc[c] = *(const float4 *)(srow + min(s0 + c * 256 + lane * 4, stride - 4));
    const Digit d = find_digit<kNT>(ghist + row * kTopkBins, kTopkBins, k, sh, &shd);
    auto selected = [&](int c, int e, uint32_t &key) -> bool {
        const float4 v = sc[c];
        key = order_key(e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w);
        return s0 + c * 256 + lane * 4 + e < s1 && (key >> (32 - kTopkBinBits)) >= d.digit;
    };
    int cnt = 0;
#pragma unroll
    for (int c = 0; c < F4; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            uint32_t key;
            cnt += __popcll(__ballot(selected(c, e, key)));
        }
    if (lane == 0) sh[NW + wv] = cnt;
    __syncthreads();
    int base = 0, M = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int v = sh[NW + i];
        base += i < wv ? v : 0;
        M += v;
    }
    __syncthreads();
    if (M > kTopkFinalItems || M != d.above + d.at) {
        select_row_global(srow, nv, k, d, orow, hist, sh, &shd);
        return;
    }
#pragma unroll
    for (int c = 0; c < F4; ++c) {
        uint32_t key[4];
        bool sel[4];
        int before = 0, chunk = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sel[e] = selected(c, e, key[e]);
            const uint64_t bm = __ballot(sel[e]);
            before += lanes_below(bm);
            chunk += __popcll(bm);
        }
        int pos = base + before;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (sel[e]) items[pos++] = IdxKey{s0 + c * 256 + lane * 4 + e, key[e]};
        base += chunk;
    }
    __syncthreads();
    select_items(items, M, k, d, orow, hist, sh, &shd);
}

// ----------------------------------------------------- long rows: filter + final
// k_topk_filter: kFT threads per workgroup, nblk workgroups per query.  Each
// workgroup writes the (index, key) pairs of its chunk whose first digit is at
// least D (kept ones and candidates alike) to the chunk's segment, in index
// order, and their number to counts.
// k_topk_final: one workgroup per query gathers the segments into LDS (the
// pairs arrive in index order), resolves the candidates and writes the kept
// indices.  (A kernel boundary separates the two: on this multi-die GPU a
// device-scope fence inside one kernel costs more.)
__global__ __launch_bounds__(kFT) void k_topk_filter(int Tq, int N, int m, int k, QPos q_pos0, int nblk,
                                                     const float *__restrict__ scores,
                                                     const uint32_t *__restrict__ ghist, IdxKey *__restrict__ seg,
                                                     int32_t *__restrict__ counts) {
    __shared__ int sh[kFT / 64];
    __shared__ Digit shd;
    const int64_t row = blockIdx.x / nblk;
    const int blk = blockIdx.x % nblk;
    const int64_t nv = n_visible(q_pos0.at(row / Tq, row % Tq), m, N);
    if (nv <= k) return;
    if ((int64_t)blk * kTopkFilterChunk >= nv) {  // a chunk past the visible entries holds no pair
        if (threadIdx.x == 0) counts[row * nblk + blk] = 0;
        return;
    }
    const int64_t stride = topk_score_stride(N);
    const float *srow = scores + row * stride;
    const int64_t j0 = (int64_t)blk * kTopkFilterChunk + threadIdx.x * kFPT;
    // the chunk's scores (16-byte vectors; past the row's end its last vector
    // is reread and masked) are in flight while the digit is found
    float4 sc[kFPT / 4];
#pragma unroll
    for (int u = 0; u < kFPT / 4; ++u) sc[u] = *(const float4 *)(srow + min(j0 + 4 * u, stride - 4));
    const Digit d = find_digit<kFT>(ghist + row * kTopkBins, kTopkBins, k, sh, &shd);
    uint32_t keys[kFPT];
    uint32_t bits = 0;
#pragma unroll
    for (int u = 0; u < kFPT / 4; ++u) {
        keys[4 * u + 0] = order_key(sc[u].x);
        keys[4 * u + 1] = order_key(sc[u].y);
        keys[4 * u + 2] = order_key(sc[u].z);
        keys[4 * u + 3] = order_key(sc[u].w);
    }
#pragma unroll
    for (int u = 0; u < kFPT; ++u)
        bits |= (uint32_t)(j0 + u < nv && (keys[u] >> (32 - kTopkBinBits)) >= d.digit) << u;
    int total;
    int pos = block_excl_scan<kFT>(__popc(bits), sh, &total);
    IdxKey *sg = seg + (row * nblk + blk) * (int64_t)kTopkFilterChunk;
#pragma unroll
    for (int u = 0; u < kFPT; ++u)
        if ((bits >> u) & 1) sg[pos++] = IdxKey{(int32_t)(j0 + u), keys[u]};
    if (threadIdx.x == 0) counts[row * nblk + blk] = total;
}

__global__ __launch_bounds__(kNT) void k_topk_final(int Tq, int N, int m, int k, QPos q_pos0, int nblk,
                                                    const float *__restrict__ scores,
                                                    const uint32_t *__restrict__ ghist,
                                                    const IdxKey *__restrict__ seg,
                                                    const int32_t *__restrict__ counts, int32_t *__restrict__ out) {
    extern __shared__ IdxKey items[];  // [kTopkFinalItems]
    __shared__ uint32_t hist[2048];
    __shared__ int pre[kNT + 1];       // segment starts (nblk <= 1023)
    __shared__ int sh[2 * kNT / 64];
    __shared__ Digit shd;
    const int64_t row = blockIdx.x;
    const int64_t nv = n_visible(q_pos0.at(row / Tq, row % Tq), m, N);
    int32_t *orow = out + row * k;
    if (trivial_row(nv, k, orow)) return;
    // the segment sizes are fetched alongside the histogram
    const int cnt = (int)threadIdx.x < nblk ? counts[row * nblk + threadIdx.x] : 0;
    const Digit d = find_digit<kNT>(ghist + row * kTopkBins, kTopkBins, k, sh, &shd);
    int M;
    const int x = block_excl_scan<kNT>(cnt, sh, &M);
    if ((int)threadIdx.x <= nblk) pre[threadIdx.x] = (int)threadIdx.x < nblk ? x : M;
    __syncthreads();
    if (M > kTopkFinalItems || M != d.above + d.at) {
        // more pairs than LDS holds
        select_row_global(scores + row * topk_score_stride(N), nv, k, d, orow, hist, sh, &shd);
        return;
    }
    // gather: batches of four pairs per thread, all loads in flight together
    const IdxKey *segr = seg + row * nblk * (int64_t)kTopkFilterChunk;
    for (int i0 = 0; i0 < M; i0 += 4 * kNT) {
        IdxKey v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = min(i0 + u * kNT + (int)threadIdx.x, M - 1);
            int lo = 0, hi = nblk;  // last segment b with pre[b] <= i
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (pre[mid] <= i) lo = mid; else hi = mid;
            }
            v[u] = segr[lo * (int64_t)kTopkFilterChunk + (i - pre[lo])];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = i0 + u * kNT + (int)threadIdx.x;
            if (i < M) items[i] = v[u];
        }
    }
    __syncthreads();
    select_items(items, M, k, d, orow, hist, sh, &shd);
}

// ------------------------------------------------------------------ host side
TopkPlan topk_plan(int64_t rows, int64_t N) {
    TopkPlan p;
    // one pass needs enough queries to spread the score rows over the CUs (one
    // CU streaming a 128 KiB row is slower than eight CUs filtering it)
    p.filter = rows < kTopkCompactMinRows || N > kTopkCompactMax;
    p.nblk = (N + kTopkFilterChunk - 1) / kTopkFilterChunk;
    if (p.nblk < 1) p.nblk = 1;
    return p;
}

// scratch layout: histograms [rows][kTopkBins] u32 (cleared before the
// indexer), then (filter path) counts [rows][nblk] i32 and segments
// [rows][nblk][chunk] of (index, key) pairs
static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

size_t topk_clear_words(int64_t rows, int64_t N) {
    (void)N;
    return (size_t)rows * kTopkBins;
}

size_t topk_scratch_bytes(int64_t rows, int64_t N) {
    const TopkPlan p = topk_plan(rows, N);
    size_t bytes = align256(topk_clear_words(rows, N) * 4);
    if (p.filter) bytes += align256((size_t)rows * p.nblk * 4) + (size_t)rows * p.nblk * kTopkFilterChunk * 8;
    return bytes;
}

hipError_t launch_fill_u32(uint32_t *p, int64_t n, uint32_t v, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)blocks), dim3(256), 0, st, p, n, v);
    return hipGetLastError();
}

template <int KPL>
static hipError_t launch_compact(int64_t rows, int Tq, int N, int m, int k, QPos q_pos0, const float *scores,
                                 const uint32_t *hist, int32_t *out, hipStream_t st) {
    static_assert(KPL * kNT <= kTopkCompactMax, "row longer than the one-pass limit");
    const size_t lds = (size_t)kTopkFinalItems * sizeof(IdxKey);
    static const hipError_t attr =
        hipFuncSetAttribute((const void *)k_topk_compact<KPL>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(k_topk_compact<KPL>, dim3((unsigned)rows), dim3(kNT), lds, st, Tq, N, m, k, q_pos0, scores,
                       hist, out);
    return hipGetLastError();
}

hipError_t launch_topk(int B, int Tq, int N, int m, int k, QPos q_pos0, const float *scores, void *scratch,
                       int32_t *out, hipStream_t st) {
    const int64_t rows = (int64_t)B * Tq;
    const TopkPlan p = topk_plan(rows, N);
    uint32_t *hist = (uint32_t *)scratch;
    if (!p.filter) {
        if (N <= 8 * kNT) return launch_compact<8>(rows, Tq, N, m, k, q_pos0, scores, hist, out, st);
        if (N <= 16 * kNT) return launch_compact<16>(rows, Tq, N, m, k, q_pos0, scores, hist, out, st);
        if (N <= 32 * kNT) return launch_compact<32>(rows, Tq, N, m, k, q_pos0, scores, hist, out, st);
        return launch_compact<64>(rows, Tq, N, m, k, q_pos0, scores, hist, out, st);
    }
    char *base = (char *)scratch + align256(topk_clear_words(rows, N) * 4);
    int32_t *counts = (int32_t *)base;
    IdxKey *seg = (IdxKey *)(base + align256((size_t)rows * p.nblk * 4));
    if (N > 0) {
        hipLaunchKernelGGL(k_topk_filter, dim3((unsigned)(rows * p.nblk)), dim3(kFT), 0, st, Tq, N, m, k, q_pos0,
                           (int)p.nblk, scores, hist, seg, counts);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const size_t lds = (size_t)kTopkFinalItems * sizeof(IdxKey);
    static const hipError_t attr =
        hipFuncSetAttribute((const void *)k_topk_final, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(k_topk_final, dim3((unsigned)rows), dim3(kNT), lds, st, Tq, N, m, k, q_pos0, (int)p.nblk,
                       scores, hist, seg, counts, out);
    return hipGetLastError();
}

}  // namespace csa
