// Per-query top-k over the indexer scores (DeepSeek-V4 overview page,
// section 2.2 step 2: keep only the top-k most relevant compressed entries).
//
// Order: score descending, then entry index ascending, so the kept set is
// unique even with equal scores.  Output: kept indices ascending, -1 padded.
//
// Method: exact radix select on order-preserving 32-bit keys.  The first
// digit (topk_bin: the key's top 13 bits in a window of 2048 bins, keys
// outside the window in the two end bins) is counted by the indexer epilogue
// into a per-query histogram, so no workgroup here rescans a row for it.
// From the histogram the digit D holding the k-th key follows; keys with a
// higher digit are kept, keys with digit D are the candidates, resolved by
// more digits in LDS histograms (the key's remaining 19 bits for an interior
// bin, all 32 for an end bin) and, for keys that are fully equal, by index.
//
// Many queries with rows of up to kTopkCompactMax scores (prefill chunks):
// one workgroup per query, several per CU, reads its row twice (count, then
// pack the pairs of digit >= D into LDS) and resolves the pairs there.  Few
// queries (decode) or long rows (1M context): the row is cut into chunks of
// kTopkFilterChunk scores; a workgroup per chunk writes
// the (index, key) pairs of its chunk whose digit is >= D, in index order, to
// a segment of the workspace; then one workgroup per query gathers all
// segments into LDS and resolves them.  Either way the kept set leaves in
// ascending index order through one exchange of per-wavefront totals and
// in-wave ballots, never a sort.
#include "compress_fold.h"

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

// the least key of first-digit bin b: topk_bin(key) >= b exactly when
// key >= topk_bin_floor(b)
__device__ __forceinline__ uint32_t topk_bin_floor(uint32_t b) {
    return b == 0u ? 0u : (b + kTopkWindow0) << kTopkKeyShift;
}

struct Digit {
    uint32_t digit;
    int above;  // keys in higher bins
    int at;     // keys in the digit's bin
};

// Find D with count(bin > D) < rem <= count(bin >= D) over nbins bins.
template <int NT>
__device__ Digit find_digit(const uint32_t *hist, int nbins, int rem, int *sh, Digit *shd) {
    const int per = nbins >= NT ? nbins / NT : 1;  // bins per thread (threads past nbins hold none)
    const int tid = threadIdx.x;
    const bool holds = tid * per < nbins;
    // (a histogram holding fewer than rem keys has no such digit: then digit 0
    // with nothing above it, so the selection stays inside the row and k)
    if (tid == 0) *shd = Digit{0u, 0, 0};
    int own = 0;
    if (holds)
        for (int q = 0; q < per; ++q) own += (int)hist[tid * per + q];
    int total;
    const int before = block_excl_scan<NT>(own, sh, &total);
    const int incl = total - before;  // keys in bins >= tid*per
    const int excl = incl - own;      // keys in bins >= (tid+1)*per
    if (holds && excl < rem && incl >= rem) {
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

// The selection below the first digit D (the bin of the k-th key): keys of
// a higher bin are kept outright; keys of bin D compare (key & mask) with
// prefix, which the refinement extends digit by digit, and `rem` of those
// equal to it are kept.  An interior bin is one 13-bit key prefix, so its
// keys go on with bits [18:8] and [7:0]; an end bin gathers keys of many
// prefixes and starts again from the top: bits [31:21], [20:10], [9:0].
struct Sel {
    uint32_t D, prefix, mask;
    int rem;
    __device__ static Sel start(const Digit &d, int k) {
        Sel s;
        const bool interior = d.digit > 0u && d.digit < (uint32_t)(kTopkBins - 1);
        s.D = d.digit;
        s.prefix = interior ? (d.digit + kTopkWindow0) << kTopkKeyShift : 0u;
        s.mask = interior ? ~0u << kTopkKeyShift : 0u;
        s.rem = k - d.above;
        return s;
    }
    // 1: kept outright; 0: in bin D and equal to the prefix so far; -1: not kept
    __device__ __forceinline__ int cmp(uint32_t key) const {
        const uint32_t b = topk_bin(key);
        if (b != D) return b > D ? 1 : -1;
        const uint32_t km = key & mask;
        return km > prefix ? 1 : (km == prefix ? 0 : -1);
    }
};

// Narrow bin D down to one full key value (keys key_at(0 .. n-1)).
template <int NT, class KeyAt>
__device__ void refine(KeyAt key_at, int64_t n, Sel &s, uint32_t *hist, int *sh, Digit *shd) {
    const bool interior = s.mask != 0u;
    const int passes = interior ? 2 : 3;
    for (int pass = 0; pass < passes; ++pass) {
        const int shift = interior ? (pass == 0 ? 8 : 0) : (pass == 0 ? 21 : pass == 1 ? 10 : 0);
        const int nbins = interior ? (pass == 0 ? 2048 : 256) : (pass < 2 ? 2048 : 1024);
        for (int i = threadIdx.x; i < nbins; i += NT) hist[i] = 0;
        __syncthreads();
        for (int64_t j = threadIdx.x; j < n; j += NT) {
            const uint32_t key = key_at(j);
            if (s.cmp(key) == 0) atomicAdd(&hist[(key >> shift) & (nbins - 1)], 1u);
        }
        __syncthreads();
        const Digit d = find_digit<NT>(hist, nbins, s.rem, sh, shd);
        s.rem -= d.above;
        s.prefix |= d.digit << shift;
        s.mask |= (uint32_t)(nbins - 1) << shift;
        if (d.at == s.rem) break;  // every key equal to the prefix is kept
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
__device__ void ordered_keep(KeyAt key_at, int64_t n, const Sel &s, int *sh, Emit emit) {
    const int rem = s.rem;
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t per = ((n + NW - 1) / NW + 63) / 64 * 64;
    const int64_t s0 = min(n, (int64_t)wv * per), s1 = min(n, s0 + per);
    int gt = 0, eq = 0;
    for (int64_t c = s0; c < s1; c += 64) {
        const int64_t i = c + lane;
        const int cv = i < s1 ? s.cmp(key_at(i)) : -1;
        gt += __popcll(__ballot(cv == 1));
        eq += __popcll(__ballot(cv == 0));
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
        const int cv = i < s1 ? s.cmp(key_at(i)) : -1;
        const bool e = cv == 0;
        const uint64_t em = __ballot(e);
        const bool sel = cv == 1 || (e && eq_b + lanes_below(em) < rem);
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

// Zero a query's first-digit histogram once nothing reads it any more, so
// that every call leaves the histograms as zero as it needs them: a caller
// that keeps one workspace for calls of one shape clears it only once.
__device__ __forceinline__ void clear_row_hist(uint32_t *h) {
    for (int i = threadIdx.x * 4; i < kTopkBins; i += blockDim.x * 4) *(u32x4 *)(h + i) = u32x4{0u, 0u, 0u, 0u};
}

struct IdxKey {
    int32_t j;
    uint32_t key;
};

// Exact select straight over a score row in global memory (used only when
// the pairs of digit >= D do not fit in LDS).
template <int NT>
__device__ void select_row_global(const float *srow, int64_t nv, int k, Digit d, int32_t *orow, uint32_t *hist,
                                  int *sh, Digit *shd) {
    Sel s = Sel::start(d, k);
    auto key_at = [&](int64_t j) -> uint32_t { return order_key(srow[j]); };
    if (d.at != s.rem) refine<NT>(key_at, nv, s, hist, sh, shd);
    ordered_keep<NT>(key_at, nv, s, sh, [&](int pos, int64_t j) {
        if (pos >= 0 && pos < k) orow[pos] = (int32_t)j;
    });
}

// The M pairs of digit >= D sit in LDS in index order: resolve digit D with
// the lower digits and write the kept indices, ascending.
template <int NT>
__device__ void select_items(const IdxKey *items, int M, int k, Digit d, int32_t *orow, uint32_t *hist, int *sh,
                             Digit *shd) {
    Sel s = Sel::start(d, k);  // keys of digit D to keep: s.rem
    auto key_at = [&](int64_t i) -> uint32_t { return items[i].key; };
    if (d.at != s.rem) refine<NT>(key_at, M, s, hist, sh, shd);
    ordered_keep<NT>(key_at, M, s, sh, [&](int pos, int64_t i) {
        if (pos >= 0 && pos < k) orow[pos] = items[i].j;
    });
}

// ------------------------------------ streaming one pass, several rows per CU
// One workgroup of kST threads per query, the row read twice from memory
// instead of held in registers (the second read mostly from cache), so that
// a workgroup needs few registers and kStreamItems pairs of LDS and several
// rows are selected on one CU at once.  Wavefront w owns a contiguous run of
// the row: a first read counts its pairs of digit >= D, one exchange of the
// counts gives each run its offset, a second read packs the pairs into LDS in
// index order (in-run offsets from ballots), and they are resolved there.
// Rows with more pairs than that take the global select.
constexpr int kST = 512;
constexpr int kStreamItems = 4096;
constexpr int kStreamBatch = 4;  // 16-byte vectors per lane in flight per batch

__global__ __launch_bounds__(kST) void k_topk_stream(int Tq, int N, int m, int k, QPos q_pos0,
                                                     const float *__restrict__ scores,
                                                     uint32_t *__restrict__ ghist, int32_t *__restrict__ out) {
    __shared__ IdxKey items[kStreamItems];
    __shared__ uint32_t hist[2048];
    __shared__ int sh[2 * kST / 64];
    __shared__ Digit shd;
    constexpr int NW = kST / 64;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t row = blockIdx.x;
    const int64_t nv = n_visible(q_pos0.at(row / Tq, row % Tq), m, N);
    int32_t *orow = out + row * k;
    uint32_t *hrow = ghist + row * kTopkBins;
    if (trivial_row(nv, k, orow)) {
        clear_row_hist(hrow);
        return;
    }
    const int stride = (int)topk_score_stride(N);
    const float *srow = scores + row * stride;
    const int per = (int)((nv + NW * 256 - 1) / (NW * 256)) * 256;  // run length (a multiple of 256 scores)
    const int s0 = wv * per;
    const int s1 = (int)min((int64_t)s0 + per, nv);
    const Digit d = find_digit<kST>(hrow, kTopkBins, k, sh, &shd);
    clear_row_hist(hrow);
    const uint32_t kmin = topk_bin_floor(d.digit);  // keys of digit >= D
    // batches of kStreamBatch vectors of four consecutive scores per lane, all
    // in flight together (past the row's end the last vector is reread and
    // masked); f(c, e, selected, key) per score in index order of (c, lane, e)
    auto for_run = [&](auto f) {
        for (int b0 = s0; b0 < s1; b0 += kStreamBatch * 256) {
            float4 v[kStreamBatch];
#pragma unroll
            for (int u = 0; u < kStreamBatch; ++u)
                v[u] = *(const float4 *)(srow + min(b0 + u * 256 + lane * 4, stride - 4));
#pragma unroll
            for (int u = 0; u < kStreamBatch; ++u) {
                const int c = b0 + u * 256;
                if (c >= s1) break;  // (uniform)
                f(c, v[u]);
            }
        }
    };
    auto select4 = [&](int c, const float4 &v, uint32_t (&key)[4], bool (&sel)[4]) {
        key[0] = order_key(v.x);
        key[1] = order_key(v.y);
        key[2] = order_key(v.z);
        key[3] = order_key(v.w);
#pragma unroll
        for (int e = 0; e < 4; ++e) sel[e] = c + lane * 4 + e < s1 && key[e] >= kmin;
    };
    int cnt = 0;
    for_run([&](int c, const float4 &v) {
        uint32_t key[4];
        bool sel[4];
        select4(c, v, key, sel);
#pragma unroll
        for (int e = 0; e < 4; ++e) cnt += __popcll(__ballot(sel[e]));
    });
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
    if (M > kStreamItems || M != d.above + d.at) {
        select_row_global<kST>(srow, nv, k, d, orow, hist, sh, &shd);
        return;
    }
    for_run([&](int c, const float4 &v) {
        uint32_t key[4];
        bool sel[4];
        select4(c, v, key, sel);
        int before = 0, chunk = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint64_t bm = __ballot(sel[e]);
            before += lanes_below(bm);
            chunk += __popcll(bm);
        }
        int pos = base + before;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (sel[e]) items[pos++] = IdxKey{c + lane * 4 + e, key[e]};
        base += chunk;
    });
    __syncthreads();
    select_items<kST>(items, M, k, d, orow, hist, sh, &shd);
}

// ----------------------------------------------------- long rows: filter + final
// k_topk_filter: kFT threads per workgroup, nblk workgroups per query.  Each
// workgroup writes the (index, key) pairs of its chunk whose first digit is at
// least D (kept ones and candidates alike) to the chunk's segment, in index
// order, and their number to counts.
// k_topk_final: one workgroup per query gathers the segments into LDS (the
// pairs arrive in index order), resolves the candidates, writes the kept
// indices and zeroes the row's histogram.  (A kernel boundary separates the
// two: on this multi-die GPU a device-scope fence inside one kernel costs
// more.)  Workgroups past the filter's own (filter_blocks) run extra work of
// the same call that neither reads nor writes what the filter touches: a
// decode step's compression, which then needs no launch of its own.
struct NoExtra {
    __device__ __forceinline__ void run(int) const {}
};

template <class Extra>
__global__ __launch_bounds__(kFT) void k_topk_filter(int Tq, int N, int m, int k, QPos q_pos0, int nblk,
                                                     const float *__restrict__ scores,
                                                     const uint32_t *__restrict__ ghist, IdxKey *__restrict__ seg,
                                                     int32_t *__restrict__ counts, int filter_blocks, Extra extra) {
    __shared__ int sh[kFT / 64];
    __shared__ Digit shd;
    if ((int)blockIdx.x >= filter_blocks) {  // (uniform per workgroup: before any barrier)
        extra.run((int)blockIdx.x - filter_blocks);
        return;
    }
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
    const uint32_t kmin = topk_bin_floor(d.digit);  // keys of digit >= D
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
        bits |= (uint32_t)(j0 + u < nv && keys[u] >= kmin) << u;
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
                                                    uint32_t *__restrict__ ghist,
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
    uint32_t *hrow = ghist + row * kTopkBins;
    if (trivial_row(nv, k, orow)) {
        clear_row_hist(hrow);
        return;
    }
    // the segment sizes are fetched alongside the histogram
    const int cnt = (int)threadIdx.x < nblk ? counts[row * nblk + threadIdx.x] : 0;
    const Digit d = find_digit<kNT>(hrow, kTopkBins, k, sh, &shd);
    clear_row_hist(hrow);
    int M;
    const int x = block_excl_scan<kNT>(cnt, sh, &M);
    if ((int)threadIdx.x <= nblk) pre[threadIdx.x] = (int)threadIdx.x < nblk ? x : M;
    __syncthreads();
    if (M > kTopkFinalItems || M != d.above + d.at) {
        // more pairs than LDS holds
        select_row_global<kNT>(scores + row * topk_score_stride(N), nv, k, d, orow, hist, sh, &shd);
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
    select_items<kNT>(items, M, k, d, orow, hist, sh, &shd);
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

// extra_blocks workgroups of `extra` follow the filter's (filter path only)
template <class Extra>
static hipError_t launch_topk_x(int B, int Tq, int N, int m, int k, QPos q_pos0, const float *scores, void *scratch,
                                int32_t *out, hipStream_t st, const Extra &extra, int64_t extra_blocks) {
    const int64_t rows = (int64_t)B * Tq;
    const TopkPlan p = topk_plan(rows, N);
    uint32_t *hist = (uint32_t *)scratch;
    if (!p.filter) {
        if (extra_blocks) return hipErrorInvalidValue;
        hipLaunchKernelGGL(k_topk_stream, dim3((unsigned)rows), dim3(kST), 0, st, Tq, N, m, k, q_pos0, scores, hist,
                           out);
        return hipGetLastError();
    }
    char *base = (char *)scratch + align256(topk_clear_words(rows, N) * 4);
    int32_t *counts = (int32_t *)base;
    IdxKey *seg = (IdxKey *)(base + align256((size_t)rows * p.nblk * 4));
    if (N > 0) {
        const int64_t fb = rows * p.nblk;
        hipLaunchKernelGGL(k_topk_filter<Extra>, dim3((unsigned)(fb + extra_blocks)), dim3(kFT), 0, st, Tq, N, m, k,
                           q_pos0, (int)p.nblk, scores, hist, seg, counts, (int)fb, extra);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    } else if (extra_blocks) {
        return hipErrorInvalidValue;
    }
    const size_t lds = (size_t)kTopkFinalItems * sizeof(IdxKey);
    static const hipError_t attr =
        hipFuncSetAttribute((const void *)k_topk_final, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(k_topk_final, dim3((unsigned)rows), dim3(kNT), lds, st, Tq, N, m, k, q_pos0, (int)p.nblk,
                       scores, hist, seg, counts, out);
    return hipGetLastError();
}

hipError_t launch_topk(int B, int Tq, int N, int m, int k, QPos q_pos0, const float *scores, void *scratch,
                       int32_t *out, hipStream_t st) {
    return launch_topk_x(B, Tq, N, m, k, q_pos0, scores, scratch, out, st, NoExtra{}, 0);
}

template <typename T>
static hipError_t launch_topk_folded_t(int B, int Tq, int N, int m, int k, QPos q_pos0, const float *scores,
                                       void *scratch, int32_t *out, hipStream_t st, const FoldedCompress &c) {
    int tpr, slices;
    if (!compress_partition(c.d, c.m, 16 / (int)sizeof(T), &tpr, &slices)) return hipErrorInvalidValue;
    if (c.ragged) {
        const RaggedCompressBlocks<T> x{c.m, c.d, tpr, slices, c.pos, (const T *)c.raw, c.raw_bs, c.logits,
                                        c.log_bs, c.ring, (T *)c.out, c.omap, c.out_rows};
        return launch_topk_x(B, Tq, N, m, k, q_pos0, scores, scratch, out, st, x, (int64_t)c.B * slices);
    }
    const CompressBlocks<T> x{c.G, c.m, c.d, tpr, slices, (const T *)c.raw, c.raw_bs, c.logits, c.log_bs,
                              (T *)c.out, c.out_bs};
    return launch_topk_x(B, Tq, N, m, k, q_pos0, scores, scratch, out, st, x, (int64_t)c.B * c.G * slices);
}

hipError_t launch_topk_folded(int B, int Tq, int N, int m, int k, QPos q_pos0, const float *scores, void *scratch,
                              int32_t *out, hipStream_t st, const FoldedCompress &fc) {
    if (fc.dt == 0) return launch_topk_folded_t<float>(B, Tq, N, m, k, q_pos0, scores, scratch, out, st, fc);
    return launch_topk_folded_t<bf16_t>(B, Tq, N, m, k, q_pos0, scores, scratch, out, st, fc);
}

}  // namespace csa
