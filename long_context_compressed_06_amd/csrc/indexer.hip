// Lightning indexer (DeepSeek-V4 overview page, section 2.2 step 2):
//     s[t, j] = sum_h w[t, h] * ReLU(qI[t, h, :] . kI[j, :])
// for every entry j visible to query t; invisible entries get -inf.
//
// Mapping.  A query's entries are read in batches of four 16-entry tiles,
// dealt round-robin to the query's wavefronts (so that they sweep the keys
// front to back together).
// The query's index heads sit in registers as the MFMA A operand (M = 16
// heads per block, K = d_I); each 16-entry tile of index keys is streamed
// from HBM straight into registers as the B operand (N = 16 entries), so
// every key byte is read exactly once with 16-byte loads that cover whole
// rows.  The 16x16 output tile holds four heads per lane for one entry: the
// ReLU, the head weight and the head sum happen in registers, and two
// cross-lane exchanges finish the sum over the four lane groups.  Keys are
// read with non-temporal loads in batches of UNROLL tiles, double-buffered so
// one batch is in flight while the previous one is scored.
//
// Optionally (hist != nullptr) the epilogue also counts every visible score
// by the top 11 bits of its order-preserving key (the first radix digit of
// the top-k selection): per-wave LDS histograms, flushed to the query's
// global histogram with one atomic per non-empty bin.
#include "kernels.h"

namespace csa {

template <typename T, int DI, int MB>
__global__ __launch_bounds__(256) void k_index_scores(int Tq, int N, int HI, int m, QPos q_pos0, int64_t n_items,
                                                       int chunks_per_row,
                                                       const T *__restrict__ qI, const float *__restrict__ w,
                                                       const T *__restrict__ kI, int64_t k_bs,
                                                       float *__restrict__ scores, int64_t s_stride,
                                                       float *__restrict__ scores2, uint32_t *__restrict__ hist) {
    using E = Elem<T>;
    constexpr int KS = DI / E::KSTEP;
    constexpr int UNROLL = 4;
    __shared__ uint32_t whist[4][kTopkBins];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t item = (int64_t)blockIdx.x * 4 + wv;
    if (hist) {
        for (int i = lane; i < kTopkBins; i += 64) whist[wv][i] = 0;
    }
    if (item >= n_items) return;
    const int64_t row = item / chunks_per_row;
    const int chunk = (int)(item % chunks_per_row);
    const int64_t b = row / Tq, ti = row % Tq;
    const int64_t nv = n_visible(q_pos0.at(b, ti), m, N);
    const int g = lane >> 4, c = lane & 15;

    typename E::frag a[MB][KS];
    float wgt[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int head = mb * 16 + c;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const typename E::frag v = E::load(qI + (row * HI + min(head, HI - 1)) * DI + ks * E::KSTEP + g * E::KPL);
            a[mb][ks] = head < HI ? v : E::zero();
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int hh = mb * 16 + 4 * g + e;
            const float wv_ = w[row * HI + min(hh, HI - 1)];
            wgt[mb][e] = hh < HI ? wv_ : 0.f;
        }
    }

    const T *kb = kI + b * k_bs + g * E::KPL;
    float *srow = scores + row * s_stride;
    float *srow2 = scores2 ? scores2 + row * (int64_t)N : nullptr;
    constexpr int BATCH = 16 * UNROLL;  // entries per batch of tiles
    // the row's batches are dealt round-robin to its chunks_per_row waves, so
    // that together they sweep the keys front to back
    const int64_t j_lo = (int64_t)chunk * BATCH;
    const int64_t j_hi = N;
    const int64_t jstep = (int64_t)chunks_per_row * BATCH;

    if (nv == 0) {  // nothing visible: the wave's batches are all -inf
        for (int64_t j0 = j_lo; j0 < j_hi; j0 += jstep)
            for (int64_t j = j0 + lane; j < min(j0 + BATCH, j_hi); j += 64) {
                srow[j] = -INFINITY;
                if (srow2) srow2[j] = -INFINITY;
            }
    } else {
    // one batch: UNROLL tiles of 16 index keys, straight from HBM to registers.
    // Loads are unconditional so the compiler can wait for exactly one batch:
    // lanes past the visible entries reread the last visible row.
    const int64_t j_last = nv - 1;
    auto load_batch = [&](int64_t j0, typename E::frag (&bf)[UNROLL][KS]) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            int64_t jr = j0 + u * 16 + c;
            jr = jr < j_last ? jr : j_last;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) bf[u][ks] = E::load_nt(kb + jr * DI + ks * E::KSTEP);
        }
    };
    auto score_batch = [&](int64_t j0, const typename E::frag (&bf)[UNROLL][KS]) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t j = j0 + u * 16 + c;
            floatx4 acc[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) acc[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) acc[mb] = E::mma(a[mb][ks], bf[u][ks], acc[mb]);
            float s = 0.f;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int e = 0; e < 4; ++e) s += wgt[mb][e] * fmaxf(acc[mb][e], 0.f);
            s += __shfl_xor(s, 16);
            s += __shfl_xor(s, 32);
            if (g == 0 && j < j_hi) {
                srow[j] = j < nv ? s : -INFINITY;
                if (srow2) srow2[j] = j < nv ? s : -INFINITY;
            }
            if (hist && g == 0 && j < j_hi && j < nv)
                atomicAdd(&whist[wv][topk_bin(order_key(s))], 1u);
        }
    };
    // double-buffered: the next batch is in flight while this one is scored
    typename E::frag b0[UNROLL][KS], b1[UNROLL][KS];
    if (j_lo < j_hi) load_batch(j_lo, b0);
    for (int64_t j0 = j_lo; j0 < j_hi; j0 += 2 * jstep) {
        load_batch(j0 + jstep, b1);
        score_batch(j0, b0);
        load_batch(j0 + 2 * jstep, b0);
        if (j0 + jstep < j_hi) score_batch(j0 + jstep, b1);
    }
    }
    if (hist) {
        // LDS operations of one wave complete in order: the counts are final here
        uint32_t *grow = hist + row * kTopkBins;
        for (int i = lane; i < kTopkBins; i += 64) {
            const uint32_t v = whist[wv][i];
            if (v) atomicAdd(&grow[i], v);
        }
    }
}

// ---------------------------------------------------------------------------
// bf16 keys: LDS-DMA streaming.
//
// One workgroup of kIdxWaves wavefronts works on one query; a query's 16-entry
// key tiles are dealt round-robin to the wavefronts of its workgroups.  Each
// wavefront streams its tiles HBM -> LDS with global_load_lds_dwordx4 into a
// private ring of kIdxStages tiles (no VGPRs held by loads in flight, and each
// instruction reads one contiguous KiB).  Within every key row the 16-byte
// chunks are stored XOR-swizzled by the row, so that the MFMA B-operand reads
// (ds_read_b128: 16 rows, one chunk each) hit 16 distinct bank groups.  The
// query's index heads are staged once per workgroup through LDS into the MFMA
// A operand; the epilogue (ReLU * w, head sum, score store, optional first
// top-k digit count) is the same as above, with one LDS histogram per
// workgroup.
constexpr int kIdxWaves = 4;

template <int DI>
struct IdxDma {
    static constexpr int RB = DI * 2;        // bytes per key row
    static constexpr int CPR = RB / 16;      // 16-byte chunks per row
    static constexpr int TB = 16 * RB;       // bytes per 16-row tile
    static constexpr int IPT = TB / 1024;    // DMA instructions per tile
    static constexpr int RPS = 16 / CPR;     // consecutive rows sharing one swizzle
    static constexpr int STAGES = 8;         // ring slots per wavefront
    static constexpr int RING = kIdxWaves * STAGES * TB;
    static constexpr int QS = 64 * DI * 2;   // staged index query (up to 64 heads)
    static constexpr int LDS = RING + QS + kTopkBins * 4 + kMaxPagesPerSeq * 4;  // (+ page list, paged caches)
    // chunk position of row r's chunk ch (an involution, so it also maps back)
    static __device__ __forceinline__ int swz(int r, int ch) { return ch ^ ((r / RPS) % CPR); }
};

// 16 bytes per lane from `src` into LDS at lds_addr + 16 * lane, non-temporal
// (the keys are read once).  Inline assembly keeps the compiler from draining
// the loads in flight before every LDS read; completion is awaited explicitly.
// One wait state separates the M0 write from the LDS-DMA instruction.
__device__ __forceinline__ void lds_dma16_nt(uint32_t lds_addr, const void *src) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(lds_addr), "v"(src)
                 : "memory", "m0");
}
// The same from a wave-uniform base address in scalar registers plus a 32-bit
// per-lane byte offset.  Five wait states before the load: the base may have
// just been written by the vector unit (readfirstlane), which the code
// generator does not track into inline assembly.
__device__ __forceinline__ void lds_dma16_nt_s(uint32_t lds_addr, uint32_t voff, uint64_t base) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(lds_addr), "v"(voff),
                 "s"(base)
                 : "memory", "m0");
}

// max(x, 0) on the bit pattern: negative floats are negative integers, so one
// integer max (no NaN canonicalisation of the MFMA result first)
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// sum over the four 16-lane groups (each lane gets the sum for its l % 16)
__device__ __forceinline__ float sum_lane_groups(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

template <int DI, int MB, bool PAGED>
__global__ __launch_bounds__(kIdxWaves * 64) void k_index_dma(int Tq, int N, int HI, int m, QPos q_pos0,
                                                               int blocks_per_row, const bf16_t *__restrict__ qI,
                                                               const float *__restrict__ w,
                                                               const bf16_t *__restrict__ kI, RowMap kl,
                                                               float *__restrict__ scores, int64_t s_stride,
                                                               float *__restrict__ scores2,
                                                               uint32_t *__restrict__ hist) {
    using S = IdxDma<DI>;
    constexpr int KS = DI / 32;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    unsigned char *ring = lds;
    bf16_t *qs = (bf16_t *)(lds + S::RING);
    uint32_t *bh = (uint32_t *)(lds + S::RING + S::QS);
    int32_t *pl = (int32_t *)(lds + S::RING + S::QS + kTopkBins * 4);  // the query's pages (paged caches)

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // (uniform: keeps tile logic scalar)
    const int g = lane >> 4, c = lane & 15;
    const int rank = xcd_rank(gridDim.x);
    int64_t row = rank / blocks_per_row;
    int part = rank % blocks_per_row, parts = blocks_per_row;
    if (q_pos0.pos && !ragged_share(q_pos0.pos, (int)(gridDim.x / blocks_per_row), m, N, gridDim.x, rank, &row, &part,
                                    &parts))
        return;  // (ragged rows: workgroups shared by visible tiles; uniform per workgroup)
    const int64_t b = row / Tq, ti = row % Tq;
    const int64_t nv = n_visible(q_pos0.at(b, ti), m, N);
    const int wpr = parts * kIdxWaves;                // wavefronts per query
    const int gw = part * kIdxWaves + wv;             // this wavefront's rank
    const int tiles = (N + 15) / 16;
    const int vtiles = (int)((nv + 15) / 16);
    const int n_all = tiles > gw ? (tiles - gw + wpr - 1) / wpr : 0;    // tiles of this wavefront
    const int n_vis = vtiles > gw ? (vtiles - gw + wpr - 1) / wpr : 0;  // ... holding visible entries

    // ---- DMA of one tile into ring slot `slot`.  Lane addresses step by a
    // fixed stride from tile to tile; in the tile that holds the last visible
    // entry, rows past it reread that entry's row (their scores are masked).
    const bf16_t *kb = kI + (PAGED ? 0 : b * kl.bstride);
    unsigned char *my_ring = ring + wv * S::STAGES * S::TB;
    const uint32_t ring_addr = (uint32_t)(uintptr_t)my_ring;
    // A whole tile (16 rows, contiguous in memory: pages are multiples of 16
    // rows) is one wave-uniform base address plus a fixed byte offset per lane.
    uint32_t voff[S::IPT];
#pragma unroll
    for (int ip = 0; ip < S::IPT; ++ip) {
        const int byte = ip * 1024 + lane * 16;  // within the tile
        const int r = byte / S::RB, pos = (byte % S::RB) / 16;
        voff[ip] = (uint32_t)((r * DI + S::swz(r, pos) * 8) * 2);
    }
    // paged: the page of the next tile to issue, read from LDS one issue ahead
    // (so no issue waits on its own page lookup)
    int32_t pg_next = 0;
    auto page_entry = [&](int i) -> int32_t {
        const int64_t t = gw + (int64_t)i * wpr;
        return pl[min((t * 16) >> kl.pshift, (int64_t)kMaxPagesPerSeq - 1)];
    };
    auto issue = [&](int i) {
        const int t = gw + i * wpr;
        const int slot = i % S::STAGES;
        const bool whole = (int64_t)t * 16 + 16 <= nv;
        // earlier reads of the slot (and the page lookup) are done
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        // first row of the tile: the pool row (paged) or the row in the sequence
        int64_t row0 = (int64_t)t * 16;
        if constexpr (PAGED) {
            const int64_t pg = (uint32_t)__builtin_amdgcn_readfirstlane(pg_next);
            row0 = (pg << kl.pshift) | (row0 & ((1 << kl.pshift) - 1));
            if (i + 1 < n_vis) pg_next = page_entry(i + 1);
        }
        const uint32_t lds0 = __builtin_amdgcn_readfirstlane(ring_addr + slot * S::TB);
        if (whole) {
            // (wave-uniform; readfirstlane makes it scalar for the compiler too)
            const uint64_t b64 = (uint64_t)((PAGED ? kI : kb) + row0 * DI);
            const uint64_t base = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b64 >> 32)) << 32) |
                                  (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b64);
#pragma unroll
            for (int ip = 0; ip < S::IPT; ++ip) lds_dma16_nt_s(lds0 + ip * 1024, voff[ip], base);
        } else {
            // the tile holding the last visible entry: rows past it reread that entry
#pragma unroll
            for (int ip = 0; ip < S::IPT; ++ip) {
                const int byte = ip * 1024 + lane * 16;
                const int r = byte / S::RB, pos = (byte % S::RB) / 16;
                const int64_t rr = min((int64_t)t * 16 + r, nv - 1) - (int64_t)t * 16;
                const bf16_t *src = (PAGED ? kI : kb) + (row0 + rr) * DI + S::swz(r, pos) * 8;
                lds_dma16_nt(lds0 + ip * 1024, src);
            }
        }
    };

    // ---- the head weights, then the index query staged in LDS (each
    // thread's loads issued together, from clamped positions: one memory
    // round trip for all of them) and the histogram cleared
    float wgt[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) wgt[mb][e] = w[row * HI + min(mb * 16 + 4 * g + e, HI - 1)];
    const int n_pages = PAGED ? (int)min((nv + (1 << kl.pshift) - 1) >> kl.pshift, (int64_t)kl.pstride) : 0;
    PageStage<kIdxWaves * 64> pages;
    if constexpr (PAGED) pages.load(kl, b, n_pages);
    {
        constexpr int kQU = (16 * MB * DI / 8 + kIdxWaves * 64 - 1) / (kIdxWaves * 64);
        const int nq = HI * DI / 8;
        u32x4 qv[kQU];
#pragma unroll
        for (int u = 0; u < kQU; ++u)
            qv[u] = *(const u32x4 *)(qI + row * HI * DI + min((int)threadIdx.x + u * kIdxWaves * 64, nq - 1) * 8);
#pragma unroll
        for (int u = 0; u < kQU; ++u) {
            const int i = (int)threadIdx.x + u * kIdxWaves * 64;
            if (i < nq) *(u32x4 *)(qs + i * 8) = qv[u];
        }
    }
    if (hist)
        for (int i = threadIdx.x; i < kTopkBins; i += kIdxWaves * 64) bh[i] = 0;
    if constexpr (PAGED) pages.store(kl, pl, n_pages);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (mb * 16 + 4 * g + e >= HI) wgt[mb][e] = 0.f;
    __syncthreads();
    bf16x8 a[MB][KS];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int head = mb * 16 + c;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            bf16x8 v = *(const bf16x8 *)(qs + min(head, HI - 1) * DI + ks * 32 + g * 8);
            if (head >= HI) v = Elem<bf16_t>::zero();
            a[mb][ks] = v;
        }
    }
    // (issued after the barrier above, which waits for every load in flight)
    if constexpr (PAGED)
        if (n_vis > 0) pg_next = page_entry(0);
    for (int i = 0; i < S::STAGES - 1 && i < n_vis; ++i) issue(i);

    float *srow = scores + row * s_stride;
    float *srow2 = scores2 ? scores2 + row * (int64_t)N : nullptr;
    for (int i = 0; i < n_vis; ++i) {
        if (i + S::STAGES - 1 < n_vis) {
            issue(i + S::STAGES - 1);
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"((S::STAGES - 1) * S::IPT) : "memory");
        } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        const unsigned char *tile = my_ring + (i % S::STAGES) * S::TB;
        bf16x8 kf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            kf[ks] = *(const bf16x8 *)(tile + c * S::RB + S::swz(c, ks * 4 + g) * 16);
        floatx4 acc[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mb][ks], kf[ks], acc[mb], 0, 0, 0);
        float sc = 0.f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int e = 0; e < 4; ++e) sc += wgt[mb][e] * relu(acc[mb][e]);
        sc = sum_lane_groups(sc);
        const int64_t j = (int64_t)(gw + i * wpr) * 16 + c;
        if (g == 0 && j < N) {
            const float v = j < nv ? sc : -INFINITY;
            srow[j] = v;
            if (srow2) srow2[j] = v;
            if (hist && j < nv) atomicAdd(&bh[topk_bin(order_key(sc))], 1u);
        }
    }
    // tiles with no visible entry
    for (int i = n_vis; i < n_all; ++i) {
        const int64_t j = (int64_t)(gw + i * wpr) * 16 + lane;
        if (lane < 16 && j < N) {
            srow[j] = -INFINITY;
            if (srow2) srow2[j] = -INFINITY;
        }
    }
    if (hist) {
        __syncthreads();
        uint32_t *grow = hist + row * kTopkBins;
        for (int i = threadIdx.x; i < kTopkBins; i += kIdxWaves * 64) {
            const uint32_t v = bh[i];
            if (v) atomicAdd(&grow[i], v);
        }
    }
}

template <int DI, int MB, bool PAGED>
static hipError_t launch_dma_p(int B, int Tq, int N, int HI, int m, QPos q_pos0, const void *qI, const float *w,
                               const void *kI, RowMap k_bs, float *scores, int64_t s_stride, float *scores2,
                               uint32_t *hist, hipStream_t st) {
    using S = IdxDma<DI>;
    constexpr int lds = PAGED ? S::LDS : S::LDS - kMaxPagesPerSeq * 4;  // (the page list: paged keys only)
    static const hipError_t attr = hipFuncSetAttribute((const void *)k_index_dma<DI, MB, PAGED>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (attr != hipSuccess) return attr;
    const int64_t rows = (int64_t)B * Tq;
    const int64_t tiles = (N + 15) / 16;
    // one workgroup per CU in total when there are few queries, at least one per query
    int64_t bpr = (256 + rows - 1) / rows;
    const int64_t max_bpr = (tiles + kIdxWaves - 1) / kIdxWaves;
    if (bpr > max_bpr) bpr = max_bpr;
    if (bpr < 1) bpr = 1;
    hipLaunchKernelGGL((k_index_dma<DI, MB, PAGED>), dim3((unsigned)(rows * bpr)), dim3(kIdxWaves * 64), lds, st,
                       Tq, N, HI, m, q_pos0, (int)bpr, (const bf16_t *)qI, w, (const bf16_t *)kI, k_bs, scores,
                       s_stride, scores2, hist);
    return hipGetLastError();
}

// paging is a template parameter: the contiguous kernel carries no page-table code
template <int DI, int MB>
static hipError_t launch_dma(int B, int Tq, int N, int HI, int m, QPos q_pos0, const void *qI, const float *w,
                             const void *kI, RowMap k_bs, float *scores, int64_t s_stride, float *scores2,
                             uint32_t *hist, hipStream_t st) {
    if (k_bs.ptab)
        return launch_dma_p<DI, MB, true>(B, Tq, N, HI, m, q_pos0, qI, w, kI, k_bs, scores, s_stride, scores2, hist,
                                          st);
    return launch_dma_p<DI, MB, false>(B, Tq, N, HI, m, q_pos0, qI, w, kI, k_bs, scores, s_stride, scores2, hist, st);
}

template <typename T, int DI, int MB>
static hipError_t launch_t(int B, int Tq, int N, int HI, int m, QPos q_pos0, const void *qI, const float *w,
                           const void *kI, RowMap k_bs, float *scores, int64_t s_stride, float *scores2, uint32_t *hist, hipStream_t st) {
    const int64_t rows = (int64_t)B * Tq;
    const int64_t batches = (N + 63) / 64;  // batches of four 16-entry tiles
    // aim for ~2048 wavefronts in flight (8 per CU) when there are few queries
    int64_t chunks = (2048 + rows - 1) / rows;
    if (chunks > batches) chunks = batches;
    if (chunks < 1) chunks = 1;
    const int64_t items = rows * chunks;
    const int64_t blocks = (items + 3) / 4;
    hipLaunchKernelGGL((k_index_scores<T, DI, MB>), dim3((unsigned)blocks), dim3(256), 0, st, Tq, N, HI, m, q_pos0,
                       items, (int)chunks, (const T *)qI, w, (const T *)kI, k_bs.bstride, scores, s_stride,
                       scores2, hist);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// bf16 keys, many queries (prefill chunks): query-blocked.
//
// One workgroup of kPreWaves wavefronts serves kPreWaves consecutive queries
// of one sequence, one query per wavefront, so every key tile staged in LDS
// feeds kPreWaves queries (a decode-style kernel would stream the keys once
// per query).  Each wavefront keeps its query's index heads in registers as
// the MFMA A operand and computes a 64-entry x H_I tile per step: 4 K-steps x
// 4 entry blocks x MB head blocks of v_mfma_f32_16x16x32_bf16, reading the
// key fragments (B operand) from the shared LDS tile; the epilogue is the
// decode kernel's (ReLU, head weights, head sum across lane groups), with one
// LDS histogram per query for the first top-k digit.  Key tiles of 64 rows
// stream HBM -> LDS by LDS-DMA with kPreStages tiles in flight, rows
// XOR-swizzled as in k_index_dma.  Entries past a query's visible count are
// -inf; tiles past every query of the workgroup are not computed.
constexpr int kPreWaves = 8;
constexpr int kPreMinQueries = 64;  // queries per sequence from which the query-blocked kernel is used
constexpr int kPreRows = 128;      // entries per key tile
static_assert(kPreRows % 64 == 0, "epilogues take four 16-entry blocks at a time");
constexpr int kPreStages = 3;

template <int DI>
struct IdxPre {
    static constexpr int RB = DI * 2;                 // bytes per key row
    static constexpr int CPR = RB / 16;               // 16-byte chunks per row
    static constexpr int RPS = 16 / CPR;              // consecutive rows sharing one swizzle
    static constexpr int TB = kPreRows * RB;          // bytes per key tile
    static constexpr int IPT = TB / 1024;             // DMA instructions per tile
    static constexpr int LDS = kPreStages * TB + kPreWaves * kTopkBins * 4;
    static __device__ __forceinline__ int swz(int r, int ch) { return ch ^ ((r / RPS) % CPR); }
};

template <int DI, int MB>
__global__ __launch_bounds__(kPreWaves * 64) void k_index_prefill(int Tq, int N, int HI, int m, QPos q_pos0,
                                                                   int blocks_per_seq, const bf16_t *__restrict__ qI,
                                                                   const float *__restrict__ w,
                                                                   const bf16_t *__restrict__ kI, int64_t k_bs,
                                                                   float *__restrict__ scores, int64_t s_stride,
                                                                   float *__restrict__ scores2,
                                                                   uint32_t *__restrict__ hist) {
    using S = IdxPre<DI>;
    constexpr int KS = DI / 32;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    unsigned char *ring = lds;
    uint32_t *qh = (uint32_t *)(lds + kPreStages * S::TB);  // [kPreWaves][kTopkBins]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c = lane & 15;
    const int64_t b = blockIdx.x / blocks_per_seq;
    const int q0 = (blockIdx.x % blocks_per_seq) * kPreWaves;  // first query of the workgroup
    const int ti = q0 + wv;
    const bool on = ti < Tq;
    const int64_t row = b * Tq + min(ti, Tq - 1);
    const int64_t nv = on ? n_visible(q_pos0.at(b, ti), m, N) : 0;
    // visible entries of the workgroup's last query bound every tile it computes
    const int64_t nv_max = n_visible(q_pos0.at(b, min(q0 + kPreWaves, Tq) - 1), m, N);
    const int vtiles = (int)((nv_max + kPreRows - 1) / kPreRows);

    if (hist)
        for (int i = lane; i < kTopkBins; i += 64) qh[wv * kTopkBins + i] = 0;
    // the query's index heads (A operand) and head weights
    bf16x8 a[MB][KS];
    float wgt[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int head = mb * 16 + c;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 v = *(const bf16x8 *)(qI + (row * HI + min(head, HI - 1)) * DI + ks * 32 + g * 8);
            a[mb][ks] = head < HI ? v : Elem<bf16_t>::zero();
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int hh = mb * 16 + 4 * g + e;
            const float v = w[row * HI + min(hh, HI - 1)];
            wgt[mb][e] = hh < HI ? v : 0.f;
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // (vmcnt(0): the loads above are done before the DMAs start)

    // DMA of key tile t into stage t % kPreStages: wave wv moves KiB wv, wv + kPreWaves, ...
    const bf16_t *kb = kI + b * k_bs;
    const uint32_t ring_addr = (uint32_t)(uintptr_t)ring;
    auto issue = [&](int t) {
        const uint32_t stage = ring_addr + (t % kPreStages) * S::TB;
        for (int ip = wv; ip < S::IPT; ip += kPreWaves) {
            const int byte = ip * 1024 + lane * 16;
            const int r = byte / S::RB, pos = (byte % S::RB) / 16;
            const int64_t jr = min((int64_t)t * kPreRows + r, nv_max - 1);
            lds_dma16_nt(__builtin_amdgcn_readfirstlane(stage + ip * 1024), kb + jr * DI + S::swz(r, pos) * 8);
        }
    };
    // DMA instructions per wave per tile: every wave moves IPW KiB, or (short
    // tiles) IPW or none, so vmcnt((stages - 2) * IPW) always covers the older tiles
    constexpr int IPW = (S::IPT + kPreWaves - 1) / kPreWaves;
    static_assert(S::IPT % kPreWaves == 0 || S::IPT < kPreWaves, "uneven shares of a tile's DMA");
    for (int t = 0; t < kPreStages - 1 && t < vtiles; ++t) issue(t);

    float *srow = scores + row * s_stride;
    float *srow2 = scores2 ? scores2 + row * (int64_t)N : nullptr;
    for (int t = 0; t < vtiles; ++t) {
        // this wave's share of tile t has landed (kPreStages-2 younger tiles may fly), then
        // the barrier: every share has landed and every wave is done with tile t-1
        if (t + kPreStages - 2 < vtiles)
            asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((kPreStages - 2) * IPW) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        if (t + kPreStages - 1 < vtiles) issue(t + kPreStages - 1);
        const unsigned char *tile = ring + (t % kPreStages) * S::TB;
        // four 16-entry blocks at a time: their head sums finish together, after
        // which every lane holds one score (block g, entry c: tile row 16 g + c of
        // the four) for the stores and the histogram
#pragma unroll
        for (int q4 = 0; q4 < kPreRows / 64; ++q4) {
            float part[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int r = (q4 * 4 + u) * 16 + c;
                bf16x8 kf[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) kf[ks] = *(const bf16x8 *)(tile + r * S::RB + S::swz(r, ks * 4 + g) * 16);
                floatx4 acc[MB];
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) acc[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mb][ks], kf[ks], acc[mb], 0, 0, 0);
                float sc = 0.f;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) sc += wgt[mb][e] * relu(acc[mb][e]);
                part[u] = sc;
            }
            const float sc = sum_lane_groups4(part);
            const int64_t j = (int64_t)t * kPreRows + q4 * 64 + lane;
            if (on && j < N) {
                const float v = j < nv ? sc : -INFINITY;
                srow[j] = v;
                if (srow2) srow2[j] = v;
                if (hist && j < nv) atomicAdd(&qh[wv * kTopkBins + topk_bin(order_key(sc))], 1u);
            }
        }
    }
    // entries past every query of the workgroup
    if (on)
        for (int64_t j = (int64_t)vtiles * kPreRows + lane; j < N; j += 64) {
            srow[j] = -INFINITY;
            if (srow2) srow2[j] = -INFINITY;
        }
    if (hist && on) {
        // LDS operations of one wave complete in order: its histogram is final here
        uint32_t *grow = hist + row * kTopkBins;
        for (int i = lane; i < kTopkBins; i += 64) {
            const uint32_t v = qh[wv * kTopkBins + i];
            if (v) atomicAdd(&grow[i], v);
        }
    }
}

template <int DI, int MB>
static hipError_t launch_prefill(int B, int Tq, int N, int HI, int m, QPos q_pos0, const void *qI, const float *w,
                                 const void *kI, RowMap k_bs, float *scores, int64_t s_stride, float *scores2,
                                 uint32_t *hist, hipStream_t st) {
    using S = IdxPre<DI>;
    static const hipError_t attr = hipFuncSetAttribute((const void *)k_index_prefill<DI, MB>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, S::LDS);
    if (attr != hipSuccess) return attr;
    const int bps = (Tq + kPreWaves - 1) / kPreWaves;
    hipLaunchKernelGGL((k_index_prefill<DI, MB>), dim3((unsigned)((int64_t)B * bps)), dim3(kPreWaves * 64), S::LDS,
                       st, Tq, N, HI, m, q_pos0, bps, (const bf16_t *)qI, w, (const bf16_t *)kI, k_bs.bstride, scores,
                       s_stride, scores2, hist);
    return hipGetLastError();
}

template <typename T, int DI>
static hipError_t launch_di(int B, int Tq, int N, int HI, int m, QPos q_pos0, const void *qI, const float *w,
                            const void *kI, RowMap k_bs, float *scores, int64_t s_stride, float *scores2, uint32_t *hist, hipStream_t st) {
    if constexpr (sizeof(T) == 2) {
        // many queries per sequence: the query-blocked kernel (contiguous keys only)
        if (Tq >= kPreMinQueries && !k_bs.ptab) {
            if (HI <= 16) return launch_prefill<DI, 1>(B, Tq, N, HI, m, q_pos0, qI, w, kI, k_bs, scores, s_stride,
                                                       scores2, hist, st);
            if (HI <= 32) return launch_prefill<DI, 2>(B, Tq, N, HI, m, q_pos0, qI, w, kI, k_bs, scores, s_stride,
                                                       scores2, hist, st);
            return launch_prefill<DI, 4>(B, Tq, N, HI, m, q_pos0, qI, w, kI, k_bs, scores, s_stride, scores2, hist, st);
        }
        if (HI <= 16) return launch_dma<DI, 1>(B, Tq, N, HI, m, q_pos0, qI, w, kI, k_bs, scores, s_stride, scores2,
                                               hist, st);
        if (HI <= 32) return launch_dma<DI, 2>(B, Tq, N, HI, m, q_pos0, qI, w, kI, k_bs, scores, s_stride, scores2,
                                               hist, st);
        return launch_dma<DI, 4>(B, Tq, N, HI, m, q_pos0, qI, w, kI, k_bs, scores, s_stride, scores2, hist, st);
    }
    if (HI <= 16) return launch_t<T, DI, 1>(B, Tq, N, HI, m, q_pos0, qI, w, kI, k_bs, scores, s_stride, scores2,
                                                   hist, st);
    if (HI <= 32) return launch_t<T, DI, 2>(B, Tq, N, HI, m, q_pos0, qI, w, kI, k_bs, scores, s_stride, scores2,
                                                   hist, st);
    return launch_t<T, DI, 4>(B, Tq, N, HI, m, q_pos0, qI, w, kI, k_bs, scores, s_stride, scores2,
                                                   hist, st);
}

template <typename T>
static hipError_t launch_dt(int B, int Tq, int N, int HI, int dI, int m, QPos q_pos0, const void *qI,
                            const float *w, const void *kI, RowMap k_bs, float *scores, int64_t s_stride, float *scores2,
                            uint32_t *hist, hipStream_t st) {
    switch (dI) {
        case 32: return launch_di<T, 32>(B, Tq, N, HI, m, q_pos0, qI, w, kI, k_bs, scores, s_stride, scores2,
                                                   hist, st);
        case 64: return launch_di<T, 64>(B, Tq, N, HI, m, q_pos0, qI, w, kI, k_bs, scores, s_stride, scores2,
                                                   hist, st);
        default: return launch_di<T, 128>(B, Tq, N, HI, m, q_pos0, qI, w, kI, k_bs, scores, s_stride, scores2,
                                                   hist, st);
    }
}

hipError_t launch_index_scores(int dt, int B, int Tq, int N, int HI, int dI, int m, QPos q_pos0, const void *qI,
                               const float *w, const void *kI, RowMap k_bs, float *scores, int64_t s_stride, float *scores2,
                               uint32_t *hist, hipStream_t st) {
    if (dt == 0) return launch_dt<float>(B, Tq, N, HI, dI, m, q_pos0, qI, w, kI, k_bs, scores, s_stride,
                                          scores2, hist, st);
    return launch_dt<bf16_t>(B, Tq, N, HI, dI, m, q_pos0, qI, w, kI, k_bs, scores, s_stride,
                                          scores2, hist, st);
}

}  // namespace csa
