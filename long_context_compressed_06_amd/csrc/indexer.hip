// Lightning indexer (DeepSeek-V4 overview page, section 2.2 step 2):
//     s[t, j] = sum_h w[t, h] * ReLU(qI[t, h, :] . kI[j, :])
// for every entry j visible to query t; invisible entries get -inf.
//
// Mapping.  One wavefront owns one query and a contiguous chunk of entries.
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
__global__ __launch_bounds__(256) void k_index_scores(int Tq, int N, int HI, int m, int64_t q_pos0, int64_t n_items,
                                                       int chunks_per_row, int tiles_per_chunk,
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
    const int64_t nv = n_visible(q_pos0 + ti, m, N);
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
    const int64_t j_lo = (int64_t)chunk * tiles_per_chunk * 16;
    const int64_t j_hi = min((int64_t)N, j_lo + (int64_t)tiles_per_chunk * 16);
    constexpr int BATCH = 16 * UNROLL;  // entries per batch of tiles

    if (nv == 0) {  // nothing visible: the chunk is all -inf
        for (int64_t j = j_lo + lane; j < j_hi; j += 64) {
            srow[j] = -INFINITY;
            if (srow2) srow2[j] = -INFINITY;
        }
    } else {
    // one batch: UNROLL tiles of 16 index keys, straight from HBM to registers.
    // Loads are unconditional so the compiler can wait for exactly one batch:
    // lanes past the chunk (or past the visible entries) reread its last row.
    const int64_t j_last = min(j_hi, nv) - 1;
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
                atomicAdd(&whist[wv][order_key(s) >> (32 - kTopkBinBits)], 1u);
        }
    };
    // double-buffered: the next batch is in flight while this one is scored
    typename E::frag b0[UNROLL][KS], b1[UNROLL][KS];
    if (j_lo < j_hi) load_batch(j_lo, b0);
    for (int64_t j0 = j_lo; j0 < j_hi; j0 += 2 * BATCH) {
        load_batch(j0 + BATCH, b1);
        score_batch(j0, b0);
        load_batch(j0 + 2 * BATCH, b0);
        if (j0 + BATCH < j_hi) score_batch(j0 + BATCH, b1);
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

template <typename T, int DI, int MB>
static hipError_t launch_t(int B, int Tq, int N, int HI, int m, int64_t q_pos0, const void *qI, const float *w,
                           const void *kI, int64_t k_bs, float *scores, int64_t s_stride, float *scores2, uint32_t *hist, hipStream_t st) {
    const int64_t rows = (int64_t)B * Tq;
    const int64_t tiles = (N + 15) / 16;
    // aim for ~2048 wavefronts in flight (8 per CU) when there are few queries
    int64_t chunks = (2048 + rows - 1) / rows;
    if (chunks > tiles) chunks = tiles;
    if (chunks < 1) chunks = 1;
    int64_t tpc = (tiles + chunks - 1) / chunks;
    tpc = (tpc + 3) / 4 * 4;
    chunks = (tiles + tpc - 1) / tpc;
    if (chunks < 1) chunks = 1;
    const int64_t items = rows * chunks;
    const int64_t blocks = (items + 3) / 4;
    hipLaunchKernelGGL((k_index_scores<T, DI, MB>), dim3((unsigned)blocks), dim3(256), 0, st, Tq, N, HI, m, q_pos0,
                       items, (int)chunks, (int)tpc, (const T *)qI, w, (const T *)kI, k_bs, scores, s_stride,
                       scores2, hist);
    return hipGetLastError();
}

template <typename T, int DI>
static hipError_t launch_di(int B, int Tq, int N, int HI, int m, int64_t q_pos0, const void *qI, const float *w,
                            const void *kI, int64_t k_bs, float *scores, int64_t s_stride, float *scores2, uint32_t *hist, hipStream_t st) {
    if (HI <= 16) return launch_t<T, DI, 1>(B, Tq, N, HI, m, q_pos0, qI, w, kI, k_bs, scores, s_stride, scores2,
                                                   hist, st);
    if (HI <= 32) return launch_t<T, DI, 2>(B, Tq, N, HI, m, q_pos0, qI, w, kI, k_bs, scores, s_stride, scores2,
                                                   hist, st);
    return launch_t<T, DI, 4>(B, Tq, N, HI, m, q_pos0, qI, w, kI, k_bs, scores, s_stride, scores2,
                                                   hist, st);
}

template <typename T>
static hipError_t launch_dt(int B, int Tq, int N, int HI, int dI, int m, int64_t q_pos0, const void *qI,
                            const float *w, const void *kI, int64_t k_bs, float *scores, int64_t s_stride, float *scores2,
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

hipError_t launch_index_scores(int dt, int B, int Tq, int N, int HI, int dI, int m, int64_t q_pos0, const void *qI,
                               const float *w, const void *kI, int64_t k_bs, float *scores, int64_t s_stride, float *scores2,
                               uint32_t *hist, hipStream_t st) {
    if (dt == 0) return launch_dt<float>(B, Tq, N, HI, dI, m, q_pos0, qI, w, kI, k_bs, scores, s_stride,
                                          scores2, hist, st);
    return launch_dt<bf16_t>(B, Tq, N, HI, dI, m, q_pos0, qI, w, kI, k_bs, scores, s_stride,
                                          scores2, hist, st);
}

}  // namespace csa
