// FP4 operands of the lightning indexer (DeepSeek-V4 overview page, section
// 9, summary of key innovations, item 5: the indexer's queries and keys are
// quantised to FP4).  The block format is OCP MXFP4, the format gfx950's
// scaled MFMA consumes: 32 consecutive elements share one E8M0 scale
// X = 2^(E - 127), each element is FP4 E2M1 (magnitudes 0, 0.5, 1, 1.5, 2,
// 3, 4, 6), two codes per byte with the even element in the low nibble.
//
// k_mx4_quantize: one thread per 32-element block.  X = 2^(floor(log2 max|v|)
// - 2) with the exponent kept inside [-127, 127]; v / X (exact: a power-of-two
// scaling) rounds to the nearest magnitude, ties to the even mantissa,
// saturating at 6, by the hardware's scaled FP4 conversion (or, for a
// subnormal X, a sum of threshold tests: strict at the ties that round down,
// inclusive at the ties that round up); the sign bit is the sign bit of v.  A
// block of zeros gets E = 0 and zero codes.
//
// k_index_mx4: the decode indexer of indexer.hip with FP4 operands.  The
// query's index heads arrive in the element type and are quantised in the
// prologue by the same block routine (lane (g, c) of a head block holds
// exactly one 32-element block).  A query's entries are read in batches of
// 16-entry tiles dealt round-robin to its wavefronts; one v_mfma_scale_f32_16x16x128_f8f6f4 per 16 heads x 16 entries
// covers all of d_I = 128 (lane l holds 32 consecutive K values of row / column
// l % 16, block l / 16, with that block's scale byte), so each tile is one
// 16-byte load per lane (the tile's 16 rows of 64 code bytes, contiguous) and
// one scale-byte load.  The epilogue is the bf16 kernel's: ReLU, head weight,
// head sum across the lane groups, score store and the first top-k digit.
#include "kernels.h"

namespace csa {

typedef int int32x8 __attribute__((ext_vector_type(8)));

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// one 32-element block (32 consecutive elements at src, 16-byte aligned) ->
// 16 code bytes and its scale byte.  The element conversion is gfx950's scaled
// FP4 conversion (v / X to the nearest E2M1 value, ties to even, saturating,
// the sign bit taken from v), four bytes per dword by byte select; a block
// whose scale would be a subnormal float (max |v| < 2^-124) takes the same
// rule in software.
template <typename T>
__device__ __forceinline__ void quantize_block32(const T *src, u32x4 &packed, uint32_t &e8) {
    constexpr int NQ = 32 * (int)sizeof(T) / 16;  // 16-byte pieces of the block
    u32x4 r[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) r[q] = ((const u32x4 *)src)[q];
    float amax;
    if constexpr (sizeof(T) == 2) {
        // |bf16| bit patterns order like the values: a packed 16-bit integer max
        u16x2 mx = {0, 0};
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, r[q][e] & 0x7fff7fffu));
        amax = __uint_as_float((uint32_t)(mx[0] > mx[1] ? mx[0] : mx[1]) << 16);
    } else {
        amax = 0.f;
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fabsf(__uint_as_float(r[q][e])));
    }
    packed = u32x4{0u, 0u, 0u, 0u};
    e8 = 0;
    if (!(amax > 0.f)) return;  // a block of zeros
    int ex;
    (void)frexpf(amax, &ex);  // amax = f * 2^ex, 0.5 <= f < 1: floor(log2 amax) = ex - 1
    int se = ex - 1 - 2;
    se = se < -127 ? -127 : (se > 127 ? 127 : se);
    e8 = (uint32_t)(se + 127);
    if (se >= -126) {
        const float X = __uint_as_float((uint32_t)(se + 127) << 23);  // 2^se, a normal float
        // byte bt of dword wd holds elements 8*wd + 2*bt (low nibble) and the next one
#define CSA_CVT_BYTE(BT)                                                                                  \
    if constexpr (sizeof(T) == 2) {                                                                       \
        const int i = 8 * wd + 2 * (BT);                                                                  \
        const uint32_t pr = r[i / 8][(i % 8) / 2];                                                        \
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, __uint_as_float(pr << 16),                        \
                                                     __uint_as_float(pr & 0xffff0000u), X, BT);           \
    } else {                                                                                              \
        const int i = 8 * wd + 2 * (BT);                                                                  \
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, __uint_as_float(r[i / 4][i % 4]),                 \
                                                     __uint_as_float(r[i / 4][i % 4 + 1]), X, BT);        \
    }
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
            uint32_t w = 0;
            CSA_CVT_BYTE(0)
            CSA_CVT_BYTE(1)
            CSA_CVT_BYTE(2)
            CSA_CVT_BYTE(3)
            packed[wd] = w;
        }
#undef CSA_CVT_BYTE
    } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const float v = sizeof(T) == 2 ? __uint_as_float(((r[i / 8][(i % 8) / 2] >> (16 * (i % 2))) & 0xffffu) << 16)
                                           : __uint_as_float(r[i / 4][i % 4]);
            const float a = fabsf(ldexpf(v, -se));
            uint32_t code = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                            (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                            (uint32_t)(a > 5.f);
            if (signbit(v)) code |= 8u;
            packed[i / 8] |= code << (4 * (i % 8));
        }
    }
}

template <typename T>
__global__ __launch_bounds__(256) void k_mx4_quantize(int64_t n_blocks, const T *__restrict__ x,
                                                      uint8_t *__restrict__ codes, uint8_t *__restrict__ scales) {
    const int64_t blk = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (blk >= n_blocks) return;
    u32x4 packed;
    uint32_t e8;
    quantize_block32(x + blk * 32, packed, e8);
    *(u32x4 *)(codes + blk * 16) = packed;
    scales[blk] = (uint8_t)e8;
}

// sum over the four 16-lane groups (each lane gets the sum for its l % 16)
__device__ __forceinline__ float mx4_sum_lane_groups(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}
// max(x, 0) on the bit pattern (one integer max, no NaN canonicalisation of the MFMA result)
__device__ __forceinline__ float mx4_relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

template <typename T, int DI, int MB>
__global__ __launch_bounds__(256) void k_index_mx4(int Tq, int N, int HI, int m, QPos q_pos0, int64_t n_items,
                                                   int chunks_per_row, const T *__restrict__ qI,
                                                   const float *__restrict__ w,
                                                   const uint8_t *__restrict__ kc, const uint8_t *__restrict__ ks,
                                                   int64_t k_bs, float *__restrict__ scores, int64_t s_stride,
                                                   float *__restrict__ scores2, uint32_t *__restrict__ hist) {
    constexpr int KB = DI / 32;  // 32-element blocks per row
    constexpr int RB = DI / 2;   // code bytes per row
    constexpr int UNROLL = 4;    // tiles per batch (more waves per SIMD beat deeper batches)
    constexpr int BATCH = 16 * UNROLL;
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
    const bool kon = g < KB;  // lanes that hold a K block (d_I < 128 leaves the rest zero)

    // the query's index heads quantised in place (A operand: lane (g, c) holds
    // block g of head mb*16 + c, exactly one MXFP4 block), and head weights
    int32x8 a[MB];
    int as[MB];
    float wgt[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int head = mb * 16 + c;
        const int64_t hr = row * HI + min(head, HI - 1);
        u32x4 v = {0u, 0u, 0u, 0u};
        uint32_t sc = 127;
        if (kon && head < HI) quantize_block32(qI + hr * DI + g * 32, v, sc);
        a[mb] = int32x8{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
        as[mb] = (int)sc;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int hh = mb * 16 + 4 * g + e;
            const float wv_ = w[row * HI + min(hh, HI - 1)];
            wgt[mb][e] = hh < HI ? wv_ : 0.f;
        }
    }

    const uint8_t *kcb = kc + b * k_bs * RB + (kon ? g : 0) * 16;
    const uint8_t *ksb = ks + b * k_bs * KB + (kon ? g : 0);
    float *srow = scores + row * s_stride;
    float *srow2 = scores2 ? scores2 + row * (int64_t)N : nullptr;
    // the row's batches are dealt round-robin to its chunks_per_row waves
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
        // one batch: UNROLL tiles of 16 keys.  Loads are unconditional (lanes
        // past the visible entries reread the last visible row) so the
        // compiler can wait for exactly one batch.
        const int64_t j_last = nv - 1;
        auto load_batch = [&](int64_t j0, u32x4 (&kd)[UNROLL], int (&kx)[UNROLL]) {
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                int64_t jr = j0 + u * 16 + c;
                jr = jr < j_last ? jr : j_last;
                kd[u] = __builtin_nontemporal_load((const u32x4 *)(kcb + jr * RB));
                kx[u] = ksb[jr * KB];
            }
        };
        // the batch's four tiles finish their head sums together: lane group g
        // then holds tile g's scores (entry j0 + 16 g + c = j0 + lane)
        static_assert(UNROLL == 4, "one tile per lane group");
        auto score_batch = [&](int64_t j0, const u32x4 (&kd)[UNROLL], const int (&kx)[UNROLL]) {
            float part[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const u32x4 z = kon ? kd[u] : u32x4{0u, 0u, 0u, 0u};
                const int32x8 bk = {(int)z[0], (int)z[1], (int)z[2], (int)z[3], 0, 0, 0, 0};
                const int bs = kon ? kx[u] : 127;
                float s = 0.f;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const floatx4 acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        a[mb], bk, floatx4{0.f, 0.f, 0.f, 0.f}, 4, 4, 0, as[mb], 0, bs);
#pragma unroll
                    for (int e = 0; e < 4; ++e) s += wgt[mb][e] * mx4_relu(acc[e]);
                }
                part[u] = s;
            }
            const float s = sum_lane_groups4(part);
            const int64_t j = j0 + lane;
            if (j < j_hi) {
                srow[j] = j < nv ? s : -INFINITY;
                if (srow2) srow2[j] = j < nv ? s : -INFINITY;
            }
            if (hist && j < j_hi && j < nv) atomicAdd(&whist[wv][topk_bin(order_key(s))], 1u);
        };
        // double-buffered: the next batch is in flight while this one is scored
        u32x4 d0[UNROLL], d1[UNROLL];
        int x0[UNROLL], x1[UNROLL];
        if (j_lo < j_hi) load_batch(j_lo, d0, x0);
        for (int64_t j0 = j_lo; j0 < j_hi; j0 += 2 * jstep) {
            load_batch(j0 + jstep, d1, x1);
            score_batch(j0, d0, x0);
            load_batch(j0 + 2 * jstep, d0, x0);
            if (j0 + jstep < j_hi) score_batch(j0 + jstep, d1, x1);
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
// FP4 keys, d_I = 128: LDS-DMA streaming (the structure of k_index_dma).
//
// One workgroup of kMx4Waves wavefronts works on one query; the query's
// 16-entry tiles are dealt round-robin to the wavefronts of its workgroups,
// and each wavefront streams its tiles HBM -> LDS into a private ring of
// kMx4Stages slots: the tile's 1 KiB of codes with one non-temporal
// global_load_lds_dwordx4 (16-byte chunks XOR-swizzled by row, so the B
// operand reads are conflict-free) and its 16 rows' scale dwords with one
// global_load_lds_dword (16 lanes, a row each).  In the tile that holds the
// last visible entry, rows past it reread that entry (their scores are
// masked).  The workgroup quantises the query once (one 32-element block per
// thread) into LDS, from where every wavefront takes its A operands.
constexpr int kMx4Waves = 4;
constexpr int kMx4Stages = 4;
constexpr int kMx4Slot = 1024 + 64;  // codes of 16 rows of 64 bytes, then their 16 scale dwords
constexpr int kMx4Ring = kMx4Waves * kMx4Stages * kMx4Slot;
constexpr int kMx4QBlocks = 64 * 4;  // the query's 32-element blocks: 64 heads x 4
// ring, query codes + scales, histogram, page list (paged caches)
constexpr int kMx4Lds = kMx4Ring + kMx4QBlocks * (16 + 4) + kTopkBins * 4 + kMaxPagesPerSeq * 4;

// chunk position of row r's 16-byte chunk ch (an involution): four rows share one swizzle
__device__ __forceinline__ int mx4_swz(int r, int ch) { return ch ^ ((r >> 2) & 3); }

__device__ __forceinline__ void lds_dma16_nt_mx4(uint32_t lds_addr, const void *src) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(lds_addr), "v"(src)
                 : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4_nt_mx4(uint32_t lds_addr, const void *src) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off nt" ::"s"(lds_addr), "v"(src)
                 : "memory", "m0");
}

template <typename T, int MB, bool PAGED>
__global__ __launch_bounds__(kMx4Waves * 64) void k_index_mx4_dma(int Tq, int N, int HI, int m, QPos q_pos0,
                                                                 int blocks_per_row, const T *__restrict__ qI,
                                                                 const float *__restrict__ w,
                                                                 const uint8_t *__restrict__ kc,
                                                                 const uint8_t *__restrict__ ks, RowMap kl,
                                                                 float *__restrict__ scores, int64_t s_stride,
                                                                 float *__restrict__ scores2,
                                                                 uint32_t *__restrict__ hist) {
    constexpr int DI = 128, RB = 64, KB = 4;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    unsigned char *ring = lds;
    u32x4 *qcodes = (u32x4 *)(lds + kMx4Ring);                             // [head][block] 16 bytes
    uint32_t *qscale = (uint32_t *)(lds + kMx4Ring + kMx4QBlocks * 16);    // [head][block]
    uint32_t *bh = (uint32_t *)(lds + kMx4Ring + kMx4QBlocks * (16 + 4));
    int32_t *pl = (int32_t *)(lds + kMx4Ring + kMx4QBlocks * (16 + 4) + kTopkBins * 4);  // the query's pages

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, c = lane & 15;
    const int rank = xcd_rank(gridDim.x);
    int64_t row = rank / blocks_per_row;
    int part = rank % blocks_per_row, parts = blocks_per_row;
    if (q_pos0.pos && !ragged_share(q_pos0.pos, (int)(gridDim.x / blocks_per_row), m, N, gridDim.x, rank, &row, &part,
                                    &parts))
        return;  // (ragged rows: workgroups shared by visible tiles; uniform per workgroup)
    const int64_t b = row / Tq, ti = row % Tq;
    const int64_t nv = n_visible(q_pos0.at(b, ti), m, N);
    const int wpr = parts * kMx4Waves;
    const int gw = part * kMx4Waves + wv;
    const int tiles = (N + 15) / 16;
    const int vtiles = (int)((nv + 15) / 16);
    const int n_all = tiles > gw ? (tiles - gw + wpr - 1) / wpr : 0;
    const int n_vis = vtiles > gw ? (vtiles - gw + wpr - 1) / wpr : 0;

    const int64_t kb_rows = PAGED ? 0 : b * kl.bstride;
    const uint8_t *kcb = kc + kb_rows * RB;
    const uint8_t *ksb = ks + kb_rows * KB;
    unsigned char *my_ring = ring + wv * kMx4Stages * kMx4Slot;
    const uint32_t ring_addr = (uint32_t)(uintptr_t)my_ring;
    // this lane's chunk of a tile's codes: row r = lane / 4, position lane % 4 holding source chunk swz(r, pos)
    const int cr = lane >> 2, cpos = lane & 3;
    const int64_t tstride_c = (int64_t)wpr * 16 * RB;  // code bytes between this wavefront's tiles
    const uint8_t *csrc0 = kcb + ((int64_t)gw * 16 + cr) * RB + mx4_swz(cr, cpos) * 16;
    const uint8_t *ssrc0 = ksb + ((int64_t)gw * 16 + (lane & 15)) * KB;
    auto issue = [&](int i) {
        const int t = gw + i * wpr;
        const int slot = i % kMx4Stages;
        const bool whole = (int64_t)t * 16 + 16 <= nv;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // earlier reads of the slot are done
        const uint8_t *cs = csrc0 + i * tstride_c;
        const uint8_t *ss = ssrc0 + (int64_t)i * wpr * 16 * KB;
        if constexpr (PAGED) {  // the tile's 16 rows lie in one page (pages are multiples of 16 rows)
            const int64_t r0 = (int64_t)t * 16;
            const int64_t prow = ((int64_t)pl[r0 >> kl.pshift] << kl.pshift) | (r0 & ((1 << kl.pshift) - 1));
            const int64_t rc = whole ? cr : min(r0 + cr, nv - 1) - r0;
            const int64_t rs = whole ? (lane & 15) : min(r0 + (lane & 15), nv - 1) - r0;
            cs = kc + (prow + rc) * RB + mx4_swz(cr, cpos) * 16;
            ss = ks + (prow + rs) * KB;
        } else if (!whole) {
            cs = kcb + min((int64_t)t * 16 + cr, nv - 1) * RB + mx4_swz(cr, cpos) * 16;
            ss = ksb + min((int64_t)t * 16 + (lane & 15), nv - 1) * KB;
        }
        const uint32_t base = __builtin_amdgcn_readfirstlane(ring_addr + slot * kMx4Slot);
        lds_dma16_nt_mx4(base, cs);
        if (lane < 16) lds_dma4_nt_mx4(base + 1024, ss);
    };

    // paged caches: the query's page list first (the tile addresses need it)
    if constexpr (PAGED) {
        const int n_pages = (int)min((nv + (1 << kl.pshift) - 1) >> kl.pshift, (int64_t)kl.pstride);
        PageStage<kMx4Waves * 64> pages;
        pages.load(kl, b, n_pages);
        pages.store(kl, pl, n_pages);
        __syncthreads();
    }
    // the first tiles stream in while the query is quantised (the ring is
    // disjoint from the query and histogram areas)
    for (int i = 0; i < kMx4Stages - 1 && i < n_vis; ++i) issue(i);

    // ---- the head weights (their loads in flight with the query's), the
    // query quantised once per workgroup, the histogram cleared
    float wgt[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) wgt[mb][e] = w[row * HI + min(mb * 16 + 4 * g + e, HI - 1)];
    {
        static_assert(kMx4Waves * 64 == kMx4QBlocks, "one query block per thread");
        const int blk = threadIdx.x;
        const int head = blk >> 2;
        u32x4 v = {0u, 0u, 0u, 0u};
        uint32_t sc = 127;
        if (head < HI) quantize_block32(qI + (row * HI + head) * DI + (blk & 3) * 32, v, sc);
        qcodes[blk] = v;
        qscale[blk] = sc;
    }
    if (hist)
        for (int i = threadIdx.x; i < kTopkBins; i += kMx4Waves * 64) bh[i] = 0;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (mb * 16 + 4 * g + e >= HI) wgt[mb][e] = 0.f;
    __syncthreads();
    int32x8 a[MB];
    int as[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int head = mb * 16 + c;  // (heads past HI were quantised as zero blocks)
        const u32x4 v = qcodes[head * 4 + g];
        a[mb] = int32x8{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
        as[mb] = (int)qscale[head * 4 + g];
    }

    float *srow = scores + row * s_stride;
    float *srow2 = scores2 ? scores2 + row * (int64_t)N : nullptr;
    for (int i = 0; i < n_vis; ++i) {
        // two DMA instructions per tile (the scale one only in 16 lanes, still one count)
        if (i + kMx4Stages - 1 < n_vis) {
            issue(i + kMx4Stages - 1);
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kMx4Stages - 1) * 2) : "memory");
        } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        const unsigned char *tile = my_ring + (i % kMx4Stages) * kMx4Slot;
        const u32x4 kd = *(const u32x4 *)(tile + c * RB + mx4_swz(c, g) * 16);
        const int bs = tile[1024 + c * 4 + g];
        const int32x8 bk = {(int)kd[0], (int)kd[1], (int)kd[2], (int)kd[3], 0, 0, 0, 0};
        float sc = 0.f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const floatx4 acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                a[mb], bk, floatx4{0.f, 0.f, 0.f, 0.f}, 4, 4, 0, as[mb], 0, bs);
#pragma unroll
            for (int e = 0; e < 4; ++e) sc += wgt[mb][e] * mx4_relu(acc[e]);
        }
        sc = mx4_sum_lane_groups(sc);
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
        for (int i = threadIdx.x; i < kTopkBins; i += kMx4Waves * 64) {
            const uint32_t v = bh[i];
            if (v) atomicAdd(&grow[i], v);
        }
    }
}

template <typename T, int MB, bool PAGED>
static hipError_t launch_mx4_dma_p(int B, int Tq, int N, int HI, int m, QPos q_pos0, const void *qI, const float *w,
                                   const uint8_t *kc, const uint8_t *ks, RowMap k_bs, float *scores,
                                   int64_t s_stride, float *scores2, uint32_t *hist, hipStream_t st) {
    constexpr int lds = PAGED ? kMx4Lds : kMx4Lds - kMaxPagesPerSeq * 4;  // (the page list: paged keys only)
    static const hipError_t attr = hipFuncSetAttribute((const void *)k_index_mx4_dma<T, MB, PAGED>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (attr != hipSuccess) return attr;
    const int64_t rows = (int64_t)B * Tq;
    const int64_t tiles = (N + 15) / 16;
    int64_t bpr = (1280 + rows - 1) / rows;  // five workgroups per CU in total when there are few queries
    const int64_t max_bpr = (tiles + kMx4Waves - 1) / kMx4Waves;
    if (bpr > max_bpr) bpr = max_bpr;
    if (bpr < 1) bpr = 1;
    hipLaunchKernelGGL((k_index_mx4_dma<T, MB, PAGED>), dim3((unsigned)(rows * bpr)), dim3(kMx4Waves * 64), lds, st,
                       Tq, N, HI, m, q_pos0, (int)bpr, (const T *)qI, w, kc, ks, k_bs, scores, s_stride, scores2,
                       hist);
    return hipGetLastError();
}

// paging is a template parameter: the contiguous kernel carries no page-table code
template <typename T, int MB>
static hipError_t launch_mx4_dma(int B, int Tq, int N, int HI, int m, QPos q_pos0, const void *qI, const float *w,
                                 const uint8_t *kc, const uint8_t *ks, RowMap k_bs, float *scores, int64_t s_stride,
                                 float *scores2, uint32_t *hist, hipStream_t st) {
    if (k_bs.ptab)
        return launch_mx4_dma_p<T, MB, true>(B, Tq, N, HI, m, q_pos0, qI, w, kc, ks, k_bs, scores, s_stride, scores2,
                                             hist, st);
    return launch_mx4_dma_p<T, MB, false>(B, Tq, N, HI, m, q_pos0, qI, w, kc, ks, k_bs, scores, s_stride, scores2,
                                          hist, st);
}

hipError_t launch_mx4_quantize(int dt, int64_t n_blocks, const void *x, uint8_t *codes, uint8_t *scales,
                               hipStream_t st) {
    if (n_blocks <= 0) return hipSuccess;
    const unsigned grid = (unsigned)((n_blocks + 255) / 256);
    if (dt == 0)
        hipLaunchKernelGGL(k_mx4_quantize<float>, dim3(grid), dim3(256), 0, st, n_blocks, (const float *)x, codes,
                           scales);
    else
        hipLaunchKernelGGL(k_mx4_quantize<bf16_t>, dim3(grid), dim3(256), 0, st, n_blocks, (const bf16_t *)x, codes,
                           scales);
    return hipGetLastError();
}

template <typename T, int DI, int MB>
static hipError_t launch_mx4_t(int B, int Tq, int N, int HI, int m, QPos q_pos0, const void *qI, const float *w,
                               const uint8_t *kc, const uint8_t *ks, RowMap k_bs, float *scores, int64_t s_stride,
                               float *scores2, uint32_t *hist, hipStream_t st) {
    const int64_t rows = (int64_t)B * Tq;
    const int64_t batches = (N + 63) / 64;  // batches of four 16-entry tiles
    // aim for ~2048 wavefronts in flight (8 per CU) when there are few queries
    int64_t chunks = (2048 + rows - 1) / rows;
    if (chunks > batches) chunks = batches;
    if (chunks < 1) chunks = 1;
    const int64_t items = rows * chunks;
    const int64_t blocks = (items + 3) / 4;
    hipLaunchKernelGGL((k_index_mx4<T, DI, MB>), dim3((unsigned)blocks), dim3(256), 0, st, Tq, N, HI, m, q_pos0,
                       items, (int)chunks, (const T *)qI, w, kc, ks, k_bs.bstride, scores, s_stride, scores2, hist);
    return hipGetLastError();
}

template <typename T, int DI>
static hipError_t launch_mx4_di(int B, int Tq, int N, int HI, int m, QPos q_pos0, const void *qI, const float *w,
                                const uint8_t *kc, const uint8_t *ks, RowMap k_bs, float *scores, int64_t s_stride,
                                float *scores2, uint32_t *hist, hipStream_t st) {
    if (HI <= 16)
        return launch_mx4_t<T, DI, 1>(B, Tq, N, HI, m, q_pos0, qI, w, kc, ks, k_bs, scores, s_stride, scores2, hist,
                                      st);
    if (HI <= 32)
        return launch_mx4_t<T, DI, 2>(B, Tq, N, HI, m, q_pos0, qI, w, kc, ks, k_bs, scores, s_stride, scores2, hist,
                                      st);
    return launch_mx4_t<T, DI, 4>(B, Tq, N, HI, m, q_pos0, qI, w, kc, ks, k_bs, scores, s_stride, scores2, hist, st);
}

// ---------------------------------------------------------------------------
// Many queries per sequence (prefill chunks) with MXFP4 operands: query-blocked
// like the bf16 prefill indexer (indexer.hip).  One workgroup of kPmWaves
// wavefronts serves kPmWaves consecutive queries of one sequence, one per
// wavefront, so every key tile staged in LDS feeds kPmWaves queries.  A lane
// (g, c) quantises exactly the blocks its A operands need (block g of heads
// mb*16 + c), so the query never passes through LDS.  Key tiles of kPmRows
// entries (their codes, 64 bytes per row, chunks swizzled as in
// k_index_mx4_dma, then their scale dwords) stream HBM -> LDS by LDS-DMA with
// kPmStages tiles in flight: per tile each wavefront moves one KiB of codes
// and the scale dwords of 16 rows.  Per 16-entry block and head block, one
// scaled 16x16x128 MFMA; the epilogue is the decode kernels' (ReLU, head
// weight, head sum across the lane groups, score store, first top-k digit in a
// per-query LDS histogram).
constexpr int kPmWaves = 8;
constexpr int kPmMinQueries = 64;  // queries per sequence from which the query-blocked kernel is used
constexpr int kPmRows = 128;                        // entries per key tile
static_assert(kPmRows % 64 == 0, "epilogues take four 16-entry blocks at a time");
constexpr int kPmStages = 4;
constexpr int kPmCodeB = kPmRows * 64;              // code bytes per tile (8 KiB: one KiB per wavefront)
constexpr int kPmTile = kPmCodeB + kPmRows * 4;     // + the scale dwords
constexpr int kPmLds = kPmStages * kPmTile + kPmWaves * kTopkBins * 4;
static_assert(kPmCodeB == kPmWaves * 1024 && kPmRows == kPmWaves * 16, "one KiB and 16 scale rows per wavefront");

template <typename T, int MB>
__global__ __launch_bounds__(kPmWaves * 64) void k_index_prefill_mx4(int Tq, int N, int HI, int m, QPos q_pos0,
                                                                     int blocks_per_seq, const T *__restrict__ qI,
                                                                     const float *__restrict__ w,
                                                                     const uint8_t *__restrict__ kc,
                                                                     const uint8_t *__restrict__ ks, int64_t k_bs,
                                                                     float *__restrict__ scores, int64_t s_stride,
                                                                     float *__restrict__ scores2,
                                                                     uint32_t *__restrict__ hist) {
    constexpr int DI = 128, RB = 64, KB = 4;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    unsigned char *ring = lds;
    uint32_t *qh = (uint32_t *)(lds + kPmStages * kPmTile);  // [kPmWaves][kTopkBins]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c = lane & 15;
    const int64_t b = blockIdx.x / blocks_per_seq;
    const int q0 = (blockIdx.x % blocks_per_seq) * kPmWaves;  // first query of the workgroup
    const int ti = q0 + wv;
    const bool on = ti < Tq;
    const int64_t row = b * Tq + min(ti, Tq - 1);
    const int64_t nv = on ? n_visible(q_pos0.at(b, ti), m, N) : 0;
    // visible entries of the workgroup's last query bound every tile it computes
    const int64_t nv_max = n_visible(q_pos0.at(b, min(q0 + kPmWaves, Tq) - 1), m, N);
    const int vtiles = (int)((nv_max + kPmRows - 1) / kPmRows);

    if (hist)
        for (int i = lane; i < kTopkBins; i += 64) qh[wv * kTopkBins + i] = 0;
    // the query's index heads as MXFP4 A operands (block g of head mb*16 + c),
    // and the head weights
    int32x8 a[MB];
    int as[MB];
    float wgt[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int head = mb * 16 + c;
        u32x4 v = {0u, 0u, 0u, 0u};
        uint32_t sc = 127;
        if (head < HI) quantize_block32(qI + (row * HI + head) * DI + g * 32, v, sc);
        a[mb] = int32x8{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
        as[mb] = (int)sc;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int hh = mb * 16 + 4 * g + e;
            const float v = w[row * HI + min(hh, HI - 1)];
            wgt[mb][e] = hh < HI ? v : 0.f;
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // (vmcnt(0): the loads above are done before the DMAs start)

    // DMA of key tile t into stage t % kPmStages: wavefront wv moves KiB wv of
    // the codes (rows 16 wv .. 16 wv + 15) and, in 16 lanes, those rows' scale
    // dwords.  Rows past the last visible entry reread it.
    const uint8_t *kcb = kc + b * k_bs * RB;
    const uint8_t *ksb = ks + b * k_bs * KB;
    const uint32_t ring_addr = (uint32_t)(uintptr_t)ring;
    const int cr = 16 * wv + (lane >> 2), cpos = lane & 3;  // this lane's code row and chunk position
    const int sr = 16 * wv + (lane & 15);                   // its scale row (lanes 0-15)
    auto issue = [&](int t) {
        const uint32_t stage = ring_addr + (t % kPmStages) * kPmTile;
        const int64_t jc = min((int64_t)t * kPmRows + cr, nv_max - 1);
        const int64_t js = min((int64_t)t * kPmRows + sr, nv_max - 1);
        lds_dma16_nt_mx4(__builtin_amdgcn_readfirstlane(stage + wv * 1024), kcb + jc * RB + mx4_swz(cr, cpos) * 16);
        if (lane < 16) lds_dma4_nt_mx4(__builtin_amdgcn_readfirstlane(stage + kPmCodeB + wv * 64), ksb + js * KB);
    };
    // two DMA instructions per wavefront per tile (the scale one in 16 lanes, one count)
    for (int t = 0; t < kPmStages - 1 && t < vtiles; ++t) issue(t);

    float *srow = scores + row * s_stride;
    float *srow2 = scores2 ? scores2 + row * (int64_t)N : nullptr;
    for (int t = 0; t < vtiles; ++t) {
        // this wave's share of tile t has landed (kPmStages-2 younger tiles may fly), then
        // the barrier: every share has landed and every wave is done with tile t-1
        if (t + kPmStages - 2 < vtiles)
            asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((kPmStages - 2) * 2) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        if (t + kPmStages - 1 < vtiles) issue(t + kPmStages - 1);
        const unsigned char *tile = ring + (t % kPmStages) * kPmTile;
        // four 16-entry blocks at a time: their head sums finish together, after
        // which every lane holds one score (block g, entry c: tile row 16 g + c of
        // the four) for the stores and the histogram
#pragma unroll
        for (int q4 = 0; q4 < kPmRows / 64; ++q4) {
            float part[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int r = (q4 * 4 + u) * 16 + c;
                const u32x4 kd = *(const u32x4 *)(tile + r * RB + mx4_swz(r, g) * 16);
                const int bs = tile[kPmCodeB + r * KB + g];
                const int32x8 bk = {(int)kd[0], (int)kd[1], (int)kd[2], (int)kd[3], 0, 0, 0, 0};
                float sc = 0.f;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const floatx4 acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        a[mb], bk, floatx4{0.f, 0.f, 0.f, 0.f}, 4, 4, 0, as[mb], 0, bs);
#pragma unroll
                    for (int e = 0; e < 4; ++e) sc += wgt[mb][e] * mx4_relu(acc[e]);
                }
                part[u] = sc;
            }
            const float sc = sum_lane_groups4(part);
            const int64_t j = (int64_t)t * kPmRows + q4 * 64 + lane;
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
        for (int64_t j = (int64_t)vtiles * kPmRows + lane; j < N; j += 64) {
            srow[j] = -INFINITY;
            if (srow2) srow2[j] = -INFINITY;
        }
    // (the loads issued past the last tile land before the workgroup's LDS is released)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (hist && on) {
        // LDS operations of one wave complete in order: its histogram is final here
        uint32_t *grow = hist + row * kTopkBins;
        for (int i = lane; i < kTopkBins; i += 64) {
            const uint32_t v = qh[wv * kTopkBins + i];
            if (v) atomicAdd(&grow[i], v);
        }
    }
}

template <typename T, int MB>
static hipError_t launch_prefill_mx4(int B, int Tq, int N, int HI, int m, QPos q_pos0, const void *qI, const float *w,
                                     const uint8_t *kc, const uint8_t *ks, RowMap k_bs, float *scores,
                                     int64_t s_stride, float *scores2, uint32_t *hist, hipStream_t st) {
    static const hipError_t attr = hipFuncSetAttribute((const void *)k_index_prefill_mx4<T, MB>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kPmLds);
    if (attr != hipSuccess) return attr;
    const int bps = (Tq + kPmWaves - 1) / kPmWaves;
    hipLaunchKernelGGL((k_index_prefill_mx4<T, MB>), dim3((unsigned)((int64_t)B * bps)), dim3(kPmWaves * 64),
                       kPmLds, st, Tq, N, HI, m, q_pos0, bps, (const T *)qI, w, kc, ks, k_bs.bstride, scores,
                       s_stride, scores2, hist);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_mx4_dt(int B, int Tq, int N, int HI, int dI, int m, QPos q_pos0, const void *qI,
                                const float *w, const uint8_t *kc, const uint8_t *ks, RowMap k_bs, float *scores,
                                int64_t s_stride, float *scores2, uint32_t *hist, hipStream_t st) {
    if (dI == 128 && ((uintptr_t)ks % 4) == 0) {  // (scale rows move as dwords)
        // many queries per sequence, contiguous keys: the query-blocked kernel
        if (Tq >= kPmMinQueries && !k_bs.ptab) {
            if (HI <= 16)
                return launch_prefill_mx4<T, 1>(B, Tq, N, HI, m, q_pos0, qI, w, kc, ks, k_bs, scores, s_stride,
                                                scores2, hist, st);
            if (HI <= 32)
                return launch_prefill_mx4<T, 2>(B, Tq, N, HI, m, q_pos0, qI, w, kc, ks, k_bs, scores, s_stride,
                                                scores2, hist, st);
            return launch_prefill_mx4<T, 4>(B, Tq, N, HI, m, q_pos0, qI, w, kc, ks, k_bs, scores, s_stride, scores2,
                                            hist, st);
        }
        if (HI <= 16)
            return launch_mx4_dma<T, 1>(B, Tq, N, HI, m, q_pos0, qI, w, kc, ks, k_bs, scores, s_stride, scores2,
                                        hist, st);
        if (HI <= 32)
            return launch_mx4_dma<T, 2>(B, Tq, N, HI, m, q_pos0, qI, w, kc, ks, k_bs, scores, s_stride, scores2,
                                        hist, st);
        return launch_mx4_dma<T, 4>(B, Tq, N, HI, m, q_pos0, qI, w, kc, ks, k_bs, scores, s_stride, scores2, hist,
                                    st);
    }
    switch (dI) {
        case 32:
            return launch_mx4_di<T, 32>(B, Tq, N, HI, m, q_pos0, qI, w, kc, ks, k_bs, scores, s_stride, scores2, hist,
                                        st);
        case 64:
            return launch_mx4_di<T, 64>(B, Tq, N, HI, m, q_pos0, qI, w, kc, ks, k_bs, scores, s_stride, scores2, hist,
                                        st);
        default:
            return launch_mx4_di<T, 128>(B, Tq, N, HI, m, q_pos0, qI, w, kc, ks, k_bs, scores, s_stride, scores2,
                                         hist, st);
    }
}

hipError_t launch_index_mx4(int dt, int B, int Tq, int N, int HI, int dI, int m, QPos q_pos0, const void *qI,
                            const float *w, const uint8_t *kc, const uint8_t *ks, RowMap k_bs, float *scores,
                            int64_t s_stride, float *scores2, uint32_t *hist, hipStream_t st) {
    if (dt == 0)
        return launch_mx4_dt<float>(B, Tq, N, HI, dI, m, q_pos0, qI, w, kc, ks, k_bs, scores, s_stride, scores2, hist,
                                    st);
    return launch_mx4_dt<bf16_t>(B, Tq, N, HI, dI, m, q_pos0, qI, w, kc, ks, k_bs, scores, s_stride, scores2, hist,
                                 st);
}

}  // namespace csa
