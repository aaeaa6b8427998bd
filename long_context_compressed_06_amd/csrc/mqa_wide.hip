// Shared-KV multi-query attention for the wide configuration: bf16 rows of
// d = 512 and 33..64 query heads (DeepSeek-V4 overview page, section 2.2
// step 3: the selected entries are both key and value and all query heads
// share them; section 2.3: HCA attends to every visible entry).  Same
// arguments, row list, masking, split-K partials and merge as k_mqa.
//
// Workgroup: four wavefronts, one per SIMD.  Wave w owns the 32 query heads
// of group w / 2 and the half w % 2 of d, so each K = V row read from LDS
// feeds 32 heads of a 32x32x16 bf16 MFMA (half the LDS reads of 16-head
// waves).  Per 32-row tile, per wave:
//   S^T[32 rows x 32 heads] = K . Q^T over the wave's half of d (16 MFMAs;
//       K rows by ds_read_b128, Q^T held in registers for the whole loop),
//       summed with the partner wave's half through LDS
//   online softmax per head in the base-2 domain (lane l owns head l % 32;
//       the reference maximum only moves when the tile maximum exceeds it by
//       2^8, and it is settled right after the tile's logits are known, so
//       the weights never wait for it), P split into bf16 high and low parts: one rounding of the
//       weights to bf16 (2^-9 relative) times |v - o| of rows scaled up to
//       ~30 would reach the bf16 output tolerance
//   O^T[256 d x 32 heads] += V^T . P^T (2 x 16 MFMAs; V^T straight from the
//       row-major tile with the transposing ds_read_b64_tr_b16).  P^T needs
//       no data movement: lane l holds head l % 32 in both the logits result
//       and the weights operand, and the weighted sum takes the 32 rows in
//       the order the logits result holds them.
// Pipeline (one wave per SIMD, so everything a wave does between its MFMAs
// is interleaved with them in its own instruction stream): per tile t, the
// logits MFMAs of tile t run with tile t-1's weights (VALU) between them; after
// the exchange barrier the weighted-sum MFMAs of tile t-1 run with the
// partner's logits, the reference update and the row loads of tile t+2
// between them.  Two barriers per
// tile (tile landed; partial logits published), four LDS stages: the tile
// whose weighted sum is pending, the tile whose logits are being computed,
// and two in flight.
#include "mqa.h"

namespace csa {

namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kWT = 256;                // threads (four wavefronts)
constexpr int kTR = 32;                 // rows per tile
constexpr int kD = 512;                 // latent width
constexpr int kRS = kD * 2 + 16;        // LDS row stride (bytes, padded)
constexpr int kTileB = kTR * kRS;       // LDS bytes per tile
constexpr int kStages = 4;
constexpr int kXch = 4 * 64 * 16 * 4;   // partial logits: 4 waves x 64 lanes x 16 floats
constexpr int kDmaPerWave = kTR / 4;    // rows (one 1 KiB DMA each) per wave per tile

__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS slot of tile row r (rows 1040 bytes apart, i.e. 16 bytes apart modulo
// the 256 bytes that the 64 four-byte banks serve per cycle).  The logits read
// 16 bytes of 16 consecutive rows per 16 lanes: their slots must differ modulo
// 16.  A transposing read serves 32 lanes per cycle: 32 bytes of each of the
// four rows 4g .. 4g+3 (g = r/4 within a 16-row block) at two column offsets
// 32 bytes apart, so those rows' slots must be 4 apart modulo 16.  Slot
// 16 (r/16) + 4 (r%4) + (r/4)%4 gives both (measured: 232 and 192 bytes per
// clock per CU for the two read patterns, against 233 and 122 with the slot
// order of the 16-head kernel).
__device__ __forceinline__ int wide_slot(int r) { return (r & 16) | ((r & 3) << 2) | ((r >> 2) & 3); }

}  // namespace

size_t mqa_wide_lds_bytes(int tiles_per_split) {
    return (size_t)kStages * kTileB + kXch + (size_t)tiles_per_split * (kTR * sizeof(void *) + 4);
}

__global__ __launch_bounds__(kWT) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_mqa_wide(const MqaArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char *tiles = smem;
    floatx4 *xch = (floatx4 *)(smem + kStages * kTileB);
    const bf16_t **rtab = (const bf16_t **)(smem + kStages * kTileB + kXch);
    uint32_t *vmask = (uint32_t *)(rtab + a.tiles_per_split * kTR);

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int hg = wv >> 1, dh = wv & 1;        // head group of 32, half of d
    const int j = lane & 31, hh = lane >> 5;    // head within the group; lane half
    // the splits of one query on one XCD (their partials are merged there)
    const int rank = xcd_rank((int)gridDim.x);
    const int64_t row = rank / a.n_splits;
    const int split = rank % a.n_splits;
    const int64_t b = row / a.Tq, t = (a.pos ? a.pos[b] : a.q_pos0) + row % a.Tq;
    const int64_t nv = n_visible(t, a.m, a.N);
    const int64_t n_slots = a.k > 0 ? a.k : nv;
    const int64_t w0 = t - a.W + 1 > 0 ? t - a.W + 1 : 0;
    const int64_t n_win = a.W > 0 ? t - w0 + 1 : 0;
    const int64_t n_rows = n_slots + n_win;
    const int64_t n_tiles_all = (n_rows + kTR - 1) / kTR;
    const int64_t tile_lo = (int64_t)split * a.tiles_per_split;
    const int ntiles = (int)max((int64_t)0, min(n_tiles_all, tile_lo + a.tiles_per_split) - tile_lo);
    const int head = hg * 32 + j;
    const float scale2 = a.scale * kLog2e;
    const int dcol0 = dh * (kD / 2);

    // Q^T fragments (B operand of the logits): K-step ks covers columns
    // dcol0 + 16 ks .. +15; this lane supplies Q[head][dcol0 + 16 ks + 8 hh .. +7]
    bf16x8 qf[16];
    {
        const bf16_t *qrow = (const bf16_t *)a.q + (row * a.H + min(head, a.H - 1)) * (int64_t)kD + dcol0 + 8 * hh;
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
            const bf16x8 v = Elem<bf16_t>::load(qrow + 16 * ks);
            qf[ks] = head < a.H ? v : Elem<bf16_t>::zero();
        }
    }

    // the split's row addresses, once; masked rows (weight 0, marked in vmask)
    // load the query's own first row, in bounds and finite
    const bf16_t *ent = (const bf16_t *)a.entries;
    const bf16_t *raw_b = (const bf16_t *)a.raw + b * a.raw_bs;
    const bf16_t *fallback = (const bf16_t *)a.q + row * a.H * (int64_t)kD;
    const int nr = ntiles * kTR;
    for (int i0 = 0; i0 < nr; i0 += kWT) {
        const int i = i0 + tid;
        const bf16_t *src = nullptr;
        if (i < nr) {
            const int64_t r = tile_lo * kTR + i;
            if (r < n_slots) {
                const int64_t jj = a.k > 0 ? (int64_t)a.idx[row * a.k + r] : r;
                if (jj >= 0 && jj < nv) src = ent + a.em.offset(b, jj, kD);
            } else if (r < n_rows) {
                const int64_t p = w0 + (r - n_slots);
                src = raw_b + (a.raw_ring ? p % a.raw_ring : p - a.raw_pos0) * kD;
            }
            rtab[i] = src ? src : fallback;
        }
        const uint64_t bal = __ballot(src != nullptr);  // lanes 0-31: tile i/32; lanes 32-63: the next
        if (i < nr && (lane & 31) == 0) vmask[i >> 5] = (uint32_t)(lane ? bal >> 32 : bal);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the Q^T loads have landed
    __syncthreads();

    floatx16 o[8];  // O^T: block nb = columns dcol0 + 32 nb .. +31 (rows of the 32x32 result) x 32 heads
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[nb][e] = 0.f;
    float m_ref = -INFINITY, l_run = 0.f;  // base-2 reference maximum, running sum of the weights

    if (ntiles > 0) {
        // Row sources of local tile lt for this wave (rows 8 wv .. 8 wv + 7).
        // Tiles past the split's last one (issued so that every wave always has
        // two tiles in flight and the waits below never change) load the query's
        // own row into a stage nobody reads any more.
        auto row_src = [&](int lt, int u) -> const unsigned char * {
            const bf16_t *p = rtab[min(lt, ntiles - 1) * kTR + wv * kDmaPerWave + u];  // (always in the table)
            return (const unsigned char *)(lt < ntiles ? p : fallback) + lane * 16;
        };
        auto dma_row = [&](int lt, int u, const unsigned char *src) {
            dma16(tiles + (lt % kStages) * kTileB + wide_slot(wv * kDmaPerWave + u) * kRS, src);
        };
#pragma unroll
        for (int lt = 0; lt < 2; ++lt) {
            const unsigned char *src[kDmaPerWave];
#pragma unroll
            for (int u = 0; u < kDmaPerWave; ++u) src[u] = row_src(lt, u);
#pragma unroll
            for (int u = 0; u < kDmaPerWave; ++u) dma_row(lt, u, src[u]);
        }

        // K fragments (A operand of the logits): row j, columns dcol0 + 16 ks + 8 hh .. +7
        const int k_off = wide_slot(j) * kRS + (dcol0 + 8 * hh) * 2;
        // V^T fragments (A operand of the weighted sum) by transposing reads: in
        // each 16-lane group (column half ch of a 32-column block, lane half hh)
        // lane c addresses row base + c/4 at column 4 (c%4), base = 16 ks + 4 hh
        // (+8 for the second read, sel = 1), and receives its column of those
        // four rows.  wide_slot(16 ks + 8 sel + 4 hh + e) = 16 ks + 4 e + 2 sel + hh.
        const int c16 = lane & 15, ch = (lane >> 4) & 1;
        const int v_off = (4 * (c16 >> 2) + hh) * kRS + (dcol0 + 16 * ch + 4 * (c16 & 3)) * 2;

        auto read_v = [&](int lt, int ks, int nb) -> bf16x8 {
            const unsigned char *p0 = tiles + (lt % kStages) * kTileB + v_off + 16 * ks * kRS + nb * 64;
            const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)(p0));
            const v4s hi =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)(p0 + 2 * kRS));
            return __builtin_shufflevector(__builtin_bit_cast(bf16x4_t, lo), __builtin_bit_cast(bf16x4_t, hi), 0, 1,
                                           2, 3, 4, 5, 6, 7);
        };
        // The top of iteration lt: this wave's loads of tile lt have landed (those
        // of tile lt+1 may still fly), its LDS accesses are complete, and after the
        // barrier every wave's are: tile lt is readable and the stage of tile lt-2
        // is free for tile lt+2.
        auto barrier_a = [&]() { asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
        // the tile's full logits with masked rows at -inf.  Register r of this
        // lane holds row 8 (r/4) + 4 hh + r%4 of the tile for head j.
        auto masked = [&](int lt, floatx16 sv) -> floatx16 {
            const uint32_t vm = vmask[lt];
            if (vm != 0xffffffffu) {  // (wave-uniform; only partial tiles)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (!((vm >> (8 * (r >> 2) + 4 * hh + (r & 3))) & 1u)) sv[r] = -INFINITY;
            }
            return sv;
        };
        // The reference maximum of head j (base 2) is settled as soon as a tile's
        // logits are known, before that tile's weights are formed: it moves only
        // when the tile maximum outgrows it by 2^8, and then the accumulator and
        // the running sum (which so far hold the weighted sums of the earlier
        // tiles, relative to the old reference) are rescaled.  Weights are
        // therefore at most 2^8 and need nothing but the reference in force.
        auto settle_reference = [&](const floatx16 &sv) {
            float mx = sv[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sv[r]);
            {  // with lane l ^ 32 (the other half of the tile's rows), without an LDS round trip
                const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
                mx = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
            }
            mx *= scale2;  // base-2 maximum of this tile for head j (scale2 > 0 keeps the order)
            const bool grow = mx > m_ref + kLazyRescale;
            if (__ballot(grow)) {  // (wave-uniform; the first valid tile, then rarely)
                // exp2(-inf) = 0 when the first valid tile arrives
                const float alpha = __builtin_amdgcn_exp2f(grow ? m_ref - mx : 0.f);
                l_run *= alpha;
#pragma unroll
                for (int nb = 0; nb < 8; ++nb) o[nb] *= alpha;
                m_ref = grow ? mx : m_ref;
            }
        };
        // weights of one tile relative to the reference in force (at most 2^8),
        // split into bf16 high and low parts; their sum joins the running sum.
        // While no row has been valid m_ref is -inf and every logit -inf: 0 is
        // then used as the reference, so that every weight is exp2(-inf) = 0.
        auto weights = [&](const floatx16 &sv, bf16x8 (&pw)[2], bf16x8 (&pl)[2]) {
            const float mneg = m_ref == -INFINITY ? 0.f : -m_ref;
            float lsum = 0.f;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float pr = __builtin_amdgcn_exp2f(fmaf(sv[8 * ks + e], scale2, mneg));
                    const __bf16 w = (__bf16)pr;
                    pw[ks][e] = w;
                    pl[ks][e] = (__bf16)(pr - (float)w);
                    lsum += pr;
                }
            l_run += lsum;
        };

        // Iteration lt:
        //   barrier A: tile lt landed, the stage of tile lt-2 free
        //   block 1: the K reads of tile lt and the V^T reads of tile lt-1; the
        //     logits MFMAs of tile lt with the weights of tile lt-1 (VALU, which
        //     need only the reference settled for it) between them; this
        //     wave's half of tile lt's logits published
        //   barrier B
        //   block 2: the weighted sum of tile lt-1 (hi, then lo parts) with the
        //     partner's half of tile lt's logits, their maximum and the DMAs of
        //     tile lt+2 between its MFMAs; then the reference settled for tile
        //     lt (the rare rescale comes after the weighted sum it applies to)
        floatx16 s_prev;  // full logits of the previous tile
        for (int lt = 0; lt < ntiles; ++lt) {
            barrier_a();
            const unsigned char *cur = tiles + (lt % kStages) * kTileB;
            bf16x8 kf[16];
#pragma unroll
            for (int ks = 0; ks < 16; ++ks) kf[ks] = *(const bf16x8 *)(cur + k_off + 32 * ks);
            floatx16 a0, a1;
#pragma unroll
            for (int e = 0; e < 16; ++e) a0[e] = a1[e] = 0.f;
            bf16x8 vf[2][8], ph[2], pl[2];
            if (lt > 0) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int nb = 0; nb < 8; ++nb) vf[ks][nb] = read_v(lt - 1, ks, nb);
            }
#pragma unroll
            for (int ks = 0; ks < 16; ks += 2) {
                a0 = mfma32(kf[ks], qf[ks], a0);
                a1 = mfma32(kf[ks + 1], qf[ks + 1], a1);
            }
            if (lt > 0) weights(s_prev, ph, pl);
            const floatx16 acc = a0 + a1;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                xch[(wv * 4 + q) * 64 + lane] = floatx4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
            const unsigned char *nsrc[kDmaPerWave];
#pragma unroll
            for (int u = 0; u < kDmaPerWave; ++u) nsrc[u] = row_src(lt + 2, u);
            lds_barrier();
            floatx16 sv = acc;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const floatx4 v = xch[((wv ^ 1) * 4 + q) * 64 + lane];
#pragma unroll
                for (int e = 0; e < 4; ++e) sv[4 * q + e] += v[e];
            }
            if (lt > 0) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                    for (int nb = 0; nb < 8; ++nb) {
                        o[nb] = mfma32(vf[ks][nb], ph[ks], o[nb]);
                        if ((nb & 3) == 3) dma_row(lt + 2, 4 * ks + (nb >> 2), nsrc[4 * ks + (nb >> 2)]);
                    }
#pragma unroll
                    for (int nb = 0; nb < 8; ++nb) {
                        o[nb] = mfma32(vf[ks][nb], pl[ks], o[nb]);
                        if ((nb & 3) == 3) dma_row(lt + 2, 4 * ks + 2 + (nb >> 2), nsrc[4 * ks + 2 + (nb >> 2)]);
                    }
                }
            } else {
#pragma unroll
                for (int u = 0; u < kDmaPerWave; ++u) dma_row(lt + 2, u, nsrc[u]);
            }
            s_prev = masked(lt, sv);
            settle_reference(s_prev);
        }
        // the last tile's weights and weighted sum
        {
            bf16x8 ph[2], pl[2];
            weights(s_prev, ph, pl);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                bf16x8 v[8];
#pragma unroll
                for (int nb = 0; nb < 8; ++nb) {
                    v[nb] = read_v(ntiles - 1, ks, nb);
                    o[nb] = mfma32(v[nb], ph[ks], o[nb]);
                }
#pragma unroll
                for (int nb = 0; nb < 8; ++nb) o[nb] = mfma32(v[nb], pl[ks], o[nb]);
            }
        }
        // the loads issued past the last tile land before the workgroup's LDS is released
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }

    // lanes j and j + 32 hold the two halves of head j's rows
    float l = l_run + __shfl_xor(l_run, 32);
    if (head >= a.H) return;
    // O^T register r of block nb: column dcol0 + 32 nb + 8 (r/4) + 4 hh + r%4
    if (a.n_splits == 1) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        float *orow = a.out + (row * a.H + head) * (int64_t)kD + dcol0 + 4 * hh;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *(floatx4 *)(orow + nb * 32 + 8 * q) =
                    floatx4{o[nb][4 * q], o[nb][4 * q + 1], o[nb][4 * q + 2], o[nb][4 * q + 3]} * inv;
        if (a.lse && hh == 0 && dh == 0) a.lse[row * a.H + head] = l > 0.f ? (m_ref + __log2f(l)) * kLn2 : -INFINITY;
    } else {
        const int64_t slot = (row * a.n_splits + split) * a.H + head;
        float *po = a.part_o + slot * kD + dcol0 + 4 * hh;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *(floatx4 *)(po + nb * 32 + 8 * q) =
                    floatx4{o[nb][4 * q], o[nb][4 * q + 1], o[nb][4 * q + 2], o[nb][4 * q + 3]};
        if (hh == 0 && dh == 0) {
            a.part_ml[slot * 2 + 0] = m_ref;  // base 2
            a.part_ml[slot * 2 + 1] = l;
        }
    }
}

hipError_t launch_mqa_wide(const MqaArgs &a, int64_t rows, hipStream_t st) {
    static const hipError_t attr =
        hipFuncSetAttribute((const void *)k_mqa_wide, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (attr != hipSuccess) return attr;
    const size_t lds = mqa_wide_lds_bytes(a.tiles_per_split);
    if (lds > 160 * 1024) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_mqa_wide, dim3((unsigned)(rows * a.n_splits)), dim3(kWT), lds, st, a);
    return hipGetLastError();
}

}  // namespace csa
