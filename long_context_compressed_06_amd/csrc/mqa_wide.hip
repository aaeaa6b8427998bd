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
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 halfx4 __attribute__((ext_vector_type(4)));

constexpr int kWT = 256;                // threads (four wavefronts)
constexpr int kTR = 32;                 // rows per tile
constexpr int kD = 512;                 // latent width
constexpr int kRS = kD * 2 + 16;        // LDS row stride (bytes, padded)
constexpr int kTileB = kTR * kRS;       // LDS bytes per tile
constexpr int kStages = 4;
constexpr int kXch = 4 * 64 * 16 * 4;   // partial logits: 4 waves x 64 lanes x 16 floats
constexpr int kDmaPerWave = kTR / 4;    // rows (one 1 KiB DMA each) per wave per tile
constexpr int kOutRS = kD + 4;          // floats per head row of the output staging (16 bytes of padding)
static_assert(64 * kOutRS * 4 <= kStages * kTileB, "the output block fits in the tile stages");

// 16 bytes per lane from src + voff into LDS at lds_base + 16 * lane, the
// address in scalar registers (see dma16).  Five wait states before the load:
// the address may have just been written by the vector unit (readfirstlane),
// which the code generator does not track into inline assembly.
__device__ __forceinline__ void dma16_s(uint32_t lds_base, uint32_t voff, uint64_t src) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_base), "v"(voff), "s"(src)
                 : "memory", "m0");
}

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
    return (size_t)kStages * kTileB + kXch + (size_t)(tiles_per_split + 2) * kTR * sizeof(void *) +
           (size_t)tiles_per_split * 4;
}

__global__ __launch_bounds__(kWT) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_mqa_wide(const MqaArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char *tiles = smem;
    floatx4 *xch = (floatx4 *)(smem + kStages * kTileB);
    const bf16_t **rtab = (const bf16_t **)(smem + kStages * kTileB + kXch);
    uint32_t *vmask = (uint32_t *)(rtab + (a.tiles_per_split + 2) * kTR);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // (wave-uniform: scalar)
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

    // The query's 64 head rows (1 KiB each) go HBM -> LDS first, into tile
    // stages 2 and 3 (idle until tile 2 is loaded), laid out like a tile of K
    // rows so that the Q^T fragment reads below are the conflict-free K reads;
    // wave w moves heads 16 w .. 16 w + 15 (heads past H load head H - 1: their
    // results are never stored).  One transfer per head row, in flight while
    // the row table is built.
    const uint32_t lane16 = (uint32_t)lane * 16;
    if (ntiles > 0) {
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int hq = wv * 16 + u;
            const uint64_t src = (uint64_t)(uintptr_t)((const bf16_t *)a.q + (row * a.H + min(hq, a.H - 1)) * (int64_t)kD);
            const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(src >> 32));
            const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)src);
            const uint32_t l = (uint32_t)(uintptr_t)(tiles + (2 + (hq >> 5)) * kTileB + wide_slot(hq & 31) * kRS);
            dma16_s(__builtin_amdgcn_readfirstlane(l), lane16, ((uint64_t)hi << 32) | (uint64_t)lo);
        }
    }

    // The split's row addresses next (their index loads start the longest
    // chain of the prologue), kRtU table entries per thread per pass with all
    // their index loads in flight together (unconditional, from clamped
    // positions, so that no branch waits for one); masked rows (weight 0,
    // marked in vmask) load the query's own first row, in bounds and finite.
    const bf16_t *ent = (const bf16_t *)a.entries;
    const bf16_t *raw_b = (const bf16_t *)a.raw + b * a.raw_bs;
    const bf16_t *fallback = (const bf16_t *)a.q + row * a.H * (int64_t)kD;
    const int nr = ntiles * kTR;
    // (two tiles past the last one, all fallback rows: loads issued beyond the
    // split land in a stage that is never read again)
    // Window rows are positions w0 .. t; in a ring of raw_ring slots position p
    // sits in slot p mod raw_ring, taken here as (w0 mod raw_ring) + offset with
    // one wrap-around (a window longer than the ring takes the modulo per row).
    const int64_t ring_w0 = a.raw_ring > 0 ? w0 % a.raw_ring : 0;
    const bool ring_step = n_win <= a.raw_ring;
    constexpr int kRtU = 8;
    for (int i0 = 0; i0 < nr + 2 * kTR; i0 += kWT * kRtU) {
        int64_t jj[kRtU];
        if (a.k > 0) {  // (uniform)
            int32_t ld[kRtU];
#pragma unroll
            for (int u = 0; u < kRtU; ++u)
                ld[u] = a.idx[row * a.k + min(tile_lo * kTR + i0 + u * kWT + tid, (int64_t)a.k - 1)];
#pragma unroll
            for (int u = 0; u < kRtU; ++u) jj[u] = ld[u];
        }
#pragma unroll
        for (int u = 0; u < kRtU; ++u) {
            const int64_t r = tile_lo * kTR + i0 + u * kWT + tid;
            if (a.k == 0 || r >= n_slots) jj[u] = r;
        }
#pragma unroll
        for (int u = 0; u < kRtU; ++u) {
            if (i0 + u * kWT >= nr + 2 * kTR) break;  // (uniform: no entries of this pass remain)
            const int i = i0 + u * kWT + tid;
            const bf16_t *src = nullptr;
            if (i < nr) {
                const int64_t r = tile_lo * kTR + i;
                if (r < n_slots) {
                    if (jj[u] >= 0 && jj[u] < nv) src = ent + a.em.offset(b, jj[u], kD);
                } else if (r < n_rows) {
                    const int64_t off = r - n_slots;
                    int64_t slot;
                    if (a.raw_ring == 0) {
                        slot = w0 + off - a.raw_pos0;
                    } else if (ring_step) {
                        slot = ring_w0 + off;
                        if (slot >= a.raw_ring) slot -= a.raw_ring;
                    } else {
                        slot = (w0 + off) % a.raw_ring;
                    }
                    src = raw_b + slot * kD;
                }
            }
            if (i < nr + 2 * kTR) rtab[i] = src ? src : fallback;
            const uint64_t bal = __ballot(src != nullptr);  // lanes 0-31: tile i/32; lanes 32-63: the next
            if (i < nr && (lane & 31) == 0) vmask[i >> 5] = (uint32_t)(lane ? bal >> 32 : bal);
        }
    }

    lds_barrier();  // the row table and vmask are visible to every wave

    bf16x8 qf[16];
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
        // The eight row addresses of this wave for tile lt, wave-uniform: the
        // loads take them from scalar registers (lane l adds 16 l).
        auto next_sources = [&](int lt, uint64_t (&nsrc)[kDmaPerWave]) {
            const uint64_t *t = (const uint64_t *)rtab + lt * kTR + wv * kDmaPerWave;
#pragma unroll
            for (int u = 0; u < kDmaPerWave; ++u) {
                const uint64_t v = t[u];
                // (readfirstlane returns int: both halves are widened unsigned)
                const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
                const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
                nsrc[u] = ((uint64_t)hi << 32) | (uint64_t)lo;
            }
        };
        auto dma_row = [&](int lt, int u, uint64_t src) {
            const uint32_t l = (uint32_t)(uintptr_t)(tiles + (lt % kStages) * kTileB +
                                                      wide_slot(wv * kDmaPerWave + u) * kRS);
            dma16_s(__builtin_amdgcn_readfirstlane(l), lane16, src);
        };
#pragma unroll
        for (int lt = 0; lt < 2; ++lt) {
            uint64_t src[kDmaPerWave];
            next_sources(lt, src);
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
        // this wave's half of the logits of tile lt (one chain of 16 MFMAs) in
        // a fixed order (scheduling barriers between the steps): eight K reads
        // ahead of the chain keep it fed; per MFMA the next K read and, on even
        // steps, one row load of tile lt+2.  The returned partial is this
        // wave's half of d.
        auto block1 = [&](int lt, const uint64_t (&nsrc)[kDmaPerWave]) -> floatx16 {
            const unsigned char *cur = tiles + (lt % kStages) * kTileB + k_off;
            bf16x8 kf[16];
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) kf[ks] = *(const bf16x8 *)(cur + 32 * ks);
            __builtin_amdgcn_sched_barrier(0);
            floatx16 acc;
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
            for (int ks = 0; ks < 16; ++ks) {
                acc = mfma32(kf[ks], qf[ks], acc);
                if (ks + 8 < 16) kf[ks + 8] = *(const bf16x8 *)(cur + 32 * (ks + 8));
                if ((ks & 1) == 0) dma_row(lt + 2, ks >> 1, nsrc[ks >> 1]);
                // (ties the MFMA to its step: the code generator otherwise places
                // the whole chain after the loads)
                asm volatile("" : "+v"(acc));
                __builtin_amdgcn_sched_barrier(0);
            }
            return acc;
        };
        auto publish = [&](const floatx16 &acc) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                xch[(wv * 4 + q) * 64 + lane] = floatx4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
        };
        auto with_partner = [&](floatx16 sv) -> floatx16 {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const floatx4 v = xch[((wv ^ 1) * 4 + q) * 64 + lane];
#pragma unroll
                for (int e = 0; e < 4; ++e) sv[4 * q + e] += v[e];
            }
            return sv;
        };
        // Q^T stays in the accumulation registers, which the MFMAs read directly
        auto pin_q = [&]() {
#pragma unroll
            for (int ks = 0; ks < 16; ++ks) asm volatile("" : "+a"(qf[ks]));
        };
        // The reference maximum of head j (base 2) moves only when a tile's
        // maximum outgrows it by 2^8; the weights of that tile are then taken
        // relative to the new reference, and the accumulator and running sum
        // (the earlier tiles' weighted sums, relative to the old one) are
        // scaled by alpha once the pending weighted sum has been added.  So the
        // weights are at most 2^8 and never wait for a rescale.
        struct Ref {
            float m, alpha;
            bool grow;
        };
        auto new_reference = [&](float mx) -> Ref {
            {  // with lane l ^ 32 (the other half of the tile's rows), without an LDS round trip
                const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
                mx = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
            }
            mx *= scale2;  // base-2 maximum of this tile for head j (scale2 > 0 keeps the order)
            Ref r;
            r.grow = mx > m_ref + kLazyRescale;
            r.m = r.grow ? mx : m_ref;
            // exp2(-inf) = 0 when the first valid tile arrives (nothing accumulated yet)
            r.alpha = __builtin_amdgcn_exp2f(r.grow ? m_ref - mx : 0.f);
            return r;
        };
        // Weights of one tile relative to reference m (at most 2^8), split into
        // a high part (the weight truncated to bf16) and a low part (the exact
        // remainder, rounded to bf16); their sum is returned.  While no row has
        // been valid m is -inf and every logit -inf: 0 is then used as the
        // reference, so that every weight is exp2(-inf) = 0.
        auto weight_pair = [&](float p0, float p1, bf16x8 &pw, bf16x8 &pl, int e, float &lsum) {
            const uint32_t b0 = __float_as_uint(p0) & 0xffff0000u, b1 = __float_as_uint(p1) & 0xffff0000u;
            const bf16x2_t h2 = __builtin_bit_cast(bf16x2_t, __builtin_amdgcn_perm(b1, b0, 0x07060302u));
            const bf16x2_t lo = {(__bf16)(p0 - __uint_as_float(b0)), (__bf16)(p1 - __uint_as_float(b1))};
            pw[e - 1] = h2[0];
            pw[e] = h2[1];
            pl[e - 1] = lo[0];
            pl[e] = lo[1];
            lsum += p0 + p1;
        };
        auto weights = [&](const floatx16 &sv, float m, bf16x8 (&pw)[2], bf16x8 (&pl)[2]) -> float {
            const float mneg = m == -INFINITY ? 0.f : -m;
            float lsum = 0.f;
#pragma unroll
            for (int e = 1; e < 16; e += 2)
                weight_pair(__builtin_amdgcn_exp2f(fmaf(sv[e - 1], scale2, mneg)),
                            __builtin_amdgcn_exp2f(fmaf(sv[e], scale2, mneg)), pw[e >> 3], pl[e >> 3], e & 7, lsum);
            return lsum;
        };
        // weighted sum of the tile whose V^T fragments are vf, hi then lo parts
        auto weighted_sum = [&](const bf16x8 (&vf)[2][8], const bf16x8 (&ph)[2], const bf16x8 (&pl)[2]) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int nb = 0; nb < 8; ++nb) o[nb] = mfma32(vf[ks][nb], ph[ks], o[nb]);
#pragma unroll
                for (int nb = 0; nb < 8; ++nb) o[nb] = mfma32(vf[ks][nb], pl[ks], o[nb]);
            }
        };

        // Iteration lt (tile 0 is peeled: no weighted sum is pending before it):
        //   barrier A: tile lt landed, the stage of tile lt-2 free
        //   block 1: the logits of tile lt with the K reads of tile lt and the
        //     row loads of tile lt+2; this wave's half of the logits published
        //   barrier B
        //   block 2: the weighted sum of tile lt-1 (32 MFMAs, its V^T fragments
        //     already in registers) with, between them, the partner's half of
        //     tile lt's logits, tile lt's maximum, reference and weights, and the
        //     V^T reads of tile lt (each fragment right after its last use);
        //     then the rare rescale, after the weighted sum it applies to.
        // Block 1 is bound by the LDS reads of K, block 2 by its MFMAs; the V^T
        // reads go where the LDS has room.
        bf16x8 ph[2], pl[2];         // weights of the pending tile
        bf16x8 vf[2][8];             // its V^T fragments
        uint64_t nsrc[kDmaPerWave];  // row addresses of the next tile to load
        next_sources(2, nsrc);
        {
            barrier_a();  // (also: every wave's share of Q has landed, it was loaded before tile 0)
            // Q^T fragments (B operand of the logits): K-step ks covers columns
            // dcol0 + 16 ks .. +15; this lane supplies Q[head][dcol0 + 16 ks + 8 hh .. +7]
            {
                const unsigned char *qs = tiles + (2 + hg) * kTileB + k_off;
#pragma unroll
                for (int ks = 0; ks < 16; ++ks) qf[ks] = *(const bf16x8 *)(qs + 32 * ks);
            }
            lds_barrier();  // every wave has its Q^T before tile 2 is loaded over it
            pin_q();
            const floatx16 acc = block1(0, nsrc);
            publish(acc);
            lds_barrier();
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int nb = 0; nb < 8; ++nb) vf[ks][nb] = read_v(0, ks, nb);
            next_sources(min(3, ntiles + 1), nsrc);  // (tiles past ntiles + 1: not in the table)
            const floatx16 sv = masked(0, with_partner(acc));
            float mx = sv[0];
#pragma unroll
            for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sv[i]);
            const Ref r = new_reference(mx);
            m_ref = r.m;  // (nothing is accumulated yet)
            l_run = weights(sv, m_ref, ph, pl);
        }
        for (int lt = 1; lt < ntiles; ++lt) {
            barrier_a();
            pin_q();
            const floatx16 acc = block1(lt, nsrc);
            publish(acc);
            lds_barrier();
            // (the weighted sum stays after the barrier: its MFMAs fill the wait
            // for the partner's logits)
            asm volatile("" : "+v"(ph[0]), "+v"(ph[1]), "+v"(pl[0]), "+v"(pl[1]));
            // the first eighth of the weighted sum covers the partner's reads
            floatx4 pv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                o[q] = mfma32(vf[0][q], ph[0], o[q]);
                pv[q] = xch[((wv ^ 1) * 4 + q) * 64 + lane];
                __builtin_amdgcn_sched_barrier(0);
            }
            floatx16 full = acc;
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e) full[4 * q + e] += pv[q][e];
            // the next iteration's row addresses (tiles past ntiles + 1 are all
            // fallback rows, like tile ntiles + 1)
            next_sources(min(lt + 3, ntiles + 1), nsrc);
            const floatx16 sv = masked(lt, full);
            // The other 28 MFMAs in a fixed order (MFMA i: K-step i/16, high
            // part for i%16 < 8, block i%8), each with a slice of tile lt's work:
            // its maximum (steps 4-7), reference (8), one weight per step
            // (9-24), and the V^T fragment that MFMA i used for the last time.
            float m4[4], pr[16];
            Ref r;
            float mneg = 0.f, lsum = 0.f;
            bf16x8 nh[2], nl[2];
#pragma unroll
            for (int i = 4; i < 32; ++i) {
                const int ks = i >> 4, nb = i & 7;
                const bool lo = (i & 8) != 0;
                o[nb] = mfma32(vf[ks][nb], lo ? pl[ks] : ph[ks], o[nb]);
                if (lo) vf[ks][nb] = read_v(lt, ks, nb);
                if (i >= 4 && i < 8) {
                    const int q = i - 4;
                    m4[q] = fmaxf(fmaxf(sv[4 * q], sv[4 * q + 1]), fmaxf(sv[4 * q + 2], sv[4 * q + 3]));
                }
                if (i == 8) {
                    r = new_reference(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
                    mneg = r.m == -INFINITY ? 0.f : -r.m;
                    // (kept here: otherwise this is sunk past the MFMAs)
                    asm volatile("" : "+v"(mneg), "+v"(r.m), "+v"(r.alpha));
                }
                if (i >= 9 && i < 25) {
                    const int e = i - 9;
                    pr[e] = __builtin_amdgcn_exp2f(fmaf(sv[e], scale2, mneg));
                    if (e & 1) weight_pair(pr[e - 1], pr[e], nh[e >> 3], nl[e >> 3], e & 7, lsum);
                }
                if (i == 24) asm volatile("" : "+v"(nh[0]), "+v"(nh[1]), "+v"(nl[0]), "+v"(nl[1]), "+v"(lsum));
                __builtin_amdgcn_sched_barrier(0);
            }
            if (__ballot(r.grow)) {  // (wave-uniform; rare after the first valid tile)
                l_run *= r.alpha;
#pragma unroll
                for (int nb = 0; nb < 8; ++nb) o[nb] *= r.alpha;
            }
            m_ref = r.m;
            l_run += lsum;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                ph[ks] = nh[ks];
                pl[ks] = nl[ks];
            }
        }
        // the last tile's weighted sum
        weighted_sum(vf, ph, pl);
        // the loads issued past the last tile land before the workgroup's LDS is released
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }

    // lanes j and j + 32 hold the two halves of head j's rows
    const float l = l_run + __shfl_xor(l_run, 32);
    // The block of outputs is H rows of kD values, contiguous in memory: the
    // final output (f32) or, with several splits, the split's normalised
    // partial O / l in f16 (half the bytes of the f32 sum: the merge of the
    // partials reads them all back), scaled by a power of two sigma that keeps
    // the block's largest magnitude below 2^14 (sigma = 1 unless the values are
    // that large).  O^T registers hold 16-byte pieces of 32 different rows per
    // store, so the block is first transposed through the (now idle) tile
    // stages and then written in whole lines per wavefront.
    // (Every wave's loads have landed: the wait after the loop; after this
    // barrier no wave reads a tile any more.)
    __syncthreads();
    float *stage = (float *)smem;  // [64 heads][kOutRS]
    const float f = l > 0.f ? 1.f / l : 0.f;
    // O^T register r of block nb: column dcol0 + 32 nb + 8 (r/4) + 4 hh + r%4
    float amax = 0.f;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const floatx4 v = floatx4{o[nb][4 * q], o[nb][4 * q + 1], o[nb][4 * q + 2], o[nb][4 * q + 3]} * f;
            *(floatx4 *)(stage + head * kOutRS + dcol0 + 32 * nb + 8 * q + 4 * hh) = v;
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
        }
    if (head >= a.H) amax = 0.f;
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) amax = fmaxf(amax, __shfl_xor(amax, sh));
    float *red = (float *)xch;  // (the logits exchange area is idle too)
    if (lane == 0) red[wv] = amax;
    if (head < a.H && hh == 0 && dh == 0) {
        if (a.n_splits == 1) {
            if (a.lse) a.lse[row * a.H + head] = l > 0.f ? (m_ref + __log2f(l)) * kLn2 : -INFINITY;
        } else {
            const int64_t slot = (row * a.n_splits + split) * a.H + head;
            a.part_ml[slot * 2 + 0] = m_ref;  // base 2
            a.part_ml[slot * 2 + 1] = l;
        }
    }
    __syncthreads();
    const int n4 = a.H * (kD / 4);
    if (a.n_splits == 1) {
        float *dst = a.out + row * a.H * (int64_t)kD;
        for (int f4 = tid; f4 < n4; f4 += kWT)
            *(floatx4 *)(dst + 4 * (int64_t)f4) = *(const floatx4 *)(stage + (f4 >> 7) * kOutRS + 4 * (f4 & 127));
    } else {
        const float bmax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        int e = 0;
        (void)frexpf(bmax, &e);  // bmax < 2^e
        const int se = e > 14 ? min(e - 14, 115) : 0;
        const float inv_sigma = __uint_as_float((uint32_t)(127 - se) << 23);  // 2^-se (se <= 115)
        halfx4 *dst = (halfx4 *)a.part_o + (row * a.n_splits + split) * a.H * (int64_t)(kD / 4);
        for (int f4 = tid; f4 < n4; f4 += kWT)
            dst[f4] = __builtin_convertvector(
                *(const floatx4 *)(stage + (f4 >> 7) * kOutRS + 4 * (f4 & 127)) * inv_sigma, halfx4);
        if (tid == 0) a.part_sc[row * a.n_splits + split] = __uint_as_float((uint32_t)(127 + se) << 23);
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
