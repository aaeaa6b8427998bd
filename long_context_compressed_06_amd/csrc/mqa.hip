// Shared-KV multi-query attention over compressed entries plus a window of
// raw tokens, in one softmax (DeepSeek-V4 overview page, section 2.2 step 3:
// the selected entries are both key and value and every query head shares
// them; section 2.3: HCA attends to every entry).
//
// Grid.  One 512-thread workgroup per (query, split) of the query's row
// list; split-K partials (unnormalised O, running max, running sum) are merged
// by k_combine.  With a single split the workgroup writes the final output.
//
// Workgroup.  Eight wavefronts: wave w owns the 16 query heads of group
// w % 4 and the half w / 4 of the latent width d (SPLITD = 2; narrow rows use
// one wave per head group with the whole width).  The split's row addresses
// (gathered entries, then raw window rows) are resolved once into an LDS
// table, with a 32-bit validity mask per tile (masked rows point at the
// query's own first row: in bounds, finite, weight 0).  Tiles of 32 rows then stream
// HBM -> LDS with asynchronous 16-byte LDS-DMA loads
// (global_load_lds_dwordx4), STAGES tiles in flight, so no register staging
// and no dependent global load sits in the loop.  One DMA instruction moves
// up to 1 KiB of one row; rows sit 16 bytes apart beyond their length in LDS,
// in a permuted order (row_slot) that keeps both read patterns free of bank
// conflicts, and the loop's LDS offsets are fixed per lane (the compiler folds
// them into immediates).  Per wave and tile:
//   S^T[32 rows x 16 heads] = K . Q^T over the wave's half of d (MFMA, K rows
//       read with ds_read_b128, Q^T in registers); the two halves are summed
//       through LDS, and both waves of the pair run the same softmax
//   online softmax per head in the base-2 domain; the reference maximum only
//   moves when the running maximum exceeds it by 2^8, so the accumulator is
//   rarely rescaled (weights stay <= 256, exact in fp32)
//   O^T[d/2 x 16 heads] += V^T . P^T (MFMA; V^T read straight from the
//       row-major tile with the gfx950 transposing ds_read_b64_tr_b16, all
//       of a tile's reads issued before its MFMAs; P is split into bf16 high
//       and low parts so the weights keep ~16 bits)
// Splitting d keeps per-wave state at 16 x 256 fp32 accumulators, so two
// waves per SIMD hide LDS and MFMA latency.  fp32 data uses the 16x16x4 f32
// MFMA with scalar LDS reads instead.
#include "mqa.h"

namespace csa {

template <typename T, int D>
struct MqaShape {
    static constexpr int TR = 32;                          // rows per tile
    static constexpr int ROWB = D * (int)sizeof(T);        // bytes per row
    static constexpr int RS = ROWB + 16;                   // LDS row stride (padded)
    static constexpr int TILEB = TR * RS;                  // LDS bytes per tile
    static constexpr int IPR = ROWB >= 1024 ? ROWB / 1024 : 1;  // DMA instructions per row
    static constexpr int LPI = ROWB >= 1024 ? 64 : ROWB / 16;   // active lanes per DMA instruction
    static constexpr int NW = kMqaThreads / 64;            // wavefronts
    static constexpr int LPW = (TR / NW) * IPR;            // DMA instructions per wave per tile
    static constexpr int SPLITD = (D / 2) % Elem<T>::KSTEP == 0 && (D / 2) % 16 == 0 ? 2 : 1;
    static constexpr int DW = D / SPLITD;                  // latent columns per wave
    static constexpr int XCH1 = NW * 64 * 8 * 4;                  // one partial-logit exchange buffer
    // three stages with a double-buffered exchange (one barrier per tile) when
    // they fit, else two stages with one exchange buffer (two barriers per tile)
    static constexpr bool PIPE = SPLITD == 2 && 3 * TILEB + 2 * XCH1 <= 136 * 1024;
    static constexpr int STAGES = PIPE || (SPLITD == 1 && 3 * TILEB <= 120 * 1024) ? 3 : 2;  // tiles in flight
    static constexpr int XCH = SPLITD == 2 ? (PIPE ? 2 : 1) * XCH1 : 0;  // exchange bytes
    static size_t lds_bytes(int tiles_per_split) {
        return (size_t)STAGES * TILEB + XCH + (size_t)tiles_per_split * (TR * sizeof(void *) + 4);
    }
};

template <typename T, int D>
__global__ __launch_bounds__(kMqaThreads) void k_mqa(const MqaArgs a) {
    using E = Elem<T>;
    using S = MqaShape<T, D>;
    constexpr int KS = S::DW / E::KSTEP;   // logits K-steps per wave
    constexpr int NB = S::DW / 16;         // accumulator tiles per wave
    constexpr int NHG = S::NW / S::SPLITD; // head groups served
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char *tiles = smem;
    floatx4 *xch = (floatx4 *)(smem + S::STAGES * S::TILEB);
    const T **rtab = (const T **)(smem + S::STAGES * S::TILEB + S::XCH);
    uint32_t *vmask = (uint32_t *)(rtab + a.tiles_per_split * S::TR);

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, c = lane & 15;
    const int hg = wv % NHG, dh = wv / NHG;  // head group, half of d
    const int64_t row = blockIdx.x / a.n_splits;
    const int split = blockIdx.x % a.n_splits;
    const int64_t b = row / a.Tq, t = (a.pos ? a.pos[b] : a.q_pos0) + row % a.Tq;
    const int64_t nv = n_visible(t, a.m, a.N);
    const int64_t n_slots = a.k > 0 ? a.k : nv;
    const int64_t w0 = t - a.W + 1 > 0 ? t - a.W + 1 : 0;
    const int64_t n_win = a.W > 0 ? t - w0 + 1 : 0;
    const int64_t n_rows = n_slots + n_win;
    const int64_t n_tiles_all = (n_rows + S::TR - 1) / S::TR;
    const int64_t tile_lo = (int64_t)split * a.tiles_per_split;
    const int ntiles = (int)max((int64_t)0, min(n_tiles_all, tile_lo + a.tiles_per_split) - tile_lo);
    const int head = hg * 16 + c;
    const bool wave_on = hg * 16 < a.H && (S::SPLITD == 2 || wv < NHG);
    const float scale2 = a.scale * kLog2e;
    const int dcol0 = dh * S::DW;  // first latent column of this wave

    // Q^T fragments over the wave's columns (B operand of the logits product)
    const T *qrow = (const T *)a.q + (row * a.H + min(head, a.H - 1)) * (int64_t)D + dcol0 + g * E::KPL;
    typename E::frag qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const typename E::frag v = E::load(qrow + ks * E::KSTEP);
        qf[ks] = head < a.H ? v : E::zero();
    }

    // resolve the split's row addresses once; masked rows (weight 0, marked in
    // vmask) load the query's own first row, in bounds and finite
    const T *ent = (const T *)a.entries;
    const T *raw_b = (const T *)a.raw + b * a.raw_bs;
    const T *fallback = (const T *)a.q + row * a.H * (int64_t)D;
    const int nr = ntiles * S::TR;
    for (int i0 = 0; i0 < nr; i0 += kMqaThreads) {
        const int i = i0 + tid;
        const T *src = nullptr;
        if (i < nr) {
            const int64_t r = tile_lo * S::TR + i;
            if (r < n_slots) {
                const int64_t j = a.k > 0 ? (int64_t)a.idx[row * a.k + r] : r;
                if (j >= 0 && j < nv) src = ent + a.em.offset(b, j, D);
            } else if (r < n_rows) {
                const int64_t p = w0 + (r - n_slots);
                src = raw_b + (a.raw_ring ? p % a.raw_ring : p - a.raw_pos0) * D;
            }
            rtab[i] = src ? src : fallback;
        }
        const uint64_t bal = __ballot(src != nullptr);  // bits of tiles i/32 (lanes 0-31) and i/32+1
        if (i < nr && (lane & 31) == 0) vmask[i >> 5] = (uint32_t)(lane ? bal >> 32 : bal);
    }
    // vmcnt(0) through the intrinsic, so the compiler knows the Q^T loads have
    // landed and puts no wait for them inside the tile loop
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();

    floatx4 o[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[nb] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m_ref = -INFINITY, l_run = 0.f;  // base-2 reference maximum, running sum

    if (ntiles > 0) {
        // wave wv loads rows wv*TR/NW .. of local tile lt into stage lt % STAGES
        auto issue = [&](int lt) {
            unsigned char *buf = tiles + (lt % S::STAGES) * S::TILEB;
#pragma unroll
            for (int u = 0; u < S::TR / S::NW; ++u) {
                const int r = wv * (S::TR / S::NW) + u;
                const unsigned char *gp = (const unsigned char *)rtab[lt * S::TR + r] + lane * 16;
#pragma unroll
                for (int ip = 0; ip < S::IPR; ++ip) {
                    if (S::LPI == 64 || lane < S::LPI)
                        dma16(buf + row_slot(r) * S::RS + ip * 1024, gp + ip * 1024);
                }
            }
        };
#pragma unroll
        for (int s = 0; s < S::STAGES - 1; ++s)
            if (s < ntiles) issue(s);

        // per-lane LDS byte offsets (the rest are immediates)
        const int cb = dcol0 * (int)sizeof(T);
        const int k_off = row_slot(c) * S::RS + cb + g * E::KPL * (int)sizeof(T);  // logits, rows c (+16)
        const int v_off1 = row_slot(4 * g + (c >> 2)) * S::RS + cb + 8 * (c & 3);  // transposing, rows 4g..

        // logits of tile lt over this wave's half of d (S^T: rows 4g+e (+16), head c)
        auto logits = [&](int lt, floatx4 (&sacc)[2]) {
            const unsigned char *buf = tiles + (lt % S::STAGES) * S::TILEB;
            // all K fragments of both row blocks first, so the reads overlap;
            // then four independent accumulation chains (row block x K-step parity)
            typename E::frag kf[2][KS];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    kf[rb][ks] = *(const typename E::frag *)(buf + k_off + rb * 16 * S::RS +
                                                             ks * E::KSTEP * (int)sizeof(T));
            __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of their MFMAs
            floatx4 acc[2][2];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) acc[rb][0] = acc[rb][1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) acc[rb][ks & 1] = E::mma(kf[rb][ks], qf[ks], acc[rb][ks & 1]);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) sacc[rb] = acc[rb][0] + acc[rb][1];
        };
        // online softmax of tile lt's logits and the weighted sum of its rows
        auto softmax_pv = [&](int lt, const floatx4 (&sacc)[2]) {
            const unsigned char *buf = tiles + (lt % S::STAGES) * S::TILEB;
            const uint32_t vm = vmask[lt];
            // raw logits (masked rows -inf); scale2 > 0 keeps the order
            float sv[8];
            if (vm == 0xffffffffu) {
#pragma unroll
                for (int q = 0; q < 8; ++q) sv[q] = sacc[q >> 2][q & 3];
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int rl = (q >> 2) * 16 + 4 * g + (q & 3);
                    sv[q] = (vm >> rl) & 1u ? sacc[q >> 2][q & 3] : -INFINITY;
                }
            }
            float mx = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                             fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            mx *= scale2;  // base-2 logit maximum of this tile
            // move the reference only when the maximum outgrows it by 2^8
            if (mx > m_ref + kLazyRescale) {
                const float alpha = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - mx);
                l_run *= alpha;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) o[nb] *= alpha;
                m_ref = mx;
            }
            // m_ref stays -inf only while no row has been valid: nothing to add
            if (m_ref == -INFINITY) return;
            float p[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                p[q] = __builtin_amdgcn_exp2f(fmaf(sv[q], scale2, -m_ref));  // exp2(-inf) = 0
                l_run += p[q];
            }
            if constexpr (sizeof(T) == 2) {
                bf16x8 hi, lo;
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const __bf16 h = (__bf16)p[q];
                    hi[q] = h;
                    lo[q] = (__bf16)(p[q] - (float)h);
                }
                // lane (g, c) addresses rows 4g + c/4 (and +16), columns nb*16 + 4*(c%4) .. +3; the
                // transposing read hands lane c the column nb*16 + c of rows 4g..4g+3.  Every read of
                // the tile is issued first (the compiler waits for each only before its MFMA), then
                // the high-part products of all column blocks, then the low-part ones
                bf16x8 va[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const v4s v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4s *)(buf + v_off1 + nb * 32));
                    const v4s v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4s *)(buf + v_off1 + 16 * S::RS + nb * 32));
                    va[nb] = __builtin_shufflevector(__builtin_bit_cast(bf16x4_t, v1), __builtin_bit_cast(bf16x4_t, v2),
                                                     0, 1, 2, 3, 4, 5, 6, 7);
                }
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[nb], hi, o[nb], 0, 0, 0);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[nb], lo, o[nb], 0, 0, 0);
            } else {
                // fp32: 16x16x4 steps, one row per lane group: lane (g, c) gives
                // V[rb*16 + 4g + e][nb*16 + c] with the weight of that row
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const int r = (q >> 2) * 16 + 4 * g + (q & 3);
                        const float v = *(const float *)(buf + row_slot(r) * S::RS + cb + (nb * 16 + c) * 4);
                        o[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(v, p[q], o[nb], 0, 0, 0);
                    }
            }
        };
        if constexpr (S::PIPE) {
            // One barrier per tile.  Iteration lt: publish tile lt's partial
            // logits, wait for this wave's share of tile lt+1, barrier (so the
            // logits exchange, tile lt+1 and the end of every wave's use of
            // tile lt-1 are all settled), refill tile lt-1's stage, then the
            // softmax and weighted sum of tile lt and the logits of tile lt+1
            // run back to back.  The exchange is double-buffered by tile parity.
            floatx4 sacc[2];
            if (S::STAGES == 3 && ntiles > 1)
                wait_vm_barrier<S::LPW>();
            else
                wait_vm_barrier<0>();
            if (wave_on) logits(0, sacc);
            for (int lt = 0; lt < ntiles; ++lt) {
                floatx4 *xb = xch + (lt & 1) * (S::NW * 2 * 64);
                if (wave_on) {
                    xb[(wv * 2 + 0) * 64 + lane] = sacc[0];
                    xb[(wv * 2 + 1) * 64 + lane] = sacc[1];
                }
                wait_vm_barrier<0>();
                if (lt + S::STAGES - 1 < ntiles) issue(lt + S::STAGES - 1);
                if (wave_on) {
                    const int pw = wv ^ NHG;
                    sacc[0] += xb[(pw * 2 + 0) * 64 + lane];
                    sacc[1] += xb[(pw * 2 + 1) * 64 + lane];
                    softmax_pv(lt, sacc);
                    if (lt + 1 < ntiles) logits(lt + 1, sacc);
                }
            }
        } else {
            for (int lt = 0; lt < ntiles; ++lt) {
                // wait until this tile's loads landed (STAGES-2 younger tiles may
                // still fly); the barrier also proves every wave is done with the
                // previous tile, whose stage the next DMA reuses
                const int younger = min(ntiles - 1 - lt, S::STAGES - 2);
                if (S::STAGES == 3 && younger == 1)
                    wait_vm_barrier<S::LPW>();
                else
                    wait_vm_barrier<0>();
                if (lt + S::STAGES - 1 < ntiles) issue(lt + S::STAGES - 1);
                floatx4 sacc[2];
                if (wave_on) logits(lt, sacc);
                if constexpr (S::SPLITD == 2) {
                    // sum the two halves of the logits: publish, barrier, add the partner's
                    if (wave_on) {
                        xch[(wv * 2 + 0) * 64 + lane] = sacc[0];
                        xch[(wv * 2 + 1) * 64 + lane] = sacc[1];
                    }
                    lds_barrier();
                    if (wave_on) {
                        const int pw = wv ^ NHG;
                        sacc[0] += xch[(pw * 2 + 0) * 64 + lane];
                        sacc[1] += xch[(pw * 2 + 1) * 64 + lane];
                    }
                }
                if (wave_on) softmax_pv(lt, sacc);
            }
        }
    }

    if (!wave_on) return;
    float l = l_run;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (head >= a.H) return;
    if (a.n_splits == 1) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        float *orow = a.out + (row * a.H + head) * (int64_t)D + dcol0 + 4 * g;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) *(floatx4 *)(orow + nb * 16) = o[nb] * inv;
        if (a.lse && g == 0 && dh == 0) a.lse[row * a.H + head] = l > 0.f ? (m_ref + __log2f(l)) * kLn2 : -INFINITY;
    } else {
        const int64_t slot = (row * a.n_splits + split) * a.H + head;
        float *po = a.part_o + slot * D + dcol0 + 4 * g;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) *(floatx4 *)(po + nb * 16) = o[nb];
        if (g == 0 && dh == 0) {
            a.part_ml[slot * 2 + 0] = m_ref;  // base 2
            a.part_ml[slot * 2 + 1] = l;
        }
    }
}

// Merge the split-K partials of one (query, head): a 4-wide column slice
// per thread.  Splits are taken CB at a time (the split count rounded up to a
// multiple of four, at most kMqaMaxSplits), every (max, sum)
// and column slice of a batch loaded up front (indices past n_splits reread
// the last split with zero weight) so the loads are in flight together.
// Maxima are base-2; empty splits carry l = 0 and get weight 0.
template <int CB>
__global__ __launch_bounds__(128) void k_combine(int H, int D, int n_splits, const float *__restrict__ part_o,
                                                 const float *__restrict__ part_ml, float *__restrict__ out,
                                                 float *__restrict__ lse) {
    // rows on the XCD whose L2 holds their partials (the attention kernels place
    // a query's splits by the same rank)
    const int64_t rh = xcd_rank((int)gridDim.x);
    const int64_t row = rh / H;
    const int h = (int)(rh % H);
    const int x = min((int)threadIdx.x * 4, D - 4);
    float M = -INFINITY, L = 0.f;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < n_splits; s0 += CB) {
        float ms[CB], ls[CB];
        floatx4 po[CB];
#pragma unroll
        for (int u = 0; u < CB; ++u) {
            const int64_t slot = (row * n_splits + min(s0 + u, n_splits - 1)) * H + h;
            ms[u] = part_ml[slot * 2];
            ls[u] = s0 + u < n_splits ? part_ml[slot * 2 + 1] : 0.f;
            po[u] = *(const floatx4 *)(part_o + slot * D + x);
        }
        float Mc = M;
#pragma unroll
        for (int u = 0; u < CB; ++u) Mc = ls[u] > 0.f ? fmaxf(Mc, ms[u]) : Mc;
        if (Mc > M) {  // (more than one batch of splits only)
            const float sc = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mc);
            L *= sc;
            acc *= sc;
            M = Mc;
        }
#pragma unroll
        for (int u = 0; u < CB; ++u) {
            const float wgt = ls[u] > 0.f ? __builtin_amdgcn_exp2f(ms[u] - M) : 0.f;
            L += ls[u] * wgt;
            acc += wgt * po[u];
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    if ((int)threadIdx.x * 4 < D) *(floatx4 *)(out + rh * D + x) = acc * inv;
    if (lse && threadIdx.x == 0) lse[rh] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

// The same merge for the wide kernel's partials: f16 normalised partials
// O_s / l_s / sigma_s, so split s enters with weight l_s 2^(m_s - M) sigma_s.
template <int CB>
__global__ __launch_bounds__(128) void k_combine16(int H, int D, int n_splits, const _Float16 *__restrict__ part_o,
                                                   const float *__restrict__ part_ml,
                                                   const float *__restrict__ part_sc, float *__restrict__ out,
                                                   float *__restrict__ lse) {
    typedef _Float16 halfx4 __attribute__((ext_vector_type(4)));
    const int64_t rh = xcd_rank((int)gridDim.x);
    const int64_t row = rh / H;
    const int h = (int)(rh % H);
    const int x = min((int)threadIdx.x * 4, D - 4);
    float M = -INFINITY, L = 0.f;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < n_splits; s0 += CB) {
        float ms[CB], ls[CB], ss[CB];
        halfx4 po[CB];
#pragma unroll
        for (int u = 0; u < CB; ++u) {
            const int64_t rs = row * n_splits + min(s0 + u, n_splits - 1);
            const int64_t slot = rs * H + h;
            ms[u] = part_ml[slot * 2];
            ls[u] = s0 + u < n_splits ? part_ml[slot * 2 + 1] : 0.f;
            ss[u] = part_sc[rs];
            po[u] = *(const halfx4 *)(part_o + slot * D + x);
        }
        float Mc = M;
#pragma unroll
        for (int u = 0; u < CB; ++u) Mc = ls[u] > 0.f ? fmaxf(Mc, ms[u]) : Mc;
        if (Mc > M) {  // (more than one batch of splits only)
            const float sc = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mc);
            L *= sc;
            acc *= sc;
            M = Mc;
        }
#pragma unroll
        for (int u = 0; u < CB; ++u) {
            const float wl = ls[u] > 0.f ? ls[u] * __builtin_amdgcn_exp2f(ms[u] - M) : 0.f;
            L += wl;
            acc += (wl * ss[u]) * __builtin_convertvector(po[u], floatx4);
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    if ((int)threadIdx.x * 4 < D) *(floatx4 *)(out + rh * D + x) = acc * inv;
    if (lse && threadIdx.x == 0) lse[rh] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

int mqa_choose_splits(int64_t rows, int64_t n_rows_max, int d, int *tiles_per_split) {
    int64_t tiles = (n_rows_max + 31) / 32;
    if (tiles < 1) tiles = 1;
    int64_t s = (kMqaTargetBlocks + rows - 1) / rows;
    if (s > kMqaMaxSplits) s = kMqaMaxSplits;
    if (s < 1) s = 1;
    if (s > tiles) s = tiles;
    int64_t tps = (tiles + s - 1) / s;
    if (tps > mqa_max_tiles_per_split(d)) tps = mqa_max_tiles_per_split(d);  // bounds the LDS row table
    s = (tiles + tps - 1) / tps;
    *tiles_per_split = (int)tps;
    return (int)s;
}

static hipError_t launch_combine(const MqaArgs &a, int64_t rows, int D, hipStream_t st) {
    if (a.n_splits == 1) return hipSuccess;
    // one batch of partial loads per thread, rounded up to a multiple of four splits
    const dim3 grid((unsigned)(rows * a.H));
    if (a.n_splits <= 4)
        hipLaunchKernelGGL(k_combine<4>, grid, dim3(128), 0, st, a.H, D, a.n_splits, a.part_o, a.part_ml, a.out,
                           a.lse);
    else if (a.n_splits <= 8)
        hipLaunchKernelGGL(k_combine<8>, grid, dim3(128), 0, st, a.H, D, a.n_splits, a.part_o, a.part_ml, a.out,
                           a.lse);
    else if (a.n_splits <= 12)
        hipLaunchKernelGGL(k_combine<12>, grid, dim3(128), 0, st, a.H, D, a.n_splits, a.part_o, a.part_ml, a.out,
                           a.lse);
    else
        hipLaunchKernelGGL(k_combine<kMqaMaxSplits>, grid, dim3(128), 0, st, a.H, D, a.n_splits, a.part_o,
                           a.part_ml, a.out, a.lse);
    return hipGetLastError();
}

static hipError_t launch_combine16(const MqaArgs &a, int64_t rows, int D, hipStream_t st) {
    if (a.n_splits == 1) return hipSuccess;
    const dim3 grid((unsigned)(rows * a.H));
    const _Float16 *po = (const _Float16 *)a.part_o;
    if (a.n_splits <= 4)
        hipLaunchKernelGGL(k_combine16<4>, grid, dim3(128), 0, st, a.H, D, a.n_splits, po, a.part_ml, a.part_sc,
                           a.out, a.lse);
    else if (a.n_splits <= 8)
        hipLaunchKernelGGL(k_combine16<8>, grid, dim3(128), 0, st, a.H, D, a.n_splits, po, a.part_ml, a.part_sc,
                           a.out, a.lse);
    else if (a.n_splits <= 12)
        hipLaunchKernelGGL(k_combine16<12>, grid, dim3(128), 0, st, a.H, D, a.n_splits, po, a.part_ml, a.part_sc,
                           a.out, a.lse);
    else
        hipLaunchKernelGGL(k_combine16<kMqaMaxSplits>, grid, dim3(128), 0, st, a.H, D, a.n_splits, po, a.part_ml,
                           a.part_sc, a.out, a.lse);
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_mqa_t(const MqaArgs &a, int64_t rows, hipStream_t st) {
    using S = MqaShape<T, D>;
    // one-time opt-in to the largest dynamic LDS this instantiation may use
    static const hipError_t attr = hipFuncSetAttribute((const void *)k_mqa<T, D>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (attr != hipSuccess) return attr;
    const size_t lds = S::lds_bytes(a.tiles_per_split);
    if (lds > 160 * 1024) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_mqa<T, D>), dim3((unsigned)(rows * a.n_splits)), dim3(kMqaThreads), lds, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_combine(a, rows, D, st);
}

template <typename T>
static hipError_t launch_mqa_dt(int d, const MqaArgs &a, int64_t rows, hipStream_t st) {
    switch (d) {
        case 32: return launch_mqa_t<T, 32>(a, rows, st);
        case 64: return launch_mqa_t<T, 64>(a, rows, st);
        case 128: return launch_mqa_t<T, 128>(a, rows, st);
        case 256: return launch_mqa_t<T, 256>(a, rows, st);
        default: return launch_mqa_t<T, 512>(a, rows, st);
    }
}

hipError_t launch_mqa(int dt, int B, int Tq, int H, int d, int N, int m, int k, int W, QPos q_pos0, float scale,
                      const void *q, const void *entries, RowMap e_bs, const int32_t *idx, const void *raw,
                      int64_t raw_bs, int64_t raw_pos0, int64_t raw_ring, float *out, float *lse, float *ws,
                      int n_splits, int tiles_per_split, hipStream_t st) {
    const int64_t rows = (int64_t)B * Tq;
    MqaArgs a;
    a.Tq = Tq; a.H = H; a.N = N; a.m = m; a.k = k; a.W = W;
    a.n_splits = n_splits; a.tiles_per_split = tiles_per_split;
    a.q_pos0 = q_pos0.q_pos0; a.pos = q_pos0.pos; a.raw_ring = raw_ring; a.raw_pos0 = raw_pos0; a.em = e_bs; a.raw_bs = raw_bs; a.scale = scale;
    a.q = q; a.entries = entries; a.raw = raw; a.idx = idx; a.out = out; a.lse = lse;
    a.part_o = ws;
    a.part_ml = ws ? ws + rows * n_splits * H * (int64_t)d : nullptr;
    // (the wide kernel's f16 partials fill half of part_o; their scales follow)
    a.part_sc = ws ? (float *)((char *)ws + rows * n_splits * H * (int64_t)d * 2) : nullptr;
    if (dt == 0) return launch_mqa_dt<float>(d, a, rows, st);
    if (d == 512 && H > 32) {
        // 32-head waves with 32x32x16 MFMAs (mqa_wide.hip)
        const hipError_t e = launch_mqa_wide(a, rows, st);
        if (e != hipSuccess) return e;
        return launch_combine16(a, rows, d, st);
    }
    return launch_mqa_dt<bf16_t>(d, a, rows, st);
}

}  // namespace csa
