// Shared-KV multi-query attention over compressed entries plus a window of
// raw tokens, in one softmax (DeepSeek-V4 overview page, section 2.2 step 3:
// the selected entries are both key and value and every query head shares
// them; section 2.3: HCA attends to every entry).
//
// Grid.  One 256-thread workgroup per (query, split) of the query's row
// list; split-K partials (unnormalised O, running max, running sum) are merged
// by k_combine.  With a single split the workgroup writes the final output.
//
// Workgroup.  Four wavefronts, each owning 16 query heads.  The split's row
// addresses (gathered entries, then raw window rows) are resolved once into
// an LDS table.  Tiles of 32 rows then stream HBM -> LDS with asynchronous
// 16-byte LDS-DMA loads (global_load_lds_dwordx4), STAGES tiles in flight,
// so no register staging and no dependent global load sits in the loop.  A
// tile is stored row-major with the 16-byte chunks of row r XOR-swizzled by
// swz(r); the swizzle is applied by choosing which source chunk each lane
// fetches.  Per wave and tile:
//   S^T[32 rows x 16 heads] = K . Q^T   (MFMA; K rows read with ds_read_b128,
//                                        Q^T held in registers)
//   online softmax per head (running max / sum per lane, fp32)
//   O^T[d x 16 heads]      += V^T . P^T  (MFMA; V^T read straight from the
//                                        row-major tile with the gfx950
//                                        transposing ds_read_b64_tr_b16; P is
//                                        split into bf16 high and low parts so
//                                        the weights keep ~16 bits)
// O^T stays in registers (d/16 accumulator tiles per wave).  fp32 data uses
// the 16x16x4 f32 MFMA with scalar LDS reads instead.
#include "kernels.h"

namespace csa {

struct MqaArgs {
    int Tq, H, N, m, k, W, n_splits, tiles_per_split;
    int64_t q_pos0, raw_pos0, e_bs, raw_bs;
    float scale;
    const void *q, *entries, *raw;
    const int32_t *idx;
    float *out, *lse, *part_o, *part_ml;
};

template <typename T, int D>
struct MqaShape {
    static constexpr int TR = 32;                      // rows per tile
    static constexpr int ROWB = D * (int)sizeof(T);    // bytes per row
    static constexpr int CPR = ROWB / 16;              // 16-byte chunks per row
    static constexpr int TILEB = TR * ROWB;            // bytes per tile
    static constexpr int NI = TILEB / 1024;            // DMA instructions per tile (1 KiB each)
    static constexpr int LPW = NI / 4;                 // ... per wavefront
    // tiles in flight: three for tiles up to 32 KiB, two up to 64 KiB; narrow
    // rows (fewer than four loads per tile) are not pipelined
    static constexpr int STAGES = LPW < 1 ? 1 : (TILEB <= 32768 ? 3 : (TILEB <= 65536 ? 2 : 1));
    static size_t lds_bytes(int tiles_per_split) {
        return (size_t)STAGES * TILEB + (size_t)tiles_per_split * TR * sizeof(void *);
    }
};

// chunk swizzle of tile row r: bijective on the low 4 bits, and rows
// 4g..4g+3 map to chunks differing in bits 1..3 so that transposing reads
// of 4 rows x 2 chunks and row-parallel reads of 16 rows avoid bank conflicts
template <int CPR>
__device__ __forceinline__ int swz(int r) {
    return ((((r & 7) << 1) | ((r >> 3) & 1)) | (r & ~15)) & (CPR - 1);
}

template <int CPR>
__device__ __forceinline__ int tile_off(int r, int byte) {
    return r * CPR * 16 + ((((byte >> 4) ^ swz<CPR>(r)) << 4) | (byte & 15));
}

// 16 bytes per lane from `src` into LDS at lds_base + 16 * lane.  Issued from
// inline assembly so that the compiler does not treat every later LDS read as
// dependent on it (it would drain all tiles in flight); completion is awaited
// explicitly with wait_vm_barrier.  One wait state separates the M0 write
// from the LDS-DMA instruction, as the ISA requires.
__device__ __forceinline__ void dma16(const void *lds_base, const void *src) {
    const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(l), "v"(src)
                 : "memory", "m0");
}
// wait until at most N vector-memory operations of this wave are in flight,
// then barrier; one statement, so no LDS access is scheduled across it
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

typedef short v4s __attribute__((ext_vector_type(4)));

template <typename T, int D>
__global__ __launch_bounds__(256) void k_mqa(const MqaArgs a) {
    using E = Elem<T>;
    using S = MqaShape<T, D>;
    constexpr int KS = D / E::KSTEP;
    constexpr int NB = D / 16;
    constexpr int CPR = S::CPR;
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char *tiles = smem;
    const T **rtab = (const T **)(smem + S::STAGES * S::TILEB);

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, c = lane & 15;
    const int64_t row = blockIdx.x / a.n_splits;
    const int split = blockIdx.x % a.n_splits;
    const int64_t b = row / a.Tq, t = a.q_pos0 + row % a.Tq;
    const int64_t nv = n_visible(t, a.m, a.N);
    const int64_t n_slots = a.k > 0 ? a.k : nv;
    const int64_t w0 = t - a.W + 1 > 0 ? t - a.W + 1 : 0;
    const int64_t n_win = a.W > 0 ? t - w0 + 1 : 0;
    const int64_t n_rows = n_slots + n_win;
    const int64_t n_tiles_all = (n_rows + S::TR - 1) / S::TR;
    const int64_t tile_lo = (int64_t)split * a.tiles_per_split;
    const int ntiles = (int)max((int64_t)0, min(n_tiles_all, tile_lo + a.tiles_per_split) - tile_lo);
    const int head = wv * 16 + c;
    const bool wave_on = wv * 16 < a.H;

    // Q^T fragments (B operand of the logits product)
    const T *qrow = (const T *)a.q + (row * a.H + head) * (int64_t)D + g * E::KPL;
    typename E::frag qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = (wave_on && head < a.H) ? E::load(qrow + ks * E::KSTEP) : E::zero();

    // resolve the split's row addresses once (nullptr = masked row)
    const T *ent_b = (const T *)a.entries + b * a.e_bs;
    const T *raw_b = (const T *)a.raw + b * a.raw_bs;
    const int nr = ntiles * S::TR;
    for (int i = tid; i < nr; i += 256) {
        const int64_t r = tile_lo * S::TR + i;
        const T *src = nullptr;
        if (r < n_slots) {
            const int64_t j = a.k > 0 ? (int64_t)a.idx[row * a.k + r] : r;
            if (j >= 0 && j < nv) src = ent_b + j * D;
        } else if (r < n_rows) {
            src = raw_b + (w0 + (r - n_slots) - a.raw_pos0) * D;
        }
        rtab[i] = src;
    }
    // vmcnt(0) through the intrinsic, so the compiler knows the Q^T loads have
    // landed and puts no wait for them inside the tile loop
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    // any valid row of the split stands in for masked rows (their weight is 0)
    const T *dummy = nullptr;
    for (int i = 0; i < nr && !dummy; ++i) dummy = rtab[i];

    floatx4 o[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[nb] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    if (dummy) {
        // issue the DMA of local tile `lt` into stage buffer lt % STAGES
        auto issue = [&](int lt) {
            unsigned char *buf = tiles + (lt % S::STAGES) * S::TILEB;
            if constexpr (S::LPW >= 1) {
#pragma unroll
                for (int u = 0; u < S::LPW; ++u) {
                    const int ins = u * 4 + wv;
                    const int q = ins * 64 + lane;  // chunk index within the tile
                    const int r = q / CPR, pc = q % CPR;
                    const T *src = rtab[lt * S::TR + r];
                    src = src ? src : dummy;
                    const unsigned char *gp = (const unsigned char *)src + ((pc ^ swz<CPR>(r)) << 4);
                    dma16(buf + ins * 1024, gp);
                }
            } else {
                // narrow rows: fewer than four 1 KiB loads per tile
                for (int ins = wv; ins < S::NI; ins += 4) {
                    const int q = ins * 64 + lane;
                    const int r = q / CPR, pc = q % CPR;
                    const T *src = rtab[lt * S::TR + r];
                    src = src ? src : dummy;
                    const unsigned char *gp = (const unsigned char *)src + ((pc ^ swz<CPR>(r)) << 4);
                    dma16(buf + ins * 1024, gp);
                }
            }
        };
#pragma unroll
        for (int s = 0; s < S::STAGES - 1; ++s)
            if (s < ntiles) issue(s);

        for (int lt = 0; lt < ntiles; ++lt) {
            // keep STAGES-1 younger tiles in flight; wait until this tile's own loads landed
            if (lt + S::STAGES - 1 < ntiles) issue(lt + S::STAGES - 1);
            const int younger = min(ntiles - 1 - lt, S::STAGES - 1);
            if (S::STAGES == 3 && younger == 2)
                wait_vm_barrier<2 * S::LPW>();
            else if (S::STAGES >= 2 && younger == 1)
                wait_vm_barrier<S::LPW>();
            else
                wait_vm_barrier<0>();
            const unsigned char *buf = tiles + (lt % S::STAGES) * S::TILEB;
            const T *const *rt = rtab + lt * S::TR;
            if (wave_on) {
                floatx4 sacc[2];
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    sacc[rb] = floatx4{0.f, 0.f, 0.f, 0.f};
                    const int r = rb * 16 + c;
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const int byte = (ks * E::KSTEP + g * E::KPL) * (int)sizeof(T);
                        const typename E::frag kf = *(const typename E::frag *)(buf + tile_off<CPR>(r, byte));
                        sacc[rb] = E::mma(kf, qf[ks], sacc[rb]);
                    }
                }
                float sv[8];
                float mx = -INFINITY;
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int rl = (q >> 2) * 16 + 4 * g + (q & 3);
                    sv[q] = rt[rl] ? sacc[q >> 2][q & 3] * a.scale : -INFINITY;
                    mx = fmaxf(mx, sv[q]);
                }
                mx = fmaxf(mx, __shfl_xor(mx, 16));
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                const float m_new = fmaxf(m_run, mx);
                const float alpha = m_new == -INFINITY ? 1.f : expf(m_run - m_new);
                float p[8], psum = 0.f;
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    p[q] = sv[q] == -INFINITY ? 0.f : expf(sv[q] - m_new);
                    psum += p[q];
                }
                l_run = l_run * alpha + psum;
                m_run = m_new;
                if (__ballot(alpha != 1.f)) {
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) o[nb] *= alpha;
                }
                if constexpr (sizeof(T) == 2) {
                    bf16x8 hi, lo;
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const bf16_t h = f32_to_bf16(p[q]);
                        hi[q] = __builtin_bit_cast(__bf16, h);
                        lo[q] = __builtin_bit_cast(__bf16, f32_to_bf16(p[q] - bf16_to_f32(h)));
                    }
                    // lane (g, c) addresses rows 4g + c/4 (and +16), columns nb*16 + 4*(c%4) .. +3;
                    // the transposing read hands lane c the column nb*16 + c of rows 4g..4g+3
                    const int r1 = 4 * g + (c >> 2), r2 = r1 + 16;
                    const int cb = 8 * (c & 3);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        const int byte = nb * 32 + cb;
                        const v4s v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) v4s *)(buf + tile_off<CPR>(r1, byte)));
                        const v4s v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) v4s *)(buf + tile_off<CPR>(r2, byte)));
                        const bf16x8 va = __builtin_shufflevector(__builtin_bit_cast(bf16x4_t, v1),
                                                                  __builtin_bit_cast(bf16x4_t, v2), 0, 1, 2, 3, 4,
                                                                  5, 6, 7);
                        o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, hi, o[nb], 0, 0, 0);
                        o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, lo, o[nb], 0, 0, 0);
                    }
                } else {
                    // fp32: 16x16x4 steps, one row per lane group: lane (g, c) gives
                    // V[rb*16 + 4g + e][nb*16 + c] with the weight of that row
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                        for (int q = 0; q < 8; ++q) {
                            const int r = (q >> 2) * 16 + 4 * g + (q & 3);
                            const float v = *(const float *)(buf + tile_off<CPR>(r, (nb * 16 + c) * 4));
                            o[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(v, p[q], o[nb], 0, 0, 0);
                        }
                }
            }
            lds_barrier();
        }
    }

    if (!wave_on) return;
    float l = l_run;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (head >= a.H) return;
    if (a.n_splits == 1) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        float *orow = a.out + (row * a.H + head) * (int64_t)D + 4 * g;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) *(floatx4 *)(orow + nb * 16) = o[nb] * inv;
        if (a.lse && g == 0) a.lse[row * a.H + head] = l > 0.f ? m_run + logf(l) : -INFINITY;
    } else {
        const int64_t slot = (row * a.n_splits + split) * a.H + head;
        float *po = a.part_o + slot * D + 4 * g;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) *(floatx4 *)(po + nb * 16) = o[nb];
        if (g == 0) {
            a.part_ml[slot * 2 + 0] = m_run;
            a.part_ml[slot * 2 + 1] = l;
        }
    }
}

// Merge the split-K partials of one (query, head): a 4-wide column slice
// per thread.  Empty splits carry l = 0 and are skipped.
__global__ __launch_bounds__(128) void k_combine(int H, int D, int n_splits, const float *__restrict__ part_o,
                                                 const float *__restrict__ part_ml, float *__restrict__ out,
                                                 float *__restrict__ lse) {
    const int64_t rh = blockIdx.x;
    const int64_t row = rh / H;
    const int h = (int)(rh % H);
    float M = -INFINITY;
    for (int s = 0; s < n_splits; ++s) {
        const int64_t slot = (row * n_splits + s) * H + h;
        if (part_ml[slot * 2 + 1] > 0.f) M = fmaxf(M, part_ml[slot * 2]);
    }
    float L = 0.f;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    const int x = threadIdx.x * 4;
    for (int s = 0; s < n_splits; ++s) {
        const int64_t slot = (row * n_splits + s) * H + h;
        const float ls = part_ml[slot * 2 + 1];
        if (ls > 0.f) {
            const float wgt = expf(part_ml[slot * 2] - M);
            L += ls * wgt;
            if (x < D) acc += wgt * *(const floatx4 *)(part_o + slot * D + x);
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    if (x < D) *(floatx4 *)(out + rh * D + x) = acc * inv;
    if (lse && threadIdx.x == 0) lse[rh] = L > 0.f ? M + logf(L) : -INFINITY;
}

int mqa_choose_splits(int64_t rows, int64_t n_rows_max, int *tiles_per_split) {
    int64_t tiles = (n_rows_max + 31) / 32;
    if (tiles < 1) tiles = 1;
    int64_t s = (kMqaTargetBlocks + rows - 1) / rows;
    if (s > kMqaMaxSplits) s = kMqaMaxSplits;
    if (s < 1) s = 1;
    if (s > tiles) s = tiles;
    int64_t tps = (tiles + s - 1) / s;
    if (tps > kMqaMaxTilesPerSplit) tps = kMqaMaxTilesPerSplit;  // bounds the LDS row table
    s = (tiles + tps - 1) / tps;
    *tiles_per_split = (int)tps;
    return (int)s;
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
    hipLaunchKernelGGL((k_mqa<T, D>), dim3((unsigned)(rows * a.n_splits)), dim3(256), lds, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.n_splits == 1) return e;
    hipLaunchKernelGGL(k_combine, dim3((unsigned)(rows * a.H)), dim3(128), 0, st, a.H, D, a.n_splits, a.part_o,
                       a.part_ml, a.out, a.lse);
    return hipGetLastError();
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

hipError_t launch_mqa(int dt, int B, int Tq, int H, int d, int N, int m, int k, int W, int64_t q_pos0, float scale,
                      const void *q, const void *entries, int64_t e_bs, const int32_t *idx, const void *raw,
                      int64_t raw_bs, int64_t raw_pos0, float *out, float *lse, float *ws, int n_splits,
                      int tiles_per_split, hipStream_t st) {
    const int64_t rows = (int64_t)B * Tq;
    MqaArgs a;
    a.Tq = Tq; a.H = H; a.N = N; a.m = m; a.k = k; a.W = W;
    a.n_splits = n_splits; a.tiles_per_split = tiles_per_split;
    a.q_pos0 = q_pos0; a.raw_pos0 = raw_pos0; a.e_bs = e_bs; a.raw_bs = raw_bs; a.scale = scale;
    a.q = q; a.entries = entries; a.raw = raw; a.idx = idx; a.out = out; a.lse = lse;
    a.part_o = ws;
    a.part_ml = ws ? ws + rows * n_splits * H * (int64_t)d : nullptr;
    if (dt == 0) return launch_mqa_dt<float>(d, a, rows, st);
    return launch_mqa_dt<bf16_t>(d, a, rows, st);
}

}  // namespace csa
