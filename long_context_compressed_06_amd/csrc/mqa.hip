// Shared-KV multi-query attention over compressed entries plus a window of
// raw tokens, in one softmax (DeepSeek-V4 overview page, section 2.2 step 3:
// the selected entries are both key and value and every query head shares
// them; section 2.3: HCA attends to every entry).
//
// Grid.  One 256-thread workgroup per (query, split) of the query's row
// list; split-K partials (unnormalised O, running max, running sum) are merged
// by k_combine.  With a single split the workgroup writes the final output.
//
// Workgroup.  Four wavefronts, each owning 16 query heads.  A tile of 32 rows
// (gathered entries or raw window rows) is copied from HBM to LDS twice:
// row-major (Kt) for the logits and d-major (Vt) for the weighted sum, with
// rows ordered inside each d-row so that every lane's MFMA operand is one
// contiguous 16-byte LDS read.  Per wave and tile:
//   S^T[32 rows x 16 heads] = Kt . Q^T   (MFMA, Q^T held in registers)
//   online softmax per head (running max / sum kept per lane, fp32)
//   O^T[d x 16 heads]     += Vt . P^T    (MFMA; P split into a bf16 high part
//                                         and a bf16 low part for bf16 data so
//                                         the weights keep ~16 bits)
// O^T lives in registers (d/16 accumulator tiles per wave).
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
    static constexpr int VEC = 16 / sizeof(T);  // elements per 16-byte chunk
    static constexpr int TR = 32;               // rows per tile
    static constexpr int KROW = D + VEC;        // padded row of Kt (elements)
    static constexpr int VROW = TR + VEC;       // padded d-row of Vt (elements)
    static constexpr size_t lds_bytes =
        (size_t)(TR * KROW + D * VROW) * sizeof(T) + TR * sizeof(void *);
};

// slot of tile row r inside a d-row of Vt: lane group g's rows {4g..4g+3,
// 16+4g..16+4g+3} become the contiguous slots 8g .. 8g+7
__device__ __forceinline__ int vt_slot(int r) { return 8 * ((r & 15) >> 2) + 4 * (r >> 4) + (r & 3); }

template <typename T, int D>
__global__ __launch_bounds__(256) void k_mqa(const MqaArgs a) {
    using E = Elem<T>;
    using S = MqaShape<T, D>;
    constexpr int KS = D / E::KSTEP;
    constexpr int NB = D / 16;
    constexpr int CPR = D / S::VEC;
    extern __shared__ __align__(16) unsigned char smem[];
    T *Kt = (T *)smem;
    T *Vt = Kt + S::TR * S::KROW;
    const T **rsrc = (const T **)(Vt + D * S::VROW);

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, c = lane & 15;
    const int64_t row = blockIdx.x / a.n_splits;
    const int split = blockIdx.x % a.n_splits;
    const int64_t b = row / a.Tq, t = a.q_pos0 + row % a.Tq;
    const int64_t nv = n_visible(t, a.m, a.N);
    const int64_t n_slots = a.k > 0 ? a.k : nv;
    const int64_t w0 = t - a.W + 1 > 0 ? t - a.W + 1 : 0;
    const int64_t n_win = a.W > 0 ? t - w0 + 1 : 0;
    const int64_t n_rows = n_slots + n_win;
    const int64_t n_tiles = (n_rows + S::TR - 1) / S::TR;
    const int64_t tile_lo = (int64_t)split * a.tiles_per_split;
    const int64_t tile_hi = min(n_tiles, tile_lo + a.tiles_per_split);
    const int head = wv * 16 + c;
    const bool wave_on = wv * 16 < a.H;

    const T *qrow = (const T *)a.q + (row * a.H + head) * (int64_t)D + g * E::KPL;
    typename E::frag qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = (wave_on && head < a.H) ? E::load(qrow + ks * E::KSTEP) : E::zero();

    floatx4 o[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[nb] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    const T *ent_b = (const T *)a.entries + b * a.e_bs;
    const T *raw_b = (const T *)a.raw + b * a.raw_bs;
    for (int64_t tile = tile_lo; tile < tile_hi; ++tile) {
        if (tid < S::TR) {
            const int64_t r = tile * S::TR + tid;
            const T *src = nullptr;
            if (r < n_slots) {
                const int64_t j = a.k > 0 ? (int64_t)a.idx[row * a.k + r] : r;
                if (j >= 0 && j < nv) src = ent_b + j * D;
            } else if (r < n_rows) {
                src = raw_b + (w0 + (r - n_slots) - a.raw_pos0) * D;
            }
            rsrc[tid] = src;
        }
        __syncthreads();
        for (int ci = tid; ci < S::TR * CPR; ci += 256) {
            const int rr = ci / CPR, cc = ci % CPR;
            const T *src = rsrc[rr];
            const u32x4 v = src ? *(const u32x4 *)(src + cc * S::VEC) : u32x4{0u, 0u, 0u, 0u};
            *(u32x4 *)(Kt + rr * S::KROW + cc * S::VEC) = v;
            const T *ve = (const T *)&v;
            const int slot = vt_slot(rr);
#pragma unroll
            for (int e = 0; e < S::VEC; ++e) Vt[(cc * S::VEC + e) * S::VROW + slot] = ve[e];
        }
        __syncthreads();
        if (wave_on) {
            floatx4 sacc[2];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                sacc[rb] = floatx4{0.f, 0.f, 0.f, 0.f};
                const T *kr = Kt + (rb * 16 + c) * S::KROW + g * E::KPL;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) sacc[rb] = E::mma(E::load(kr + ks * E::KSTEP), qf[ks], sacc[rb]);
            }
            float sv[8];
            float mx = -INFINITY;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int rl = (q >> 2) * 16 + 4 * g + (q & 3);
                sv[q] = rsrc[rl] ? sacc[q >> 2][q & 3] * a.scale : -INFINITY;
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
            const T *vr = Vt + c * S::VROW + 8 * g;
            if constexpr (sizeof(T) == 2) {
                bf16x8 hi, lo;
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const bf16_t h = f32_to_bf16(p[q]);
                    hi[q] = __builtin_bit_cast(__bf16, h);
                    lo[q] = __builtin_bit_cast(__bf16, f32_to_bf16(p[q] - bf16_to_f32(h)));
                }
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const bf16x8 va = *(const bf16x8 *)(vr + nb * 16 * S::VROW);
                    o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, hi, o[nb], 0, 0, 0);
                    o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, lo, o[nb], 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int q = 0; q < 8; ++q)
                        o[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(((const float *)vr)[nb * 16 * S::VROW + q], p[q],
                                                                     o[nb], 0, 0, 0);
            }
        }
        __syncthreads();
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
    int64_t s = (256 + rows - 1) / rows;
    if (s < 1) s = 1;
    if (s > tiles) s = tiles;
    int64_t tps = (tiles + s - 1) / s;
    s = (tiles + tps - 1) / tps;
    *tiles_per_split = (int)tps;
    return (int)s;
}

template <typename T, int D>
static hipError_t launch_mqa_t(const MqaArgs &a, int64_t rows, hipStream_t st) {
    using S = MqaShape<T, D>;
    // one-time opt-in to more than 64 KiB of dynamic LDS for this instantiation
    static const hipError_t attr = hipFuncSetAttribute(
        (const void *)k_mqa<T, D>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)S::lds_bytes);
    if (attr != hipSuccess) return attr;
    hipError_t e;
    hipLaunchKernelGGL((k_mqa<T, D>), dim3((unsigned)(rows * a.n_splits)), dim3(256), S::lds_bytes, st, a);
    e = hipGetLastError();
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
