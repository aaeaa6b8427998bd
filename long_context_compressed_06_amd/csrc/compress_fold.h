// Group compression as workgroup bodies (DeepSeek-V4 overview page, section
// 2.2 step 1 for m=4 and section 2.3 for m=128), shared by the compression
// kernels and by the top-k filter launch that can carry a decode step's
// compression in workgroups of its own.
#pragma once

#include "kernels.h"

namespace csa {

constexpr int kRowsPerThread = 4;

// One workgroup's share of one group: rows = the group's first row at this
// slice's first column (rows d apart), z = its m logits, o = the entry at this
// slice's first column.
template <typename T>
__device__ __forceinline__ void compress_group(const T *__restrict__ rows, const float *__restrict__ z, int m, int d,
                                               int tpr, T *__restrict__ o) {
    constexpr int VEC = 16 / sizeof(T);  // elements per 16-byte vector
    __shared__ float alpha[128];
    __shared__ float red[256 * VEC];

    const int tid = threadIdx.x, lane = tid & 63;
    const int rpar = 256 / tpr;        // rows accumulated in parallel
    const int c = tid % tpr, rs = tid / tpr;
    const int width = tpr * VEC;       // columns of this slice
    rows += c * VEC;
    u32x4 v[kRowsPerThread];
#pragma unroll
    for (int u = 0; u < kRowsPerThread; ++u) {
        const int i = rs + u * rpar;
        v[u] = i < m ? *(const u32x4 *)(rows + (int64_t)i * d) : u32x4{0u, 0u, 0u, 0u};
    }
    if (tid < 64) {
        const float z0 = lane < m ? z[lane] : -INFINITY;
        const float z1 = lane + 64 < m ? z[lane + 64] : -INFINITY;
        const float mx = wave_max(fmaxf(z0, z1));
        const float e0 = lane < m ? expf(z0 - mx) : 0.f;
        const float e1 = lane + 64 < m ? expf(z1 - mx) : 0.f;
        const float s = wave_sum(e0 + e1);
        if (lane < m) alpha[lane] = e0 / s;
        if (lane + 64 < m) alpha[lane + 64] = e1 / s;
    }
    __syncthreads();

    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
#pragma unroll
    for (int u = 0; u < kRowsPerThread; ++u) {
        const int i = rs + u * rpar;
        const float a = i < m ? alpha[i] : 0.f;
        const T *ve = (const T *)&v[u];
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] += a * Elem<T>::to_f32(ve[e]);
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) red[rs * width + c * VEC + e] = acc[e];
    __syncthreads();
    for (int x = tid; x < width; x += 256) {
        float s = 0.f;
        for (int r = 0; r < rpar; ++r) s += red[r * width + x];
        o[x] = Elem<T>::from_f32(s);
    }
}


// threads per row slice (tpr) and slices per row of a 256-thread compression
// workgroup: a whole row if its slots cover the m rows with kRowsPerThread
// loads per thread, else halved until they do; false if no such split exists
inline bool compress_partition(int d, int m, int vec, int *tpr, int *slices) {
    int t = d / vec;
    if (t > 256 || t < 1) return false;
    while (t > 1 && (256 / t) * kRowsPerThread < m) t /= 2;
    if ((256 / t) * kRowsPerThread < m) return false;
    *tpr = t;
    *slices = d / vec / t;
    return true;
}

// One 256-thread workgroup per (batch, group, slice): workgroup blk's share.
template <typename T>
struct CompressBlocks {
    int G, m, d, tpr, slices;
    const T *raw;
    int64_t raw_bs;
    const float *logits;
    int64_t log_bs;
    T *out;
    int64_t out_bs;
    __device__ __forceinline__ void run(int blk) const {
        const int sl = blk % slices;
        const int bg = blk / slices;
        const int b = bg / G, g = bg % G;
        const int width = tpr * (16 / (int)sizeof(T));
        compress_group(raw + b * raw_bs + (int64_t)g * m * d + sl * width, logits + b * log_bs + (int64_t)g * m, m,
                       d, tpr, out + b * out_bs + (int64_t)g * d + sl * width);
    }
};

// Ragged batches: sequence b's newest token is at position pos[b]; when it
// completes a group (pos[b] + 1 a multiple of m) that group g = (pos[b]+1)/m - 1
// is pooled out of the mirrored raw and logit rings (position p at row p mod
// ring; the group's m rows are consecutive from row (g*m) mod ring) into entry g,
// if g < out_rows.  Other sequences' workgroups return at once.  One workgroup
// per (sequence, slice).
template <typename T>
struct RaggedCompressBlocks {
    int m, d, tpr, slices;
    const int64_t *pos;
    const T *raw;
    int64_t raw_bs;
    const float *logits;
    int64_t log_bs, ring;
    T *out;
    RowMap om;
    int64_t out_rows;
    __device__ __forceinline__ void run(int blk) const {
        const int sl = blk % slices;
        const int64_t b = blk / slices;
        const int64_t p = pos[b];
        if (p < 0 || (p + 1) % m != 0) return;
        const int64_t g = (p + 1) / m - 1;
        if (g >= out_rows) return;
        const int64_t r0 = (g * m) % ring;
        const int width = tpr * (16 / (int)sizeof(T));
        compress_group(raw + b * raw_bs + r0 * d + sl * width, logits + b * log_bs + r0, m, d, tpr,
                       out + om.offset(b, g, d) + sl * width);
    }
};

// A checked compression that an index call folds into its top-k filter
// launch (the compression's workgroups follow the filter's): its operands as
// launch_compress (ragged = false) or launch_compress_ragged (ragged = true)
// take them.
struct FoldedCompress {
    bool ragged;
    int dt, B, G, m, d;
    const void *raw;
    int64_t raw_bs;
    const float *logits;
    int64_t log_bs;
    void *out;
    int64_t out_bs;
    const int64_t *pos;  // ragged only
    int64_t ring;
    RowMap omap;
    int64_t out_rows;
};
// launch_topk with the compression's workgroups in the filter launch; only
// for a plan that takes the filter path (topk_plan(B*Tq, N).filter, N > 0)
hipError_t launch_topk_folded(int B, int Tq, int N, int m, int k, QPos q_pos0, const float *scores, void *scratch,
                              int32_t *out, hipStream_t st, const FoldedCompress &fc);

}  // namespace csa
