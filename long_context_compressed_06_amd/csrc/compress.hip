// Group compression: one compressed entry per group of m consecutive tokens,
// pooled with softmax weights over the tokens' learned logits (DeepSeek-V4
// overview page, section 2.2 step 1 for m=4 and section 2.3 for m=128).
//
// One 256-thread workgroup per (batch, group, slice of d).  The slice is as
// wide as it can be while the workgroup still covers all m rows with at most
// kRowsPerThread 16-byte loads per thread (m = 128 uses eight 64-wide slices,
// m = 4 one full row), so every load of a thread is in flight at once.  The
// loads are issued before wave 0 turns the m <= 128 logits into softmax
// weights in LDS; each thread then accumulates alpha_i * row in float32 and
// the partial sums of the row slots are reduced through LDS.  The entry is
// rounded once to the cache type.
#include "compress_fold.h"

namespace csa {

// Small groups (m no larger than the row slots of k_compress with a whole-row
// slice, and at most kWaveRows): one wavefront per (batch, group, slice of
// 64 vectors) pools the m rows itself, without LDS, so it can run beside
// kernels that hold a CU's LDS.  The weights are computed as k_compress
// computes them (one wavefront, lane i holding row i's), each product is
// rounded on its own and the products are added in row order from zero, as
// k_compress's LDS reduction adds them: the entries are bit-identical.
constexpr int kWaveRows = 8;

// Workgroups past a compression launch's own work zero words [0, n) of p (n a
// multiple of 4, p 16-byte aligned), so a clear the next call needs rides in
// the same launch; workgroup blk of the nblk clearing ones takes a grid stride.
__device__ __forceinline__ void clear_words(uint32_t *__restrict__ p, int64_t n, int blk, int nblk) {
    for (int64_t i = ((int64_t)blk * blockDim.x + threadIdx.x) * 4; i < n; i += (int64_t)nblk * blockDim.x * 4)
        *(u32x4 *)(p + i) = u32x4{0u, 0u, 0u, 0u};
}
// the clearing workgroups a launch of `threads`-thread workgroups appends: one
// 16-byte store per thread per pass, at most 256 of them
static int64_t clear_blocks(int64_t clr_words, int threads) {
    const int64_t b = (clr_words / 4 + threads - 1) / threads;
    return b < 256 ? b : 256;
}

template <typename T>
__global__ __launch_bounds__(64) void k_compress_wave(int G, int m, int d, int slices, const T *__restrict__ raw,
                                                      int64_t raw_bs, const float *__restrict__ logits,
                                                      int64_t log_bs, T *__restrict__ out, int64_t out_bs,
                                                      int work_blocks, uint32_t *__restrict__ clr,
                                                      int64_t clr_words) {
#pragma clang fp contract(off)  // each product rounded before it is added, as in the LDS reduction
    constexpr int VEC = 16 / sizeof(T);
    if ((int)blockIdx.x >= work_blocks) {
        clear_words(clr, clr_words, (int)blockIdx.x - work_blocks, (int)gridDim.x - work_blocks);
        return;
    }
    const int lane = threadIdx.x;
    const int sl = blockIdx.x % slices;
    const int64_t bg = blockIdx.x / slices;
    const int64_t b = bg / G, g = bg % G;
    const T *rows = raw + b * raw_bs + g * m * (int64_t)d;
    const float *z = logits + b * log_bs + g * m;
    const int col = (sl * 64 + lane) * VEC;
    const bool on = col < d;
    u32x4 v[kWaveRows];
#pragma unroll
    for (int i = 0; i < kWaveRows; ++i)
        v[i] = on && i < m ? *(const u32x4 *)(rows + (int64_t)i * d + col) : u32x4{0u, 0u, 0u, 0u};
    const float z0 = lane < m ? z[lane] : -INFINITY;
    const float mx = wave_max(fmaxf(z0, -INFINITY));
    const float e0 = lane < m ? expf(z0 - mx) : 0.f;
    const float s = wave_sum(e0 + 0.f);
    const float al = e0 / s;
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
#pragma unroll
    for (int i = 0; i < kWaveRows; ++i) {
        if (i >= m) break;
        const float a = __shfl(al, i);
        const T *ve = (const T *)&v[i];
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = acc[e] + a * Elem<T>::to_f32(ve[e]);
    }
    if (on) {
        T *o = out + b * out_bs + g * (int64_t)d + col;
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[e] = Elem<T>::from_f32(acc[e]);
    }
}

template <typename T>
__global__ __launch_bounds__(256) void k_compress(int G, int m, int d, int tpr, int slices, const T *__restrict__ raw,
                                                   int64_t raw_bs, const float *__restrict__ logits,
                                                   int64_t log_bs, T *__restrict__ out, int64_t out_bs,
                                                   int work_blocks, uint32_t *__restrict__ clr, int64_t clr_words) {
    if ((int)blockIdx.x >= work_blocks) {  // (uniform per workgroup: before any barrier)
        clear_words(clr, clr_words, (int)blockIdx.x - work_blocks, (int)gridDim.x - work_blocks);
        return;
    }
    CompressBlocks<T>{G, m, d, tpr, slices, raw, raw_bs, logits, log_bs, out, out_bs}.run((int)blockIdx.x);
}

// Ragged batches: the group each sequence's newest token completes (RaggedCompressBlocks).
template <typename T>
__global__ __launch_bounds__(256) void k_compress_ragged(int m, int d, int tpr, int slices,
                                                          const int64_t *__restrict__ pos, const T *__restrict__ raw,
                                                          int64_t raw_bs, const float *__restrict__ logits,
                                                          int64_t log_bs, int64_t ring, T *__restrict__ out,
                                                          RowMap om, int64_t out_rows, int work_blocks,
                                                          uint32_t *__restrict__ clr, int64_t clr_words) {
    if ((int)blockIdx.x >= work_blocks) {  // (uniform per workgroup: before any barrier)
        clear_words(clr, clr_words, (int)blockIdx.x - work_blocks, (int)gridDim.x - work_blocks);
        return;
    }
    RaggedCompressBlocks<T>{m, d, tpr, slices, pos, raw, raw_bs, logits, log_bs, ring, out, om, out_rows}.run(
        (int)blockIdx.x);
}

// Per-channel pooling logits: channel x of entry g pools channel x of the
// group's m rows with the softmax over those rows of logits[., x].  Same
// partition as k_compress (row slots x 16-byte column vectors, at most
// kRowsPerThread rows per thread, every load in flight at once); each thread
// keeps, per column, the maximum of its rows' logits, the sum of their
// exponentials and the weighted sum of the rows, and the row slots are merged
// through LDS by rescaling to the common maximum.
template <typename T>
__global__ __launch_bounds__(256) void k_compress_channels(int G, int m, int d, int tpr, int slices,
                                                           const T *__restrict__ raw, int64_t raw_bs,
                                                           const float *__restrict__ logits, int64_t log_bs,
                                                           T *__restrict__ out, int64_t out_bs) {
    constexpr int VEC = 16 / sizeof(T);
    __shared__ float red[3][256 * VEC];  // per row slot and column: max, sum of exponentials, weighted sum

    const int sl = blockIdx.x % slices;
    const int bg = blockIdx.x / slices;
    const int b = bg / G, g = bg % G;
    const int tid = threadIdx.x;
    const int rpar = 256 / tpr;
    const int c = tid % tpr, rs = tid / tpr;
    const int width = tpr * VEC;
    const int64_t col0 = (int64_t)sl * width + c * VEC;
    const T *rows = raw + b * raw_bs + (int64_t)g * m * d + col0;
    const float *zr = logits + b * log_bs + (int64_t)g * m * d + col0;
    u32x4 v[kRowsPerThread];
    float z[kRowsPerThread][VEC];
#pragma unroll
    for (int u = 0; u < kRowsPerThread; ++u) {
        const int i = rs + u * rpar;
        v[u] = i < m ? *(const u32x4 *)(rows + (int64_t)i * d) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int q = 0; q < VEC / 4; ++q) {
            const floatx4 zz = i < m ? *(const floatx4 *)(zr + (int64_t)i * d + 4 * q)
                                     : floatx4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
            for (int e = 0; e < 4; ++e) z[u][4 * q + e] = zz[e];
        }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        float mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < kRowsPerThread; ++u) mx = fmaxf(mx, z[u][e]);
        float s = 0.f, a = 0.f;
        if (mx > -INFINITY) {
#pragma unroll
            for (int u = 0; u < kRowsPerThread; ++u) {
                const float w = expf(z[u][e] - mx);  // rows past m: exp(-inf) = 0
                s += w;
                a += w * Elem<T>::to_f32(((const T *)&v[u])[e]);
            }
        }
        const int x = rs * width + c * VEC + e;
        red[0][x] = mx;
        red[1][x] = s;
        red[2][x] = a;
    }
    __syncthreads();
    T *o = out + b * out_bs + (int64_t)g * d + (int64_t)sl * width;
    for (int x = tid; x < width; x += 256) {
        float M = -INFINITY;
        for (int r = 0; r < rpar; ++r) M = fmaxf(M, red[0][r * width + x]);
        float S = 0.f, A = 0.f;
        for (int r = 0; r < rpar; ++r) {
            const float mr = red[0][r * width + x];
            if (mr > -INFINITY) {
                const float f = expf(mr - M);
                S += f * red[1][r * width + x];
                A += f * red[2][r * width + x];
            }
        }
        o[x] = Elem<T>::from_f32(A / S);
    }
}

template <typename T>
hipError_t launch_compress_t(int B, int G, int m, int d, const void *raw, int64_t raw_bs, const float *logits,
                             int64_t log_bs, void *out, int64_t out_bs, hipStream_t st, uint32_t *clr,
                             int64_t clr_words) {
    constexpr int VEC = 16 / sizeof(T);
    // threads per row slice: d/VEC (a whole row), halved until the workgroup's
    // row slots times kRowsPerThread cover the m rows
    int tpr = d / VEC;
    if (tpr > 256) return hipErrorInvalidValue;
    while (tpr > 1 && (256 / tpr) * kRowsPerThread < m) tpr /= 2;
    if ((256 / tpr) * kRowsPerThread < m) return hipErrorInvalidValue;
    const int slices = d / VEC / tpr;
    if (tpr == d / VEC && m <= 256 / tpr && m <= kWaveRows) {  // each row slot holds one row: the LDS-free form
        const int wslices = (d / VEC + 63) / 64;
        const int64_t work = (int64_t)B * G * wslices;
        hipLaunchKernelGGL(k_compress_wave<T>, dim3((unsigned)(work + clear_blocks(clr_words, 64))), dim3(64), 0, st, G, m, d,
                           wslices, (const T *)raw, raw_bs, logits, log_bs, (T *)out, out_bs, (int)work, clr,
                           clr_words);
        return hipGetLastError();
    }
    const int64_t work = (int64_t)B * G * slices;
    hipLaunchKernelGGL(k_compress<T>, dim3((unsigned)(work + clear_blocks(clr_words, 256))), dim3(256), 0, st, G, m, d, tpr,
                       slices, (const T *)raw, raw_bs, logits, log_bs, (T *)out, out_bs, (int)work, clr, clr_words);
    return hipGetLastError();
}
template <typename T>
hipError_t launch_compress_ragged_t(int B, int m, int d, const int64_t *pos, const void *raw, int64_t raw_bs,
                                    const float *logits, int64_t log_bs, int64_t ring, void *out, RowMap out_bs,
                                    int64_t out_rows, hipStream_t st, uint32_t *clr, int64_t clr_words) {
    constexpr int VEC = 16 / sizeof(T);
    int tpr = d / VEC;
    if (tpr > 256) return hipErrorInvalidValue;
    while (tpr > 1 && (256 / tpr) * kRowsPerThread < m) tpr /= 2;
    if ((256 / tpr) * kRowsPerThread < m) return hipErrorInvalidValue;
    const int slices = d / VEC / tpr;
    const int64_t work = (int64_t)B * slices;
    hipLaunchKernelGGL(k_compress_ragged<T>, dim3((unsigned)(work + clear_blocks(clr_words, 256))), dim3(256), 0, st,
                       m, d, tpr, slices, pos, (const T *)raw, raw_bs, logits, log_bs, ring, (T *)out, out_bs,
                       out_rows, (int)work, clr, clr_words);
    return hipGetLastError();
}
hipError_t launch_compress_ragged(int dt, int B, int m, int d, const int64_t *pos, const void *raw, int64_t raw_bs,
                                  const float *logits, int64_t log_bs, int64_t ring, void *out, RowMap out_bs,
                                  int64_t out_rows, hipStream_t st, uint32_t *clr, int64_t clr_words) {
    if (dt == 0)
        return launch_compress_ragged_t<float>(B, m, d, pos, raw, raw_bs, logits, log_bs, ring, out, out_bs,
                                               out_rows, st, clr, clr_words);
    return launch_compress_ragged_t<bf16_t>(B, m, d, pos, raw, raw_bs, logits, log_bs, ring, out, out_bs, out_rows,
                                            st, clr, clr_words);
}

template <typename T>
hipError_t launch_compress_channels_t(int B, int G, int m, int d, const void *raw, int64_t raw_bs,
                                      const float *logits, int64_t log_bs, void *out, int64_t out_bs,
                                      hipStream_t st) {
    constexpr int VEC = 16 / sizeof(T);
    int tpr = d / VEC;
    if (tpr > 256 || tpr < 1) return hipErrorInvalidValue;
    while (tpr > 1 && (256 / tpr) * kRowsPerThread < m) tpr /= 2;
    if ((256 / tpr) * kRowsPerThread < m) return hipErrorInvalidValue;
    const int slices = d / VEC / tpr;
    hipLaunchKernelGGL(k_compress_channels<T>, dim3((unsigned)((int64_t)B * G * slices)), dim3(256), 0, st, G, m,
                       d, tpr, slices, (const T *)raw, raw_bs, logits, log_bs, (T *)out, out_bs);
    return hipGetLastError();
}
hipError_t launch_compress_channels(int dt, int B, int G, int m, int d, const void *raw, int64_t raw_bs,
                                    const float *logits, int64_t log_bs, void *out, int64_t out_bs,
                                    hipStream_t st) {
    if (dt == 0)
        return launch_compress_channels_t<float>(B, G, m, d, raw, raw_bs, logits, log_bs, out, out_bs, st);
    return launch_compress_channels_t<bf16_t>(B, G, m, d, raw, raw_bs, logits, log_bs, out, out_bs, st);
}
hipError_t launch_compress(int dt, int B, int G, int m, int d, const void *raw, int64_t raw_bs,
                           const float *logits, int64_t log_bs, void *out, int64_t out_bs, hipStream_t st,
                           uint32_t *clr, int64_t clr_words) {
    if ((int64_t)B * G == 0 && clr_words == 0) return hipSuccess;
    if (dt == 0)
        return launch_compress_t<float>(B, G, m, d, raw, raw_bs, logits, log_bs, out, out_bs, st, clr, clr_words);
    return launch_compress_t<bf16_t>(B, G, m, d, raw, raw_bs, logits, log_bs, out, out_bs, st, clr, clr_words);
}

}  // namespace csa
