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
#include "kernels.h"

namespace csa {

constexpr int kRowsPerThread = 4;

template <typename T>
__global__ __launch_bounds__(256) void k_compress(int G, int m, int d, int tpr, int slices, const T *__restrict__ raw,
                                                   int64_t raw_bs, const float *__restrict__ logits,
                                                   int64_t log_bs, T *__restrict__ out, int64_t out_bs) {
    constexpr int VEC = 16 / sizeof(T);  // elements per 16-byte vector
    __shared__ float alpha[128];
    __shared__ float red[256 * VEC];

    const int sl = blockIdx.x % slices;
    const int bg = blockIdx.x / slices;
    const int b = bg / G, g = bg % G;
    const int tid = threadIdx.x, lane = tid & 63;
    const int rpar = 256 / tpr;        // rows accumulated in parallel
    const int c = tid % tpr, rs = tid / tpr;
    const int width = tpr * VEC;       // columns of this slice
    const T *rows = raw + b * raw_bs + (int64_t)g * m * d + sl * width + c * VEC;
    u32x4 v[kRowsPerThread];
#pragma unroll
    for (int u = 0; u < kRowsPerThread; ++u) {
        const int i = rs + u * rpar;
        v[u] = i < m ? *(const u32x4 *)(rows + (int64_t)i * d) : u32x4{0u, 0u, 0u, 0u};
    }
    const float *z = logits + b * log_bs + (int64_t)g * m;
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
    T *o = out + b * out_bs + (int64_t)g * d + sl * width;
    for (int x = tid; x < width; x += 256) {
        float s = 0.f;
        for (int r = 0; r < rpar; ++r) s += red[r * width + x];
        o[x] = Elem<T>::from_f32(s);
    }
}

template <typename T>
hipError_t launch_compress_t(int B, int G, int m, int d, const void *raw, int64_t raw_bs, const float *logits,
                             int64_t log_bs, void *out, int64_t out_bs, hipStream_t st) {
    constexpr int VEC = 16 / sizeof(T);
    // threads per row slice: d/VEC (a whole row), halved until the workgroup's
    // row slots times kRowsPerThread cover the m rows
    int tpr = d / VEC;
    if (tpr > 256) return hipErrorInvalidValue;
    while (tpr > 1 && (256 / tpr) * kRowsPerThread < m) tpr /= 2;
    if ((256 / tpr) * kRowsPerThread < m) return hipErrorInvalidValue;
    const int slices = d / VEC / tpr;
    hipLaunchKernelGGL(k_compress<T>, dim3((unsigned)((int64_t)B * G * slices)), dim3(256), 0, st, G, m, d, tpr,
                       slices, (const T *)raw, raw_bs, logits, log_bs, (T *)out, out_bs);
    return hipGetLastError();
}
hipError_t launch_compress(int dt, int B, int G, int m, int d, const void *raw, int64_t raw_bs,
                           const float *logits, int64_t log_bs, void *out, int64_t out_bs, hipStream_t st) {
    if (dt == 0) return launch_compress_t<float>(B, G, m, d, raw, raw_bs, logits, log_bs, out, out_bs, st);
    return launch_compress_t<bf16_t>(B, G, m, d, raw, raw_bs, logits, log_bs, out, out_bs, st);
}

}  // namespace csa
