// Group compression: one compressed entry per group of m consecutive tokens,
// pooled with softmax weights over the tokens' learned logits (DeepSeek-V4
// overview page, section 2.2 step 1 for m=4 and section 2.3 for m=128).
//
// One 256-thread workgroup per (batch, group).  Wave 0 turns the m <= 128
// logits into softmax weights in LDS; then every thread streams 16-byte
// vectors of the group's rows (coalesced along d), accumulates alpha_i * row
// in float32 and the partial sums of the row slots are reduced through LDS.
// The entry is rounded once to the cache type.
#include "kernels.h"

namespace csa {

template <typename T>
__global__ __launch_bounds__(256) void k_compress(int G, int m, int d, const T *__restrict__ raw,
                                                   int64_t raw_bs, const float *__restrict__ logits,
                                                   int64_t log_bs, T *__restrict__ out, int64_t out_bs) {
    constexpr int VEC = 16 / sizeof(T);  // elements per 16-byte vector
    __shared__ float alpha[128];
    __shared__ float red[256 * VEC];

    const int b = blockIdx.x / G, g = blockIdx.x % G;
    const int tid = threadIdx.x, lane = tid & 63;
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

    const int tpr = d / VEC;       // threads covering one row
    const int rpar = 256 / tpr;    // rows accumulated in parallel
    const int c = tid % tpr, rs = tid / tpr;
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
    const T *rows = raw + b * raw_bs + (int64_t)g * m * d + c * VEC;
    for (int i = rs; i < m; i += rpar) {
        const u32x4 v = *(const u32x4 *)(rows + (int64_t)i * d);
        const float a = alpha[i];
        const T *ve = (const T *)&v;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] += a * Elem<T>::to_f32(ve[e]);
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) red[rs * d + c * VEC + e] = acc[e];
    __syncthreads();
    T *o = out + b * out_bs + (int64_t)g * d;
    for (int x = tid; x < d; x += 256) {
        float s = 0.f;
        for (int r = 0; r < rpar; ++r) s += red[r * d + x];
        o[x] = Elem<T>::from_f32(s);
    }
}

template <typename T>
hipError_t launch_compress_t(int B, int G, int m, int d, const void *raw, int64_t raw_bs, const float *logits,
                             int64_t log_bs, void *out, int64_t out_bs, hipStream_t st) {
    hipLaunchKernelGGL(k_compress<T>, dim3(B * G), dim3(256), 0, st, G, m, d, (const T *)raw, raw_bs, logits,
                       log_bs, (T *)out, out_bs);
    return hipGetLastError();
}

hipError_t launch_compress(int dt, int B, int G, int m, int d, const void *raw, int64_t raw_bs,
                           const float *logits, int64_t log_bs, void *out, int64_t out_bs, hipStream_t st) {
    if (dt == 0) return launch_compress_t<float>(B, G, m, d, raw, raw_bs, logits, log_bs, out, out_bs, st);
    return launch_compress_t<bf16_t>(B, G, m, d, raw, raw_bs, logits, log_bs, out, out_bs, st);
}

}  // namespace csa
