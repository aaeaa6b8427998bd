// Cache maintenance between attention steps: new rows enter a cache at the
// next free positions, or a raw-token ring buffer (the window of raw tokens
// and the tokens of the group being filled, DeepSeek-V4 overview page,
// section 2.2 step 1: every m tokens become one entry).
//
// The ring is mirrored: a ring of R positions has 2R row slots and position p
// is written to slots p mod R and p mod R + R, so any R consecutive positions
// sit in consecutive slots (starting at the first one's p mod R) and the
// compression and attention kernels read a window out of the ring as a plain
// strided tensor.  Rows are opaque bytes: element rows, pooling logits,
// FP4 codes and scale bytes all move through the same kernel.
//
// k_append_rows: a grid-stride copy per batch (blockIdx.y), VW-byte vectors.
// k_append_multi: up to eight such copies in one launch (blockIdx.z); a job
// may take each batch's position from device memory (ragged batches) and may
// keep only the token that completes a group, writing it to that group's row.
#include "kernels.h"

namespace csa {

template <int VW>
struct Vec;
template <>
struct Vec<16> { typedef u32x4 T; };
template <>
struct Vec<8> { typedef uint64_t T; };
template <>
struct Vec<4> { typedef uint32_t T; };
template <>
struct Vec<2> { typedef uint16_t T; };
template <>
struct Vec<1> { typedef uint8_t T; };

template <int VW>
__global__ __launch_bounds__(256) void k_append_rows(int64_t n, int64_t vpr, const unsigned char *__restrict__ src,
                                                     int64_t src_bs, unsigned char *__restrict__ dst,
                                                     int64_t dst_bs, int64_t pos0, int64_t ring) {
    typedef typename Vec<VW>::T V;
    const int64_t b = blockIdx.y;
    const int64_t row_bytes = vpr * VW;
    const unsigned char *s = src + b * src_bs;
    unsigned char *d = dst + b * dst_bs;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n * vpr; e += (int64_t)gridDim.x * 256) {
        const int64_t i = e / vpr, v = e % vpr;
        const V x = *(const V *)(s + i * row_bytes + v * VW);
        const int64_t p = pos0 + i;
        if (ring == 0) {
            *(V *)(d + p * row_bytes + v * VW) = x;
        } else {
            const int64_t slot = p % ring;
            *(V *)(d + slot * row_bytes + v * VW) = x;
            *(V *)(d + (slot + ring) * row_bytes + v * VW) = x;
        }
    }
}

// several appends in one launch: blockIdx.z selects the job, blockIdx.y the batch
template <int VW>
__device__ __forceinline__ void append_job_body(const AppendJob &J) {
    typedef typename Vec<VW>::T V;
    const int64_t b = blockIdx.y;
    const int64_t vpr = J.row_bytes / VW;
    const unsigned char *s = J.src + b * J.src_bs;
    unsigned char *d = J.dst + (J.dmap.ptab ? 0 : b * J.dst_bs);  // (paged: rows of the pool)
    const int64_t base = J.pos0 + (J.pos ? J.pos[b] : 0);
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < J.n * vpr; e += (int64_t)gridDim.x * 256) {
        const int64_t i = e / vpr, v = e % vpr;
        int64_t p = base + i;
        if (J.every > 0) {  // only the token that completes a group: its row goes to that group's index
            if (p < 0 || (p + 1) % J.every != 0) continue;
            p = (p + 1) / J.every - 1;
        }
        if (p < 0) continue;  // (positions read from memory are not checked by the host)
        const V x = *(const V *)(s + i * J.row_bytes + v * VW);
        if (J.ring == 0) {
            if (p >= J.dst_rows) continue;
            const int64_t row = J.dmap.ptab ? J.dmap.paged_row(b, p) : p;
            *(V *)(d + row * J.row_bytes + v * VW) = x;
        } else {
            const int64_t slot = p % J.ring;
            *(V *)(d + slot * J.row_bytes + v * VW) = x;
            *(V *)(d + (slot + J.ring) * J.row_bytes + v * VW) = x;
        }
    }
}

__global__ __launch_bounds__(256) void k_append_multi(AppendJobs jobs) {
    const AppendJob &J = jobs.j[blockIdx.z];
    if ((int)blockIdx.y >= J.B) return;
    switch (J.vw) {
        case 16: append_job_body<16>(J); break;
        case 8: append_job_body<8>(J); break;
        case 4: append_job_body<4>(J); break;
        case 2: append_job_body<2>(J); break;
        default: append_job_body<1>(J); break;
    }
}

hipError_t launch_append_multi(const AppendJobs &jobs, int count, hipStream_t st) {
    int64_t blocks = 1, bmax = 1;
    for (int i = 0; i < count; ++i) {
        const int64_t b = (jobs.j[i].n * (jobs.j[i].row_bytes / jobs.j[i].vw) + 255) / 256;
        blocks = b > blocks ? b : blocks;
        bmax = jobs.j[i].B > bmax ? jobs.j[i].B : bmax;
    }
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(k_append_multi, dim3((unsigned)blocks, (unsigned)bmax, (unsigned)count), dim3(256), 0, st,
                       jobs);
    return hipGetLastError();
}

__global__ void k_positions_advance(int B, int64_t *pos, int64_t delta) {
    const int b = blockIdx.x * 256 + threadIdx.x;
    if (b < B) pos[b] += delta;
}

hipError_t launch_positions_advance(int B, int64_t *pos, int64_t delta, hipStream_t st) {
    if (B <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_positions_advance, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, st, B, pos, delta);
    return hipGetLastError();
}

hipError_t launch_append_rows(int B, int64_t n, int64_t row_bytes, int vw, const void *src, int64_t src_bs,
                              void *dst, int64_t dst_bs, int64_t pos0, int64_t ring, hipStream_t st) {
    const int64_t vpr = row_bytes / vw;
    int64_t blocks = (n * vpr + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    if (blocks < 1) blocks = 1;
    const dim3 grid((unsigned)blocks, (unsigned)B);
    const unsigned char *s = (const unsigned char *)src;
    unsigned char *d = (unsigned char *)dst;
    switch (vw) {
        case 16: hipLaunchKernelGGL(k_append_rows<16>, grid, dim3(256), 0, st, n, vpr, s, src_bs, d, dst_bs, pos0, ring); break;
        case 8: hipLaunchKernelGGL(k_append_rows<8>, grid, dim3(256), 0, st, n, vpr, s, src_bs, d, dst_bs, pos0, ring); break;
        case 4: hipLaunchKernelGGL(k_append_rows<4>, grid, dim3(256), 0, st, n, vpr, s, src_bs, d, dst_bs, pos0, ring); break;
        case 2: hipLaunchKernelGGL(k_append_rows<2>, grid, dim3(256), 0, st, n, vpr, s, src_bs, d, dst_bs, pos0, ring); break;
        default: hipLaunchKernelGGL(k_append_rows<1>, grid, dim3(256), 0, st, n, vpr, s, src_bs, d, dst_bs, pos0, ring); break;
    }
    return hipGetLastError();
}

}  // namespace csa
