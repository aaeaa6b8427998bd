// Measurement helper, not part of the method: a streaming read of a device
// buffer, the reference the lightning indexer's HBM rate is compared with.
// Same load path as the indexer: each wavefront moves 1 KiB per non-temporal
// global_load_lds_dwordx4 into a private LDS ring of kProbeSlots slots (that
// many KiB in flight per wavefront).  The buffer is cut into F contiguous
// fronts read at the same time (the indexer streams one front per query):
// wavefront w reads front w mod F, its KiB chunks dealt round-robin to that
// front's wavefronts.  One word per wavefront is XOR-folded into the sink.
#include "kernels.h"

namespace csa {

constexpr int kProbeSlots = 32;
constexpr int kProbeWaves = 4;
constexpr int kProbeBlocks = 256;

__global__ __launch_bounds__(kProbeWaves * 64) void k_stream_read(const unsigned char *__restrict__ p,
                                                                  int64_t chunks_per_front, int fronts,
                                                                  uint32_t *__restrict__ sink) {
    __shared__ __attribute__((aligned(16))) unsigned char ring[kProbeWaves][kProbeSlots][1024];
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * kProbeWaves + w, nw = (int64_t)gridDim.x * kProbeWaves;
    const int64_t per_front = nw / fronts;  // wavefronts per front
    const int64_t f = wave % fronts, wf = wave / fronts;
    const unsigned char *base = p + f * chunks_per_front * 1024;
    int k = 0;
    for (int64_t c = wf; c < chunks_per_front; c += per_front, ++k) {
        const unsigned char *src = base + c * 1024 + l * 16;
        const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&ring[w][k % kProbeSlots][0]);
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(lds), "v"(src)
                     : "memory", "m0");
        if (k >= kProbeSlots - 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kProbeSlots - 1) : "memory");
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (l == 0) atomicXor(&sink[wave % 64], *(const uint32_t *)&ring[w][0][0]);
}

hipError_t launch_stream_read(const void *p, int64_t bytes, int fronts, uint32_t *sink, hipStream_t st) {
    const int64_t chunks_per_front = bytes / 1024 / fronts;
    hipLaunchKernelGGL(k_stream_read, dim3(kProbeBlocks), dim3(kProbeWaves * 64), 0, st, (const unsigned char *)p,
                       chunks_per_front, fronts, sink);
    return hipGetLastError();
}

}  // namespace csa
