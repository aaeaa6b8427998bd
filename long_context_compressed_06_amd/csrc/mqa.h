// Pieces shared by the attention kernels (mqa.hip, mqa_wide.hip): the
// argument block, LDS-DMA issue and waits, and the LDS slot order of a tile's
// rows.
#pragma once

#include "kernels.h"

namespace csa {

struct MqaArgs {
    int Tq, H, N, m, k, W, n_splits, tiles_per_split;
    int64_t q_pos0, raw_pos0, raw_bs;
    RowMap em;           // entry rows (a batch stride or a page table)
    const int64_t *pos;  // optional: sequence b's query position (ragged batches, Tq = 1)
    int64_t raw_ring;    // 0: raw rows are positions raw_pos0 ..; R: position p is ring row p mod R
    float scale;
    const void *q, *entries, *raw;
    const int32_t *idx;
    float *out, *lse, *part_o, *part_ml;
    // the wide kernel's split partials: part_o holds f16 values O / l / sigma,
    // part_sc the power of two sigma of each (query, split)
    float *part_sc;
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazyRescale = 8.f;  // base-2 headroom of the reference maximum
constexpr int kMqaThreads = 512;


// 16 bytes per active lane from `src` into LDS at lds_base + 16 * lane.
// Issued from inline assembly so that the compiler does not treat every
// later LDS read as dependent on it (it would drain all tiles in flight);
// completion is awaited explicitly with wait_vm_barrier.  One wait state
// separates the M0 write from the LDS-DMA instruction, as the ISA requires.
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

// LDS slot of tile row r.  LDS serves 128 bytes (32 four-byte banks) per
// cycle, and the row stride is 4 banks (mod 32): the logits product reads 16
// bytes of rows c and c+8 in one cycle per eight lanes, so rows 0-7 (and
// 8-15, ...) need slots distinct mod 8; a transposing read takes 8 bytes of
// rows 4g..4g+3 in one cycle per sixteen lanes, so those four rows need slots
// two apart mod 8 (disjoint 8-bank windows): rows 4g..4g+3 go to even slots
// for even g and odd slots for odd g.
__device__ __forceinline__ int row_slot(int r) { return (r & 24) | ((r & 3) << 1) | ((r >> 2) & 1); }

}  // namespace csa
