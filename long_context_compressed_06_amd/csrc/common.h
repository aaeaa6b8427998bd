// Device-side building blocks shared by the gfx950 kernels of libcsa.
//
// Element types: `float` for the fp32 path and `bf16_t` (raw 16-bit storage)
// for the bf16 path.  All arithmetic is float32.  Matrix products use the
// CDNA MFMA instructions with 16x16 output tiles and 64-lane wavefronts:
//   bf16: v_mfma_f32_16x16x32_bf16  (K = 32, 8 K-values per lane)
//   fp32: v_mfma_f32_16x16x4_f32    (K = 4,  1 K-value per lane)
// Operand layout (both instructions): lane l supplies A[l % 16][kgrp] and
// B[kgrp][l % 16], where kgrp is the lane group g = l / 16's share of K; the
// result tile lands with lane l holding D[4*g + e][l % 16] for e = 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

typedef uint16_t bf16_t;
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// round-to-nearest-even float32 -> bf16 (inputs are finite in this library)
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

template <typename T> struct Elem;

template <> struct Elem<float> {
    static constexpr int KPL = 1;    // K values held per lane by one MFMA operand
    static constexpr int KSTEP = 4;  // K of one MFMA
    typedef float frag;
    static __device__ __forceinline__ float to_f32(float v) { return v; }
    static __device__ __forceinline__ float from_f32(float v) { return v; }
    static __device__ __forceinline__ floatx4 mma(frag a, frag b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    // load the KPL consecutive elements starting at p
    static __device__ __forceinline__ frag load(const float *p) { return *p; }
    // streaming load that is not kept in the caches
    static __device__ __forceinline__ frag load_nt(const float *p) { return __builtin_nontemporal_load(p); }
    static __device__ __forceinline__ frag zero() { return 0.f; }
};

template <> struct Elem<bf16_t> {
    static constexpr int KPL = 8;
    static constexpr int KSTEP = 32;
    typedef bf16x8 frag;
    static __device__ __forceinline__ float to_f32(bf16_t v) { return bf16_to_f32(v); }
    static __device__ __forceinline__ bf16_t from_f32(float v) { return f32_to_bf16(v); }
    static __device__ __forceinline__ floatx4 mma(frag a, frag b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ frag load(const bf16_t *p) { return *(const bf16x8 *)p; }
    static __device__ __forceinline__ frag load_nt(const bf16_t *p) {
        return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load((const u32x4 *)p));
    }
    static __device__ __forceinline__ frag zero() {
        frag z;
        for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.0f;
        return z;
    }
};

// Query positions: every sequence's queries at q_pos0, q_pos0 + 1, ...
// (uniform batches), or, with `pos` set, sequence b's queries at pos[b],
// pos[b] + 1, ... read from device memory (ragged batches: each sequence at
// its own length).  Converts from a plain position.
struct QPos {
    int64_t q_pos0;
    const int64_t *pos;
    __host__ __device__ QPos(int64_t p = 0, const int64_t *ps = nullptr) : q_pos0(p), pos(ps) {}
    __device__ __forceinline__ int64_t at(int64_t b, int64_t ti) const { return (pos ? pos[b] : q_pos0) + ti; }
};

// Rows of a per-sequence cache (entries or index keys).  Contiguous caches:
// sequence b starts bstride units into the buffer (the unit is the caller's:
// offset() takes it in elements).  Paged caches (ptab set): row j of sequence
// b is row j & (2^pshift - 1) of page ptab[b * pstride + (j >> pshift)] of
// one pool of npages pages of 2^pshift rows; page ids read from memory are
// clamped into the pool.  Converts from a plain batch stride.
struct RowMap {
    int64_t bstride;
    const int32_t *ptab;
    int pstride, pshift;
    int64_t npages;
    __host__ __device__ RowMap(int64_t bs = 0, const int32_t *t = nullptr, int ps = 0, int sh = 0, int64_t np = 0)
        : bstride(bs), ptab(t), pstride(ps), pshift(sh), npages(np) {}
    __device__ __forceinline__ int64_t page_of(int64_t b, int64_t pidx) const {
        int64_t pg = ptab[b * pstride + pidx];
        return pg < 0 ? 0 : (pg >= npages ? npages - 1 : pg);
    }
    // pool row of sequence b's row j (paged maps only)
    __device__ __forceinline__ int64_t paged_row(int64_t b, int64_t j) const {
        return (page_of(b, j >> pshift) << pshift) | (j & ((1 << pshift) - 1));
    }
    // element offset of sequence b's row j, rows of rowlen elements (bstride in elements)
    __device__ __forceinline__ int64_t offset(int64_t b, int64_t j, int64_t rowlen) const {
        return ptab ? paged_row(b, j) * rowlen : b * bstride + j * rowlen;
    }
};
// Indexer epilogues: the head sum of four 16-entry blocks at once.  Lane
// (g, c) = (lane / 16, lane % 16) holds x[u], block u's partial score of entry
// c over its lane group's heads; on return it holds block g's total for entry
// c, i.e. the four lane groups end with the four blocks.  One 32-lane swap
// pairs blocks 0/2 and 1/3 across the wave halves, one 16-lane swap finishes
// (three swaps and three adds for four blocks; the additions are paired as
// (g0 + g2) + (g1 + g3), the order of the one-block sum).
__device__ __forceinline__ float sum_lane_groups4(const float (&x)[4]) {
    // v_permlane32_swap: lanes 32-63 of the first operand <-> lanes 0-31 of the second
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[0]), __float_as_uint(x[2]), false, false);
    const float r02 = __uint_as_float(p[0]) + __uint_as_float(p[1]);  // halves: block 0 (lanes 0-31), 2
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[1]), __float_as_uint(x[3]), false, false);
    const float r13 = __uint_as_float(q[0]) + __uint_as_float(q[1]);  // halves: block 1, 3
    // v_permlane16_swap: odd 16-lane rows of the first operand <-> even rows of the second
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(r02), __float_as_uint(r13), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// page list of one sequence staged in LDS by the indexers (pages of at most
// this many entries per sequence)
constexpr int kMaxPagesPerSeq = 1024;

// Sequence b's first n page ids (n <= kMaxPagesPerSeq) into LDS pl[0, n), by
// a workgroup of NT threads, in two parts so that other loads can be issued
// in between: load() issues each thread's loads together, from clamped
// (always valid) positions, store() writes them; one memory round trip.
template <int NT>
struct PageStage {
    static constexpr int U = (kMaxPagesPerSeq + NT - 1) / NT;
    int32_t v[U];
    __device__ __forceinline__ void load(const RowMap &kl, int64_t b, int n) {
        if (n <= 0) return;
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = kl.ptab[b * kl.pstride + min((int)threadIdx.x + u * NT, n - 1)];
    }
    // (the page ids are clamped into the pool here, as page_of does)
    __device__ __forceinline__ void store(const RowMap &kl, int32_t *pl, int n) const {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = (int)threadIdx.x + u * NT;
            if (i < n) pl[i] = (int32_t)(v[u] < 0 ? 0 : (v[u] >= kl.npages ? kl.npages - 1 : v[u]));
        }
    }
};

// Entries visible to a query at absolute position t: complete groups only.
__device__ __forceinline__ int64_t n_visible(int64_t t, int m, int64_t N) {
    if (t < 0) return 0;
    int64_t n = (t + 1) / m;
    return n < N ? n : N;
}

// Rank of this workgroup with consecutive ranks on one XCD.  The dispatcher
// deals workgroups to the 8 XCDs round-robin (workgroup i to XCD i mod 8),
// so rank (i mod 8) * (G / 8) + i / 8 gives XCD x the ranks [x G/8, (x+1) G/8)
// when G, the grid size, is a multiple of 8 (else the rank is i).  The
// indexers map consecutive ranks to the workgroups of one query row, which
// keeps a row's key stream, query and histogram on one XCD.
__device__ __forceinline__ int xcd_rank(int G) {
    const int i = blockIdx.x;
    return (G & 7) ? i : (i & 7) * (G >> 3) + (i >> 3);
}

// Ragged batches (one query per row, rows = B, row b at position pos[b]):
// share the G workgroups of a launch among the rows in proportion to their
// visible 16-entry tiles, every row getting at least one:
//     parts_b = 1 + tiles_b * (G - B) / sum_j tiles_j      (G >= B)
// and workgroup i serves row b with parts_{<b} <= i < parts_{<=b}.  Every
// wavefront computes the same answer from pos (no barrier); false for the
// workgroups left over by the rounding.
__device__ __forceinline__ bool ragged_share(const int64_t *__restrict__ pos, int B, int m, int64_t N, int G, int i,
                                             int64_t *row, int *part, int *parts) {
    const int lane = threadIdx.x & 63;
    auto tiles_of = [&](int b) -> int64_t { return b < B ? (n_visible(pos[b], m, N) + 15) / 16 : 0; };
    int64_t total = 0;
    for (int b0 = 0; b0 < B; b0 += 64) {
        int64_t t = tiles_of(b0 + lane);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o);
        total += t;
    }
    const int64_t spare = G - B;
    int64_t base = 0;
    for (int b0 = 0; b0 < B; b0 += 64) {
        const int b = b0 + lane;
        const int64_t pb = b < B ? 1 + (total > 0 ? tiles_of(b) * spare / total : 0) : 0;
        int64_t incl = pb;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int64_t y = __shfl_up(incl, o);
            if (lane >= o) incl += y;
        }
        const int64_t lo = base + incl - pb;
        const uint64_t hit = __ballot(b < B && lo <= i && i < base + incl);
        if (hit) {
            const int src = __builtin_ctzll(hit);
            *row = b0 + src;
            *part = (int)(i - __shfl(lo, src));
            *parts = (int)__shfl(pb, src);
            return true;
        }
        base += __shfl(incl, 63);
    }
    return false;
}

// order-preserving map of a float score to uint32 (larger score, larger key;
// -0 ranks with +0)
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float wave_max(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

}  // namespace csa
