// Launchers of the gfx950 kernels (one translation unit per kernel family).
// dt: 0 = float32 elements, 1 = bf16 elements.  All pointers are device
// pointers; every launcher only enqueues on `st` and returns the launch
// status.  Argument checking happens in abi.cpp before any launcher runs.
#pragma once

#include "common.h"

namespace csa {

// first radix digit of the top-k select, counted per query by the indexer
// epilogue: the top 13 bits of the score key (sign, exponent, four mantissa
// bits, so 16 bins per binade) offset into a window of kTopkBins values that
// holds the binades 2^-63 .. 2^64 of non-negative scores; every key below the
// window counts in bin 0, every key above it in the last bin.  An interior
// bin is one 13-bit key prefix; the two end bins are not.
constexpr int kTopkBinBits = 11;
constexpr int kTopkBins = 1 << kTopkBinBits;
constexpr int kTopkKeyShift = 19;                            // key bits below the 13-bit prefix
constexpr uint32_t kTopkWindow0 = (1u << 12) + (64u << 4);   // the prefix at bin 0's upper edge
__device__ __forceinline__ uint32_t topk_bin(uint32_t key) {
    const uint32_t t = key >> kTopkKeyShift;
    return t <= kTopkWindow0 ? 0u : min(t - kTopkWindow0, (uint32_t)(kTopkBins - 1));
}
// decode (few queries) top-k: scores per filter workgroup, (index, key)
// pairs the final workgroup gathers into LDS, and the longest row accepted
constexpr int kTopkFilterChunk = 4096;
constexpr int kTopkFinalItems = 16384;
// with at least kTopkCompactMinRows queries, rows of up to kTopkCompactMax
// scores are selected in one pass by one workgroup per query (several per
// CU); otherwise the filter + final path spreads each row over CUs
constexpr int kTopkCompactMax = 65536;
constexpr int kTopkCompactMinRows = 256;
constexpr int64_t kTopkMaxEntries = (int64_t)kTopkFilterChunk * 1023;

struct TopkPlan {
    bool filter;     // multi-workgroup filter + final path (else one pass, one workgroup per query)
    int64_t nblk;    // filter workgroups per query
};
TopkPlan topk_plan(int64_t rows, int64_t N);
// top-k scratch after the score rows; its first topk_clear_words(rows, N)
// 32-bit words must be zero when the indexer starts (histograms, counters)
size_t topk_scratch_bytes(int64_t rows, int64_t N);
size_t topk_clear_words(int64_t rows, int64_t N);

// clr / clr_words (optional, here and in launch_compress_ragged): words also
// zeroed by the same launch (clr_words a multiple of 4, clr 16-byte aligned),
// e.g. the top-k histograms of the index call that follows
hipError_t launch_compress(int dt, int B, int G, int m, int d, const void *raw, int64_t raw_bs,
                           const float *logits, int64_t log_bs, void *out, int64_t out_bs, hipStream_t st,
                           uint32_t *clr = nullptr, int64_t clr_words = 0);
// ragged batches: per sequence, the group completed by its newest token (position pos[b]), read out of
// mirrored raw / logit rings of `ring` positions, into entry row (pos[b]+1)/m - 1 when below out_rows
hipError_t launch_compress_ragged(int dt, int B, int m, int d, const int64_t *pos, const void *raw, int64_t raw_bs,
                                  const float *logits, int64_t log_bs, int64_t ring, void *out, RowMap out_map,
                                  int64_t out_rows, hipStream_t st, uint32_t *clr = nullptr, int64_t clr_words = 0);
// logits: [B][G*m][d] f32 (per channel), batch stride log_bs elements
hipError_t launch_compress_channels(int dt, int B, int G, int m, int d, const void *raw, int64_t raw_bs,
                                    const float *logits, int64_t log_bs, void *out, int64_t out_bs,
                                    hipStream_t st);

// scores: [rows][s_stride] (s_stride >= N); scores2: optional second copy,
// [rows][N]; hist: optional [rows, kTopkBins] counts, must be zero on entry
// k_bs: the key cache's rows (a batch stride, or a page table: d_I = 128 bf16 only)
hipError_t launch_index_scores(int dt, int B, int Tq, int N, int HI, int dI, int m, QPos q_pos0, const void *qI,
                               const float *w, const void *kI, RowMap k_bs, float *scores, int64_t s_stride,
                               float *scores2, uint32_t *hist, hipStream_t st);

// MXFP4 operands (32-element blocks, one E8M0 scale byte each, E2M1 codes two
// per byte): quantise n_blocks blocks of x (dt elements) into codes
// [n_blocks][16] and scales [n_blocks]
hipError_t launch_mx4_quantize(int dt, int64_t n_blocks, const void *x, uint8_t *codes, uint8_t *scales,
                               hipStream_t st);
// the indexer on MXFP4 operands: queries qI [rows, HI, dI] in element type dt,
// quantised inside the kernel; keys as codes [B][k_bs rows][dI/2] and scales
// [B][k_bs rows][dI/32]; outputs as launch_index_scores
hipError_t launch_index_mx4(int dt, int B, int Tq, int N, int HI, int dI, int m, QPos q_pos0, const void *qI,
                            const float *w, const uint8_t *kc, const uint8_t *ks, RowMap k_bs, float *scores,
                            int64_t s_stride, float *scores2, uint32_t *hist, hipStream_t st);

// row stride of the score rows the top-k reads: N rounded up to 64 floats, so
// every row starts 256-byte aligned and 16-byte loads never leave the row
constexpr int64_t topk_score_stride(int64_t N) { return (N + 63) / 64 * 64; }

hipError_t launch_fill_u32(uint32_t *p, int64_t n, uint32_t v, hipStream_t st);

// rows [B][n] of row_bytes (packed, batch stride src_bs bytes) -> dst rows
// pos0 .. (ring == 0) or the mirrored ring of `ring` positions (2*ring slots);
// vw: bytes per vector, dividing row_bytes, both pointers and both strides
hipError_t launch_append_rows(int B, int64_t n, int64_t row_bytes, int vw, const void *src, int64_t src_bs,
                              void *dst, int64_t dst_bs, int64_t pos0, int64_t ring, hipStream_t st);
// up to kMaxAppendJobs appends (each as launch_append_rows) in one launch
constexpr int kMaxAppendJobs = 8;
struct AppendJob {
    const unsigned char *src;
    unsigned char *dst;
    const int64_t *pos;  // optional per-batch position added to pos0
    int64_t n, row_bytes, src_bs, dst_bs, dst_rows, pos0, ring, every;
    int vw, B;
    RowMap dmap;         // with a page table: destination rows of a paged cache (ring == 0)
};
struct AppendJobs {
    AppendJob j[kMaxAppendJobs];
};
hipError_t launch_append_multi(const AppendJobs &jobs, int count, hipStream_t st);
// measurement helper: stream-read `bytes` (a multiple of 16 KiB * fronts, 16-byte aligned) as `fronts` concurrent
// contiguous fronts, XOR-folding into sink[0..63]
hipError_t launch_stream_read(const void *p, int64_t bytes, int fronts, uint32_t *sink, hipStream_t st);
// pos[b] += delta for b < B
hipError_t launch_positions_advance(int B, int64_t *pos, int64_t delta, hipStream_t st);

// scores: [rows][topk_score_stride(N)], 16-byte aligned.  scratch:
// topk_scratch_bytes(rows, N) bytes; its histogram part must have been filled
// by launch_index_scores (zeroed before it)
hipError_t launch_topk(int B, int Tq, int N, int m, int k, QPos q_pos0, const float *scores, void *scratch,
                       int32_t *out, hipStream_t st);

// attention work split: aim for this many workgroups, at most this many
// splits of one query's rows, and at most this many 32-row tiles per split
constexpr int kMqaTargetBlocks = 256;
constexpr int kMqaMaxSplits = 16;
// (the row table shares LDS with the tile stages: four stages of bf16 rows of
// d=512, or three of fp32 ones, leave room for 48 tiles)
constexpr int kMqaMaxTilesPerSplit = 120;
constexpr int mqa_max_tiles_per_split(int d) { return d >= 512 ? 48 : kMqaMaxTilesPerSplit; }

// split count and tiles (of 32 rows) per split for `rows` queries whose row
// lists hold at most n_rows_max rows
int mqa_choose_splits(int64_t rows, int64_t n_rows_max, int d, int *tiles_per_split);
struct MqaArgs;
// bf16 rows of d = 512 with 33..64 heads: the 32-head-wave kernel (its split-K
// partials are merged by the caller)
hipError_t launch_mqa_wide(const MqaArgs &a, int64_t rows, hipStream_t st);
size_t mqa_wide_lds_bytes(int tiles_per_split);

// ws: split-K partials, rows*n_splits*H*(d+2) floats (unused when n_splits == 1)
// raw_ring: 0 -> raw row r is position raw_pos0 + r; R > 0 -> position p is raw row p mod R
hipError_t launch_mqa(int dt, int B, int Tq, int H, int d, int N, int m, int k, int W, QPos q_pos0, float scale,
                      const void *q, const void *entries, RowMap e_bs, const int32_t *idx, const void *raw,
                      int64_t raw_bs, int64_t raw_pos0, int64_t raw_ring, float *out, float *lse, float *ws,
                      int n_splits, int tiles_per_split, hipStream_t st);

}  // namespace csa
