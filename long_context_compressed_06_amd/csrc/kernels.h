// Launchers of the gfx950 kernels (one translation unit per kernel family).
// dt: 0 = float32 elements, 1 = bf16 elements.  All pointers are device
// pointers; every launcher only enqueues on `st` and returns the launch
// status.  Argument checking happens in abi.cpp before any launcher runs.
#pragma once

#include "common.h"

namespace csa {

// longest score row that the top-k kernel stages in LDS (128 KiB of keys)
constexpr int kTopkLdsKeys = 32768;

hipError_t launch_compress(int dt, int B, int G, int m, int d, const void *raw, int64_t raw_bs,
                           const float *logits, int64_t log_bs, void *out, int64_t out_bs, hipStream_t st);

hipError_t launch_index_scores(int dt, int B, int Tq, int N, int HI, int dI, int m, int64_t q_pos0, const void *qI,
                               const float *w, const void *kI, int64_t k_bs, float *scores, hipStream_t st);

hipError_t launch_topk(int B, int Tq, int N, int m, int k, int64_t q_pos0, const float *scores, int32_t *out,
                       hipStream_t st);

// split count and tiles (of 32 rows) per split for `rows` queries whose row
// lists hold at most n_rows_max rows
int mqa_choose_splits(int64_t rows, int64_t n_rows_max, int *tiles_per_split);

// ws: split-K partials, rows*n_splits*H*(d+2) floats (unused when n_splits == 1)
hipError_t launch_mqa(int dt, int B, int Tq, int H, int d, int N, int m, int k, int W, int64_t q_pos0, float scale,
                      const void *q, const void *entries, int64_t e_bs, const int32_t *idx, const void *raw,
                      int64_t raw_bs, int64_t raw_pos0, float *out, float *lse, float *ws, int n_splits,
                      int tiles_per_split, hipStream_t st);

}  // namespace csa
