/*
 * csa.h -- C ABI of the MI355X (gfx950) compressed-attention library libcsa.so.
 *
 * The library computes one layer of DeepSeek-V4's hybrid compressed
 * attention, as the DeepSeek-V4 overview page (gitcode.csdn.net) states it
 * in section 2 ("hybrid attention architecture"):
 *
 *   csa_compress    -- section 2.2, CSA step 1 (and 2.3 for HCA): every m
 *                      adjacent tokens' KV latents are pooled into one entry
 *                      with weights from a softmax over learned logits.
 *   csa_index_topk  -- section 2.2, step 2: a lightweight "lightning indexer"
 *                      scores the query against every causally visible entry
 *                      and only the top-k entries are kept.
 *   csa_sparse_mqa  -- section 2.2, step 3: the kept entries serve as both key
 *                      and value, shared by all query heads (multi-query
 *                      attention), in one softmax with a window of recent raw
 *                      tokens.
 *   hca_dense_mqa   -- section 2.3: the same attention over every visible
 *                      entry (no selection), for m=128 compression.
 *
 * Conventions common to every call
 * --------------------------------
 * Memory.   Every tensor argument is a DEVICE pointer to caller-owned memory.
 *           The library never allocates, frees, synchronises or prints, and
 *           keeps no state between calls except a per-thread error string.
 * Streams.  `stream` is a hipStream_t passed as void*.  NULL is the default
 *           stream.  Every call only enqueues work on that stream and returns;
 *           a fault during execution surfaces at the caller's next
 *           synchronisation on that stream.
 * Types.    `dt` (csa_dtype_t) is the element type of raw latents, compressed
 *           entries, queries and indexer keys/queries: CSA_F32 or CSA_BF16.
 *           Pooling logits, indexer head weights, scores, outputs and lse are
 *           always float32; selections are int32.  Arithmetic is float32
 *           (bf16 products are exact in float32; sums accumulate in float32).
 * Layout.   Row-major with the innermost dimension packed.  The batch stride of
 *           raw / entries / indexer keys is an explicit argument in ELEMENTS,
 *           so a cache may have capacity beyond N.  Every tensor pointer must
 *           be 16-byte aligned and every batch stride a multiple of 8 elements.
 * Position. A query's absolute position is t = q_pos0 + i for query row i.
 *           Compressed entry g covers positions [g*m, g*m+m); it is visible to
 *           t when g*m+m-1 <= t, so n_visible(t) = min(N, floor((t+1)/m)).
 *           The window of t is positions max(0, t-W+1) .. t (W rows, t
 *           included); raw row r of a batch holds position raw_pos0 + r.
 * Errors.   Every call returns 0 (CSA_OK) or a negative csa_status_t.  On an
 *           error nothing has been enqueued; csa_last_error_detail() (per
 *           thread) says which argument was wrong.  CSA_EHIP reports a failed
 *           kernel launch.
 * Sizes.    d in {32, 64, 128, 256, 512}; d_I in {32, 64, 128}; H <= 64;
 *           H_I <= 64; m in 1..128; 0 < k <= 2048.  Other values return
 *           CSA_EUNSUPPORTED.
 */
#ifndef CSA_H_
#define CSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CSA_OK = 0,
    CSA_EINVAL = -1,       /* inconsistent sizes, positions or NULL pointers   */
    CSA_EDTYPE = -2,       /* unknown element type                             */
    CSA_EALIGN = -3,       /* pointer or stride not aligned as required        */
    CSA_EWORKSPACE = -4,   /* workspace smaller than *_workspace_bytes() says  */
    CSA_EHIP = -5,         /* a kernel launch failed                           */
    CSA_EUNSUPPORTED = -6  /* size outside the supported set                   */
} csa_status_t;

typedef enum { CSA_F32 = 0, CSA_BF16 = 1 } csa_dtype_t;

/* Version of this ABI (incremented on any incompatible change). */
int csa_abi_version(void);
/* Static description of a status code. */
const char *csa_status_string(int status);
/* Detail of the last error returned on the calling thread ("" if none). */
const char *csa_last_error_detail(void);

/*
 * csa_compress -- group compression (overview page, section 2.2 step 1;
 * section 2.3 for m=128).  For batch b and group g < G:
 *     alpha_i = softmax_i(logits[b, g*m + i]),  i < m
 *     out[b, g, :] = sum_i alpha_i * raw[b, g*m + i, :]
 * rounded once to `dt` (round-to-nearest-even for bf16).
 *   raw     [B, G*m, d]  dt,  batch stride raw_bstride elements
 *   logits  [B, G*m]     f32, batch stride logit_bstride elements
 *   out     [B, G, d]    dt,  batch stride out_bstride elements (may point
 *                        into a cache at entry g0: out = cache + g0*d)
 * `out` must not overlap `raw` or `logits`.
 */
int csa_compress(int dt, int B, int G, int m, int d,
                 const void *raw, int64_t raw_bstride,
                 const float *logits, int64_t logit_bstride,
                 void *out, int64_t out_bstride, void *stream);

/*
 * csa_compress_channels -- group compression with per-channel pooling
 * logits (overview page, section 2.2 step 1: the compression weights come
 * from a learnable softmax normalisation; this is the per-channel form of
 * it).  For batch b, group g < G and channel x < d:
 *     alpha_i[x] = softmax_i(logits[b, g*m + i, x]),  i < m
 *     out[b, g, x] = sum_i alpha_i[x] * raw[b, g*m + i, x]
 * rounded once to `dt`.  The same call pools an index-key stream into the
 * entries' index keys (d = d_I) when those keys are produced by the compressor.
 *   raw     [B, G*m, d]  dt,  batch stride raw_bstride elements
 *   logits  [B, G*m, d]  f32, batch stride logit_bstride elements (multiple of 4)
 *   out     [B, G, d]    dt,  batch stride out_bstride elements
 * raw, logits and out 16-byte aligned; `out` must not overlap raw or logits.
 */
int csa_compress_channels(int dt, int B, int G, int m, int d,
                          const void *raw, int64_t raw_bstride,
                          const float *logits, int64_t logit_bstride,
                          void *out, int64_t out_bstride, void *stream);

/*
 * csa_append_rows -- cache maintenance between steps (overview page, section
 * 2.2 step 1: the raw tokens of a group are kept until its m-th token
 * arrives and the group becomes one entry; the window of raw tokens is kept
 * for the attention).  Copies rows into a cache or a raw-token ring:
 *     ring == 0:  dst[b, pos0 + i] = rows[b, i]
 *     ring == R:  dst[b, (pos0+i) mod R] = dst[b, (pos0+i) mod R + R] = rows[b, i]
 * for b < B, i < n.  The ring is mirrored (2R slots), so positions
 * p .. p+L-1 (L <= R) of a ring sit in slots p mod R .. p mod R + L - 1 and a
 * window of the raw stream is a plain strided view of it.  Rows are opaque
 * bytes (element rows, f32 logits, FP4 codes or scale bytes).
 *   rows  [B, n] rows of row_bytes bytes, packed; batch stride rows_bstride BYTES
 *   dst   [B, dst_rows] rows of row_bytes bytes; batch stride dst_bstride BYTES
 *         (ring == 0: pos0 + n <= dst_rows; ring > 0: n <= ring, 2*ring <= dst_rows)
 * `rows` must not overlap `dst`.  B <= 65535.  Any alignment (wider moves
 * when row_bytes, pointers and strides allow).
 */
int csa_append_rows(int B, int n, int64_t row_bytes, const void *rows, int64_t rows_bstride,
                    void *dst, int64_t dst_bstride, int64_t dst_rows, int64_t pos0, int64_t ring,
                    void *stream);

/*
 * csa_append_rows_multi -- several csa_append_rows in one launch (a decode
 * step appends a token's raw row, its logits and, with pooled index keys,
 * its index key and their logits).  With pos == NULL and every == 0, job i
 * does exactly what csa_append_rows(jobs[i].B, jobs[i].n, ...) does, with the
 * same checks.  Two extensions serve ragged batches (each sequence at its own
 * position):
 *   pos    device array [B] (int64): batch b's rows start at position
 *          pos0 + pos[b] instead of pos0;
 *   every  > 0: only the row of a token that completes a group of `every`
 *          tokens is kept (position p with (p+1) mod every == 0), written to
 *          that group's row (p+1)/every - 1 (an entry's index key enters
 *          the cache when its group is emitted).
 * Positions read from memory are not checked by the host: the kernel skips
 * rows whose destination falls outside [0, dst_rows) (ring == 0) or whose
 * position is negative.  No job's destination may overlap another job's rows
 * or destination.  count <= 8; the job array is read during the call only.
 * Errors name the job.
 */
typedef struct {
    int B, n;
    int64_t row_bytes;
    const void *rows;
    int64_t rows_bstride;
    void *dst;
    int64_t dst_bstride, dst_rows, pos0, ring;
    const int64_t *pos;
    int64_t every;
    const int32_t *page_table;  /* paged destination (ring == 0): see "Paged caches" below */
    int max_pages, page_rows;
    int64_t n_pages;
} csa_append_job;
int csa_append_rows_multi(int count, const csa_append_job *jobs, void *stream);

/*
 * Ragged batches: B sequences, each at its own length, decoding one token
 * each.  pos is a device array [B] (int64) holding each sequence's newest
 * token position t_b; it is read by the kernels, so a step captured in a HIP
 * graph keeps working as the positions advance (csa_positions_advance).  The
 * host cannot check device positions: every ragged call is memory-safe for
 * any values (visibility is clamped to N, ring rows are taken mod ring,
 * destinations outside a cache are skipped), and positions outside what the
 * caches hold give meaningless but bounded results.
 *
 * csa_positions_advance -- pos[b] += delta for b < B.
 *
 * csa_ragged_compress -- a1 for ragged batches (overview page, section 2.2
 * step 1: a group becomes an entry when its m-th token arrives).  For every
 * sequence whose newest token completes a group ((t_b + 1) mod m == 0) the
 * group g = (t_b+1)/m - 1 is pooled as csa_compress does, from its m rows
 * and logits in mirrored rings (position p at ring row p mod ring; the rings
 * hold 2*ring rows, m <= ring), into out[b, g] if g < out_rows.
 *   raw_ring    [B, 2*ring, d]  dt,  batch stride ring_bstride elements
 *   logit_ring  [B, 2*ring]     f32, batch stride logit_bstride elements
 *   out         [B, out_rows, d] dt, batch stride out_bstride elements
 *
 * csa_ragged_index_topk / csa_ragged_index_topk_mx4 -- csa_index_topk /
 * csa_index_topk_mx4 with one query per sequence at position t_b (Tq = 1;
 * n_visible(t_b) entries of the N in the cache are scored).  Same workspace
 * (csa_index_topk_workspace_bytes(B, 1, N, H_I, k)) and outputs.
 *
 * csa_ragged_sparse_mqa / hca_ragged_dense_mqa -- csa_sparse_mqa /
 * hca_dense_mqa with one query per sequence at position t_b; the window's
 * raw rows come from a ring (position p at row p mod ring, ring >= W), so no
 * raw_pos0 is needed.  q [B, 1, H, d]; workspace as for Tq = 1.
 *
 * Paged caches (every ragged call and append job that addresses a cache):
 * with page_table == NULL a cache is [B, rows, row] with the batch stride
 * given; otherwise it is a pool of n_pages pages of page_rows rows (a power
 * of two >= 16) shared by the batch, row j of sequence b lying in row
 * j mod page_rows of page page_table[b * max_pages + j / page_rows]
 * (int32, max_pages <= 1024 entries per sequence, covering N / out_rows).
 * The batch stride is then ignored.  Page ids read from memory are clamped
 * into [0, n_pages).  Paged index keys need d_I = 128 (bf16 keys, or FP4
 * codes with 4-byte aligned scales).  Entries and index keys of one layer
 * may share one table.
 */
int csa_positions_advance(int B, int64_t *pos, int64_t delta, void *stream);
int csa_ragged_compress(int dt, int B, int m, int d, const int64_t *pos,
                        const void *raw_ring, int64_t ring_bstride,
                        const float *logit_ring, int64_t logit_bstride, int64_t ring,
                        void *out, int64_t out_bstride, int64_t out_rows,
                        const int32_t *page_table, int max_pages, int page_rows, int64_t n_pages,
                        void *stream);
int csa_ragged_index_topk(int dt, int B, int N, int H_I, int d_I, int m, int k, const int64_t *pos,
                          const void *q_idx, const float *w_idx,
                          const void *k_idx, int64_t k_bstride,
                          const int32_t *page_table, int max_pages, int page_rows, int64_t n_pages,
                          int32_t *topk_idx, float *scores_out,
                          void *workspace, size_t workspace_bytes, void *stream);
int csa_ragged_index_topk_mx4(int dt, int B, int N, int H_I, int d_I, int m, int k, const int64_t *pos,
                              const void *q_idx, const float *w_idx,
                              const uint8_t *k_codes, const uint8_t *k_scales, int64_t k_bstride,
                              const int32_t *page_table, int max_pages, int page_rows, int64_t n_pages,
                              int32_t *topk_idx, float *scores_out,
                              void *workspace, size_t workspace_bytes, void *stream);
/*
 * flags of the fused compress + index calls.
 * CSA_HIST_ZERO: the caller vouches that the top-k histograms in the
 *   workspace are zero, as they are in a zero-filled workspace and after any
 *   call of these or the index calls whose most recent predecessor on the
 *   workspace had the same B, Tq and N (every index call leaves its
 *   histograms zero).  The call then clears nothing first: on the selection's
 *   multi-workgroup path (few queries: decode) the compression runs in the
 *   top-k filter launch instead, one launch fewer per step; otherwise in a
 *   launch of its own before the indexer.  Results are unchanged.  With
 *   nonzero histograms the selection is wrong (the kernels still touch no
 *   memory outside the call's operands and workspace).
 * Other bits: CSA_EINVAL.
 */
#define CSA_HIST_ZERO 1

/*
 * csa_ragged_compress_index_topk (+ _mx4) -- csa_ragged_compress followed by
 * csa_ragged_index_topk (csa_ragged_index_topk_mx4) on the same stream, the
 * compression running in the launch that clears the selection's histograms,
 * as csa_compress_index_topk does for uniform batches.  The arguments are the
 * two calls' own, in order (dt, B, m and pos shared; the e_ page arguments
 * are the compression's, the others the index keys'); the results equal
 * those of the two calls bit for bit.  Besides each call's checks,
 * entries_out may overlap no index operand, output or the workspace, and the
 * rings and pos may overlap neither the workspace nor an index output
 * (CSA_EINVAL).  flags: 0 or CSA_HIST_ZERO (above).
 */
int csa_ragged_compress_index_topk(int dt, int B, int m, int d, const int64_t *pos,
                                   const void *raw_ring, int64_t ring_bstride,
                                   const float *logit_ring, int64_t logit_bstride, int64_t ring,
                                   void *entries_out, int64_t out_bstride, int64_t out_rows,
                                   const int32_t *e_page_table, int e_max_pages, int e_page_rows,
                                   int64_t e_n_pages,
                                   int N, int H_I, int d_I, int k,
                                   const void *q_idx, const float *w_idx,
                                   const void *k_idx, int64_t k_bstride,
                                   const int32_t *page_table, int max_pages, int page_rows, int64_t n_pages,
                                   int32_t *topk_idx, float *scores_out,
                                   void *workspace, size_t workspace_bytes, int flags, void *stream);
int csa_ragged_compress_index_topk_mx4(int dt, int B, int m, int d, const int64_t *pos,
                                       const void *raw_ring, int64_t ring_bstride,
                                       const float *logit_ring, int64_t logit_bstride, int64_t ring,
                                       void *entries_out, int64_t out_bstride, int64_t out_rows,
                                       const int32_t *e_page_table, int e_max_pages, int e_page_rows,
                                       int64_t e_n_pages,
                                       int N, int H_I, int d_I, int k,
                                       const void *q_idx, const float *w_idx,
                                       const uint8_t *k_codes, const uint8_t *k_scales, int64_t k_bstride,
                                       const int32_t *page_table, int max_pages, int page_rows, int64_t n_pages,
                                       int32_t *topk_idx, float *scores_out,
                                       void *workspace, size_t workspace_bytes, int flags, void *stream);
int csa_ragged_sparse_mqa(int dt, int B, int H, int d, int N, int m, int k, int W,
                          const int64_t *pos, float scale,
                          const void *q,
                          const void *entries, int64_t e_bstride,
                          const int32_t *page_table, int max_pages, int page_rows, int64_t n_pages,
                          const int32_t *topk_idx,
                          const void *raw_ring, int64_t ring_bstride, int64_t ring,
                          float *out, float *lse,
                          void *workspace, size_t workspace_bytes, void *stream);
int hca_ragged_dense_mqa(int dt, int B, int H, int d, int N, int m, int W,
                         const int64_t *pos, float scale,
                         const void *q,
                         const void *entries, int64_t e_bstride,
                         const int32_t *page_table, int max_pages, int page_rows, int64_t n_pages,
                         const void *raw_ring, int64_t ring_bstride, int64_t ring,
                         float *out, float *lse,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * csa_index_topk -- lightning indexer and per-query top-k (overview page,
 * section 2.2 step 2; indexer form fixed as a sum over index heads of a
 * head weight times ReLU of a query-key dot product).  For query row i of
 * batch b at position t = q_pos0 + i and entry j < n_visible(t):
 *     s[j] = sum_h w_idx[b,i,h] * max(0, q_idx[b,i,h,:] . k_idx[b,j,:])
 * The k entries first in the order (s descending, j ascending) are kept; if
 * n_visible(t) <= k all visible entries are kept.  topk_idx[b,i,:] holds
 * the kept indices in ascending order followed by -1 padding.
 *   q_idx     [B, Tq, H_I, d_I]  dt
 *   w_idx     [B, Tq, H_I]       f32
 *   k_idx     [B, N, d_I]        dt, batch stride k_bstride elements
 *   topk_idx  [B, Tq, k]         int32 (output)
 *   scores_out optional [B, Tq, N] f32 (output): s[j] for visible j, -inf
 *             for j >= n_visible(t).  NULL: scores stay in the workspace.
 *   workspace device scratch of at least
 *             csa_index_topk_workspace_bytes(B, Tq, N, H_I, k) bytes (always
 *             required: it also holds the selection's histograms); it must
 *             not overlap any argument.  N <= 4190208.
 * Scores must not be NaN (inputs must be finite).
 */
size_t csa_index_topk_workspace_bytes(int B, int Tq, int N, int H_I, int k);
int csa_index_topk(int dt, int B, int Tq, int N, int H_I, int d_I, int m, int k,
                   int64_t q_pos0,
                   const void *q_idx, const float *w_idx,
                   const void *k_idx, int64_t k_bstride,
                   int32_t *topk_idx, float *scores_out,
                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * csa_index_scores -- the lightning indexer alone (overview page, section 2.2
 * step 2, scoring part): writes scores[b, i, j] = s[j] as defined for
 * csa_index_topk for every visible entry and -inf for j >= n_visible(t).
 * Same arguments and rules as csa_index_topk; no selection, no workspace.
 *   scores    [B, Tq, N] f32 (output)
 */
int csa_index_scores(int dt, int B, int Tq, int N, int H_I, int d_I, int m, int64_t q_pos0,
                     const void *q_idx, const float *w_idx,
                     const void *k_idx, int64_t k_bstride,
                     float *scores, void *stream);

/*
 * FP4 indexer operands (overview page, section 9, summary of key innovations,
 * item 5: the indexer's queries and keys are quantised to FP4).  The block
 * format is OCP MXFP4, the one gfx950's scaled MFMA consumes: each run of 32
 * consecutive elements shares one scale byte E (E8M0: the value 2^(E-127));
 * each element is a 4-bit E2M1 code (bit 3 sign, bits 2..1 exponent with bias
 * 1, bit 0 mantissa: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), two codes per
 * byte with the even element in the low nibble.  A row of d_I elements is
 * d_I/2 code bytes and d_I/32 scale bytes.
 *
 * csa_mx4_quantize -- codes and scales of n_rows rows of d elements (d a
 * multiple of 32).  Per block: E = 127 + clamp(floor(log2 max|v|) - 2, -127,
 * 127); each v / 2^(E-127) goes to the nearest E2M1 magnitude, ties to the even
 * mantissa, magnitudes beyond 6 saturate to 6; the sign bit is v's sign bit.
 * A block of zeros gets E = 0 and zero codes.  Inputs must be finite.
 *   x       [n_rows, d]      dt (dense)
 *   codes   [n_rows, d/2]    uint8 (output, dense)
 *   scales  [n_rows, d/32]   uint8 (output, dense)
 * x and codes 16-byte aligned; outputs must not overlap the input.
 */
int csa_mx4_quantize(int dt, int64_t n_rows, int d, const void *x,
                     uint8_t *codes, uint8_t *scales, void *stream);

/*
 * csa_index_topk_mx4 -- csa_index_topk with MXFP4 index operands: the index
 * queries arrive in the element type dt and are quantised inside the call
 * exactly as csa_mx4_quantize does; the keys arrive as MXFP4 codes and scales
 * (quantised once, when they entered the cache).  The scores are the same
 * formula on the exact values the codes and scales stand for, accumulated in
 * float32.
 *   q_idx     [B, Tq, H_I, d_I]     dt
 *   w_idx     [B, Tq, H_I]          f32
 *   k_codes   [B, N, d_I/2]         uint8     k_scales [B, N, d_I/32]  uint8
 *             both with a batch stride of k_bstride ROWS (entries)
 *   topk_idx, scores_out, workspace: as csa_index_topk, with the same
 *             workspace size (csa_index_topk_workspace_bytes).
 * q_idx and k_codes 16-byte aligned.  d_I in {32, 64, 128}.
 */
int csa_index_topk_mx4(int dt, int B, int Tq, int N, int H_I, int d_I, int m, int k,
                       int64_t q_pos0,
                       const void *q_idx, const float *w_idx,
                       const uint8_t *k_codes, const uint8_t *k_scales, int64_t k_bstride,
                       int32_t *topk_idx, float *scores_out,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * csa_index_scores_mx4 -- the FP4 lightning indexer alone: the scores of
 * csa_index_topk_mx4 (same operands, quantisation and rules), -inf for
 * j >= n_visible(t); no selection, no workspace.
 *   scores    [B, Tq, N] f32 (output, dense)
 */
int csa_index_scores_mx4(int dt, int B, int Tq, int N, int H_I, int d_I, int m, int64_t q_pos0,
                         const void *q_idx, const float *w_idx,
                         const uint8_t *k_codes, const uint8_t *k_scales, int64_t k_bstride,
                         float *scores, void *stream);

/*
 * csa_compress_index_topk / csa_compress_index_topk_mx4 -- csa_compress
 * followed by csa_index_topk (or csa_index_topk_mx4) on the same stream, as
 * one CSA step issues them (overview page, section 2.2: the new groups are
 * compressed, then the indexer selects among the cached entries).  The
 * compression goes into the launch that also clears the selection's
 * histograms, which saves one launch per step.  Its output is the attention's
 * entries cache, not the index keys, so the indexer does not read it.
 *   raw .. out_bstride  exactly csa_compress's arguments (dt, B, m and the
 *                       rules are shared with the index call; G = 0 skips the
 *                       compression)
 *   Tq .. stream        exactly csa_index_topk's (csa_index_topk_mx4's)
 *                       arguments after B and m
 * Both results equal those of the two separate calls, bit for bit.  Besides
 * each call's own checks, entries_out may overlap no index operand, output or
 * the workspace, and raw / logits may overlap neither the workspace nor an
 * index output (CSA_EINVAL).  flags: 0 or CSA_HIST_ZERO (defined above
 * csa_ragged_compress_index_topk).  On an error nothing is launched.
 */
int csa_compress_index_topk(int dt, int B, int G, int m, int d,
                            const void *raw, int64_t raw_bstride,
                            const float *logits, int64_t logit_bstride,
                            void *entries_out, int64_t out_bstride,
                            int Tq, int N, int H_I, int d_I, int k, int64_t q_pos0,
                            const void *q_idx, const float *w_idx,
                            const void *k_idx, int64_t k_bstride,
                            int32_t *topk_idx, float *scores_out,
                            void *workspace, size_t workspace_bytes, int flags, void *stream);
int csa_compress_index_topk_mx4(int dt, int B, int G, int m, int d,
                                const void *raw, int64_t raw_bstride,
                                const float *logits, int64_t logit_bstride,
                                void *entries_out, int64_t out_bstride,
                                int Tq, int N, int H_I, int d_I, int k, int64_t q_pos0,
                                const void *q_idx, const float *w_idx,
                                const uint8_t *k_codes, const uint8_t *k_scales, int64_t k_bstride,
                                int32_t *topk_idx, float *scores_out,
                                void *workspace, size_t workspace_bytes, int flags, void *stream);

/*
 * csa_sparse_mqa -- shared-KV multi-query attention over the selected
 * entries plus the raw window, one softmax (overview page, section 2.2
 * step 3: selected entries act as both key and value, all heads share them).
 * For query row i (position t) the row set is
 *     R = { entries[b, j] : j in topk_idx[b,i,:], 0 <= j < n_visible(t) }
 *       + { raw[b, p - raw_pos0] : max(0, t-W+1) <= p <= t }
 * (slots holding -1 or an index outside [0, n_visible(t)) are skipped), and
 * for every head h
 *     l_r = scale * q[b,i,h,:] . R_r,   o = sum_r softmax(l)_r R_r,
 *     lse = log sum_r exp(l_r).
 * An empty row set gives o = 0 and lse = -inf.
 *   q         [B, Tq, H, d]    dt
 *   entries   [B, N, d]        dt, batch stride e_bstride elements
 *   topk_idx  [B, Tq, k]       int32
 *   raw       [B, raw_len, d]  dt, batch stride raw_bstride elements;
 *             must cover the window: raw_pos0 <= max(0, q_pos0-W+1) and
 *             raw_pos0 + raw_len >= q_pos0 + Tq  (checked, CSA_EINVAL)
 *   out       [B, Tq, H, d]    f32 (output)
 *   lse       [B, Tq, H]       f32 (output, optional: NULL)
 *   workspace at least csa_mqa_workspace_bytes(B, Tq, H, d, k + W) bytes.
 */
size_t csa_mqa_workspace_bytes(int B, int Tq, int H, int d, int n_rows_max);
int csa_sparse_mqa(int dt, int B, int Tq, int H, int d, int N, int m, int k, int W,
                   int64_t q_pos0, float scale,
                   const void *q,
                   const void *entries, int64_t e_bstride,
                   const int32_t *topk_idx,
                   const void *raw, int64_t raw_bstride, int64_t raw_pos0, int raw_len,
                   float *out, float *lse,
                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * hca_dense_mqa -- HCA attention (overview page, section 2.3: no sparse
 * selection, dense attention over all compressed entries).  Same as
 * csa_sparse_mqa with the row set { entries[b, j] : j < n_visible(t) } plus
 * the same raw window.  workspace: csa_mqa_workspace_bytes(B, Tq, H, d, N + W).
 */
int hca_dense_mqa(int dt, int B, int Tq, int H, int d, int N, int m, int W,
                  int64_t q_pos0, float scale,
                  const void *q,
                  const void *entries, int64_t e_bstride,
                  const void *raw, int64_t raw_bstride, int64_t raw_pos0, int raw_len,
                  float *out, float *lse,
                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * csa_index_topk_noalloc -- csa_index_topk for callers that cannot allocate
 * (code under HIP graph capture that may not call hipMalloc, tight serving
 * loops, harnesses that forbid allocation).  Same arguments, outputs and
 * errors as csa_index_topk, without the workspace: the call uses a
 * scratch array of CSA_NOALLOC_SCRATCH_BYTES held in the library, one per
 * GPU, allocated when the library is loaded on that GPU and kept until the
 * process ends.  It calls no allocator.  Sizes whose
 * csa_index_topk_workspace_bytes(B, Tq, N, H_I, k) exceeds
 * CSA_NOALLOC_SCRATCH_BYTES return CSA_EWORKSPACE before anything is
 * enqueued (16 MiB holds e.g. 32 decode queries over 32768 entries or 4
 * over 262144).  Every call on one GPU shares that GPU's array and the array
 * keeps the last call's contents (the part that must start at zero is
 * cleared by the call itself): calls that overlap in time on one GPU (on
 * different streams, or from different threads without ordering) race and
 * must be serialised by the caller.  The first call on each device looks up
 * the array's device address (hipGetSymbolAddress) with that device
 * current; a failure there returns CSA_EHIP.
 */
#define CSA_NOALLOC_SCRATCH_BYTES (16u << 20)
int csa_index_topk_noalloc(int dt, int B, int Tq, int N, int H_I, int d_I, int m, int k,
                           int64_t q_pos0,
                           const void *q_idx, const float *w_idx,
                           const void *k_idx, int64_t k_bstride,
                           int32_t *topk_idx, float *scores_out, void *stream);

/*
 * csa_stream_read -- measurement helper (not part of the method): reads
 * `bytes` of `buf` as `fronts` contiguous fronts streamed at the same time,
 * with the indexer's load path (1 KiB non-temporal LDS-DMA per instruction,
 * 32 KiB in flight per wavefront, 1024 wavefronts), and XOR-folds one word
 * per wavefront into sink[0..63] (uint32, caller-owned, read-modify-write).
 * The lightning indexer streams one front per query; this is the reference
 * its HBM rate is compared with.  fronts a divisor of 1024, bytes a multiple
 * of 1 KiB * fronts, buf 16-byte aligned.
 */
int csa_stream_read(const void *buf, int64_t bytes, int fronts, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H_ */
