/*
 * CPU oracle for DeepSeek-V4 hybrid compressed attention (CSA / HCA).
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load this library.  It
 * shares no source, header, table or helper with the HIP library.
 *
 * Everything is plain C: scalar loops, double accumulation, no SIMD
 * intrinsics, no fast-math, one pthread pool over independent rows.  Inputs
 * arrive as float arrays (bf16 and fp32 inputs convert to float exactly) and
 * are widened to double on read.  Arrays are dense, row-major, no strides.
 *
 * Sources (the DeepSeek-V4 overview page on gitcode.csdn.net, section 2
 * "hybrid attention architecture"):
 *   2.2 step 1  -- every m=4 adjacent tokens' KV pooled into one entry with
 *                  weights from a learnable softmax normalisation;
 *   2.2 step 2  -- a lightweight "lightning indexer" scores each query
 *                  against the compressed entries; keep the top-k (k=1024);
 *   2.2 step 3  -- the selected entries act as both key and value, shared
 *                  by all query heads (MQA);
 *   2.3         -- HCA pools 128 tokens per entry and attends densely.
 * The indexer form  s_j = sum_h w_h * ReLU(q_h . k_j)  and the sliding window
 * of recent raw tokens inside the same softmax are fixed by the project
 * statement of the method, not by the pages.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* A minimal parallel-for over independent work items.                 */
/* ------------------------------------------------------------------ */
typedef void (*item_fn)(void *ctx, long item);

typedef struct {
    item_fn fn;
    void *ctx;
    long n_items;
    long next;
    pthread_mutex_t lock;
} pool_t;

static void *pool_worker(void *arg) {
    pool_t *p = (pool_t *)arg;
    for (;;) {
        long it;
        pthread_mutex_lock(&p->lock);
        it = p->next++;
        pthread_mutex_unlock(&p->lock);
        if (it >= p->n_items) break;
        p->fn(p->ctx, it);
    }
    return NULL;
}

static void parallel_for(long n_items, int nthreads, item_fn fn, void *ctx) {
    pool_t p;
    pthread_t th[256];
    int i, nt;
    if (n_items <= 0) return;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > n_items) nthreads = (int)n_items;
    p.fn = fn;
    p.ctx = ctx;
    p.n_items = n_items;
    p.next = 0;
    pthread_mutex_init(&p.lock, NULL);
    nt = 0;
    for (i = 1; i < nthreads; i++) {
        if (pthread_create(&th[nt], NULL, pool_worker, &p) == 0) nt++;
    }
    pool_worker(&p);
    for (i = 0; i < nt; i++) pthread_join(th[i], NULL);
    pthread_mutex_destroy(&p.lock);
}

/* ------------------------------------------------------------------ */
/* Causal bookkeeping.                                                 */
/* A group g covers positions [g*m, g*m+m).  It is visible to a query  */
/* at position t once all of its tokens are at or before t, so the     */
/* query sees groups 0 .. floor((t+1)/m)-1, capped by the N entries    */
/* that exist.  Incomplete groups are never emitted.                   */
/* ------------------------------------------------------------------ */
long oracle_n_visible(long t, int m, long N) {
    long n;
    if (t < 0 || m <= 0) return 0;
    n = (t + 1) / m;
    return n < N ? n : N;
}

/* first raw position of the sliding window that ends at (and includes) t */
long oracle_window_start(long t, int W) {
    long s = t - (long)W + 1;
    return s > 0 ? s : 0;
}

/* ------------------------------------------------------------------ */
/* Step 1: group compression (CSA m=4, HCA m=128).                     */
/* e_g = sum_i alpha_i * c[g*m+i],  alpha = softmax over the group's   */
/* m scalar logits.  Output is the exact (unrounded) double value.     */
/* ------------------------------------------------------------------ */
typedef struct {
    int G, m, d;
    const float *raw;    /* [B, G*m, d] */
    const float *logits; /* [B, G*m]    */
    double *out;         /* [B, G, d]   */
} compress_ctx;

static void compress_item(void *vctx, long item) {
    compress_ctx *c = (compress_ctx *)vctx;
    long b = item / c->G, g = item % c->G;
    const float *z = c->logits + (b * c->G + g) * c->m;
    const float *rows = c->raw + (b * c->G + g) * (long)c->m * c->d;
    double *e = c->out + (b * c->G + g) * (long)c->d;
    double zmax = -INFINITY, denom = 0.0;
    double *alpha = (double *)malloc(sizeof(double) * c->m);
    int i, x;
    for (i = 0; i < c->m; i++)
        if ((double)z[i] > zmax) zmax = (double)z[i];
    for (i = 0; i < c->m; i++) {
        alpha[i] = exp((double)z[i] - zmax);
        denom += alpha[i];
    }
    for (i = 0; i < c->m; i++) alpha[i] /= denom;
    for (x = 0; x < c->d; x++) {
        double acc = 0.0;
        for (i = 0; i < c->m; i++) acc += alpha[i] * (double)rows[(long)i * c->d + x];
        e[x] = acc;
    }
    free(alpha);
}

void oracle_compress(int B, int G, int m, int d, const float *raw, const float *logits,
                     double *out, int nthreads) {
    compress_ctx c = {G, m, d, raw, logits, out};
    parallel_for((long)B * G, nthreads, compress_item, &c);
}

/* ------------------------------------------------------------------ */
/* Step 1 with per-channel pooling logits (a reading of the overview   */
/* page, section 2.2 step 1, which leaves the form of the learnable    */
/* softmax weights open): channel x of entry g pools channel x of its  */
/* m tokens with the softmax over the group of that channel's logits,  */
/*   e_g[x] = sum_i softmax_i(z[g*m+i, x]) * c[g*m+i, x].              */
/* Output is the exact (unrounded) double value.                        */
/* ------------------------------------------------------------------ */
static void compress_channels_item(void *vctx, long item) {
    compress_ctx *c = (compress_ctx *)vctx;
    long b = item / c->G, g = item % c->G;
    const float *z = c->logits + (b * c->G + g) * (long)c->m * c->d;  /* [m, d] */
    const float *rows = c->raw + (b * c->G + g) * (long)c->m * c->d;  /* [m, d] */
    double *e = c->out + (b * c->G + g) * (long)c->d;
    int i, x;
    for (x = 0; x < c->d; x++) {
        double zmax = -INFINITY, denom = 0.0, acc = 0.0;
        for (i = 0; i < c->m; i++)
            if ((double)z[(long)i * c->d + x] > zmax) zmax = (double)z[(long)i * c->d + x];
        for (i = 0; i < c->m; i++) {
            double a = exp((double)z[(long)i * c->d + x] - zmax);
            denom += a;
            acc += a * (double)rows[(long)i * c->d + x];
        }
        e[x] = acc / denom;
    }
}

void oracle_compress_channels(int B, int G, int m, int d, const float *raw, const float *logits,
                              double *out, int nthreads) {
    compress_ctx c = {G, m, d, raw, logits, out};
    parallel_for((long)B * G, nthreads, compress_channels_item, &c);
}

/* Round-to-nearest-even of a double to the bfloat16 grid (8 significant
 * bits, exponent range of IEEE single), returned as a float.  This is the
 * rounding the compressed cache applies when it is stored in bf16. */
static double round_to_bf16(double v) {
    int ex;
    double f, q;
    if (v == 0.0 || isnan(v) || isinf(v)) return v;
    f = frexp(v, &ex);           /* v = f * 2^ex, 0.5 <= |f| < 1 */
    (void)f;
    ex = ex - 8;                 /* quantum for 8 significant bits */
    if (ex < -133) ex = -133;    /* bf16 subnormal quantum 2^-133  */
    q = ldexp(1.0, ex);
    v = nearbyint(v / q) * q;    /* default rounding mode: ties to even */
    if (fabs(v) > 3.3895313892515355e38) v = v > 0 ? INFINITY : -INFINITY;
    return v;
}

void oracle_round_bf16(long n, const double *x, float *y) {
    long i;
    for (i = 0; i < n; i++) y[i] = (float)round_to_bf16(x[i]);
}

/* ------------------------------------------------------------------ */
/* Step 2: lightning indexer.                                          */
/* s[t, j] = sum_h w[t, h] * max(0, qI[t, h, :] . kI[j, :])            */
/* for j < n_visible(t); entries that are not visible get -inf.        */
/* Work items are (batch, query, chunk of entries).                    */
/* ------------------------------------------------------------------ */
#define IDX_CHUNK 2048

typedef struct {
    int Tq, N, HI, dI, m;
    long q_pos0;
    const float *qI; /* [B, Tq, HI, dI] */
    const float *w;  /* [B, Tq, HI]     */
    const float *kI; /* [B, N, dI]      */
    double *scores;  /* [B, Tq, N]      */
    long n_chunks;
} index_ctx;

static void index_item(void *vctx, long item) {
    index_ctx *c = (index_ctx *)vctx;
    long row = item / c->n_chunks, chunk = item % c->n_chunks;
    long b = row / c->Tq, ti = row % c->Tq;
    long t = c->q_pos0 + ti;
    long nv = oracle_n_visible(t, c->m, c->N);
    long j0 = chunk * IDX_CHUNK, j1 = j0 + IDX_CHUNK, j;
    const float *q = c->qI + row * (long)c->HI * c->dI;
    const float *w = c->w + row * (long)c->HI;
    double *s = c->scores + row * (long)c->N;
    if (j1 > c->N) j1 = c->N;
    for (j = j0; j < j1; j++) {
        const float *k = c->kI + (b * c->N + j) * (long)c->dI;
        double acc = 0.0;
        int h, x;
        if (j >= nv) {
            s[j] = -INFINITY;
            continue;
        }
        for (h = 0; h < c->HI; h++) {
            double dot = 0.0;
            for (x = 0; x < c->dI; x++) dot += (double)q[(long)h * c->dI + x] * (double)k[x];
            if (dot > 0.0) acc += (double)w[h] * dot;
        }
        s[j] = acc;
    }
}

void oracle_index_scores(int B, int Tq, int N, int HI, int dI, int m, long q_pos0,
                         const float *qI, const float *w, const float *kI, double *scores,
                         int nthreads) {
    index_ctx c;
    c.Tq = Tq; c.N = N; c.HI = HI; c.dI = dI; c.m = m; c.q_pos0 = q_pos0;
    c.qI = qI; c.w = w; c.kI = kI; c.scores = scores;
    c.n_chunks = (N + IDX_CHUNK - 1) / IDX_CHUNK;
    if (c.n_chunks < 1) c.n_chunks = 1;
    parallel_for((long)B * Tq * c.n_chunks, nthreads, index_item, &c);
}

/* ------------------------------------------------------------------ */
/* Low-precision indexer operands: MXFP4.                              */
/* The overview page (section 9, summary of key innovations, item 5)   */
/* quantises the indexer's queries and keys to FP4 without giving the  */
/* block format.  The reading here is the OCP microscaling format      */
/* MXFP4: every 32 consecutive elements share one E8M0 scale           */
/* X = 2^(E - 127); the elements are FP4 E2M1 (a sign, 2 exponent bits */
/* with bias 1, 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6).*/
/* Conversion of a block: X = 2^(floor(log2 max|v|) - 2), 2 being the  */
/* largest E2M1 exponent, with the exponent kept inside E8M0's range   */
/* [-127, 127]; each v / X goes to the nearest magnitude, a tie to the */
/* one whose mantissa bit is 0, and magnitudes past 6 saturate to 6; a */
/* code's sign bit is v's sign bit (so -0 and negatives that round to */
/* zero encode as negative zero).  A block whose elements are all zero */
/* gets E = 0 and zero codes.  Two codes per byte, the even            */
/* element in the low nibble.  Inputs must be finite.                  */
/* ------------------------------------------------------------------ */
static const double fp4_magnitude[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* nearest E2M1 code of v (already divided by the block scale) */
static int fp4_code(double v) {
    double a = fabs(v), best_err = INFINITY;
    int best = 0, i;
    for (i = 0; i < 8; i++) {
        double err = fabs(a - fp4_magnitude[i]);
        if (err < best_err || (err == best_err && (i & 1) == 0)) {
            best_err = err;
            best = i;
        }
    }
    return (signbit(v) ? 8 : 0) | best;
}

void oracle_mx4_quantize(long n_blocks, const float *x, uint8_t *codes, uint8_t *scales) {
    long blk;
    int i;
    for (blk = 0; blk < n_blocks; blk++) {
        const float *v = x + blk * 32;
        uint8_t *cb = codes + blk * 16;
        double amax = 0.0, X;
        int se, ex;
        for (i = 0; i < 32; i++)
            if (fabs((double)v[i]) > amax) amax = fabs((double)v[i]);
        if (amax == 0.0) {
            scales[blk] = 0;
            memset(cb, 0, 16);
            continue;
        }
        (void)frexp(amax, &ex);  /* amax = f * 2^ex, 0.5 <= f < 1: floor(log2 amax) = ex - 1 */
        se = ex - 1 - 2;
        if (se < -127) se = -127;
        if (se > 127) se = 127;
        scales[blk] = (uint8_t)(se + 127);
        X = ldexp(1.0, se);
        for (i = 0; i < 32; i += 2) {
            int lo = fp4_code((double)v[i] / X), hi = fp4_code((double)v[i + 1] / X);
            cb[i / 2] = (uint8_t)(lo | (hi << 4));
        }
    }
}

/* the exact value of every element (representable in float) */
void oracle_mx4_dequantize(long n_blocks, const uint8_t *codes, const uint8_t *scales, float *out) {
    long blk;
    int i;
    for (blk = 0; blk < n_blocks; blk++) {
        double X = ldexp(1.0, (int)scales[blk] - 127);
        for (i = 0; i < 32; i++) {
            int c = (codes[blk * 16 + i / 2] >> (4 * (i & 1))) & 15;
            double mag = fp4_magnitude[c & 7] * X;
            out[blk * 32 + i] = (float)((c & 8) ? -mag : mag);
        }
    }
}

/* ------------------------------------------------------------------ */
/* Step 3: per-query top-k.                                            */
/* Keep the k visible entries that come first in the total order       */
/* (score descending, index ascending).  If n_visible <= k every       */
/* visible entry is kept.  Output: indices ascending, then -1 padding. */
/* ------------------------------------------------------------------ */
typedef struct {
    double s;
    int32_t j;
} scored_t;

static int by_score_then_index(const void *a, const void *b) {
    const scored_t *x = (const scored_t *)a, *y = (const scored_t *)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->j > y->j) - (x->j < y->j);
}

static int ascending_int(const void *a, const void *b) {
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

typedef struct {
    int Tq, N, k, m;
    long q_pos0;
    const double *scores; /* [B, Tq, N] */
    int32_t *idx;         /* [B, Tq, k] */
} topk_ctx;

static void topk_item(void *vctx, long row) {
    topk_ctx *c = (topk_ctx *)vctx;
    long ti = row % c->Tq;
    long nv = oracle_n_visible(c->q_pos0 + ti, c->m, c->N);
    const double *s = c->scores + row * (long)c->N;
    int32_t *out = c->idx + row * (long)c->k;
    long i, n_sel;
    if (nv <= c->k) {
        for (i = 0; i < nv; i++) out[i] = (int32_t)i;
        n_sel = nv;
    } else {
        scored_t *all = (scored_t *)malloc(sizeof(scored_t) * nv);
        for (i = 0; i < nv; i++) {
            all[i].s = s[i];
            all[i].j = (int32_t)i;
        }
        qsort(all, nv, sizeof(scored_t), by_score_then_index);
        for (i = 0; i < c->k; i++) out[i] = all[i].j;
        free(all);
        n_sel = c->k;
        qsort(out, n_sel, sizeof(int32_t), ascending_int);
    }
    for (i = n_sel; i < c->k; i++) out[i] = -1;
}

void oracle_topk(int B, int Tq, int N, int k, int m, long q_pos0, const double *scores,
                 int32_t *idx, int nthreads) {
    topk_ctx c = {Tq, N, k, m, q_pos0, scores, idx};
    parallel_for((long)B * Tq, nthreads, topk_item, &c);
}

/* ------------------------------------------------------------------ */
/* Step 4: shared-KV multi-query attention.                            */
/* The row set of query t is the selected compressed entries followed  */
/* by the raw rows of positions window_start(t) .. t.  Every row is    */
/* both key and value.  For each head h:                               */
/*   l_r = scale * q_h . R_r ,  p_r = exp(l_r - max l),                */
/*   o_h = sum_r p_r R_r / sum_r p_r ,  lse_h = max l + log sum_r p_r. */
/* An empty row set gives o = 0 and lse = -inf.                        */
/* ------------------------------------------------------------------ */
typedef struct {
    int Tq, H, d, N, k, W, m, dense;
    long q_pos0, raw_pos0;
    int raw_len;
    double scale;
    const float *q;       /* [B, Tq, H, d] */
    const float *entries; /* [B, N, d]     */
    const int32_t *idx;   /* [B, Tq, k] (sparse only) */
    const float *raw;     /* [B, raw_len, d] */
    double *out;          /* [B, Tq, H, d] */
    double *lse;          /* [B, Tq, H]    */
} attn_ctx;

static void attn_item(void *vctx, long row) {
    attn_ctx *c = (attn_ctx *)vctx;
    long b = row / c->Tq, ti = row % c->Tq;
    long t = c->q_pos0 + ti;
    long n_sel = 0, n_rows, r, i;
    long w0 = oracle_window_start(t, c->W);
    long n_win = c->W > 0 ? t - w0 + 1 : 0;
    const float **rows;
    double *logit;
    int h, x;

    if (c->dense) {
        n_sel = oracle_n_visible(t, c->m, c->N);
    } else {
        const int32_t *sel = c->idx + row * (long)c->k;
        for (i = 0; i < c->k; i++)
            if (sel[i] >= 0) n_sel++;
    }
    n_rows = n_sel + n_win;
    rows = (const float **)malloc(sizeof(float *) * (n_rows > 0 ? n_rows : 1));
    logit = (double *)malloc(sizeof(double) * (n_rows > 0 ? n_rows : 1));
    r = 0;
    if (c->dense) {
        for (i = 0; i < n_sel; i++) rows[r++] = c->entries + (b * c->N + i) * (long)c->d;
    } else {
        const int32_t *sel = c->idx + row * (long)c->k;
        for (i = 0; i < c->k; i++)
            if (sel[i] >= 0) rows[r++] = c->entries + (b * c->N + sel[i]) * (long)c->d;
    }
    for (i = 0; i < n_win; i++)
        rows[r++] = c->raw + (b * (long)c->raw_len + (w0 + i - c->raw_pos0)) * c->d;

    for (h = 0; h < c->H; h++) {
        const float *qh = c->q + (row * c->H + h) * (long)c->d;
        double *o = c->out + (row * c->H + h) * (long)c->d;
        double mx = -INFINITY, sum = 0.0;
        for (x = 0; x < c->d; x++) o[x] = 0.0;
        if (n_rows == 0) {
            if (c->lse) c->lse[row * c->H + h] = -INFINITY;
            continue;
        }
        for (r = 0; r < n_rows; r++) {
            double dot = 0.0;
            for (x = 0; x < c->d; x++) dot += (double)qh[x] * (double)rows[r][x];
            logit[r] = c->scale * dot;
            if (logit[r] > mx) mx = logit[r];
        }
        for (r = 0; r < n_rows; r++) {
            double p = exp(logit[r] - mx);
            sum += p;
            for (x = 0; x < c->d; x++) o[x] += p * (double)rows[r][x];
        }
        for (x = 0; x < c->d; x++) o[x] /= sum;
        if (c->lse) c->lse[row * c->H + h] = mx + log(sum);
    }
    free(rows);
    free(logit);
}

void oracle_sparse_mqa(int B, int Tq, int H, int d, int N, int k, int W, long q_pos0,
                       double scale, const float *q, const float *entries, const int32_t *idx,
                       const float *raw, long raw_pos0, int raw_len, double *out, double *lse,
                       int nthreads) {
    attn_ctx c;
    memset(&c, 0, sizeof(c));
    c.Tq = Tq; c.H = H; c.d = d; c.N = N; c.k = k; c.W = W; c.m = 1; c.dense = 0;
    c.q_pos0 = q_pos0; c.raw_pos0 = raw_pos0; c.raw_len = raw_len; c.scale = scale;
    c.q = q; c.entries = entries; c.idx = idx; c.raw = raw; c.out = out; c.lse = lse;
    parallel_for((long)B * Tq, nthreads, attn_item, &c);
}

/* HCA: the same attention with every visible compressed entry selected. */
void oracle_dense_mqa(int B, int Tq, int H, int d, int N, int m, int W, long q_pos0,
                      double scale, const float *q, const float *entries, const float *raw,
                      long raw_pos0, int raw_len, double *out, double *lse, int nthreads) {
    attn_ctx c;
    memset(&c, 0, sizeof(c));
    c.Tq = Tq; c.H = H; c.d = d; c.N = N; c.k = 0; c.W = W; c.m = m; c.dense = 1;
    c.q_pos0 = q_pos0; c.raw_pos0 = raw_pos0; c.raw_len = raw_len; c.scale = scale;
    c.q = q; c.entries = entries; c.idx = NULL; c.raw = raw; c.out = out; c.lse = lse;
    parallel_for((long)B * Tq, nthreads, attn_item, &c);
}
