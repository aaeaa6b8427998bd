// extern "C" boundary of libcsa: argument checking, workspace sizing, status
// strings and dispatch to the kernel launchers.  Nothing here allocates,
// synchronises or throws; every error returns before anything is enqueued.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/csa.h"
#include "compress_fold.h"

namespace {

thread_local std::string g_detail;

int fail(int status, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_detail = buf;
    return status;
}

int ok() {
    g_detail.clear();
    return CSA_OK;
}

bool d_supported(int d) { return d == 32 || d == 64 || d == 128 || d == 256 || d == 512; }
bool dI_supported(int d) { return d == 32 || d == 64 || d == 128; }
size_t esize(int dt) { return dt == CSA_F32 ? 4 : 2; }
bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// byte range [lo, hi) of a batched tensor: B batches of `inner` elements, `bstride` apart
struct Span {
    uintptr_t lo, hi;
};
Span span(const void *p, int64_t B, int64_t bstride, int64_t inner, size_t es) {
    Span s{(uintptr_t)p, (uintptr_t)p};
    if (p && B > 0 && inner > 0) s.hi = s.lo + (size_t)((B - 1) * bstride + inner) * es;
    return s;
}
bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

int check_dt(int dt) {
    if (dt != CSA_F32 && dt != CSA_BF16) return fail(CSA_EDTYPE, "dt=%d is neither CSA_F32 nor CSA_BF16", dt);
    return CSA_OK;
}

int hip_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(CSA_EHIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// a paged cache: page_rows a power of two >= 16, at most kMaxPagesPerSeq pages per sequence covering N rows,
// a pool of n_pages pages; on success *map addresses the pool
int check_pages(const int32_t *page_table, int B, int max_pages, int page_rows, int64_t n_pages, int64_t N,
                       csa::RowMap *map) {
    if (page_rows < 16 || (page_rows & (page_rows - 1)))
        return fail(CSA_EUNSUPPORTED, "page_rows=%d is not a power of two >= 16", page_rows);
    if (max_pages < 1 || max_pages > csa::kMaxPagesPerSeq)
        return fail(CSA_EUNSUPPORTED, "max_pages=%d outside 1..%d", max_pages, csa::kMaxPagesPerSeq);
    if ((int64_t)max_pages * page_rows < N)
        return fail(CSA_EINVAL, "%d pages of %d rows do not cover N=%lld", max_pages, page_rows, (long long)N);
    if (n_pages < 1) return fail(CSA_EINVAL, "n_pages must be >= 1");
    if (!aligned(page_table, 4)) return fail(CSA_EALIGN, "page_table needs 4-byte alignment");
    int sh = 0;
    while ((1 << sh) < page_rows) ++sh;
    *map = csa::RowMap(0, page_table, max_pages, sh, n_pages);
    (void)B;
    return CSA_OK;
}

// The workspace of csa_index_topk_noalloc: one array per GPU, alive until the
// process ends.  In host code `scratch` names a host-side stand-in, never a
// device address; the device address is looked up once per device
// (scratch_on_current_device) and only that pointer is handed to kernels.
static __device__ __align__(256) unsigned char scratch[CSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// device address of `scratch` on the calling thread's current device
int scratch_on_current_device(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(CSA_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(CSA_EUNSUPPORTED, "device %d outside 0..%d", dev, kMaxDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(CSA_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return CSA_OK;
}

}  // namespace

extern "C" {

int csa_abi_version(void) { return 1; }

const char *csa_status_string(int s) {
    switch (s) {
        case CSA_OK: return "ok";
        case CSA_EINVAL: return "invalid argument";
        case CSA_EDTYPE: return "unknown element type";
        case CSA_EALIGN: return "misaligned pointer or stride";
        case CSA_EWORKSPACE: return "workspace too small";
        case CSA_EHIP: return "HIP launch failure";
        case CSA_EUNSUPPORTED: return "unsupported size";
        default: return "unknown status";
    }
}

const char *csa_last_error_detail(void) { return g_detail.c_str(); }

// a compression (csa_compress's arguments), checked on its own or ahead of an index call
struct CompressJob {
    int dt, B, G, m, d;
    const void *raw;
    int64_t raw_bs;
    const float *logits;
    int64_t log_bs;
    void *out;
    int64_t out_bs;
    // the bytes each operand spans (for the overlap checks of a fused call)
    Span raw_span() const { return span(raw, B, raw_bs, (int64_t)G * m * d, esize(dt)); }
    Span log_span() const { return span(logits, B, log_bs, (int64_t)G * m, 4); }
    Span out_span() const { return span(out, B, out_bs, (int64_t)G * d, esize(dt)); }
};

// csa_compress's checks; *empty when there is nothing to compress
static int check_compress(const CompressJob &c, bool *empty) {
    *empty = true;
    if (int s = check_dt(c.dt)) return s;
    if (c.B < 0 || c.G < 0) return fail(CSA_EINVAL, "B=%d and G=%d must be >= 0", c.B, c.G);
    if (c.m < 1 || c.m > 128) return fail(CSA_EUNSUPPORTED, "m=%d outside 1..128", c.m);
    if (!d_supported(c.d)) return fail(CSA_EUNSUPPORTED, "d=%d not in {32,64,128,256,512}", c.d);
    if ((int64_t)c.B * c.G == 0) return ok();
    if (!c.raw || !c.logits || !c.out) return fail(CSA_EINVAL, "NULL tensor pointer");
    if (c.raw_bs < (int64_t)c.G * c.m * c.d || c.log_bs < (int64_t)c.G * c.m || c.out_bs < (int64_t)c.G * c.d)
        return fail(CSA_EINVAL, "a batch stride is smaller than one batch's extent");
    if (!aligned(c.raw, 16) || !aligned(c.out, 16) || !aligned(c.logits, 4) || c.raw_bs % 8 || c.out_bs % 8)
        return fail(CSA_EALIGN, "raw/out need 16-byte alignment and batch strides a multiple of 8 elements");
    if (overlap(c.out_span(), c.raw_span()) || overlap(c.out_span(), c.log_span()))
        return fail(CSA_EINVAL, "out overlaps raw or logits");
    *empty = false;
    return CSA_OK;
}

static hipError_t launch_compress_job(const CompressJob &c, hipStream_t st, uint32_t *clr = nullptr,
                                      int64_t clr_words = 0) {
    return csa::launch_compress(c.dt, c.B, c.G, c.m, c.d, c.raw, c.raw_bs, c.logits, c.log_bs, c.out, c.out_bs, st,
                                clr, clr_words);
}

int csa_compress(int dt, int B, int G, int m, int d, const void *raw, int64_t raw_bstride, const float *logits,
                 int64_t logit_bstride, void *out, int64_t out_bstride, void *stream) {
    const CompressJob c{dt, B, G, m, d, raw, raw_bstride, logits, logit_bstride, out, out_bstride};
    bool empty;
    if (int s = check_compress(c, &empty)) return s;
    if (empty) return ok();
    return hip_status(launch_compress_job(c, (hipStream_t)stream), "compress launch");
}

static_assert(csa::kTopkBins % 4 == 0, "the fused clear zeroes whole 16-byte runs");

// A checked compression that an index call runs in the launch clearing its
// top-k histograms, or (histograms already zero) in its top-k filter launch:
// the bytes it writes and reads (for the overlap checks), how to launch it
// with that clear, and its operands for the filter launch.
struct FusedCompress {
    Span out;
    Span in[3];
    int n_in;
    hipError_t (*launch)(const void *job, hipStream_t st, uint32_t *clr, int64_t clr_words);
    const void *job;
    csa::FoldedCompress fold;
};

static FusedCompress fused(const CompressJob &c) {
    return FusedCompress{c.out_span(), {c.raw_span(), c.log_span(), Span{}}, 2,
                         [](const void *j, hipStream_t st, uint32_t *clr, int64_t cw) {
                             return launch_compress_job(*(const CompressJob *)j, st, clr, cw);
                         },
                         &c,
                         csa::FoldedCompress{false, c.dt, c.B, c.G, c.m, c.d, c.raw, c.raw_bs, c.logits, c.log_bs,
                                             c.out, c.out_bs, nullptr, 0, csa::RowMap(), 0}};
}

// the compression against the index operands, outputs and workspace (its
// output may not overlap any of them, nor its inputs the workspace or the
// index outputs: it may run before, beside or after the indexer)
static int check_compress_against(const FusedCompress *fc, const Span *in, int n_in, const Span &si,
                                  const Span &ss, const Span &sw) {
    if (!fc) return CSA_OK;
    for (int i = 0; i < n_in; ++i)
        if (overlap(fc->out, in[i])) return fail(CSA_EINVAL, "the compression output overlaps an index input");
    if (overlap(fc->out, si) || overlap(fc->out, ss) || overlap(fc->out, sw))
        return fail(CSA_EINVAL, "the compression overlaps an index output or the workspace");
    for (int i = 0; i < fc->n_in; ++i)
        if (overlap(fc->in[i], sw) || overlap(fc->in[i], si) || overlap(fc->in[i], ss))
            return fail(CSA_EINVAL, "a compression input overlaps the workspace or an index output");
    return CSA_OK;
}

static int check_flags(int flags) {
    if (flags & ~CSA_HIST_ZERO) return fail(CSA_EINVAL, "unknown flags 0x%x", (unsigned)flags);
    return CSA_OK;
}

// The launches of an index call around its indexer launch: the top-k
// histograms are cleared first (in the compression's launch when there is
// one) unless the caller vouches that they are zero (CSA_HIST_ZERO: every
// call leaves them so); then the indexer; then the top-k, whose filter launch
// carries the compression when the histograms needed no clear and the
// selection takes the filter path.
extern "C++" {
template <class IndexLaunch>
static int run_index_call(int64_t rows, int N, const FusedCompress *fc, int flags, uint32_t *scratch,
                          hipStream_t st, IndexLaunch index, int B, int Tq, int m, int k, csa::QPos q_pos0,
                          const float *scores, int32_t *topk_idx) {
    const bool zero = (flags & CSA_HIST_ZERO) != 0;
    const bool fold = fc && zero && N > 0 && csa::topk_plan(rows, N).filter;
    if (N > 0) {
        if (!zero) {
            const int64_t cw = (int64_t)csa::topk_clear_words(rows, N);
            if (int s = hip_status(fc ? fc->launch(fc->job, st, scratch, cw) : csa::launch_fill_u32(scratch, cw, 0u, st),
                                   "histogram clear"))
                return s;
        } else if (fc && !fold) {
            if (int s = hip_status(fc->launch(fc->job, st, nullptr, 0), "compress launch")) return s;
        }
        if (int s = hip_status(index(), "indexer launch")) return s;
    } else if (fc) {
        if (int s = hip_status(fc->launch(fc->job, st, nullptr, 0), "compress launch")) return s;
    }
    if (fold)
        return hip_status(csa::launch_topk_folded(B, Tq, N, m, k, q_pos0, scores, scratch, topk_idx, st, fc->fold),
                          "top-k launch");
    return hip_status(csa::launch_topk(B, Tq, N, m, k, q_pos0, scores, scratch, topk_idx, st), "top-k launch");
}
}  // extern "C++"

int csa_compress_channels(int dt, int B, int G, int m, int d, const void *raw, int64_t raw_bstride,
                          const float *logits, int64_t logit_bstride, void *out, int64_t out_bstride, void *stream) {
    if (int s = check_dt(dt)) return s;
    if (B < 0 || G < 0) return fail(CSA_EINVAL, "B=%d and G=%d must be >= 0", B, G);
    if (m < 1 || m > 128) return fail(CSA_EUNSUPPORTED, "m=%d outside 1..128", m);
    if (!d_supported(d)) return fail(CSA_EUNSUPPORTED, "d=%d not in {32,64,128,256,512}", d);
    if ((int64_t)B * G == 0) return ok();
    if (!raw || !logits || !out) return fail(CSA_EINVAL, "NULL tensor pointer");
    if (raw_bstride < (int64_t)G * m * d || logit_bstride < (int64_t)G * m * d || out_bstride < (int64_t)G * d)
        return fail(CSA_EINVAL, "a batch stride is smaller than one batch's extent");
    if (!aligned(raw, 16) || !aligned(out, 16) || !aligned(logits, 16) || raw_bstride % 8 || out_bstride % 8 ||
        logit_bstride % 4)
        return fail(CSA_EALIGN, "raw/out/logits need 16-byte alignment, raw/out batch strides a multiple of 8 "
                                "elements and the logits' a multiple of 4");
    const size_t es = esize(dt);
    const Span so = span(out, B, out_bstride, (int64_t)G * d, es);
    if (overlap(so, span(raw, B, raw_bstride, (int64_t)G * m * d, es)) ||
        overlap(so, span(logits, B, logit_bstride, (int64_t)G * m * d, 4)))
        return fail(CSA_EINVAL, "out overlaps raw or logits");
    return hip_status(csa::launch_compress_channels(dt, B, G, m, d, raw, raw_bstride, logits, logit_bstride, out,
                                                    out_bstride, (hipStream_t)stream),
                      "compress launch");
}

// the checks of one append; on success *vw is the widest move the job allows
// paged: dst is a pool of dst_rows rows shared by the batch (dst_bstride unused)
static int check_append(int B, int n, int64_t row_bytes, const void *rows, int64_t rows_bstride, const void *dst,
                        int64_t dst_bstride, int64_t dst_rows, int64_t pos0, int64_t ring, int *vw,
                        bool paged = false) {
    if (B < 0 || n < 0) return fail(CSA_EINVAL, "B=%d and n=%d must be >= 0", B, n);
    if (B > 65535) return fail(CSA_EUNSUPPORTED, "B=%d above 65535", B);
    if (row_bytes < 1) return fail(CSA_EINVAL, "row_bytes=%lld must be >= 1", (long long)row_bytes);
    if (pos0 < 0 || ring < 0 || dst_rows < 0) return fail(CSA_EINVAL, "pos0, ring and dst_rows must be >= 0");
    if (ring == 0 && pos0 + n > dst_rows)
        return fail(CSA_EINVAL, "rows %lld..%lld outside the %lld destination rows", (long long)pos0,
                    (long long)(pos0 + n - 1), (long long)dst_rows);
    if (ring > 0 && (n > ring || 2 * ring > dst_rows))
        return fail(CSA_EINVAL, "a ring of %lld positions needs n <= ring and %lld slots (have %lld)",
                    (long long)ring, (long long)(2 * ring), (long long)dst_rows);
    if ((int64_t)B * n == 0) return ok();
    if (!rows || !dst) return fail(CSA_EINVAL, "NULL tensor pointer");
    if (rows_bstride < (int64_t)n * row_bytes || (!paged && dst_bstride < dst_rows * row_bytes))
        return fail(CSA_EINVAL, "a batch stride is smaller than one batch's extent");
    const Span ss = span(rows, B, rows_bstride, (int64_t)n * row_bytes, 1);
    const Span sd = paged ? span(dst, 1, 0, dst_rows * row_bytes, 1) : span(dst, B, dst_bstride, dst_rows * row_bytes, 1);
    if (overlap(ss, sd)) return fail(CSA_EINVAL, "rows overlap the destination");
    int w = 16;
    while (w > 1 &&
           (row_bytes % w || !aligned(rows, w) || !aligned(dst, w) || rows_bstride % w || (!paged && dst_bstride % w)))
        w /= 2;
    *vw = w;
    return ok();
}

int csa_append_rows_multi(int count, const csa_append_job *jobs, void *stream) {
    if (count < 0 || count > csa::kMaxAppendJobs)
        return fail(CSA_EUNSUPPORTED, "count=%d outside 0..%d", count, csa::kMaxAppendJobs);
    if (count > 0 && !jobs) return fail(CSA_EINVAL, "NULL job array");
    csa::AppendJobs aj{};
    int live = 0;
    for (int i = 0; i < count; ++i) {
        const csa_append_job &J = jobs[i];
        int vw = 1;
        if (J.every < 0) return fail(CSA_EINVAL, "job %d: every must be >= 0", i);
        csa::RowMap dmap;
        if (J.page_table) {
            if (J.ring != 0) return fail(CSA_EINVAL, "job %d: a paged destination cannot be a ring", i);
            if (int s = check_pages(J.page_table, J.B, J.max_pages, J.page_rows, J.n_pages, J.dst_rows, &dmap)) {
                std::string d = "job " + std::to_string(i) + ": " + g_detail;
                return fail(s, "%s", d.c_str());
            }
        }
        if (J.pos && !aligned(J.pos, 8)) return fail(CSA_EALIGN, "job %d: pos needs 8-byte alignment", i);
        // with positions from memory the destination rows are checked on the device (rows outside are
        // skipped); the host checks what it can: a zero base position
        // (paged destination: its pool is checked as one span of n_pages * page_rows rows)
        const int64_t d_rows = J.page_table ? J.n_pages * J.page_rows : J.dst_rows;
        if (int s = check_append(J.B, J.n, J.row_bytes, J.rows, J.rows_bstride, J.dst, J.dst_bstride, d_rows,
                                 (J.pos || J.every) ? 0 : J.pos0, J.ring, &vw, J.page_table != nullptr)) {
            std::string d = "job " + std::to_string(i) + ": " + g_detail;
            return fail(s, "%s", d.c_str());
        }
        if ((int64_t)J.B * J.n == 0) continue;
        // no job may write where another reads or writes
        const Span di = J.page_table ? span(J.dst, 1, 0, J.n_pages * J.page_rows * J.row_bytes, 1)
                                     : span(J.dst, J.B, J.dst_bstride, J.dst_rows * J.row_bytes, 1);
        for (int k = 0; k < count; ++k) {
            const csa_append_job &K = jobs[k];
            if (k == i || (int64_t)K.B * K.n == 0) continue;
            const Span dk = K.page_table ? span(K.dst, 1, 0, K.n_pages * K.page_rows * K.row_bytes, 1)
                                         : span(K.dst, K.B, K.dst_bstride, K.dst_rows * K.row_bytes, 1);
            if (overlap(di, span(K.rows, K.B, K.rows_bstride, (int64_t)K.n * K.row_bytes, 1)) ||
                (k < i && overlap(di, dk)))
                return fail(CSA_EINVAL, "job %d's destination overlaps job %d's rows or destination", i, k);
        }
        csa::AppendJob &A = aj.j[live++];
        A.src = (const unsigned char *)J.rows;
        A.dst = (unsigned char *)J.dst;
        A.n = J.n;
        A.row_bytes = J.row_bytes;
        A.src_bs = J.rows_bstride;
        A.dst_bs = J.dst_bstride;
        A.pos0 = J.pos0;
        A.ring = J.ring;
        A.pos = J.pos;
        A.every = J.every;
        A.dst_rows = J.dst_rows;
        A.dmap = dmap;
        A.vw = vw;
        A.B = J.B;
    }
    if (live == 0) return ok();
    return hip_status(csa::launch_append_multi(aj, live, (hipStream_t)stream), "append launch");
}

int csa_stream_read(const void *buf, int64_t bytes, int fronts, uint32_t *sink, void *stream) {
    if (fronts < 1 || fronts > 1024 || 1024 % fronts)
        return fail(CSA_EUNSUPPORTED, "fronts=%d is not a divisor of 1024", fronts);
    if (bytes < 0 || bytes % ((int64_t)1024 * fronts))
        return fail(CSA_EINVAL, "bytes must be a multiple of 1 KiB per front");
    if (bytes == 0) return ok();
    if (!buf || !sink) return fail(CSA_EINVAL, "NULL pointer");
    if (!aligned(buf, 16) || !aligned(sink, 4)) return fail(CSA_EALIGN, "buf needs 16-byte alignment");
    if (overlap(span(buf, 1, 0, bytes, 1), span(sink, 1, 0, 64, 4))) return fail(CSA_EINVAL, "sink overlaps buf");
    return hip_status(csa::launch_stream_read(buf, bytes, fronts, sink, (hipStream_t)stream), "stream read launch");
}

int csa_positions_advance(int B, int64_t *pos, int64_t delta, void *stream) {
    if (B < 0) return fail(CSA_EINVAL, "B=%d must be >= 0", B);
    if (B == 0) return ok();
    if (!pos) return fail(CSA_EINVAL, "NULL pos");
    if (!aligned(pos, 8)) return fail(CSA_EALIGN, "pos needs 8-byte alignment");
    return hip_status(csa::launch_positions_advance(B, pos, delta, (hipStream_t)stream), "advance launch");
}

// a ragged compression (csa_ragged_compress's arguments), checked on its own or ahead of an index call
struct RaggedCompressJob {
    int dt, B, m, d;
    const int64_t *pos;
    const void *raw_ring;
    int64_t ring_bs;
    const float *logit_ring;
    int64_t logit_bs, ring;
    void *out;
    int64_t out_bs, out_rows;
    const int32_t *page_table;
    int max_pages, page_rows;
    int64_t n_pages;
    // set by the check: the output's row map and what each operand spans
    csa::RowMap omap{0};
    Span so{}, sraw{}, slog{}, spos{};
};

// csa_ragged_compress's checks; *empty when nothing can be written
static int check_ragged_compress(RaggedCompressJob &c, bool *empty) {
    *empty = true;
    if (int s = check_dt(c.dt)) return s;
    if (c.B < 0 || c.out_rows < 0) return fail(CSA_EINVAL, "B and out_rows must be >= 0");
    if (c.m < 1 || c.m > 128) return fail(CSA_EUNSUPPORTED, "m=%d outside 1..128", c.m);
    if (!d_supported(c.d)) return fail(CSA_EUNSUPPORTED, "d=%d not in {32,64,128,256,512}", c.d);
    if (c.ring < c.m)
        return fail(CSA_EINVAL, "a ring of %lld positions cannot hold a group of %d", (long long)c.ring, c.m);
    if (c.B == 0 || c.out_rows == 0) return ok();
    if (!c.pos || !c.raw_ring || !c.logit_ring || !c.out) return fail(CSA_EINVAL, "NULL tensor pointer");
    c.omap = csa::RowMap(c.out_bs);
    int64_t o_span_b = c.B, o_span_stride = c.out_bs, o_span_inner = c.out_rows * c.d;
    if (c.page_table) {
        if (int s = check_pages(c.page_table, c.B, c.max_pages, c.page_rows, c.n_pages, c.out_rows, &c.omap))
            return s;
        o_span_b = 1, o_span_stride = 0, o_span_inner = c.n_pages * c.page_rows * c.d;
    } else if (c.out_bs < c.out_rows * c.d) {
        return fail(CSA_EINVAL, "out_bstride smaller than out_rows*d");
    }
    if (c.ring_bs < 2 * c.ring * c.d || c.logit_bs < 2 * c.ring)
        return fail(CSA_EINVAL, "a batch stride is smaller than one batch's extent (rings hold 2*ring rows)");
    if (!aligned(c.raw_ring, 16) || !aligned(c.out, 16) || !aligned(c.logit_ring, 4) || !aligned(c.pos, 8) ||
        c.ring_bs % 8 || c.out_bs % 8)
        return fail(CSA_EALIGN, "raw/out need 16-byte alignment and batch strides a multiple of 8 elements");
    const size_t es = esize(c.dt);
    c.so = span(c.out, o_span_b, o_span_stride, o_span_inner, es);
    c.sraw = span(c.raw_ring, c.B, c.ring_bs, 2 * c.ring * c.d, es);
    c.slog = span(c.logit_ring, c.B, c.logit_bs, 2 * c.ring, 4);
    c.spos = span(c.pos, 1, 0, c.B, 8);
    if (overlap(c.so, c.sraw) || overlap(c.so, c.slog) || overlap(c.so, c.spos))
        return fail(CSA_EINVAL, "out overlaps an input");
    *empty = false;
    return CSA_OK;
}

static hipError_t launch_ragged_compress_job(const RaggedCompressJob &c, hipStream_t st, uint32_t *clr = nullptr,
                                             int64_t clr_words = 0) {
    return csa::launch_compress_ragged(c.dt, c.B, c.m, c.d, c.pos, c.raw_ring, c.ring_bs, c.logit_ring, c.logit_bs,
                                       c.ring, c.out, c.omap, c.out_rows, st, clr, clr_words);
}

static FusedCompress fused(const RaggedCompressJob &c) {
    return FusedCompress{c.so, {c.sraw, c.slog, c.spos}, 3,
                         [](const void *j, hipStream_t st, uint32_t *clr, int64_t cw) {
                             return launch_ragged_compress_job(*(const RaggedCompressJob *)j, st, clr, cw);
                         },
                         &c,
                         csa::FoldedCompress{true, c.dt, c.B, 0, c.m, c.d, c.raw_ring, c.ring_bs, c.logit_ring,
                                             c.logit_bs, c.out, c.out_bs, c.pos, c.ring, c.omap, c.out_rows}};
}

int csa_ragged_compress(int dt, int B, int m, int d, const int64_t *pos, const void *raw_ring, int64_t ring_bstride,
                        const float *logit_ring, int64_t logit_bstride, int64_t ring, void *out, int64_t out_bstride,
                        int64_t out_rows, const int32_t *page_table, int max_pages, int page_rows, int64_t n_pages,
                        void *stream) {
    RaggedCompressJob c{dt, B, m, d, pos, raw_ring, ring_bstride, logit_ring, logit_bstride, ring, out, out_bstride,
                        out_rows, page_table, max_pages, page_rows, n_pages};
    bool empty;
    if (int s = check_ragged_compress(c, &empty)) return s;
    if (empty) return ok();
    return hip_status(launch_ragged_compress_job(c, (hipStream_t)stream), "compress launch");
}

int csa_append_rows(int B, int n, int64_t row_bytes, const void *rows, int64_t rows_bstride, void *dst,
                    int64_t dst_bstride, int64_t dst_rows, int64_t pos0, int64_t ring, void *stream) {
    int vw = 1;
    if (int s = check_append(B, n, row_bytes, rows, rows_bstride, dst, dst_bstride, dst_rows, pos0, ring, &vw))
        return s;
    if ((int64_t)B * n == 0) return ok();
    return hip_status(csa::launch_append_rows(B, n, row_bytes, vw, rows, rows_bstride, dst, dst_bstride, pos0, ring,
                                              (hipStream_t)stream),
                      "append launch");
}

// the score rows the top-k reads, padded to csa::topk_score_stride(N) floats
static size_t scores_bytes(int64_t rows, int64_t N) {
    return ((size_t)rows * csa::topk_score_stride(N) * sizeof(float) + 255) / 256 * 256;
}

size_t csa_index_topk_workspace_bytes(int B, int Tq, int N, int H_I, int k) {
    (void)H_I;
    (void)k;
    if (B <= 0 || Tq <= 0 || N < 0) return 0;
    const int64_t rows = (int64_t)B * Tq;
    return scores_bytes(rows, N) + (csa::topk_scratch_bytes(rows, N) + 255) / 256 * 256;
}

// positions: a uniform q_pos0 (>= 0), or per-sequence device positions with Tq = 1
static int check_qpos(csa::QPos qp, int B, int Tq) {
    if (qp.pos) {
        if (Tq != 1) return fail(CSA_EINVAL, "per-sequence positions need one query per sequence");
        if (!aligned(qp.pos, 8)) return fail(CSA_EALIGN, "pos needs 8-byte alignment");
    } else if (qp.q_pos0 < 0) {
        return fail(CSA_EINVAL, "q_pos0 must be >= 0");
    }
    (void)B;
    return CSA_OK;
}

static int index_topk_impl(int dt, int B, int Tq, int N, int H_I, int d_I, int m, int k, csa::QPos q_pos0,
                           const void *q_idx, const float *w_idx, const void *k_idx, int64_t k_bstride,
                           int32_t *topk_idx, float *scores_out, void *workspace, size_t workspace_bytes,
                           void *stream, const int32_t *page_table = nullptr, int max_pages = 0, int page_rows = 0,
                           int64_t n_pages = 0, const FusedCompress *fc = nullptr, int flags = 0) {
    if (int s = check_dt(dt)) return s;
    if (B < 0 || Tq < 0 || N < 0) return fail(CSA_EINVAL, "B, Tq and N must be >= 0");
    if (H_I < 1 || H_I > 64) return fail(CSA_EUNSUPPORTED, "H_I=%d outside 1..64", H_I);
    if (!dI_supported(d_I)) return fail(CSA_EUNSUPPORTED, "d_I=%d not in {32,64,128}", d_I);
    if (m < 1) return fail(CSA_EINVAL, "m=%d must be >= 1", m);
    if (k < 1 || k > 2048) return fail(CSA_EUNSUPPORTED, "k=%d outside 1..2048", k);
    if ((int64_t)B * Tq > 0)
        if (int s = check_qpos(q_pos0, B, Tq)) return s;
    if (N > csa::kTopkMaxEntries) return fail(CSA_EUNSUPPORTED, "N=%d above %lld entries", N, (long long)csa::kTopkMaxEntries);
    if ((int64_t)B * Tq == 0)
        return fc ? hip_status(fc->launch(fc->job, (hipStream_t)stream, nullptr, 0), "compress launch") : ok();
    if (!q_idx || !w_idx || !topk_idx || (N > 0 && !k_idx)) return fail(CSA_EINVAL, "NULL tensor pointer");
    csa::RowMap kmap(k_bstride);
    int64_t k_span_b = B, k_span_stride = k_bstride, k_span_inner = (int64_t)N * d_I;
    if (page_table) {
        if (dt != CSA_BF16 || d_I != 128)
            return fail(CSA_EUNSUPPORTED, "paged index keys need bf16 keys with d_I = 128");
        if (int s = check_pages(page_table, B, max_pages, page_rows, n_pages, N, &kmap)) return s;
        k_span_b = 1, k_span_stride = 0, k_span_inner = n_pages * page_rows * d_I;
    } else if (N > 0 && k_bstride < (int64_t)N * d_I) {
        return fail(CSA_EINVAL, "k_bstride smaller than N*d_I");
    }
    if (!aligned(q_idx, 16) || !aligned(k_idx, 16) || !aligned(w_idx, 4) || !aligned(topk_idx, 4) ||
        !aligned(scores_out, 4) || k_bstride % 8)
        return fail(CSA_EALIGN, "q_idx/k_idx need 16-byte alignment, k_bstride a multiple of 8 elements");
    const int64_t rows = (int64_t)B * Tq;
    const size_t need = csa_index_topk_workspace_bytes(B, Tq, N, H_I, k);
    if (!workspace || workspace_bytes < need)
        return fail(CSA_EWORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    if (!aligned(workspace, 16)) return fail(CSA_EALIGN, "workspace needs 16-byte alignment");
    float *scores = (float *)workspace;
    uint32_t *scratch = (uint32_t *)((char *)workspace + scores_bytes(rows, N));
    const size_t es = esize(dt);
    const Span si = span(topk_idx, B, (int64_t)Tq * k, (int64_t)Tq * k, 4);
    const Span ss = span(scores_out, B, (int64_t)Tq * N, (int64_t)Tq * N, 4);
    const Span inputs[3] = {span(q_idx, B, (int64_t)Tq * H_I * d_I, (int64_t)Tq * H_I * d_I, es),
                            span(w_idx, B, (int64_t)Tq * H_I, (int64_t)Tq * H_I, 4),
                            span(k_idx, k_span_b, k_span_stride, k_span_inner, es)};
    for (const Span &in : inputs)
        if (overlap(si, in) || overlap(ss, in)) return fail(CSA_EINVAL, "an output overlaps an input");
    if (overlap(si, ss)) return fail(CSA_EINVAL, "topk_idx overlaps scores_out");
    const Span sw = span(workspace, 1, 0, (int64_t)need, 1);
    for (const Span &in : inputs)
        if (overlap(sw, in)) return fail(CSA_EINVAL, "workspace overlaps an input");
    if (overlap(sw, si) || overlap(sw, ss)) return fail(CSA_EINVAL, "workspace overlaps an output");
    if (int s = check_compress_against(fc, inputs, 3, si, ss, sw)) return s;
    hipStream_t st = (hipStream_t)stream;
    // the first radix digit of the selection is counted by the indexer into
    // the histograms at the start of the top-k scratch
    return run_index_call(
        rows, N, fc, flags, scratch, st,
        [&] {
            return csa::launch_index_scores(dt, B, Tq, N, H_I, d_I, m, q_pos0, q_idx, w_idx, k_idx, kmap, scores,
                                            csa::topk_score_stride(N), scores_out, scratch, st);
        },
        B, Tq, m, k, q_pos0, scores, topk_idx);
}

int csa_index_topk(int dt, int B, int Tq, int N, int H_I, int d_I, int m, int k, int64_t q_pos0, const void *q_idx,
                   const float *w_idx, const void *k_idx, int64_t k_bstride, int32_t *topk_idx, float *scores_out,
                   void *workspace, size_t workspace_bytes, void *stream) {
    if (q_pos0 < 0) return fail(CSA_EINVAL, "q_pos0 must be >= 0");
    return index_topk_impl(dt, B, Tq, N, H_I, d_I, m, k, csa::QPos(q_pos0), q_idx, w_idx, k_idx, k_bstride, topk_idx,
                           scores_out, workspace, workspace_bytes, stream);
}

int csa_compress_index_topk(int dt, int B, int G, int m, int d, const void *raw, int64_t raw_bstride,
                            const float *logits, int64_t logit_bstride, void *entries_out, int64_t out_bstride,
                            int Tq, int N, int H_I, int d_I, int k, int64_t q_pos0, const void *q_idx,
                            const float *w_idx, const void *k_idx, int64_t k_bstride, int32_t *topk_idx,
                            float *scores_out, void *workspace, size_t workspace_bytes, int flags, void *stream) {
    const CompressJob c{dt, B, G, m, d, raw, raw_bstride, logits, logit_bstride, entries_out, out_bstride};
    bool empty;
    if (int s = check_compress(c, &empty)) return s;
    if (int s = check_flags(flags)) return s;
    if (q_pos0 < 0) return fail(CSA_EINVAL, "q_pos0 must be >= 0");
    const FusedCompress fc = fused(c);
    return index_topk_impl(dt, B, Tq, N, H_I, d_I, m, k, csa::QPos(q_pos0), q_idx, w_idx, k_idx, k_bstride, topk_idx,
                           scores_out, workspace, workspace_bytes, stream, nullptr, 0, 0, 0, empty ? nullptr : &fc,
                           flags);
}

int csa_index_topk_noalloc(int dt, int B, int Tq, int N, int H_I, int d_I, int m, int k, int64_t q_pos0,
                           const void *q_idx, const float *w_idx, const void *k_idx, int64_t k_bstride,
                           int32_t *topk_idx, float *scores_out, void *stream) {
    if (q_pos0 < 0) return fail(CSA_EINVAL, "q_pos0 must be >= 0");
    const size_t need = csa_index_topk_workspace_bytes(B, Tq, N, H_I, k);
    if (need > (size_t)CSA_NOALLOC_SCRATCH_BYTES)
        return fail(CSA_EWORKSPACE, "B=%d, Tq=%d, N=%d needs %zu bytes of scratch, the static scratch holds %zu", B,
                    Tq, N, need, (size_t)CSA_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    if ((int64_t)B * Tq > 0)
        if (int s = scratch_on_current_device(&ws)) return s;
    return index_topk_impl(dt, B, Tq, N, H_I, d_I, m, k, csa::QPos(q_pos0), q_idx, w_idx, k_idx, k_bstride, topk_idx,
                           scores_out, ws, CSA_NOALLOC_SCRATCH_BYTES, stream);
}

int csa_ragged_index_topk(int dt, int B, int N, int H_I, int d_I, int m, int k, const int64_t *pos,
                          const void *q_idx, const float *w_idx, const void *k_idx, int64_t k_bstride,
                          const int32_t *page_table, int max_pages, int page_rows, int64_t n_pages,
                          int32_t *topk_idx, float *scores_out, void *workspace, size_t workspace_bytes,
                          void *stream) {
    if (B > 0 && !pos) return fail(CSA_EINVAL, "NULL pos");
    return index_topk_impl(dt, B, 1, N, H_I, d_I, m, k, csa::QPos(0, pos), q_idx, w_idx, k_idx, k_bstride, topk_idx,
                           scores_out, workspace, workspace_bytes, stream, page_table, max_pages, page_rows,
                           n_pages);
}

int csa_ragged_compress_index_topk(int dt, int B, int m, int d, const int64_t *pos, const void *raw_ring,
                                   int64_t ring_bstride, const float *logit_ring, int64_t logit_bstride,
                                   int64_t ring, void *entries_out, int64_t out_bstride, int64_t out_rows,
                                   const int32_t *e_page_table, int e_max_pages, int e_page_rows,
                                   int64_t e_n_pages, int N, int H_I, int d_I, int k, const void *q_idx,
                                   const float *w_idx, const void *k_idx, int64_t k_bstride,
                                   const int32_t *page_table, int max_pages, int page_rows, int64_t n_pages,
                                   int32_t *topk_idx, float *scores_out, void *workspace, size_t workspace_bytes,
                                   int flags, void *stream) {
    RaggedCompressJob c{dt, B, m, d, pos, raw_ring, ring_bstride, logit_ring, logit_bstride, ring, entries_out,
                        out_bstride, out_rows, e_page_table, e_max_pages, e_page_rows, e_n_pages};
    bool empty;
    if (int s = check_ragged_compress(c, &empty)) return s;
    if (int s = check_flags(flags)) return s;
    if (B > 0 && !pos) return fail(CSA_EINVAL, "NULL pos");
    const FusedCompress fc = fused(c);
    return index_topk_impl(dt, B, 1, N, H_I, d_I, m, k, csa::QPos(0, pos), q_idx, w_idx, k_idx, k_bstride, topk_idx,
                           scores_out, workspace, workspace_bytes, stream, page_table, max_pages, page_rows,
                           n_pages, empty ? nullptr : &fc, flags);
}

int csa_index_scores(int dt, int B, int Tq, int N, int H_I, int d_I, int m, int64_t q_pos0, const void *q_idx,
                     const float *w_idx, const void *k_idx, int64_t k_bstride, float *scores, void *stream) {
    if (int s = check_dt(dt)) return s;
    if (B < 0 || Tq < 0 || N < 0) return fail(CSA_EINVAL, "B, Tq and N must be >= 0");
    if (H_I < 1 || H_I > 64) return fail(CSA_EUNSUPPORTED, "H_I=%d outside 1..64", H_I);
    if (!dI_supported(d_I)) return fail(CSA_EUNSUPPORTED, "d_I=%d not in {32,64,128}", d_I);
    if (m < 1) return fail(CSA_EINVAL, "m=%d must be >= 1", m);
    if (q_pos0 < 0) return fail(CSA_EINVAL, "q_pos0 must be >= 0");
    if ((int64_t)B * Tq * N == 0) return ok();
    if (!q_idx || !w_idx || !k_idx || !scores) return fail(CSA_EINVAL, "NULL tensor pointer");
    if (k_bstride < (int64_t)N * d_I) return fail(CSA_EINVAL, "k_bstride smaller than N*d_I");
    if (!aligned(q_idx, 16) || !aligned(k_idx, 16) || !aligned(w_idx, 4) || !aligned(scores, 4) || k_bstride % 8)
        return fail(CSA_EALIGN, "q_idx/k_idx need 16-byte alignment, k_bstride a multiple of 8 elements");
    const size_t es = esize(dt);
    const Span ss = span(scores, B, (int64_t)Tq * N, (int64_t)Tq * N, 4);
    if (overlap(ss, span(q_idx, B, (int64_t)Tq * H_I * d_I, (int64_t)Tq * H_I * d_I, es)) ||
        overlap(ss, span(w_idx, B, (int64_t)Tq * H_I, (int64_t)Tq * H_I, 4)) ||
        overlap(ss, span(k_idx, B, k_bstride, (int64_t)N * d_I, es)))
        return fail(CSA_EINVAL, "scores overlaps an input");
    return hip_status(csa::launch_index_scores(dt, B, Tq, N, H_I, d_I, m, q_pos0, q_idx, w_idx, k_idx, k_bstride,
                                               scores, N, nullptr, nullptr, (hipStream_t)stream),
                      "indexer launch");
}

int csa_mx4_quantize(int dt, int64_t n_rows, int d, const void *x, uint8_t *codes, uint8_t *scales, void *stream) {
    if (int s = check_dt(dt)) return s;
    if (n_rows < 0 || d < 0) return fail(CSA_EINVAL, "n_rows and d must be >= 0");
    if (d % 32) return fail(CSA_EUNSUPPORTED, "d=%d is not a multiple of 32", d);
    if (n_rows * d == 0) return ok();
    if (!x || !codes || !scales) return fail(CSA_EINVAL, "NULL tensor pointer");
    if (!aligned(x, 16) || !aligned(codes, 16)) return fail(CSA_EALIGN, "x and codes need 16-byte alignment");
    const Span sx = span(x, 1, 0, n_rows * d, esize(dt));
    const Span sc = span(codes, 1, 0, n_rows * d / 2, 1), ss = span(scales, 1, 0, n_rows * d / 32, 1);
    if (overlap(sx, sc) || overlap(sx, ss) || overlap(sc, ss)) return fail(CSA_EINVAL, "x, codes and scales overlap");
    return hip_status(csa::launch_mx4_quantize(dt, n_rows * d / 32, x, codes, scales, (hipStream_t)stream),
                      "quantise launch");
}

static int index_topk_mx4_impl(int dt, int B, int Tq, int N, int H_I, int d_I, int m, int k, csa::QPos q_pos0,
                               const void *q_idx, const float *w_idx, const uint8_t *k_codes,
                               const uint8_t *k_scales, int64_t k_bstride, int32_t *topk_idx, float *scores_out,
                               void *workspace, size_t workspace_bytes, void *stream,
                               const int32_t *page_table = nullptr, int max_pages = 0, int page_rows = 0,
                               int64_t n_pages = 0, const FusedCompress *fc = nullptr, int flags = 0) {
    if (int s = check_dt(dt)) return s;
    if (B < 0 || Tq < 0 || N < 0) return fail(CSA_EINVAL, "B, Tq and N must be >= 0");
    if (H_I < 1 || H_I > 64) return fail(CSA_EUNSUPPORTED, "H_I=%d outside 1..64", H_I);
    if (!dI_supported(d_I)) return fail(CSA_EUNSUPPORTED, "d_I=%d not in {32,64,128}", d_I);
    if (m < 1) return fail(CSA_EINVAL, "m=%d must be >= 1", m);
    if (k < 1 || k > 2048) return fail(CSA_EUNSUPPORTED, "k=%d outside 1..2048", k);
    if ((int64_t)B * Tq > 0)
        if (int s = check_qpos(q_pos0, B, Tq)) return s;
    if (N > csa::kTopkMaxEntries) return fail(CSA_EUNSUPPORTED, "N=%d above %lld entries", N, (long long)csa::kTopkMaxEntries);
    if ((int64_t)B * Tq == 0)
        return fc ? hip_status(fc->launch(fc->job, (hipStream_t)stream, nullptr, 0), "compress launch") : ok();
    if (!q_idx || !w_idx || !topk_idx || (N > 0 && (!k_codes || !k_scales)))
        return fail(CSA_EINVAL, "NULL tensor pointer");
    csa::RowMap kmap(k_bstride);
    int64_t k_span_b = B, k_span_rows = k_bstride, k_inner_rows = N;
    if (page_table) {
        if (d_I != 128 || !aligned(k_scales, 4))
            return fail(CSA_EUNSUPPORTED, "paged FP4 keys need d_I = 128 and 4-byte aligned scales");
        if (int s = check_pages(page_table, B, max_pages, page_rows, n_pages, N, &kmap)) return s;
        k_span_b = 1, k_span_rows = 0, k_inner_rows = n_pages * page_rows;
    } else if (N > 0 && k_bstride < N) {
        return fail(CSA_EINVAL, "k_bstride smaller than N rows");
    }
    if (!aligned(q_idx, 16) || !aligned(k_codes, 16) || !aligned(w_idx, 4) || !aligned(topk_idx, 4) ||
        !aligned(scores_out, 4))
        return fail(CSA_EALIGN, "q_idx/k_codes need 16-byte alignment");
    const int64_t rows = (int64_t)B * Tq;
    const size_t need = csa_index_topk_workspace_bytes(B, Tq, N, H_I, k);
    if (!workspace || workspace_bytes < need)
        return fail(CSA_EWORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    if (!aligned(workspace, 16)) return fail(CSA_EALIGN, "workspace needs 16-byte alignment");
    const int64_t rb = d_I / 2, kb = d_I / 32;
    const Span si = span(topk_idx, B, (int64_t)Tq * k, (int64_t)Tq * k, 4);
    const Span ss = span(scores_out, B, (int64_t)Tq * N, (int64_t)Tq * N, 4);
    const Span inputs[4] = {span(q_idx, 1, 0, rows * H_I * d_I, esize(dt)), span(w_idx, 1, 0, rows * H_I, 4),
                            span(k_codes, k_span_b, k_span_rows * rb, k_inner_rows * rb, 1),
                            span(k_scales, k_span_b, k_span_rows * kb, k_inner_rows * kb, 1)};
    const Span sw = span(workspace, 1, 0, (int64_t)need, 1);
    for (const Span &in : inputs)
        if (overlap(si, in) || overlap(ss, in) || overlap(sw, in))
            return fail(CSA_EINVAL, "an output or the workspace overlaps an input");
    if (overlap(si, ss) || overlap(sw, si) || overlap(sw, ss))
        return fail(CSA_EINVAL, "outputs and workspace overlap");
    if (int s = check_compress_against(fc, inputs, 4, si, ss, sw)) return s;
    float *scores = (float *)workspace;
    uint32_t *scratch = (uint32_t *)((char *)workspace + scores_bytes(rows, N));
    hipStream_t st = (hipStream_t)stream;
    return run_index_call(
        rows, N, fc, flags, scratch, st,
        [&] {
            return csa::launch_index_mx4(dt, B, Tq, N, H_I, d_I, m, q_pos0, q_idx, w_idx, k_codes, k_scales, kmap,
                                         scores, csa::topk_score_stride(N), scores_out, scratch, st);
        },
        B, Tq, m, k, q_pos0, scores, topk_idx);
}

int csa_index_topk_mx4(int dt, int B, int Tq, int N, int H_I, int d_I, int m, int k, int64_t q_pos0,
                       const void *q_idx, const float *w_idx, const uint8_t *k_codes, const uint8_t *k_scales,
                       int64_t k_bstride, int32_t *topk_idx, float *scores_out, void *workspace,
                       size_t workspace_bytes, void *stream) {
    if (q_pos0 < 0) return fail(CSA_EINVAL, "q_pos0 must be >= 0");
    return index_topk_mx4_impl(dt, B, Tq, N, H_I, d_I, m, k, csa::QPos(q_pos0), q_idx, w_idx, k_codes, k_scales,
                               k_bstride, topk_idx, scores_out, workspace, workspace_bytes, stream);
}

int csa_compress_index_topk_mx4(int dt, int B, int G, int m, int d, const void *raw, int64_t raw_bstride,
                                const float *logits, int64_t logit_bstride, void *entries_out, int64_t out_bstride,
                                int Tq, int N, int H_I, int d_I, int k, int64_t q_pos0, const void *q_idx,
                                const float *w_idx, const uint8_t *k_codes, const uint8_t *k_scales,
                                int64_t k_bstride, int32_t *topk_idx, float *scores_out, void *workspace,
                                size_t workspace_bytes, int flags, void *stream) {
    const CompressJob c{dt, B, G, m, d, raw, raw_bstride, logits, logit_bstride, entries_out, out_bstride};
    bool empty;
    if (int s = check_compress(c, &empty)) return s;
    if (int s = check_flags(flags)) return s;
    if (q_pos0 < 0) return fail(CSA_EINVAL, "q_pos0 must be >= 0");
    const FusedCompress fc = fused(c);
    return index_topk_mx4_impl(dt, B, Tq, N, H_I, d_I, m, k, csa::QPos(q_pos0), q_idx, w_idx, k_codes, k_scales,
                               k_bstride, topk_idx, scores_out, workspace, workspace_bytes, stream, nullptr, 0, 0,
                               0, empty ? nullptr : &fc, flags);
}

int csa_index_scores_mx4(int dt, int B, int Tq, int N, int H_I, int d_I, int m, int64_t q_pos0, const void *q_idx,
                         const float *w_idx, const uint8_t *k_codes, const uint8_t *k_scales, int64_t k_bstride,
                         float *scores, void *stream) {
    if (int s = check_dt(dt)) return s;
    if (B < 0 || Tq < 0 || N < 0) return fail(CSA_EINVAL, "B, Tq and N must be >= 0");
    if (H_I < 1 || H_I > 64) return fail(CSA_EUNSUPPORTED, "H_I=%d outside 1..64", H_I);
    if (!dI_supported(d_I)) return fail(CSA_EUNSUPPORTED, "d_I=%d not in {32,64,128}", d_I);
    if (m < 1) return fail(CSA_EINVAL, "m=%d must be >= 1", m);
    if (q_pos0 < 0) return fail(CSA_EINVAL, "q_pos0 must be >= 0");
    if ((int64_t)B * Tq * N == 0) return ok();
    if (!q_idx || !w_idx || !k_codes || !k_scales || !scores) return fail(CSA_EINVAL, "NULL tensor pointer");
    if (k_bstride < N) return fail(CSA_EINVAL, "k_bstride smaller than N rows");
    if (!aligned(q_idx, 16) || !aligned(k_codes, 16) || !aligned(w_idx, 4) || !aligned(scores, 4))
        return fail(CSA_EALIGN, "q_idx/k_codes need 16-byte alignment");
    const int64_t rows = (int64_t)B * Tq, rb = d_I / 2, kb = d_I / 32;
    const Span ss = span(scores, B, (int64_t)Tq * N, (int64_t)Tq * N, 4);
    if (overlap(ss, span(q_idx, 1, 0, rows * H_I * d_I, esize(dt))) || overlap(ss, span(w_idx, 1, 0, rows * H_I, 4)) ||
        overlap(ss, span(k_codes, B, k_bstride * rb, (int64_t)N * rb, 1)) ||
        overlap(ss, span(k_scales, B, k_bstride * kb, (int64_t)N * kb, 1)))
        return fail(CSA_EINVAL, "scores overlaps an input");
    return hip_status(csa::launch_index_mx4(dt, B, Tq, N, H_I, d_I, m, csa::QPos(q_pos0), q_idx, w_idx, k_codes,
                                            k_scales, csa::RowMap(k_bstride), scores, N, nullptr, nullptr,
                                            (hipStream_t)stream),
                      "indexer launch");
}

int csa_ragged_index_topk_mx4(int dt, int B, int N, int H_I, int d_I, int m, int k, const int64_t *pos,
                              const void *q_idx, const float *w_idx, const uint8_t *k_codes,
                              const uint8_t *k_scales, int64_t k_bstride, const int32_t *page_table, int max_pages,
                              int page_rows, int64_t n_pages, int32_t *topk_idx, float *scores_out,
                              void *workspace, size_t workspace_bytes, void *stream) {
    if (B > 0 && !pos) return fail(CSA_EINVAL, "NULL pos");
    return index_topk_mx4_impl(dt, B, 1, N, H_I, d_I, m, k, csa::QPos(0, pos), q_idx, w_idx, k_codes, k_scales,
                               k_bstride, topk_idx, scores_out, workspace, workspace_bytes, stream, page_table,
                               max_pages, page_rows, n_pages);
}

int csa_ragged_compress_index_topk_mx4(int dt, int B, int m, int d, const int64_t *pos, const void *raw_ring,
                                       int64_t ring_bstride, const float *logit_ring, int64_t logit_bstride,
                                       int64_t ring, void *entries_out, int64_t out_bstride, int64_t out_rows,
                                       const int32_t *e_page_table, int e_max_pages, int e_page_rows,
                                       int64_t e_n_pages, int N, int H_I, int d_I, int k, const void *q_idx,
                                       const float *w_idx, const uint8_t *k_codes, const uint8_t *k_scales,
                                       int64_t k_bstride, const int32_t *page_table, int max_pages, int page_rows,
                                       int64_t n_pages, int32_t *topk_idx, float *scores_out, void *workspace,
                                       size_t workspace_bytes, int flags, void *stream) {
    RaggedCompressJob c{dt, B, m, d, pos, raw_ring, ring_bstride, logit_ring, logit_bstride, ring, entries_out,
                        out_bstride, out_rows, e_page_table, e_max_pages, e_page_rows, e_n_pages};
    bool empty;
    if (int s = check_ragged_compress(c, &empty)) return s;
    if (int s = check_flags(flags)) return s;
    if (B > 0 && !pos) return fail(CSA_EINVAL, "NULL pos");
    const FusedCompress fc = fused(c);
    return index_topk_mx4_impl(dt, B, 1, N, H_I, d_I, m, k, csa::QPos(0, pos), q_idx, w_idx, k_codes, k_scales,
                               k_bstride, topk_idx, scores_out, workspace, workspace_bytes, stream, page_table,
                               max_pages, page_rows, n_pages, empty ? nullptr : &fc, flags);
}

size_t csa_mqa_workspace_bytes(int B, int Tq, int H, int d, int n_rows_max) {
    if (B <= 0 || Tq <= 0 || H <= 0 || d <= 0) return 0;
    int tps = 0;
    const int64_t rows = (int64_t)B * Tq;
    const int s = csa::mqa_choose_splits(rows, n_rows_max, d, &tps);
    if (s <= 1) return 0;
    const size_t bytes = (size_t)rows * s * H * (d + 2) * sizeof(float);
    return (bytes + 255) / 256 * 256;
}

// raw_ring > 0 (with per-sequence positions): the raw rows are a ring, position p at row p mod raw_ring
static int mqa_common(int dt, int B, int Tq, int H, int d, int N, int m, int k, int W, csa::QPos q_pos0, float scale,
                      const void *q, const void *entries, int64_t e_bstride, const int32_t *idx, const void *raw,
                      int64_t raw_bstride, int64_t raw_pos0, int64_t raw_len, int64_t raw_ring, float *out,
                      float *lse, void *workspace, size_t workspace_bytes, void *stream,
                      const int32_t *page_table = nullptr, int max_pages = 0, int page_rows = 0,
                      int64_t n_pages = 0) {
    if (int s = check_dt(dt)) return s;
    if (B < 0 || Tq < 0 || N < 0 || W < 0 || raw_len < 0) return fail(CSA_EINVAL, "B, Tq, N, W, raw_len must be >= 0");
    if (H < 1 || H > 64) return fail(CSA_EUNSUPPORTED, "H=%d outside 1..64", H);
    if (!d_supported(d)) return fail(CSA_EUNSUPPORTED, "d=%d not in {32,64,128,256,512}", d);
    if (m < 1) return fail(CSA_EINVAL, "m=%d must be >= 1", m);
    if (k < 0 || k > 2048) return fail(CSA_EUNSUPPORTED, "k=%d outside 1..2048", k);
    if (!(scale > 0.f) || !std::isfinite(scale)) return fail(CSA_EINVAL, "scale must be finite and > 0");
    if (raw_pos0 < 0 || raw_ring < 0) return fail(CSA_EINVAL, "positions must be >= 0");
    if ((int64_t)B * Tq == 0) return ok();
    if (int s = check_qpos(q_pos0, B, Tq)) return s;
    if (W > 0 && raw_ring > 0) {
        // per-sequence positions: the window is whatever the ring holds (any position maps inside it)
        if (raw_ring < W) return fail(CSA_EINVAL, "a ring of %lld positions cannot hold a window of %d",
                                      (long long)raw_ring, W);
        if (!raw) return fail(CSA_EINVAL, "NULL raw with W > 0");
        if (raw_bstride < raw_len * d) return fail(CSA_EINVAL, "raw_bstride smaller than the ring's rows");
    } else if (W > 0) {
        const int64_t qp = q_pos0.q_pos0;
        const int64_t win0 = qp - W + 1 > 0 ? qp - W + 1 : 0;
        if (raw_pos0 > win0 || raw_pos0 + raw_len < qp + Tq)
            return fail(CSA_EINVAL, "raw rows [%lld, %lld) do not cover the window [%lld, %lld)", (long long)raw_pos0,
                        (long long)(raw_pos0 + raw_len), (long long)win0, (long long)(qp + Tq));
        if (!raw) return fail(CSA_EINVAL, "NULL raw with W > 0");
        if (raw_bstride < (int64_t)raw_len * d) return fail(CSA_EINVAL, "raw_bstride smaller than raw_len*d");
    }
    if (!q || !out || (N > 0 && !entries) || (k > 0 && !idx)) return fail(CSA_EINVAL, "NULL tensor pointer");
    csa::RowMap emap(e_bstride);
    int64_t e_span_b = B, e_span_stride = e_bstride, e_span_inner = (int64_t)N * d;
    if (page_table) {
        if (int s = check_pages(page_table, B, max_pages, page_rows, n_pages, N, &emap)) return s;
        e_span_b = 1, e_span_stride = 0, e_span_inner = n_pages * page_rows * d;
    } else if (N > 0 && e_bstride < (int64_t)N * d) {
        return fail(CSA_EINVAL, "e_bstride smaller than N*d");
    }
    if (!aligned(q, 16) || !aligned(entries, 16) || !aligned(raw, 16) || !aligned(out, 16) || !aligned(idx, 4) ||
        !aligned(lse, 4) || e_bstride % 8 || raw_bstride % 8)
        return fail(CSA_EALIGN, "q/entries/raw/out need 16-byte alignment, strides a multiple of 8 elements");
    const size_t es = esize(dt);
    const Span so = span(out, B, (int64_t)Tq * H * d, (int64_t)Tq * H * d, 4);
    const Span sl = span(lse, B, (int64_t)Tq * H, (int64_t)Tq * H, 4);
    const Span inputs[4] = {span(q, B, (int64_t)Tq * H * d, (int64_t)Tq * H * d, es),
                            span(entries, e_span_b, e_span_stride, e_span_inner, es),
                            span(raw, B, raw_bstride, (int64_t)raw_len * d, es),
                            span(idx, B, (int64_t)Tq * k, (int64_t)Tq * k, 4)};
    for (const Span &in : inputs)
        if (overlap(so, in) || overlap(sl, in)) return fail(CSA_EINVAL, "an output overlaps an input");
    if (overlap(so, sl)) return fail(CSA_EINVAL, "out overlaps lse");
    const int64_t rows = (int64_t)B * Tq;
    const int64_t n_rows_max = (int64_t)(k > 0 ? k : N) + W;
    int tps = 0;
    const int splits = csa::mqa_choose_splits(rows, n_rows_max, d, &tps);
    float *ws = nullptr;
    if (splits > 1) {
        const size_t need = csa_mqa_workspace_bytes(B, Tq, H, d, (int)n_rows_max);
        if (!workspace || workspace_bytes < need)
            return fail(CSA_EWORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
        if (!aligned(workspace, 16)) return fail(CSA_EALIGN, "workspace needs 16-byte alignment");
        ws = (float *)workspace;
    }
    return hip_status(csa::launch_mqa(dt, B, Tq, H, d, N, m, k, W, q_pos0, scale, q, entries, emap, idx, raw,
                                      raw_bstride, raw_pos0, raw_ring, out, lse, ws, splits, tps,
                                      (hipStream_t)stream),
                      "attention launch");
}

int csa_sparse_mqa(int dt, int B, int Tq, int H, int d, int N, int m, int k, int W, int64_t q_pos0, float scale,
                   const void *q, const void *entries, int64_t e_bstride, const int32_t *topk_idx, const void *raw,
                   int64_t raw_bstride, int64_t raw_pos0, int raw_len, float *out, float *lse, void *workspace,
                   size_t workspace_bytes, void *stream) {
    if (k < 1 || k > 2048) return fail(CSA_EUNSUPPORTED, "k=%d outside 1..2048", k);
    if (q_pos0 < 0) return fail(CSA_EINVAL, "positions must be >= 0");
    return mqa_common(dt, B, Tq, H, d, N, m, k, W, csa::QPos(q_pos0), scale, q, entries, e_bstride, topk_idx, raw,
                      raw_bstride, raw_pos0, raw_len, 0, out, lse, workspace, workspace_bytes, stream);
}

int csa_ragged_sparse_mqa(int dt, int B, int H, int d, int N, int m, int k, int W, const int64_t *pos, float scale,
                          const void *q, const void *entries, int64_t e_bstride, const int32_t *page_table,
                          int max_pages, int page_rows, int64_t n_pages, const int32_t *topk_idx,
                          const void *raw_ring, int64_t ring_bstride, int64_t ring, float *out, float *lse,
                          void *workspace, size_t workspace_bytes, void *stream) {
    if (k < 1 || k > 2048) return fail(CSA_EUNSUPPORTED, "k=%d outside 1..2048", k);
    if (B > 0 && !pos) return fail(CSA_EINVAL, "NULL pos");
    if (ring < 1) return fail(CSA_EINVAL, "ring must be >= 1");
    return mqa_common(dt, B, 1, H, d, N, m, k, W, csa::QPos(0, pos), scale, q, entries, e_bstride, topk_idx,
                      raw_ring, ring_bstride, 0, ring, ring, out, lse, workspace, workspace_bytes, stream, page_table,
                      max_pages, page_rows, n_pages);
}

int hca_ragged_dense_mqa(int dt, int B, int H, int d, int N, int m, int W, const int64_t *pos, float scale,
                         const void *q, const void *entries, int64_t e_bstride, const int32_t *page_table,
                         int max_pages, int page_rows, int64_t n_pages, const void *raw_ring,
                         int64_t ring_bstride, int64_t ring, float *out, float *lse, void *workspace,
                         size_t workspace_bytes, void *stream) {
    if (B > 0 && !pos) return fail(CSA_EINVAL, "NULL pos");
    if (ring < 1) return fail(CSA_EINVAL, "ring must be >= 1");
    return mqa_common(dt, B, 1, H, d, N, m, 0, W, csa::QPos(0, pos), scale, q, entries, e_bstride, nullptr, raw_ring,
                      ring_bstride, 0, ring, ring, out, lse, workspace, workspace_bytes, stream, page_table,
                      max_pages, page_rows, n_pages);
}

int hca_dense_mqa(int dt, int B, int Tq, int H, int d, int N, int m, int W, int64_t q_pos0, float scale, const void *q,
                  const void *entries, int64_t e_bstride, const void *raw, int64_t raw_bstride, int64_t raw_pos0,
                  int raw_len, float *out, float *lse, void *workspace, size_t workspace_bytes, void *stream) {
    if (q_pos0 < 0) return fail(CSA_EINVAL, "positions must be >= 0");
    return mqa_common(dt, B, Tq, H, d, N, m, 0, W, csa::QPos(q_pos0), scale, q, entries, e_bstride, nullptr, raw,
                      raw_bstride, raw_pos0, raw_len, 0, out, lse, workspace, workspace_bytes, stream);
}

}  // extern "C"
