// Host side of the C ABI declared in include/stem_bsa.h: argument checks,
// workspace carving and kernel launches.  Nothing here allocates device
// memory or synchronises.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <vector>

#include "stem_internal.h"

using namespace stem;

namespace {
thread_local char g_err[256] = "";
}  // namespace

namespace stem {

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return STEM_OK;
}

}  // namespace stem

namespace {

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool finite_pos(float x) { return std::isfinite(x) && x > 0.0f; }

}  // namespace

namespace stem {

int check_desc(const stem_attn_desc *d, Shape *s) {
    if (!d) return fail(STEM_EINVAL, "desc is NULL");
    if (d->batch < 1 || d->seq_len < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1)
        return fail(STEM_EINVAL, "batch, seq_len and head counts must be positive");
    if (d->num_q_heads % d->num_kv_heads)
        return fail(STEM_EINVAL, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)",
                    d->num_q_heads, d->num_kv_heads);
    if (d->block_size != 64 && d->block_size != 128)
        return fail(STEM_EUNSUPPORTED, "block_size %d not built (64 or 128)", d->block_size);
    if (d->head_dim != 64 && d->head_dim != 128)
        return fail(STEM_EUNSUPPORTED, "head_dim %d not built (64 or 128)", d->head_dim);
    if (d->seq_len % d->block_size)
        return fail(STEM_EINVAL, "seq_len %d is not a multiple of block_size %d", d->seq_len,
                    d->block_size);
    const int nb = d->seq_len / d->block_size;
    if (nb > 4096) return fail(STEM_EUNSUPPORTED, "more than 4096 blocks per sequence (%d)", nb);
    if (d->dtype != STEM_F32 && d->dtype != STEM_BF16 && d->dtype != STEM_FP8_E4M3)
        return fail(STEM_EINVAL, "unknown dtype %d", d->dtype);
    if (!finite_pos(d->q_scale) || !finite_pos(d->k_scale) || !finite_pos(d->v_scale))
        return fail(STEM_EINVAL, "scales must be finite and positive");
    if (d->dtype != STEM_FP8_E4M3 && (d->q_scale != 1.0f || d->k_scale != 1.0f || d->v_scale != 1.0f))
        return fail(STEM_EINVAL, "q/k/v scales must be 1 unless dtype is STEM_FP8_E4M3");
    if (!std::isfinite(d->softmax_scale) || d->softmax_scale < 0.0f)
        return fail(STEM_EINVAL, "softmax_scale must be finite and >= 0");
    const long long elems = (long long)d->batch * d->seq_len * d->num_q_heads * d->head_dim;
    if (elems >= (1LL << 40)) return fail(STEM_EUNSUPPORTED, "tensor too large");
    s->batch = d->batch;
    s->seq = d->seq_len;
    s->hq = d->num_q_heads;
    s->hkv = d->num_kv_heads;
    s->d = d->head_dim;
    s->blk = d->block_size;
    s->nb = nb;
    s->words = (nb + 31) / 32;
    s->dtype = d->dtype;
    s->q_scale = d->q_scale;
    s->k_scale = d->k_scale;
    s->v_scale = d->v_scale;
    s->tau = d->softmax_scale > 0.0f ? d->softmax_scale : 1.0f / std::sqrt((float)d->head_dim);
    return STEM_OK;
}

int check_kv(const stem_kv_desc *kv, const Shape &s, KvView *out) {
    if (!kv) return fail(STEM_EINVAL, "kv is NULL");
    if (!kv->k || !kv->v) return fail(STEM_EINVAL, "k or v is NULL");
    out->k = kv->k;
    out->v = kv->v;
    out->table = kv->block_table;
    out->page_log2 = 0;
    out->pages_per_seq = 0;
    out->rows = (size_t)s.batch * s.seq;
    if (kv->block_table) {
        const int p = kv->page_size;
        if (p < 1 || (p & (p - 1))) return fail(STEM_EINVAL, "page_size %d is not a power of two", p);
        if ((long long)kv->pages_per_seq * p < s.seq)
            return fail(STEM_EINVAL, "pages_per_seq * page_size < seq_len");
        if (kv->num_pages < 1) return fail(STEM_EINVAL, "num_pages must be positive");
        int lg = 0;
        while ((1 << lg) < p) ++lg;
        out->page_log2 = lg;
        out->pages_per_seq = kv->pages_per_seq;
        out->rows = (size_t)kv->num_pages * p;
    }
    return STEM_OK;
}

int hip_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(STEM_EHIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// Reports an error left by earlier asynchronous work before enqueuing more.
int hip_precheck() {
    hipError_t e = hipPeekAtLastError();
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(STEM_EHIP, "earlier HIP error: %s", hipGetErrorString(e));
    }
    return STEM_OK;
}

void workspace_layout(const Shape &s, size_t *qbar, size_t *kbar, size_t *lvn, size_t *total) {
    const size_t nq = (size_t)s.batch * s.hq * s.nb * s.d * sizeof(float);
    const size_t nk = (size_t)s.batch * s.hkv * s.nb * s.d * sizeof(float);
    const size_t nl = (size_t)s.batch * s.hkv * s.nb * sizeof(float);
    *qbar = 0;
    *kbar = align256(nq);
    *lvn = *kbar + align256(nk);
    *total = *lvn + align256(nl);
}

int score_launch(const Shape &s, const void *q, const KvView *kv, float *scores, void *workspace, bool sam,
                 hipStream_t st, const char *what) {
    size_t oq, ok_, ol, total;
    workspace_layout(s, &oq, &ok_, &ol, &total);
    char *ws = static_cast<char *>(workspace);
    float *qbar = reinterpret_cast<float *>(ws + oq);
    float *kbar = reinterpret_cast<float *>(ws + ok_);
    float *lvn = sam ? nullptr : reinterpret_cast<float *>(ws + ol);
    hipError_t e = launch_pool(s, q, kv, qbar, kbar, lvn, st);
    if (e == hipSuccess) e = launch_score(s, qbar, kbar, lvn, scores, st);
    return hip_status(e, what);
}

}  // namespace stem

namespace {

// ---- debug checks (STEM_DEBUG set to anything but "" or "0") ----------------
// The kernels do not check block-table entries or list indices on the device.
// In debug mode every entry point that reads a block table copies it to the
// host first (waiting for the stream) and rejects entries outside
// [0, num_pages) with STEM_EINVAL before anything is enqueued; stem_select
// waits for its kernel and checks the lists and counts it wrote.
bool debug_on() {
    const char *e = std::getenv("STEM_DEBUG");
    return e && *e && std::strcmp(e, "0") != 0;
}

int debug_table(const stem_kv_desc *kv, const Shape &s, hipStream_t st) {
    if (!debug_on() || !kv->block_table) return STEM_OK;
    std::vector<int32_t> host((size_t)s.batch * kv->pages_per_seq);
    hipError_t e = hipMemcpyAsync(host.data(), kv->block_table, host.size() * sizeof(int32_t),
                                  hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_status(e, "STEM_DEBUG: reading the block table");
    return stem_validate_block_table(host.data(), s.batch, kv->pages_per_seq, kv->num_pages, s.seq,
                                     kv->page_size);
}

// Arguments of the attention entry points: shapes, K/V, q and o present, and
// the limits of the attention kernels (32-bit K/V offsets, pages of at least
// 16 tokens).
int check_attention(const stem_attn_desc *desc, const void *q, const stem_kv_desc *kv, void *o, Shape *s,
                    KvView *v) {
    int rc = check_desc(desc, s);
    if (rc) return rc;
    if ((rc = check_kv(kv, *s, v))) return rc;
    if (!q || !o) return fail(STEM_EINVAL, "q or o is NULL");
    const size_t es = s->dtype == STEM_F32 ? 4 : s->dtype == STEM_BF16 ? 2 : 1;
    const size_t rows = v->table ? (size_t)kv->num_pages * kv->page_size : (size_t)s->batch * s->seq;
    if (rows * s->hkv * s->d * es >= (size_t(1) << 32))
        return fail(STEM_EUNSUPPORTED, "K/V tensors of 4 GiB or more are not supported");
    if (v->table && kv->page_size < 16) return fail(STEM_EUNSUPPORTED, "page_size below 16 tokens is not supported");
    return 0;
}

// The decode kernels read a block's page entries one per lane of a wave, so
// a block may span at most 64 pages; as for the prefill kernels, pages must
// hold at least 16 tokens.
int check_decode_pages(const stem_kv_desc *kv, const KvView &v) {
    if (v.table && kv->page_size < 16) return fail(STEM_EUNSUPPORTED, "page_size below 16 tokens is not supported");
    return 0;
}

// stem_score and stem_score_sam: pool Q, K (and V) into the workspace, then
// the score GEMM (with the value term unless sam).
int score_from_kv(const stem_attn_desc *desc, const void *q, const stem_kv_desc *kv, float *scores,
                  void *workspace, size_t workspace_bytes, void *stream, bool sam) {
    Shape s;
    KvView v;
    int rc = check_desc(desc, &s);
    if (rc) return rc;
    if ((rc = check_kv(kv, s, &v))) return rc;
    if (!q || !scores || !workspace) return fail(STEM_EINVAL, "q, scores or workspace is NULL");
    size_t oq, ok_, ol, total;
    workspace_layout(s, &oq, &ok_, &ol, &total);
    if (workspace_bytes < total)
        return fail(STEM_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, total);
    if ((rc = hip_precheck())) return rc;
    if ((rc = debug_table(kv, s, static_cast<hipStream_t>(stream)))) return rc;
    return score_launch(s, q, &v, scores, workspace, sam, static_cast<hipStream_t>(stream),
                        sam ? "stem_score_sam launch" : "stem_score launch");
}

}  // namespace

extern "C" {

const char *stem_last_error(void) { return g_err; }

int stem_score_workspace_size(const stem_attn_desc *desc, size_t *bytes) {
    Shape s;
    int rc = check_desc(desc, &s);
    if (rc) return rc;
    if (!bytes) return fail(STEM_EINVAL, "bytes is NULL");
    size_t a, b, c;
    workspace_layout(s, &a, &b, &c, bytes);
    return ok();
}

int stem_score(const stem_attn_desc *desc, const void *q, const stem_kv_desc *kv, float *scores,
               void *workspace, size_t workspace_bytes, void *stream) {
    return score_from_kv(desc, q, kv, scores, workspace, workspace_bytes, stream, false);
}

int stem_score_sam(const stem_attn_desc *desc, const void *q, const stem_kv_desc *kv, float *scores,
                   void *workspace, size_t workspace_bytes, void *stream) {
    return score_from_kv(desc, q, kv, scores, workspace, workspace_bytes, stream, true);
}

int stem_score_pooled(const stem_attn_desc *desc, const void *q, const float *kbar, const float *lvn,
                      float *scores, void *workspace, size_t workspace_bytes, void *stream) {
    Shape s;
    int rc = check_desc(desc, &s);
    if (rc) return rc;
    if (!q || !kbar || !scores || !workspace)
        return fail(STEM_EINVAL, "q, kbar, scores or workspace is NULL");
    size_t oq, ok_, ol, total;
    workspace_layout(s, &oq, &ok_, &ol, &total);
    if (workspace_bytes < total)
        return fail(STEM_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, total);
    if ((rc = hip_precheck())) return rc;
    float *qbar = reinterpret_cast<float *>(static_cast<char *>(workspace) + oq);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = launch_pool(s, q, nullptr, qbar, nullptr, nullptr, st);
    if (e == hipSuccess) e = launch_score(s, qbar, kbar, lvn, scores, st);
    return hip_status(e, "stem_score_pooled launch");
}

int stem_cache_write(const stem_attn_desc *desc, const void *k_in, const void *v_in,
                     const stem_kv_desc *cache, float *kbar, float *lvn, void *stream) {
    Shape s;
    KvView v;
    int rc = check_desc(desc, &s);
    if (rc) return rc;
    if ((rc = check_kv(cache, s, &v))) return rc;
    if (!k_in || !v_in || !kbar || !lvn) return fail(STEM_EINVAL, "k_in, v_in, kbar or lvn is NULL");
    if ((rc = hip_precheck())) return rc;
    if ((rc = debug_table(cache, s, static_cast<hipStream_t>(stream)))) return rc;
    hipError_t e = launch_cache_write(s, k_in, v_in, v, kbar, lvn, static_cast<hipStream_t>(stream));
    return hip_status(e, "stem_cache_write launch");
}

int stem_tpd_budget(int32_t num_blocks, double density, double alpha, int32_t *budget_host,
                    int64_t *total) {
    TpdPlan p;
    const char *why = "";
    int rc = tpd_make_plan(num_blocks, density, alpha, &p, &why);
    if (rc) return fail(rc, "%s", why);
    if (budget_host)
        for (int i = 0; i < num_blocks; ++i) budget_host[i] = tpd_row_budget(p, i);
    if (total) *total = p.total;
    return ok();
}

int stem_select(const stem_attn_desc *desc, const float *scores, double density, double alpha,
                uint32_t *mask, int32_t *list, int32_t list_stride, int32_t *count, void *stream) {
    Shape s;
    int rc = check_desc(desc, &s);
    if (rc) return rc;
    if (!scores || !mask) return fail(STEM_EINVAL, "scores or mask is NULL");
    TpdPlan p;
    const char *why = "";
    if ((rc = tpd_make_plan(s.nb, density, alpha, &p, &why))) return fail(rc, "%s", why);
    if (list) {
        int kmax = 0;
        for (int i = 0; i < s.nb; ++i) { int k = tpd_row_budget(p, i); if (k > kmax) kmax = k; }
        if (list_stride < kmax)
            return fail(STEM_EINVAL, "list_stride %d is below the largest budget %d", list_stride, kmax);
    }
    if ((rc = hip_precheck())) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = launch_select(s, p, scores, mask, list, list_stride, count, st);
    if ((rc = hip_status(e, "stem_select launch"))) return rc;
    if (debug_on() && list && count) {
        // debug mode: the lists and counts just written, checked on the host
        const size_t rows = (size_t)s.batch * s.hq * s.nb;
        std::vector<int32_t> hl(rows * list_stride), hc(rows);
        e = hipMemcpyAsync(hl.data(), list, hl.size() * sizeof(int32_t), hipMemcpyDeviceToHost, st);
        if (e == hipSuccess) e = hipMemcpyAsync(hc.data(), count, hc.size() * sizeof(int32_t), hipMemcpyDeviceToHost, st);
        if (e == hipSuccess) e = hipStreamSynchronize(st);
        if (e != hipSuccess) return hip_status(e, "STEM_DEBUG: reading the kept lists");
        return stem_validate_lists(hl.data(), hc.data(), s.batch * s.hq, s.nb, list_stride);
    }
    return STEM_OK;
}

int bsa_prefill(const stem_attn_desc *desc, const void *q, const stem_kv_desc *kv,
                const uint32_t *mask, void *o, float *lse, void *stream) {
    Shape s;
    KvView v;
    int rc = check_attention(desc, q, kv, o, &s, &v);
    if (rc) return rc;
    if ((rc = hip_precheck())) return rc;
    if ((rc = debug_table(kv, s, static_cast<hipStream_t>(stream)))) return rc;
    hipError_t e = launch_bsa(s, q, v, mask, o, lse, static_cast<hipStream_t>(stream));
    return hip_status(e, "bsa_prefill launch");
}

int bsa_prefill_blasst(const stem_attn_desc *desc, const void *q, const stem_kv_desc *kv,
                       const uint32_t *mask, double lambda, void *o, float *lse, int32_t *skipped,
                       void *stream) {
    Shape s;
    KvView v;
    int rc = check_attention(desc, q, kv, o, &s, &v);
    if (rc) return rc;
    if (!(lambda >= 0.0 && lambda <= 1.0)) return fail(STEM_EINVAL, "lambda must lie in [0, 1]");
    if (s.d != 128 || s.blk != 128 || s.dtype == STEM_F32)
        return fail(STEM_EUNSUPPORTED, "the online skip needs head_dim 128, block_size 128 and bf16 or FP8");
    if ((rc = hip_precheck())) return rc;
    if ((rc = debug_table(kv, s, static_cast<hipStream_t>(stream)))) return rc;
    const float skip_log2 = lambda > 0.0 ? (float)std::log2(lambda) : -std::numeric_limits<float>::infinity();
    hipError_t e = launch_bsa_skip(s, q, v, mask, skip_log2, o, lse, skipped, static_cast<hipStream_t>(stream));
    return hip_status(e, "bsa_prefill_blasst launch");
}

int stem_decode_workspace_size(const stem_attn_desc *desc, size_t *bytes) {
    Shape s;
    int rc = check_desc(desc, &s);
    if (rc) return rc;
    if (!bytes) return fail(STEM_EINVAL, "bytes is NULL");
    size_t a, b, c;
    decode_workspace_layout(s, &a, &b, &c, bytes);
    return ok();
}

int stem_decode(const stem_attn_desc *desc, const void *q, const stem_kv_desc *kv,
                const int32_t *seq_lens, const int32_t *keep, const float *kbar, const float *lvn,
                void *o, float *lse, void *workspace, size_t workspace_bytes, void *stream) {
    Shape s;
    KvView v;
    int rc = check_desc(desc, &s);
    if (rc) return rc;
    if ((rc = check_kv(kv, s, &v))) return rc;
    if ((rc = check_decode_pages(kv, v))) return rc;
    if (!q || !seq_lens || !o || !workspace) return fail(STEM_EINVAL, "q, seq_lens, o or workspace is NULL");
    if (keep && !kbar) return fail(STEM_EINVAL, "kbar is NULL but keep is given");
    size_t a, b, c, total;
    decode_workspace_layout(s, &a, &b, &c, &total);
    if (workspace_bytes < total)
        return fail(STEM_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, total);
    if ((rc = hip_precheck())) return rc;
    if ((rc = debug_table(kv, s, static_cast<hipStream_t>(stream)))) return rc;
    hipError_t e = launch_decode(s, q, v, seq_lens, keep, kbar, lvn, o, lse, workspace,
                                 static_cast<hipStream_t>(stream));
    return hip_status(e, "stem_decode launch");
}

int stem_decode_blasst_workspace_size(const stem_attn_desc *desc, size_t *bytes) {
    Shape s;
    int rc = check_desc(desc, &s);
    if (rc) return rc;
    if (!bytes) return fail(STEM_EINVAL, "bytes is NULL");
    size_t a, b, c, d;
    decode_skip_layout(s, &a, &b, &c, &d, bytes);
    return ok();
}

int stem_decode_blasst(const stem_attn_desc *desc, const void *q, const stem_kv_desc *kv,
                       const int32_t *seq_lens, const int32_t *keep, const float *kbar, const float *lvn,
                       double lambda, void *o, float *lse, int32_t *skipped, void *workspace,
                       size_t workspace_bytes, void *stream) {
    Shape s;
    KvView v;
    int rc = check_desc(desc, &s);
    if (rc) return rc;
    if ((rc = check_kv(kv, s, &v))) return rc;
    if ((rc = check_decode_pages(kv, v))) return rc;
    if (!q || !seq_lens || !o || !workspace) return fail(STEM_EINVAL, "q, seq_lens, o or workspace is NULL");
    if (keep && !kbar) return fail(STEM_EINVAL, "kbar is NULL but keep is given");
    if (!(lambda >= 0.0 && lambda <= 1.0)) return fail(STEM_EINVAL, "lambda must lie in [0, 1]");
    size_t a, b, c, d, total;
    decode_skip_layout(s, &a, &b, &c, &d, &total);
    if (workspace_bytes < total)
        return fail(STEM_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, total);
    if ((rc = hip_precheck())) return rc;
    if ((rc = debug_table(kv, s, static_cast<hipStream_t>(stream)))) return rc;
    DecodeSkip sk;
    sk.log2_lambda = lambda > 0.0 ? (float)std::log2(lambda) : -std::numeric_limits<float>::infinity();
    sk.skipped = skipped;
    hipError_t e = launch_decode(s, q, v, seq_lens, keep, kbar, lvn, o, lse, workspace,
                                 static_cast<hipStream_t>(stream), &sk);
    return hip_status(e, "stem_decode_blasst launch");
}

int stem_validate_block_table(const int32_t *table, int32_t batch, int32_t pages_per_seq, int32_t num_pages,
                              int32_t seq_len, int32_t page_size) {
    if (!table) return fail(STEM_EINVAL, "table is NULL");
    if (batch < 1 || seq_len < 1 || num_pages < 1) return fail(STEM_EINVAL, "batch, seq_len and num_pages must be positive");
    if (page_size < 1 || (page_size & (page_size - 1))) return fail(STEM_EINVAL, "page_size %d is not a power of two", page_size);
    if ((long long)pages_per_seq * page_size < seq_len) return fail(STEM_EINVAL, "pages_per_seq * page_size < seq_len");
    const int used = (int)(((long long)seq_len + page_size - 1) / page_size);
    for (int b = 0; b < batch; ++b)
        for (int p = 0; p < used; ++p) {
            const int32_t e = table[(size_t)b * pages_per_seq + p];
            if (e < 0 || e >= num_pages)
                return fail(STEM_EINVAL, "block_table[%d][%d] = %d lies outside [0, %d)", b, p, e, num_pages);
        }
    return ok();
}

int stem_validate_lists(const int32_t *lists, const int32_t *counts, int32_t rows_per_block_row, int32_t num_blocks,
                        int32_t list_stride) {
    if (!lists || !counts) return fail(STEM_EINVAL, "lists or counts is NULL");
    if (rows_per_block_row < 1 || num_blocks < 1 || list_stride < 1)
        return fail(STEM_EINVAL, "row count, num_blocks and list_stride must be positive");
    for (long long r = 0; r < (long long)rows_per_block_row * num_blocks; ++r) {
        const int I = (int)(r % num_blocks);
        const int c = counts[r];
        if (c < 0 || c > I + 1 || c > list_stride)
            return fail(STEM_EINVAL, "count of row %lld (query block %d) is %d, outside [0, %d]", r, I, c,
                        I + 1 < list_stride ? I + 1 : list_stride);
        const int32_t *l = lists + r * list_stride;
        for (int e = 0; e < c; ++e) {
            if (l[e] < 0 || l[e] > I)
                return fail(STEM_EINVAL, "list of row %lld (query block %d), entry %d = %d lies outside [0, %d]", r,
                            I, e, l[e], I);
            if (e > 0 && l[e] <= l[e - 1])
                return fail(STEM_EINVAL, "list of row %lld is not strictly ascending at entry %d", r, e);
        }
    }
    return ok();
}

}  // extern "C"
