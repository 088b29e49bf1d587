// Library-internal declarations shared by the host API and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "stem_bsa.h"

namespace stem {

// Validated problem shape, passed by value to every launcher.
struct Shape {
    int batch, seq, hq, hkv, d, blk, nb, words;   // words = ceil(nb / 32)
    int dtype;                                    // stem_dtype
    float q_scale, k_scale, v_scale;
    float tau;                                    // softmax scale
};

// K/V addressing: contiguous [b, S, Hkv, d] when table == nullptr, else
// paged [num_pages, page, Hkv, d] with table [b, pages_per_seq].
struct KvView {
    const void *k, *v;
    const int32_t *table;
    int page_log2;
    int pages_per_seq;
    size_t rows;                      // token rows of each of K and V (pages x page_size when paged)
};

// The TPD budget in closed form: every row's budget follows from the single
// threshold grant (th_row, th_n), the last of the T - (2Nb - 1) grants made
// in water-filling order.  power: 1 for alpha = 0 (key n/(I+1)), 2 for
// alpha = 1/2 (key n^2/(I+1), the square of n/sqrt(I+1)), 0 for alpha = 1
// (key n).  has_threshold == 0 when no block beyond the forced ones is granted.
struct TpdPlan {
    int nb;
    int power;
    int has_threshold;
    int th_row, th_n;
    long long total;
};

// Largest n with grant (row, n) at or before grant (t_row, t_n) in the order
// (key, row).  Exact in 64-bit integers for n, row < 2^16.
__host__ __device__ inline long long tpd_nmax(int power, int row, int t_row, int t_n) {
    const bool le = row <= t_row;            // equal keys: the smaller row comes first
    const unsigned long long a = (unsigned long long)row + 1;     // I + 1
    const unsigned long long b = (unsigned long long)t_row + 1;   // I* + 1
    const unsigned long long tn = (unsigned long long)t_n;
    if (power == 0) return le ? (long long)tn : (long long)tn - 1;
    if (power == 1) {
        // n * b <= tn * a   (or <)
        const unsigned long long num = tn * a;
        return le ? (long long)(num / b) : (long long)((num - 1) / b);
    }
    // power 2:  n^2 * b <= tn^2 * a   (or <)
    const unsigned long long num = tn * tn * a;
    const unsigned long long lim = le ? num : num - 1;
    unsigned long long x = (unsigned long long)sqrt((double)lim / (double)b);
    while ((x + 1) * (x + 1) * b <= lim) ++x;
    while (x > 0 && x * x * b > lim) --x;
    return (long long)x;
}

// Budget k[I] of row I under a plan.
__host__ __device__ inline int tpd_row_budget(const TpdPlan &p, int row) {
    const int lo = row == 0 ? 1 : 2;        // forced: sink (and diagonal)
    const int hi = row + 1;                 // a row holds at most I+1 blocks
    if (!p.has_threshold || hi <= lo) return lo;
    long long n = tpd_nmax(p.power, row, p.th_row, p.th_n);
    if (n < lo) n = lo;
    if (n > hi) n = hi;
    return (int)n;
}

// Host-side argument handling shared by the entry points (api.cpp).
// fail: records the message for stem_last_error and returns code; ok: clears it.
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int ok();
int check_desc(const stem_attn_desc *d, Shape *s);
int check_kv(const stem_kv_desc *kv, const Shape &s, KvView *out);
int hip_status(hipError_t e, const char *what);
int hip_precheck();
// stem_score's workspace: offsets of qbar, kbar, lvn and the total bytes.
void workspace_layout(const Shape &s, size_t *qbar, size_t *kbar, size_t *lvn, size_t *total);
// Pools into `workspace` (stem_score's layout) and runs the score GEMM;
// returns the status of the launches (what names them in the message).
int score_launch(const Shape &s, const void *q, const KvView *kv, float *scores, void *workspace, bool sam,
                 hipStream_t st, const char *what);

// Host: builds the plan (validates density/alpha); returns STEM_OK or an error.
int tpd_make_plan(int nb, double density, double alpha, TpdPlan *out, const char **why);

// Launchers (enqueue only; return the launch status).
// launch_pool: Q always; K when kv is given; V when kv and lvn are given.
hipError_t launch_pool(const Shape &s, const void *q, const KvView *kv,
                       float *qbar, float *kbar, float *lvn, hipStream_t st);
// launch_score: lvn == nullptr leaves the value term out (SAM).
hipError_t launch_score(const Shape &s, const float *qbar, const float *kbar, const float *lvn,
                        float *scores, hipStream_t st);
hipError_t launch_cache_write(const Shape &s, const void *k_in, const void *v_in,
                              const KvView &cache, float *kbar, float *lvn, hipStream_t st);
hipError_t launch_select(const Shape &s, const TpdPlan &plan, const float *scores,
                         uint32_t *mask, int32_t *list, int list_stride, int32_t *count,
                         hipStream_t st);
hipError_t launch_bsa(const Shape &s, const void *q, const KvView &kv, const uint32_t *mask,
                      void *o, float *lse, hipStream_t st);
// The same attention with the online skip: a row drops a kept block whose
// largest logit lies more than log2(1/lambda) below its running maximum
// (skip_log2 = log2(lambda), -inf: never); skipped (nullable) receives the
// count per query row.  Only head_dim 128, block 128, bf16 or FP8.
hipError_t launch_bsa_skip(const Shape &s, const void *q, const KvView &kv, const uint32_t *mask,
                           float skip_log2, void *o, float *lse, int32_t *skipped, hipStream_t st);
// Decode: workspace offsets (kept lists, counts, split partials) and launch.
void decode_workspace_layout(const Shape &s, size_t *lists, size_t *counts, size_t *part,
                             size_t *total);
// With the online skip: block maxima, the list of entries not dropped and its
// length, and the block scores, after the decode workspace.
void decode_skip_layout(const Shape &s, size_t *bmax, size_t *live, size_t *nlive, size_t *scores,
                        size_t *total);
struct DecodeSkip {
    float log2_lambda;                // -inf: never drop
    int32_t *skipped;                 // [b, hq] dropped blocks per row, or null
};
hipError_t launch_decode(const Shape &s, const void *q, const KvView &kv, const int32_t *seq_lens,
                         const int32_t *keep, const float *kbar, const float *lvn, void *o,
                         float *lse, void *workspace, hipStream_t st, const DecodeSkip *skip = nullptr);

}  // namespace stem
