/*
 * stem_bsa.h — C ABI of the Stem block-sparse prefill-attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * The path has three steps, each one entry point:
 *   stem_score   OAM block scoring: compact per-block Q/K representations, one
 *                small GEMM per head, plus the log of each V block's norm
 *                (Stem article on cn486.com, §一.3.2 "Output-Aware Metric" and
 *                §二.2.1 "Stem operator optimisation").
 *   stem_select  TPD budget fused with top-k block selection (same article,
 *                §一.3.1 "Token Position Decay" and §二.2.1; setupai.cc summary
 *                "Technical Deep Dive").
 *   bsa_prefill  causal block-sparse flash attention over the kept blocks
 *                (same article, §二.2.2 "BSA operator optimisation"); with no
 *                mask it is the dense causal kernel used as the baseline of
 *                §二.3 "operator benchmark".
 * stem_tpd_budget exposes the budget on the host.
 *
 * Around the path:
 *   stem_score_sam     the score-only metric (SAM) that OAM is contrasted
 *                      with (setupai.cc summary, "Technical Deep Dive"): the
 *                      same scores without the value term, for ablations.
 *   stem_cache_write   writes a prefill's K and V into the (FP8, paged) cache
 *                      and computes the key-block means and value-block norms
 *                      in the same pass, so scoring does not read K and V
 *                      again (cn486.com article, §二.2.1: precomputed compact
 *                      block representations; §二.2.2: paged FP8 KV in vLLM).
 *   stem_score_pooled  scoring from those precomputed representations.
 *   stem_decode        one decode step over the cache with Stem block
 *                      selection for the new token.
 *   bsa_prefill_blasst the attention with BLASST's online skip of blocks far
 *                      below a row's running maximum, on top of the mask.
 *   stem_decode_blasst the decode step with the same skip, which leaves the
 *                      dropped blocks' V rows unread.
 *
 * Conventions for every entry point
 *   - Tensors are row-major, in caller-owned DEVICE memory unless a comment
 *     says "host".  The library never allocates or frees memory and never
 *     synchronises; all work is enqueued on `stream` (a hipStream_t passed as
 *     void*, NULL = the null stream).
 *   - Layouts: Q [batch, seq_len, num_q_heads, head_dim];
 *     contiguous K/V [batch, seq_len, num_kv_heads, head_dim];
 *     paged K/V [num_pages, page_size, num_kv_heads, head_dim] with
 *     block_table [batch, pages_per_seq] (token t of sequence b lives in page
 *     block_table[b][t / page_size], row t % page_size).
 *   - Query head h reads KV head h / (num_q_heads / num_kv_heads).
 *   - Blocks are block_size tokens; Nb = seq_len / block_size.  Positions of
 *     queries and keys are both 0..seq_len-1 (prefill, causal).
 *   - Return value: STEM_OK, or a negative stem_status.  On a non-OK return
 *     nothing has been enqueued; stem_last_error() gives a message (per
 *     thread).  A HIP error raised by earlier asynchronous work may surface
 *     as STEM_EHIP on a later call.
 *   - Calls are thread-safe; calls on one stream execute in order.
 *
 * Supported shapes: head_dim in {64, 128}; block_size in {64, 128};
 * seq_len a positive multiple of block_size with Nb <= 4096; dtype STEM_F32,
 * STEM_BF16 or STEM_FP8_E4M3 (OCP E4M3, "e4m3fn", with per-tensor fp32
 * scales: real value = code * scale).  Paged K/V: page_size a power of two;
 * the attention and decode entry points need at least 16 tokens per page.
 */
#ifndef STEM_BSA_H
#define STEM_BSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    STEM_OK = 0,
    STEM_EINVAL = -1,        /* invalid argument (null pointer, bad shape or range) */
    STEM_EUNSUPPORTED = -2,  /* valid but not built (head_dim, block_size, dtype, alpha) */
    STEM_EHIP = -3,          /* HIP runtime error */
    STEM_EWORKSPACE = -4     /* workspace smaller than stem_score_workspace_size() */
} stem_status;

typedef enum {
    STEM_F32 = 0,
    STEM_BF16 = 1,
    STEM_FP8_E4M3 = 2
} stem_dtype;

/* Problem shape, element type and scales (by value everywhere it is read). */
typedef struct {
    int32_t batch;
    int32_t seq_len;         /* multiple of block_size */
    int32_t num_q_heads;
    int32_t num_kv_heads;    /* divides num_q_heads */
    int32_t head_dim;        /* 64 or 128 */
    int32_t block_size;      /* 64 or 128 */
    int32_t dtype;           /* stem_dtype of Q, K and V */
    float q_scale, k_scale, v_scale;   /* FP8 dequantisation scales; must be 1 otherwise */
    float softmax_scale;     /* tau; 0 selects 1/sqrt(head_dim) */
} stem_attn_desc;

/* Where K and V live.  block_table == NULL: contiguous [batch, seq_len,
 * num_kv_heads, head_dim] tensors; otherwise paged (layout above) and every
 * block_table entry must lie in [0, num_pages) — entries are not checked on
 * the device (see STEM_DEBUG below for a host-side check). */
typedef struct {
    const void *k;
    const void *v;
    const int32_t *block_table;  /* device [batch, pages_per_seq] or NULL */
    int32_t page_size;           /* power of two; ignored when contiguous */
    int32_t pages_per_seq;       /* >= seq_len / page_size */
    int32_t num_pages;
} stem_kv_desc;

/* Bytes of scratch stem_score needs: the pooled representations it writes
 * there, each region starting on a 256-byte boundary, in this order:
 *   qbar [batch, num_q_heads, Nb, head_dim] fp32   mean of each block's Q rows
 *   kbar [batch, num_kv_heads, Nb, head_dim] fp32  mean of each block's K rows
 *   lvn  [batch, num_kv_heads, Nb] fp32            ln of the Frobenius norm of the block's V rows
 * (dequantised values for FP8).  They stay valid after the call. */
int stem_score_workspace_size(const stem_attn_desc *desc, size_t *bytes);

/* OAM block scores (Stem article §一.3.2, §二.2.1):
 *   scores[b, h, I, J] = tau * <qbar[b,h,I], kbar[b,g(h),J]> + lvn[b,g(h),J]   for J <= I
 * scores: fp32 [batch, num_q_heads, Nb, Nb]; entries with J > I are not
 * written (the selection never reads them).  All arithmetic is fp32 with a
 * fixed summation order, so repeated calls give identical bits.
 * workspace: device memory of at least stem_score_workspace_size() bytes. */
int stem_score(const stem_attn_desc *desc, const void *q, const stem_kv_desc *kv,
               float *scores, void *workspace, size_t workspace_bytes, void *stream);

/* SAM block scores: stem_score without the value term (the score-only
 * metric the setupai.cc summary, "Technical Deep Dive", contrasts OAM with):
 *   scores[b, h, I, J] = tau * <qbar[b,h,I], kbar[b,g(h),J]>   for J <= I (J > I not written).
 * Arguments, workspace and errors as stem_score; the lvn region of the
 * workspace is left unwritten. */
int stem_score_sam(const stem_attn_desc *desc, const void *q, const stem_kv_desc *kv,
                   float *scores, void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of device scratch stem_score_noalloc holds on each device: room for
 * stem_score's workspace (stem_score_workspace_size) up to this size, e.g.
 * 128K tokens with 64 query / 8 KV heads and head_dim 128 (36 MiB). */
#define STEM_NOALLOC_SCRATCH_BYTES (64u << 20)

/* stem_score for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same kernels and the same scores, bit for bit; the pooled representations
 * go to a scratch array the library holds on each device (fixed size,
 * STEM_NOALLOC_SCRATCH_BYTES, kept until the process ends) instead of a
 * workspace.  The call allocates nothing.
 *   stream: must belong to the current device (STEM_EINVAL otherwise).
 * A problem whose stem_score workspace exceeds STEM_NOALLOC_SCRATCH_BYTES is
 * rejected with STEM_EWORKSPACE.  All calls on one device share its scratch:
 * calls that overlap in time on one device (different streams or threads)
 * race, and the representations are not readable by the caller. */
int stem_score_noalloc(const stem_attn_desc *desc, const void *q, const stem_kv_desc *kv,
                       float *scores, void *stream);

/* Block scores from key-block representations computed earlier (by
 * stem_cache_write, or left in a stem_score workspace): pools Q into the qbar
 * region of the workspace, then the score GEMM of stem_score.
 *   kbar: fp32 [batch, num_kv_heads, Nb, head_dim], dequantised means.
 *   lvn:  fp32 [batch, num_kv_heads, Nb], or NULL for SAM scores.
 *   workspace: at least stem_score_workspace_size() bytes (only qbar is written).
 * Given the kbar and lvn stem_score would pool from the same K/V, the scores
 * are bit-identical to stem_score's. */
int stem_score_pooled(const stem_attn_desc *desc, const void *q, const float *kbar,
                      const float *lvn, float *scores, void *workspace, size_t workspace_bytes,
                      void *stream);

/* Writes one prefill's keys and values into the KV cache and, in the same
 * pass over the new tokens, the block representations scoring needs (Stem
 * article on cn486.com, §二.2.1 and §二.2.2).
 *   desc:  shape; desc->dtype is the CACHE's element type.
 *          STEM_FP8_E4M3: k_in and v_in are bf16; each element x is stored
 *          as the E4M3 code nearest to the fp32 quotient x / scale (ties to
 *          even, saturating at +-448), scale = desc->k_scale or v_scale.
 *          Inputs must be finite.
 *          STEM_BF16, STEM_F32: k_in and v_in have that type and are copied.
 *   k_in, v_in: [batch, seq_len, num_kv_heads, head_dim] (contiguous).
 *   cache: the destination, contiguous or paged exactly as stem_kv_desc
 *          describes for reading; cache->k and cache->v are WRITTEN.  Pages
 *          of different tokens must not alias.
 *   kbar:  fp32 [batch, num_kv_heads, Nb, head_dim], mean of each block's
 *          stored (dequantised) key rows.
 *   lvn:   fp32 [batch, num_kv_heads, Nb], ln of the Frobenius norm of each
 *          block's stored (dequantised) value rows.
 * kbar and lvn are bit-identical to what stem_score pools from the written
 * cache, so stem_score_pooled with them gives stem_score's scores. */
int stem_cache_write(const stem_attn_desc *desc, const void *k_in, const void *v_in,
                     const stem_kv_desc *cache, float *kbar, float *lvn, void *stream);

/* Bytes of scratch stem_decode needs.  After a call the workspace holds,
 * each region starting on a 256-byte boundary, in this order:
 *   lists  int32 [batch, num_q_heads, Nb]  kept blocks of each row, ascending
 *   counts int32 [batch, num_q_heads]      number of kept blocks
 * followed by the split-K partials. */
int stem_decode_workspace_size(const stem_attn_desc *desc, size_t *bytes);

/* One decode step of Stem block-sparse attention: for every sequence b and
 * query head h, the new token (position t = seq_lens[b] - 1, block
 * I = t / block_size) scores the complete blocks J in [1, I-1] of its cache
 * with the OAM metric (Stem article on cn486.com, §一.3.2, the token standing
 * for its query block), keeps J = 0, J = I and the best keep[b] - |{0, I}|
 * of them (score descending, equal scores to the smaller J), and attends to
 * the keys j <= t of the kept blocks only (the memory-bound decode case of
 * the BLASST summary, §2.3: skipped blocks are never read).
 *   desc:     shape of the cache: seq_len is its capacity per sequence (a
 *             multiple of block_size); dtype, scales and softmax scale as for
 *             bsa_prefill.
 *   q:        [batch, num_q_heads, head_dim] in desc->dtype (FP8 codes with
 *             q_scale).
 *   kv:       the cache (contiguous or paged), holding tokens 0..t of every
 *             sequence, the new token's K and V included.  Paged caches need
 *             pages of at least 16 tokens (STEM_EUNSUPPORTED otherwise).
 *   seq_lens: device int32 [batch], tokens in each sequence including the new
 *             one; values outside [1, seq_len] are clamped into it.
 *   keep:     device int32 [batch], blocks to keep for the new token's row
 *             (for the prefill's TPD budget: stem_tpd_budget over I + 1 rows,
 *             entry I), clamped to [|{0, I}|, I + 1]; NULL keeps every block
 *             (dense decode).
 *   kbar, lvn: the cache's block representations as stem_cache_write
 *             produces them (only complete blocks J < I are read); lvn NULL
 *             scores without the value term; both unused when keep is NULL.
 *   o:        [batch, num_q_heads, head_dim], bf16 (fp32 for STEM_F32).
 *   lse:      optional fp32 [batch, num_q_heads], natural log.
 *   workspace: at least stem_decode_workspace_size() bytes. */
int stem_decode(const stem_attn_desc *desc, const void *q, const stem_kv_desc *kv,
                const int32_t *seq_lens, const int32_t *keep, const float *kbar, const float *lvn,
                void *o, float *lse, void *workspace, size_t workspace_bytes, void *stream);

/* Workspace of stem_decode_blasst: that of stem_decode followed by, each
 * 256-byte aligned, the kept blocks' maxima fp32 [batch, num_q_heads, Nb]
 * (entry e = e-th kept block), the entries not dropped int32
 * [batch, num_q_heads, Nb] in ascending order, their number int32
 * [batch, num_q_heads], and the kept blocks' scores fp32
 * [batch, num_q_heads, Nb, block_size]. */
int stem_decode_blasst_workspace_size(const stem_attn_desc *desc, size_t *bytes);

/* stem_decode with BLASST's online skip ("BLASST: Dynamic BLocked Attention
 * Sparsity via Softmax Thresholding", gist.science summary: §2.1
 * running-maximum pruning; §2.3 decode, where skipping a block saves its V
 * loads).  Among the new token's kept blocks, in ascending J, a block is
 * dropped when its largest logit tau * q.k over the keys j <= t lies more than
 * ln(1 / lambda) below the largest of the earlier kept blocks; the first kept
 * block never is.  O and LSE are those of the blocks not dropped.  The K rows
 * of every kept block are read; the V rows of a dropped block are not.
 *   lambda:  in [0, 1] (0 drops nothing: the step is stem_decode's, with
 *            bit-identical O and LSE); NaN or values outside are
 *            STEM_EINVAL.
 *   skipped: optional int32 [batch, num_q_heads]: blocks each row dropped.
 *   workspace: at least stem_decode_blasst_workspace_size() bytes.
 * Every other argument, and every check, as for stem_decode. */
int stem_decode_blasst(const stem_attn_desc *desc, const void *q, const stem_kv_desc *kv,
                       const int32_t *seq_lens, const int32_t *keep, const float *kbar, const float *lvn,
                       double lambda, void *o, float *lse, int32_t *skipped, void *workspace,
                       size_t workspace_bytes, void *stream);

/* TPD budget on the host (Stem article §一.3.1; setupai.cc "Technical Deep
 * Dive").  T = floor(density * Nb(Nb+1)/2 + 1/2) computed in double, clamped
 * to [2*Nb - 1, Nb(Nb+1)/2].  Row 0 keeps 1 block, every other row starts at
 * 2 (sink and diagonal); the remaining T - (2*Nb - 1) blocks are granted one
 * at a time to the row I with the smallest (k[I]+1) / (I+1)^(1-alpha) among
 * rows with k[I] < I+1, equal keys to the smaller I.
 *   density in (0, 1]; alpha in {0, 0.5, 1} (0: uniform keep ratio, 0.5:
 *   ratio decaying as 1/sqrt(I+1), 1: uniform count); 1 <= num_blocks <= 65536.
 *   budget_host: host int32 [num_blocks] (may be NULL); total: host (may be NULL). */
int stem_tpd_budget(int32_t num_blocks, double density, double alpha,
                    int32_t *budget_host, int64_t *total);

/* Fused TPD budget + top-k selection (Stem article §二.2.1).  For every row
 * (b, h, I): keep J = 0 and J = I, then the budget[I] - |{0, I}| best J in
 * [1, I-1] ordered by score descending, equal scores to the smaller J, NaN
 * below every number.  The budget is the one stem_tpd_budget returns.
 *   scores: fp32 [batch, num_q_heads, Nb, Nb] (only J < I is read)
 *   mask:   uint32 [batch, num_q_heads, Nb, ceil(Nb/32)]; bit J%32 of word
 *           J/32 set when block J is kept; bits above the diagonal are 0.
 *   list:   optional int32 [batch, num_q_heads, Nb, list_stride]: the kept J
 *           in ascending order (entries past count undefined);
 *           list_stride >= max budget.  NULL to skip.
 *   count:  optional int32 [batch, num_q_heads, Nb] = budget[I].  NULL to skip. */
int stem_select(const stem_attn_desc *desc, const float *scores, double density, double alpha,
                uint32_t *mask, int32_t *list, int32_t list_stride, int32_t *count,
                void *stream);

/* Causal block-sparse attention (Stem article §二.2.2).  For every query token
 * i of block I and head h: softmax over the keys of the kept blocks J < I and
 * the keys j <= i of block I when it is kept; a skipped block counts as -inf
 * scores.  Bits above the diagonal are ignored.  A row with no kept block
 * gives O = 0 and LSE = -inf.
 *   mask: as stem_select writes it, or NULL for dense causal attention (every
 *         block J <= I; a kernel without any mask logic).
 *   o:    [batch, seq_len, num_q_heads, head_dim]: fp32 for STEM_F32 inputs,
 *         bf16 for STEM_BF16 and STEM_FP8_E4M3 inputs.
 *   lse:  optional fp32 [batch, num_q_heads, seq_len], natural log of the
 *         softmax denominator of tau * q.k (dequantised); NULL to skip. */
int bsa_prefill(const stem_attn_desc *desc, const void *q, const stem_kv_desc *kv,
                const uint32_t *mask, void *o, float *lse, void *stream);

/* bsa_prefill with the online skip of BLASST ("BLASST: Dynamic BLocked
 * Attention Sparsity via Softmax Thresholding", gist.science summary, §2.1
 * running-maximum pruning) on top of the mask.  Every row visits its kept
 * blocks in ascending J, keeping the running maximum m of the logits
 * tau * q.k it has taken in.  Block J's largest logit over the keys the row
 * sees is compared with m: when it lies more than ln(1 / lambda) below m, the
 * row drops the block (no exponentials, no sum, no product with V).  A dropped
 * block never moves m, so the test is against the largest logit of the row's
 * earlier kept blocks; a row's first block is never dropped.  O and LSE are
 * those of the blocks not dropped.  When all 32 rows that one wavefront
 * holds drop a block, its softmax is not computed at all; K and V are still
 * loaded in order (the summary's §2.3 prefill design).
 *   mask:    as for bsa_prefill (NULL: every causal block, the pages' dense
 *            setting of the skip).
 *   lambda:  in [0, 1]; 0 drops nothing (the result equals bsa_prefill's up
 *            to rounding); NaN or values outside are STEM_EINVAL.
 *   o, lse:  as for bsa_prefill.
 *   skipped: optional int32 [batch, num_q_heads, seq_len]: blocks each query
 *            row dropped.  NULL to skip.
 * Supported: head_dim 128, block_size 128, STEM_BF16 or STEM_FP8_E4M3
 * (STEM_EUNSUPPORTED otherwise). */
int bsa_prefill_blasst(const stem_attn_desc *desc, const void *q, const stem_kv_desc *kv,
                       const uint32_t *mask, double lambda, void *o, float *lse, int32_t *skipped,
                       void *stream);

/* Debug checks.  With the environment variable STEM_DEBUG set (to anything
 * but "" or "0"), every entry point that reads a block table first copies it
 * to the host, waiting for `stream`, and returns STEM_EINVAL, with nothing
 * enqueued, when an entry that one of the batch's seq_len tokens uses lies
 * outside [0, num_pages); stem_select waits for its kernel and checks the
 * lists and counts it wrote with stem_validate_lists.  Debug mode breaks the
 * no-synchronisation convention on purpose; it is for finding bad inputs, not
 * for timing.  The two checks are also callable directly on host arrays.
 *
 * stem_validate_block_table: table is HOST int32 [batch, pages_per_seq];
 * checks entries [b][p] for p < ceil(seq_len / page_size).  STEM_OK, or
 * STEM_EINVAL naming the first bad entry (or a bad argument). */
int stem_validate_block_table(const int32_t *table, int32_t batch, int32_t pages_per_seq, int32_t num_pages,
                              int32_t seq_len, int32_t page_size);

/* stem_validate_lists: lists HOST int32 [rows, num_blocks, list_stride] and
 * counts HOST int32 [rows, num_blocks] in stem_select's layout (rows = batch *
 * num_q_heads; the row of query block I is entry I).  Each count must lie in
 * [0, min(I + 1, list_stride)] and its entries must be strictly ascending
 * block indices in [0, I].  STEM_OK, or STEM_EINVAL naming the first bad
 * count or entry. */
int stem_validate_lists(const int32_t *lists, const int32_t *counts, int32_t rows, int32_t num_blocks,
                        int32_t list_stride);

/* Message for the last non-OK return on this thread ("" if none). */
const char *stem_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* STEM_BSA_H */
