"""fp64 definitions of the Stem prefill path: OAM scoring, TPD budget, top-k
block selection and causal block-sparse attention.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Not imported by the
product path.

Sources (web pages; no code exists on them):
  [Stem-cn]  "腾讯混元Stem稀疏注意力算法：长文推理加速新SOTA" (cn486.com) —
             §一.3.1 Token Position Decay, §一.3.2 Output-Aware Metric,
             §二.1 challenges of existing operators, §二.2.1 Stem operator,
             §二.2.2 BSA operator, §二.3 operator benchmark.
  [BLASST]   "BLASST: Dynamic BLocked Attention Sparsity via Softmax
             Thresholding" (gist.science summary) — §2.1 running-maximum
             pruning (the online skip on top of the block mask).
  [Stem-en]  "Tencent Hunyuan introduces Stem sparse attention algorithm"
             (setupai.cc) — "Technical Deep Dive".

Conventions (shared with the library's documented interface, not its code):
  q  [batch, S, Hq, d]     token-major, head-interleaved (as a KV cache stores it)
  k,v[batch, S, Hkv, d]    Hq % Hkv == 0, query head h reads KV head h // (Hq/Hkv)
  blocks of B tokens, Nb = S / B; I indexes query blocks, J key blocks.

Readings taken where the pages are silent (each is the plainest one the rest
of the text supports; "parity unpinned against the authors" for the OAM form,
the pooling, the norm type and the TPD shape):
  * OAM (Stem-cn §一.3.2: contribution = routing probability x value
    magnitude; §二.2.1: the metric is purely additive, needs no softmax):
    log(p_ij * |v_j|) = tau*q.k - LSE_i + ln|v_j|; the LSE is constant per
    query row, so rows are ranked by tau*q.k + ln|v|.  At block level the
    compact representation is the mean of the block's rows (the mean of all
    B x B pairwise logits equals the logit of the means, by bilinearity) and
    the value magnitude is the Frobenius norm of the block's V rows.
  * TPD (Stem-cn §一.3.1; Stem-en Deep Dive): a fixed total of kept blocks,
    redistributed towards early query blocks by water-filling; see
    ``tpd_budget``.
  * Selection: the sink block J=0 and the diagonal J=I are always kept; the
    rest of the row's budget goes to the highest-scoring J in [1, I-1], equal
    scores to the smaller J, NaN below everything.
"""

from __future__ import annotations

import heapq
import math
from fractions import Fraction

import numpy as np

E4M3_MAX = 448.0  # largest finite OCP FP8 E4M3 ("e4m3fn") value: 1.75 * 2**8


# --------------------------------------------------------------------------
# Inputs
# --------------------------------------------------------------------------

def e4m3fn_round(x):
    """Round to the nearest OCP FP8 E4M3 value (ties to even), saturating at
    +-448.  Written from the format definition: 1 sign bit, 4 exponent bits
    with bias 7, 3 mantissa bits, no infinities; normal numbers from 2**-6,
    subnormals are multiples of 2**-9.  The pages name FP8 quantisation
    (Stem-cn §二.2.2) without a rounding rule; this is the OCP default.
    Returns fp64 values (exactly representable in E4M3)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)                      # a = m * 2**e with m in [0.5, 1)
    exp = np.maximum(e - 1, -6)             # binade exponent, floored at the normal minimum
    quantum = np.ldexp(1.0, exp - 3)        # spacing of 3-bit mantissas in that binade
    r = np.round(a / quantum) * quantum     # np.round: round half to even
    r = np.minimum(r, E4M3_MAX)
    r = np.where(a == 0, 0.0, r)
    return np.copysign(r, x)


def dequantize(values, scale=1.0):
    """x = x_q * scale in fp64 (per-tensor scale; 1 for unquantised inputs)."""
    return np.asarray(values, dtype=np.float64) * float(scale)


# --------------------------------------------------------------------------
# OAM scoring  [Stem-cn §一.3.2, §二.2.1]
# --------------------------------------------------------------------------

def pool_blocks(q, k, v, block):
    """Compact per-block representations (Stem-cn §二.2.1: Q and K are first
    reduced to block-level representations, then one GEMM scores all blocks).

    Returns
      qbar [b, Hq, Nb, d]   mean of the block's query rows
      kbar [b, Hkv, Nb, d]  mean of the block's key rows
      lvn  [b, Hkv, Nb]     ln of the Frobenius norm of the block's value rows
                            (the "value magnitude" of Stem-cn §一.3.2)
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b, S, Hq, d = q.shape
    Hkv = k.shape[2]
    nb = S // block
    qbar = q.reshape(b, nb, block, Hq, d).mean(axis=2).transpose(0, 2, 1, 3)
    kbar = k.reshape(b, nb, block, Hkv, d).mean(axis=2).transpose(0, 2, 1, 3)
    sq = (v.reshape(b, nb, block, Hkv, d) ** 2).sum(axis=(2, 4))      # [b, Nb, Hkv]
    with np.errstate(divide="ignore"):
        lvn = 0.5 * np.log(sq).transpose(0, 2, 1)
    return qbar, kbar, lvn


def oam_scores(q, k, v, block, softmax_scale=None):
    """Block scores s[b, h, I, J] = tau * <qbar_hI, kbar_gJ> + lvn_gJ for J <= I,
    -inf above the diagonal (no causal block there).  tau is the attention
    softmax scale (1/sqrt(d) unless given), g = h // (Hq/Hkv)."""
    qbar, kbar, lvn = pool_blocks(q, k, v, block)
    b, Hq, nb, d = qbar.shape
    Hkv = kbar.shape[1]
    group = Hq // Hkv
    tau = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    s = np.full((b, Hq, nb, nb), -np.inf)
    upper = np.triu(np.ones((nb, nb), dtype=bool), 1)
    for bi in range(b):
        for h in range(Hq):
            g = h // group
            row = tau * (qbar[bi, h] @ kbar[bi, g].T) + lvn[bi, g][None, :]
            row[upper] = -np.inf
            s[bi, h] = row
    return s


def sam_scores(q, k, block, softmax_scale=None):
    """Score-only block scores (SAM, the metric Stem-en's Deep Dive contrasts
    OAM with: attention scores alone, no value information):
    s[b, h, I, J] = tau * <qbar_hI, kbar_gJ> for J <= I, -inf above."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    b, S, Hq, d = q.shape
    Hkv = k.shape[2]
    nb = S // block
    qbar = q.reshape(b, nb, block, Hq, d).mean(axis=2)          # [b, Nb, Hq, d]
    kbar = k.reshape(b, nb, block, Hkv, d).mean(axis=2)         # [b, Nb, Hkv, d]
    group = Hq // Hkv
    tau = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    s = np.full((b, Hq, nb, nb), -np.inf)
    for bi in range(b):
        for h in range(Hq):
            logits = tau * (qbar[bi, :, h, :] @ kbar[bi, :, h // group, :].T)
            for i in range(nb):
                s[bi, h, i, :i + 1] = logits[i, :i + 1]
    return s


# --------------------------------------------------------------------------
# KV-cache write  [Stem-cn §二.2.1 compact block representations computed
# ahead of scoring; §二.2.2 FP8 paged KV]
# --------------------------------------------------------------------------

def quantize_e4m3(x, scale):
    """E4M3 value stored for x under a per-tensor scale: the single-precision
    quotient x / scale (IEEE division, the precision the write computes in),
    then the nearest E4M3 value, ties to even, saturating at +-448.  Returns
    the stored values (not multiplied back by the scale) in fp64."""
    quotient = np.asarray(x, dtype=np.float32) / np.float32(scale)
    return e4m3fn_round(quotient.astype(np.float64))


def cache_write(k, v, block, fp8=False, k_scale=1.0, v_scale=1.0):
    """What a prefill's cache write stores and the block representations of
    the stored values.  k, v: [b, S, Hkv, d].
    Returns (k_stored, v_stored, kbar, lvn): the stored element values
    (E4M3 values when fp8, else the inputs), and kbar [b, Hkv, Nb, d] / lvn
    [b, Hkv, Nb] of the dequantised stored values (as pool_blocks defines
    them)."""
    if fp8:
        ks = quantize_e4m3(k, k_scale)
        vs = quantize_e4m3(v, v_scale)
    else:
        ks = np.asarray(k, dtype=np.float64)
        vs = np.asarray(v, dtype=np.float64)
        k_scale = v_scale = 1.0
    kd, vd = dequantize(ks, k_scale), dequantize(vs, v_scale)
    b, S, Hkv, d = kd.shape
    nb = S // block
    kbar = kd.reshape(b, nb, block, Hkv, d).mean(axis=2).transpose(0, 2, 1, 3)
    sq = (vd.reshape(b, nb, block, Hkv, d) ** 2).sum(axis=(2, 4))
    with np.errstate(divide="ignore"):
        lvn = 0.5 * np.log(sq).transpose(0, 2, 1)
    return ks, vs, kbar, lvn


# --------------------------------------------------------------------------
# TPD budget  [Stem-cn §一.3.1; Stem-en Technical Deep Dive]
# --------------------------------------------------------------------------

def causal_block_count(nb):
    """Blocks on or below the diagonal: Nb (Nb + 1) / 2."""
    return nb * (nb + 1) // 2


def tpd_total(nb, density):
    """Total kept blocks per head: T = floor(density * C + 1/2) in fp64, with
    C the causal block count, clamped to [2 Nb - 1, C] (the forced sink and
    diagonal blocks always count; Stem-cn §一.3.1 fixes the total, TPD only
    moves it)."""
    if not (0.0 < density <= 1.0):
        raise ValueError("density must lie in (0, 1]")
    c = causal_block_count(nb)
    t = int(math.floor(density * c + 0.5))
    return max(2 * nb - 1, min(c, t))


def _tpd_key(alpha, i, n):
    """Water-filling key of granting row i its n-th block: n / (i+1)**(1-alpha).
    Compared exactly: for alpha = 0 the key is n/(i+1), for alpha = 1/2 its
    square n**2/(i+1) (same order), for alpha = 1 it is n."""
    if alpha == 0.0:
        return Fraction(n, i + 1)
    if alpha == 0.5:
        return Fraction(n * n, i + 1)
    if alpha == 1.0:
        return Fraction(n)
    raise ValueError("alpha must be 0, 0.5 or 1")


def tpd_budget(nb, density, alpha=0.5):
    """Per-query-block budget k[I] (kept KV blocks in row I) and the total T.

    The pages: a position-dependent top-k inside each layer that gives early
    positions a larger share, at the same total as a uniform budget
    (Stem-cn §一.3.1; Stem-en Deep Dive).  Reading: start every row at its
    forced minimum (k[0] = 1: sink and diagonal coincide; k[I] = 2 otherwise),
    then hand out the remaining T - sum(k) blocks one at a time, each to the
    row with the smallest key (k[I]+1) / (I+1)**(1-alpha) that still has room
    (k[I] < I+1), equal keys to the smaller I.  The keep ratio then decays as
    (I+1)**-alpha; alpha = 0 is the uniform ratio, alpha = 1 a uniform count.
    """
    t = tpd_total(nb, density)
    k = [1] + [2] * (nb - 1)
    if nb == 1:
        return [1], t
    heap = []
    for i in range(nb):
        if k[i] < i + 1:
            heap.append((_tpd_key(alpha, i, k[i] + 1), i))
    heapq.heapify(heap)
    remaining = t - sum(k)
    while remaining > 0:
        _, i = heapq.heappop(heap)
        k[i] += 1
        remaining -= 1
        if k[i] < i + 1:
            heapq.heappush(heap, (_tpd_key(alpha, i, k[i] + 1), i))
    return k, t


# --------------------------------------------------------------------------
# Top-k selection  [Stem-cn §一.3.1-§一.3.2, §二.2.1]
# --------------------------------------------------------------------------

def select_row(scores_row, i, budget):
    """Kept key blocks of query block i: {0, i} plus the best (budget - |{0,i}|)
    of J in [1, i-1] ranked by score descending, ties to the smaller J, NaN
    last.  Returns a sorted list of J."""
    forced = {0, i}
    need = budget - len(forced)
    cand = np.arange(1, i)
    if need > 0 and cand.size:
        vals = np.asarray(scores_row, dtype=np.float64)[cand]
        nan = np.isnan(vals)
        # primary: NaN last; secondary: score descending; tertiary: J ascending
        order = np.lexsort((cand, -np.where(nan, 0.0, vals), nan))
        forced.update(int(j) for j in cand[order[:need]])
    return sorted(forced)


def select_blocks(scores, budget):
    """Boolean block mask [b, Hq, Nb, Nb] from block scores and per-row budget."""
    scores = np.asarray(scores, dtype=np.float64)
    b, hq, nb, _ = scores.shape
    mask = np.zeros((b, hq, nb, nb), dtype=bool)
    for bi in range(b):
        for h in range(hq):
            for i in range(nb):
                mask[bi, h, i, select_row(scores[bi, h, i], i, budget[i])] = True
    return mask


def pack_block_mask(mask):
    """Bit J of 32-bit word J // 32 in row (b, h, I) is set when block J is
    kept; words [b, Hq, Nb, ceil(Nb/32)] little-endian bit order."""
    mask = np.asarray(mask, dtype=bool)
    b, hq, nb, _ = mask.shape
    words = (nb + 31) // 32
    out = np.zeros((b, hq, nb, words), dtype=np.uint32)
    for j in range(nb):
        out[..., j // 32] |= mask[..., j].astype(np.uint32) << np.uint32(j % 32)
    return out


def unpack_block_mask(words, nb):
    words = np.asarray(words, dtype=np.uint32)
    j = np.arange(nb)
    return ((words[..., j // 32] >> (j % 32).astype(np.uint32)) & 1).astype(bool)


# --------------------------------------------------------------------------
# Block-sparse attention  [Stem-cn §二.2.2]
# --------------------------------------------------------------------------

def _visible_keys(block_mask_row, i_blk, block):
    """Token indices of the kept blocks J <= I (bits above the diagonal are
    ignored: the attention is causal)."""
    js = [j for j in range(i_blk + 1) if block_mask_row[j]]
    if not js:
        return np.zeros(0, dtype=np.int64), False
    idx = np.concatenate([np.arange(j * block, (j + 1) * block) for j in js])
    return idx, (i_blk in js)


def _attend(qrows, pos, keys_idx, diag_kept, i_blk, block, k_h, v_h, tau):
    """Softmax attention of query rows at positions `pos` over the key tokens
    `keys_idx`; inside the diagonal block a key j is visible only if j <= i.
    A skipped key block contributes nothing, exactly as a -inf logit would
    (Stem-cn §二.2.2).  Rows with no visible key give O = 0, LSE = -inf."""
    if keys_idx.size == 0:
        return np.zeros((len(pos), v_h.shape[-1])), np.full(len(pos), -np.inf)
    logits = tau * (qrows @ k_h[keys_idx].T)                     # [rows, keys]
    if diag_kept:
        diag_start = i_blk * block
        in_diag = keys_idx >= diag_start
        future = in_diag[None, :] & (keys_idx[None, :] > pos[:, None])
        logits = np.where(future, -np.inf, logits)
    m = logits.max(axis=1)
    p = np.exp(logits - m[:, None])
    l_sum = p.sum(axis=1)
    o = (p @ v_h[keys_idx]) / l_sum[:, None]
    return o, m + np.log(l_sum)


def block_sparse_attention(q, k, v, block_mask, block, softmax_scale=None):
    """O[b, S, Hq, dv] and LSE[b, Hq, S] (natural log) of causal attention that
    only sees the kept key blocks of each query block (block_mask [b,Hq,Nb,Nb]
    bool).  V may be wider or narrower than Q and K (dv = v.shape[-1]): each
    output column is the softmax-weighted mean of that column of V."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b, S, Hq, d = q.shape
    Hkv = k.shape[2]
    group = Hq // Hkv
    nb = S // block
    tau = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    o = np.zeros((b, S, Hq, v.shape[-1]))
    lse = np.full((b, Hq, S), -np.inf)
    for bi in range(b):
        for h in range(Hq):
            g = h // group
            for i_blk in range(nb):
                keys_idx, diag = _visible_keys(block_mask[bi, h, i_blk], i_blk, block)
                pos = np.arange(i_blk * block, (i_blk + 1) * block)
                oo, ll = _attend(q[bi, pos, h], pos, keys_idx, diag, i_blk, block,
                                 k[bi, :, g], v[bi, :, g], tau)
                o[bi, pos, h] = oo
                lse[bi, h, pos] = ll
    return o, lse


def attention_rows(q, k, v, block_mask, block, rows, softmax_scale=None):
    """The same definition evaluated only at the (batch, head, token) triples
    in `rows`: for sampled checks at sizes where the full oracle is too slow.
    block_mask is None for dense causal attention, else a callable
    (b, h, I) -> bool row of length Nb or an array [b, Hq, Nb, Nb].  O has V's
    width."""
    S, Hq, d = q.shape[1], q.shape[2], q.shape[3]
    Hkv = k.shape[2]
    group = Hq // Hkv
    nb = S // block
    tau = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    out_o = np.zeros((len(rows), v.shape[-1]))
    out_l = np.zeros(len(rows))
    groups = {}                                   # rows of one query block share its keys
    for n, (bi, h, i) in enumerate(rows):
        groups.setdefault((bi, h, i // block), []).append(n)
    for (bi, h, i_blk), members in groups.items():
        if block_mask is None:
            mrow = np.ones(nb, dtype=bool)
        elif callable(block_mask):
            mrow = block_mask(bi, h, i_blk)
        else:
            mrow = block_mask[bi, h, i_blk]
        keys_idx, diag = _visible_keys(mrow, i_blk, block)
        g = h // group
        pos = np.array([rows[n][2] for n in members])
        qrows = np.asarray(q[bi, pos, h], dtype=np.float64)
        kk = np.asarray(k[bi, :, g], dtype=np.float64)
        vv = np.asarray(v[bi, :, g], dtype=np.float64)
        oo, ll = _attend(qrows, pos, keys_idx, diag, i_blk, block, kk, vv, tau)
        out_o[members] = oo
        out_l[members] = ll
    return out_o, out_l


# --------------------------------------------------------------------------
# Online skip inside the block loop  [BLASST §2.1]
# --------------------------------------------------------------------------

def _attend_blasst(qrows, pos, kept_blocks, i_blk, block, k_h, v_h, tau, lam):
    """One query block's rows under the online skip of the BLASST summary
    (§2.1, running-maximum pruning) applied on top of the block mask.

    The row's kept key blocks are visited in ascending J, as a blocked online
    softmax visits them, keeping the running maximum m of the logits taken in.
    For block J the local maximum mt over the keys the row can see is compared
    with m: if mt - m < ln(lam) the row drops the block (no exponentials, no
    sum, no product with V).  A dropped block lies below m, so it never moves
    m, and m before block J is the maximum over every earlier kept block; the
    first block (m = -inf) is never dropped, and lam = 0 drops nothing.
    Returns O, LSE (natural log) over the blocks not dropped, the number of
    blocks each row dropped, and each row's smallest |mt - m - ln(lam)| over
    its blocks (how close a decision came to the threshold)."""
    rows = len(pos)
    log_lam = math.log(lam) if lam > 0 else -math.inf
    m = np.full(rows, -np.inf)
    dropped = np.zeros(rows, dtype=np.int64)
    closest = np.full(rows, np.inf)
    keys_all, logits_all = [], []
    for J in kept_blocks:
        keys = np.arange(J * block, (J + 1) * block)
        lg = tau * (qrows @ k_h[keys].T)                         # [rows, block]
        if J == i_blk:                                           # causal inside the diagonal block
            lg = np.where(keys[None, :] > pos[:, None], -np.inf, lg)
        mt = lg.max(axis=1)
        gap = mt - m                                             # +inf before the first block
        drop = _blasst_drops(gap, log_lam)
        with np.errstate(invalid="ignore"):
            margin = np.abs(gap - log_lam)                       # inf when m or ln(lam) is -inf
        closest = np.minimum(closest, np.where(np.isnan(margin), np.inf, margin))
        dropped += drop
        m = np.where(drop, m, np.maximum(m, mt))
        keys_all.append(keys)
        logits_all.append(np.where(drop[:, None], -np.inf, lg))
    if not keys_all:
        return np.zeros((rows, v_h.shape[-1])), np.full(rows, -np.inf), dropped, closest
    keys_idx = np.concatenate(keys_all)
    logits = np.concatenate(logits_all, axis=1)
    top = logits.max(axis=1)
    p = np.exp(logits - top[:, None])
    l_sum = p.sum(axis=1)
    o = (p @ v_h[keys_idx]) / l_sum[:, None]
    return o, top + np.log(l_sum), dropped, closest


def _blasst_drops(gap, log_lam):
    """The skip test of BLASST §2.1: the block's local maximum lies more than
    ln(1/lam) below the running maximum."""
    return gap < log_lam


def _blasst_check(lam):
    lam = float(lam)
    if not (0.0 <= lam <= 1.0):
        raise ValueError("lam must lie in [0, 1]")
    return lam


def blasst_attention(q, k, v, block_mask, block, lam, softmax_scale=None):
    """Block-sparse causal attention with the BLASST online skip (see
    _attend_blasst) inside every row's loop over its kept blocks.
    block_mask [b, Hq, Nb, Nb] bool, or None for every causal block (the
    pages' setting: the skip inside dense attention).  Returns O [b, S, Hq, dv]
    (V's width), LSE [b, Hq, S], dropped [b, Hq, S] and closest [b, Hq, S]."""
    lam = _blasst_check(lam)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b, S, Hq, d = q.shape
    group = Hq // k.shape[2]
    nb = S // block
    tau = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    o = np.zeros((b, S, Hq, v.shape[-1]))
    lse = np.full((b, Hq, S), -np.inf)
    dropped = np.zeros((b, Hq, S), dtype=np.int64)
    closest = np.full((b, Hq, S), np.inf)
    for bi in range(b):
        for h in range(Hq):
            g = h // group
            for i_blk in range(nb):
                row = np.ones(nb, dtype=bool) if block_mask is None else block_mask[bi, h, i_blk]
                kept = [j for j in range(i_blk + 1) if row[j]]
                pos = np.arange(i_blk * block, (i_blk + 1) * block)
                oo, ll, dd, cc = _attend_blasst(q[bi, pos, h], pos, kept, i_blk, block,
                                                k[bi, :, g], v[bi, :, g], tau, lam)
                o[bi, pos, h] = oo
                lse[bi, h, pos] = ll
                dropped[bi, h, pos] = dd
                closest[bi, h, pos] = cc
    return o, lse, dropped, closest


def blasst_attention_rows(q, k, v, block_mask, block, lam, rows, softmax_scale=None):
    """blasst_attention evaluated only at the (batch, head, token) triples in
    `rows` (block_mask as for attention_rows).  Returns O [rows, dv] (V's
    width), LSE, dropped and closest [rows]."""
    lam = _blasst_check(lam)
    S, Hq, d = q.shape[1], q.shape[2], q.shape[3]
    group = Hq // k.shape[2]
    nb = S // block
    tau = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    out_o = np.zeros((len(rows), v.shape[-1]))
    out_l = np.zeros(len(rows))
    out_d = np.zeros(len(rows), dtype=np.int64)
    out_c = np.zeros(len(rows))
    groups = {}
    for n, (bi, h, i) in enumerate(rows):
        groups.setdefault((bi, h, i // block), []).append(n)
    for (bi, h, i_blk), members in groups.items():
        if block_mask is None:
            mrow = np.ones(nb, dtype=bool)
        elif callable(block_mask):
            mrow = block_mask(bi, h, i_blk)
        else:
            mrow = block_mask[bi, h, i_blk]
        kept = [j for j in range(i_blk + 1) if mrow[j]]
        g = h // group
        pos = np.array([rows[n][2] for n in members])
        oo, ll, dd, cc = _attend_blasst(np.asarray(q[bi, pos, h], dtype=np.float64), pos, kept, i_blk,
                                        block, np.asarray(k[bi, :, g], dtype=np.float64),
                                        np.asarray(v[bi, :, g], dtype=np.float64), tau, lam)
        out_o[members] = oo
        out_l[members] = ll
        out_d[members] = dd
        out_c[members] = cc
    return out_o, out_l, out_d, out_c


def _decode_kept(q, k, v, seq_lens, block, keep, tau, value_term):
    """The kept blocks of each new token's row (sorted), by the rule of
    decode_step."""
    b, Hq, d = q.shape
    group = Hq // k.shape[2]
    kept = []
    for bi in range(b):
        t = int(seq_lens[bi]) - 1
        I = t // block
        if I > 0 and keep is not None:
            done = slice(bi, bi + 1), slice(0, I * block)
            _, kbar, lvn = pool_blocks(k[done], k[done], v[done], block)
        kept_b = []
        for h in range(Hq):
            g = h // group
            if keep is None:
                row_kept = list(range(I + 1))
            else:
                forced = 1 if I == 0 else 2
                budget = min(max(int(keep[bi]), forced), I + 1)
                row = np.full(I + 1, -np.inf)
                if I > 1:
                    row[1:I] = tau * (kbar[0, g, 1:I] @ q[bi, h])
                    if value_term:
                        row[1:I] += lvn[0, g, 1:I]
                row_kept = select_row(row, I, budget)
            kept_b.append(list(row_kept))
        kept.append(kept_b)
    return kept


def decode_step(q, k, v, seq_lens, block, keep=None, softmax_scale=None, value_term=True):
    """One decode step with Stem block selection for the new token.

    q [b, Hq, d]: the new token of each sequence; k, v [b, S, Hkv, d]: the
    cache (dequantised), sequence b holding tokens 0 .. seq_lens[b]-1 with the
    new token last, at t = seq_lens[b] - 1 in block I = t // block.
    The token scores the complete blocks J in [1, I-1] as OAM does a query
    block (Stem-cn §一.3.2, the token standing for its block's mean), with the
    block representations of pool_blocks; keep[b] blocks are kept by the rule
    of select_row (sink and own block forced), keep clamped to
    [|{0, I}|, I + 1]; keep None keeps every block.  Attention then sees the
    keys j <= t of the kept blocks (as in _attend).
    Returns (o [b, Hq, d], lse [b, Hq], kept) with kept[b][h] the sorted
    kept blocks."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b, Hq, d = q.shape
    group = Hq // k.shape[2]
    tau = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    kept = _decode_kept(q, k, v, seq_lens, block, keep, tau, value_term)
    o = np.zeros((b, Hq, d))
    lse = np.zeros((b, Hq))
    for bi in range(b):
        t = int(seq_lens[bi]) - 1
        I = t // block
        for h in range(Hq):
            g = h // group
            mrow = np.zeros(I + 1, dtype=bool)
            mrow[kept[bi][h]] = True
            keys_idx, diag = _visible_keys(mrow, I, block)
            oo, ll = _attend(q[bi, h][None, :], np.array([t]), keys_idx, diag, I, block,
                             k[bi, :, g], v[bi, :, g], tau)
            o[bi, h] = oo[0]
            lse[bi, h] = ll[0]
    return o, lse, kept


def decode_step_blasst(q, k, v, seq_lens, block, lam, keep=None, softmax_scale=None, value_term=True):
    """decode_step with the online skip of BLASST §2.1 (see _attend_blasst)
    over the new token's kept blocks, in ascending J: a block whose largest
    logit over the keys j <= t lies more than ln(1/lam) below the largest of
    the earlier kept blocks is dropped.  (BLASST §2.3 names decode, where the
    skip saves the dropped blocks' V reads.)  Returns (o [b, Hq, d],
    lse [b, Hq], kept, dropped [b, Hq], closest [b, Hq])."""
    lam = _blasst_check(lam)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b, Hq, d = q.shape
    group = Hq // k.shape[2]
    tau = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    kept = _decode_kept(q, k, v, seq_lens, block, keep, tau, value_term)
    o = np.zeros((b, Hq, d))
    lse = np.zeros((b, Hq))
    dropped = np.zeros((b, Hq), dtype=np.int64)
    closest = np.zeros((b, Hq))
    for bi in range(b):
        t = int(seq_lens[bi]) - 1
        I = t // block
        for h in range(Hq):
            g = h // group
            oo, ll, dd, cc = _attend_blasst(q[bi, h][None, :], np.array([t]), kept[bi][h], I, block,
                                            k[bi, :, g], v[bi, :, g], tau, lam)
            o[bi, h], lse[bi, h], dropped[bi, h], closest[bi, h] = oo[0], ll[0], dd[0], cc[0]
    return o, lse, kept, dropped, closest


def dense_causal_attention(q, k, v, softmax_scale=None):
    """Plain causal softmax attention, row by row over all keys j <= i: the
    dense baseline (Stem-cn §二.3) and the density-1 limit of the sparse path."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b, S, Hq, d = q.shape
    group = Hq // k.shape[2]
    tau = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    o = np.zeros((b, S, Hq, d))
    lse = np.zeros((b, Hq, S))
    for bi in range(b):
        for h in range(Hq):
            g = h // group
            for i in range(S):
                logits = tau * (k[bi, : i + 1, g] @ q[bi, i, h])
                m = logits.max()
                p = np.exp(logits - m)
                o[bi, i, h] = p @ v[bi, : i + 1, g] / p.sum()
                lse[bi, h, i] = m + np.log(p.sum())
    return o, lse


# --------------------------------------------------------------------------
# The whole path
# --------------------------------------------------------------------------

def stem_pipeline(q, k, v, block, density, alpha=0.5, softmax_scale=None):
    """Score -> budget -> select -> block-sparse attention (Stem-cn §二.1: a
    scoring stage that records each block's importance, then a sparse stage
    that computes only the selected blocks).  Returns (scores, budget, mask,
    O, LSE)."""
    s = oam_scores(q, k, v, block, softmax_scale)
    nb = s.shape[2]
    budget, _ = tpd_budget(nb, density, alpha)
    mask = select_blocks(s, budget)
    o, lse = block_sparse_attention(q, k, v, mask, block, softmax_scale)
    return s, budget, mask, o, lse
