"""Pins of the fp64 oracle to things other than itself: hand-worked fixtures
(tests/golden), brute force on tiny inputs, closed forms, invariants and
textbook library routines (torch's scaled_dot_product_attention in fp64 on
the CPU, torch's float8_e4m3fn cast).  The last section plants mistakes in
copies of oracle functions and checks that these pins catch them.
CPU only."""

import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import stem as ostem


# --------------------------------------------------------------------------
# helpers
# --------------------------------------------------------------------------

def _rand_qkv(seed, b, S, hq, hkv, d, vscale=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((b, S, hq, d))
    k = rng.standard_normal((b, S, hkv, d))
    v = rng.standard_normal((b, S, hkv, d))
    if vscale:
        v *= np.exp(0.5 * rng.standard_normal((b, S)))[:, :, None, None]
    return q, k, v


def _num(tok):
    tok = tok.strip()
    if tok == "-inf":
        return -math.inf
    if tok == "nan":
        return math.nan
    if "+" in tok and "ln" in tok:                     # "a+lnb"
        a, l = tok.split("+")
        return float(a) + math.log(float(l[2:]))
    if tok.startswith("ln"):
        return math.log(float(tok[2:]))
    if "/" in tok:
        return float(Fraction(tok))
    return float(tok)


def _lines(path):
    with open(path) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


# --------------------------------------------------------------------------
# OAM scoring
# --------------------------------------------------------------------------

def test_oam_golden(golden_dir):
    kv = {}
    for ln in _lines(os.path.join(golden_dir, "oam_worked.txt")):
        key, *vals = ln.split()
        kv[key] = vals
    tau = float(kv["tau"][0])
    B = int(kv["block"][0])
    q = np.array([float(x) for x in kv["q"]]).reshape(1, 4, 1, 2)
    k = np.array([float(x) for x in kv["k"]]).reshape(1, 4, 1, 2)
    v = np.array([float(x) for x in kv["v"]]).reshape(1, 4, 1, 2)
    s = oracle.oam_scores(q, k, v, B, softmax_scale=tau)
    for name in ("s00", "s10", "s11", "s01"):
        i, j = int(name[1]), int(name[2])
        want = _num(kv[name][0])
        if math.isinf(want):
            assert s[0, 0, i, j] == want
        else:
            assert abs(s[0, 0, i, j] - want) < 1e-14


def _oam_bruteforce(q, k, v, B, tau):
    """Full token-level logits, averaged over each B x B tile (the 'sampled
    full matmul then block reduction' form the Stem article's §二.2.1 replaces),
    plus the log Frobenius norm of each V block from numpy.linalg.norm."""
    b, S, hq, d = q.shape
    hkv = k.shape[2]
    G = hq // hkv
    nb = S // B
    out = np.full((b, hq, nb, nb), -np.inf)
    for bi in range(b):
        for h in range(hq):
            g = h // G
            L = tau * q[bi, :, h] @ k[bi, :, g].T                       # [S, S]
            for I in range(nb):
                for J in range(I + 1):
                    tile = L[I * B:(I + 1) * B, J * B:(J + 1) * B]
                    vn = np.linalg.norm(v[bi, J * B:(J + 1) * B, g], "fro")
                    out[bi, h, I, J] = tile.mean() + math.log(vn)
    return out


@pytest.mark.parametrize("shape", [(1, 64, 2, 2, 8, 16), (2, 96, 4, 2, 16, 32),
                                   (1, 128, 6, 3, 32, 16), (1, 48, 1, 1, 4, 8)])
def test_oam_equals_pairwise_block_mean(shape):
    b, S, hq, hkv, d, B = shape
    q, k, v = _rand_qkv(11, b, S, hq, hkv, d)
    tau = 1 / math.sqrt(d)
    got = oracle.oam_scores(q, k, v, B)
    want = _oam_bruteforce(q, k, v, B, tau)
    fin = np.isfinite(want)
    assert np.array_equal(fin, np.isfinite(got))
    assert np.max(np.abs(got[fin] - want[fin])) < 1e-12


def test_v_block_scaling_shifts_column_by_log():
    q, k, v = _rand_qkv(3, 1, 64, 2, 1, 8)
    B, J, c = 16, 2, 3.7
    s0 = oracle.oam_scores(q, k, v, B)
    v2 = v.copy()
    v2[:, J * B:(J + 1) * B] *= c
    s1 = oracle.oam_scores(q, k, v2, B)
    with np.errstate(invalid="ignore"):          # -inf - -inf above the diagonal
        diff = s1 - s0
    for I in range(4):
        for JJ in range(I + 1):
            want = math.log(c) if JJ == J else 0.0
            assert abs(diff[0, 0, I, JJ] - want) < 1e-12


def test_constant_v_rows_closed_form():
    B, d = 8, 4
    q, k, _ = _rand_qkv(5, 1, 32, 1, 1, d)
    row = np.array([1.0, -2.0, 2.0, 4.0])          # |row| = 5
    v = np.broadcast_to(row, (1, 32, 1, d)).copy()
    _, _, lvn = oracle.pool_blocks(q, k, v, B)
    assert np.allclose(lvn, math.log(math.sqrt(B) * 5.0), atol=1e-14)


def test_equal_value_norms_reduce_to_score_only_ranking():
    """With every V block of equal norm the V term is a constant and OAM ranks
    exactly like the score-aware metric (tau * qbar . kbar)."""
    q, k, _ = _rand_qkv(7, 1, 128, 2, 2, 8)
    v = np.ones((1, 128, 2, 8))
    B = 16
    s = oracle.oam_scores(q, k, v, B)
    qbar, kbar, _ = oracle.pool_blocks(q, k, v, B)
    for h in range(2):
        sam = qbar[0, h] @ kbar[0, h].T
        for I in range(8):
            a = np.argsort(-s[0, h, I, :I + 1], kind="stable")
            bb = np.argsort(-sam[I, :I + 1], kind="stable")
            assert list(a) == list(bb)


def test_zero_v_block_scores_minus_inf():
    q, k, v = _rand_qkv(9, 1, 32, 1, 1, 4)
    v[:, 8:16] = 0.0
    s = oracle.oam_scores(q, k, v, 8)
    assert np.all(s[0, 0, 1:, 1] == -np.inf)
    assert np.all(np.isfinite(s[0, 0, 1:, 0]))


def _sam_bruteforce(q, k, B, tau):
    """Full token-level logits averaged over each B x B tile, with no value
    information (the score-only metric of the Stem-en Deep Dive)."""
    b, S, hq, d = q.shape
    G = hq // k.shape[2]
    nb = S // B
    out = np.full((b, hq, nb, nb), -np.inf)
    for bi in range(b):
        for h in range(hq):
            L = tau * q[bi, :, h] @ k[bi, :, h // G].T
            for I in range(nb):
                for J in range(I + 1):
                    out[bi, h, I, J] = L[I * B:(I + 1) * B, J * B:(J + 1) * B].mean()
    return out


@pytest.mark.parametrize("shape", [(1, 64, 2, 2, 8, 16), (2, 96, 4, 2, 16, 32), (1, 48, 3, 1, 4, 8)])
def test_sam_equals_pairwise_block_mean(shape):
    b, S, hq, hkv, d, B = shape
    q, k, _ = _rand_qkv(13, b, S, hq, hkv, d)
    got = oracle.sam_scores(q, k, B)
    want = _sam_bruteforce(q, k, B, 1 / math.sqrt(d))
    fin = np.isfinite(want)
    assert np.array_equal(fin, np.isfinite(got))
    assert np.max(np.abs(got[fin] - want[fin])) < 1e-12


def test_sam_is_oam_with_equal_value_norms():
    """Every V row of norm 5: the V term of every block is ln(sqrt(B) * 5), so
    OAM exceeds SAM by exactly that constant on and below the diagonal."""
    B, d = 8, 4
    q, k, _ = _rand_qkv(15, 1, 64, 2, 1, d)
    rng = np.random.default_rng(1)
    v = np.zeros((1, 64, 1, d))
    v[..., 0] = 3.0
    v[..., 1] = 4.0 * np.sign(rng.standard_normal((1, 64, 1)))   # |row| = 5
    oam = oracle.oam_scores(q, k, v, B)
    sam = oracle.sam_scores(q, k, B)
    low = np.tril(np.ones((8, 8), dtype=bool))
    assert np.all(sam[..., ~low] == -np.inf)
    assert np.allclose(oam[..., low] - sam[..., low], math.log(math.sqrt(B) * 5.0), atol=1e-12)


# --------------------------------------------------------------------------
# KV-cache write
# --------------------------------------------------------------------------

def test_quantize_e4m3_closed_forms():
    # exact quotients: the rounding cases of E4M3 itself, after the division
    cases = [(2.125, 2.0, 1.0), (2.375, 2.0, 1.25), (896.0, 2.0, 448.0), (1e30, 1.0, 448.0),
             (-1e30, 1.0, -448.0), (3.0 * 2.0 ** -12, 0.25, 2.0 ** -8), (2.0 ** -11, 0.5, 0.0),
             (0.0, 3.0, 0.0), (7.5, 0.5, 15.0)]
    for x, scale, want in cases:
        assert float(oracle.quantize_e4m3(x, scale)) == want, (x, scale)


def test_quantize_e4m3_decides_on_the_single_precision_quotient():
    """x / scale is formed in fp32, as torch's CPU float32 division forms it,
    then cast by torch to float8_e4m3fn: both steps are library routines."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-12, 6, 20000))).astype(np.float32)
    for scale in (0.0123, 1.0, 3.7, 2.0 ** -5):
        xs = torch.from_numpy(x) / torch.tensor(scale, dtype=torch.float32)
        keep = (xs.abs() <= 448.0).numpy()
        want = xs[torch.from_numpy(keep)].to(torch.float8_e4m3fn).double().numpy()
        got = oracle.quantize_e4m3(x[keep], scale)
        assert np.array_equal(got, want), scale


def test_cache_write_constant_rows():
    """Constant rows: the stored value is the rounded quotient, kbar its
    dequantised value, lvn = ln(sqrt(B * d) * |value|)."""
    B, d, S = 16, 8, 64
    k = np.full((1, S, 2, d), 0.7)
    v = np.full((1, S, 2, d), -1.3)
    ks, vs, kbar, lvn = oracle.cache_write(k, v, B, fp8=True, k_scale=0.01, v_scale=0.5)
    # 0.7 / 0.01 is about 70, between the E4M3 values 64 and 72 (spacing 8 in
    # [64, 128)): stored 72.  -1.3 / 0.5 = -2.6, between -2.5 and -2.75: -2.5.
    assert np.all(ks == 72.0) and np.all(vs == -2.5)
    assert np.allclose(kbar, 72.0 * 0.01, rtol=0, atol=1e-15)
    assert np.allclose(lvn, math.log(math.sqrt(B * d) * 1.25), atol=1e-12)
    ks2, vs2, kbar2, lvn2 = oracle.cache_write(k, v, B)
    assert np.all(ks2 == 0.7) and np.allclose(kbar2, 0.7, rtol=0, atol=1e-15)
    assert np.allclose(lvn2, math.log(math.sqrt(B * d) * 1.3), atol=1e-12)


def test_cache_write_saturates_and_pools_per_block():
    B, d = 4, 2
    k = np.zeros((1, 8, 1, d))
    k[0, :4] = 1000.0            # saturates at 448 (scale 1)
    k[0, 4:] = [[[1.0, -2.0]], [[3.0, 0.5]], [[-1.0, 2.0]], [[1.0, 0.5]]]
    v = np.ones((1, 8, 1, d))
    ks, _, kbar, lvn = oracle.cache_write(k, v, B, fp8=True)
    assert np.all(ks[0, :4] == 448.0)
    assert np.array_equal(kbar[0, 0, 0], [448.0, 448.0])
    assert np.array_equal(kbar[0, 0, 1], [1.0, 0.25])
    assert np.allclose(lvn[0, 0], math.log(math.sqrt(B * d)), atol=1e-15)


# --------------------------------------------------------------------------
# TPD budget
# --------------------------------------------------------------------------

def test_tpd_golden(golden_dir):
    for ln in _lines(os.path.join(golden_dir, "tpd_budget.txt")):
        head, total, ks = [p.strip() for p in ln.split("|")]
        nb, dens, alpha = head.split()
        k, t = oracle.tpd_budget(int(nb), float(dens), float(alpha))
        assert t == int(total)
        assert k == [int(x) for x in ks.split()]


def _tpd_bruteforce(nb, density, alpha):
    """Enumerate every grant (I, n) beyond the forced minimum, sort them by
    (n / (I+1)^(1-alpha), I) as exact rationals, take the first T - sum(min)."""
    c = nb * (nb + 1) // 2
    t = max(2 * nb - 1, min(c, int(math.floor(density * c + 0.5))))
    mins = [1] + [2] * (nb - 1)
    units = []
    for i in range(nb):
        for n in range(mins[i] + 1, i + 2):
            if alpha == 0.0:
                key = Fraction(n, i + 1)
            elif alpha == 0.5:
                key = Fraction(n * n, i + 1)          # square of n/sqrt(i+1): same order
            else:
                key = Fraction(n)
            units.append((key, i))
    units.sort()
    k = list(mins)
    for _, i in units[: t - sum(mins)]:
        k[i] += 1
    return k, t


@pytest.mark.parametrize("alpha", [0.0, 0.5, 1.0])
def test_tpd_equals_bruteforce(alpha):
    for nb in list(range(1, 20)) + [31, 32, 33, 64]:
        for dens in (0.05, 0.1, 0.2, 0.25, 0.3, 0.5, 0.75, 0.9, 1.0):
            assert oracle.tpd_budget(nb, dens, alpha) == _tpd_bruteforce(nb, dens, alpha)


@pytest.mark.parametrize("nb,dens", [(32, .25), (64, .25), (512, .2), (512, .5), (512, .8),
                                     (1024, .25), (200, .33)])
def test_tpd_invariants_and_waterfill(nb, dens):
    alpha = 0.5
    k, t = oracle.tpd_budget(nb, dens, alpha)
    c = nb * (nb + 1) // 2
    assert t == max(2 * nb - 1, min(c, int(math.floor(dens * c + 0.5))))
    assert sum(k) == t
    assert k[0] == 1
    assert all(2 <= k[i] <= i + 1 for i in range(1, nb))
    # water-filling: a single threshold separates granted from refused blocks
    granted = [k[i] / math.sqrt(i + 1) for i in range(nb) if k[i] > (1 if i == 0 else 2)]
    refused = [(k[i] + 1) / math.sqrt(i + 1) for i in range(nb) if k[i] < i + 1]
    if granted and refused:
        assert max(granted) <= min(refused) + 1e-12
    # keep ratio never increases with position among unclamped rows (decay)
    ratios = [k[i] / (i + 1) for i in range(2, nb)]
    assert ratios[-1] <= ratios[0]


def test_tpd_uniform_ratio_at_alpha_zero():
    nb, dens = 256, 0.3
    k, _ = oracle.tpd_budget(nb, dens, 0.0)
    free = [i for i in range(2, nb) if 2 < k[i] < i + 1]
    theta = sum(k[i] for i in free) / sum(i + 1 for i in free)
    for i in free:
        assert abs(k[i] - theta * (i + 1)) <= 1.0 + 1e-9


def test_tpd_density_one_is_dense():
    for nb in (1, 2, 7, 64):
        k, t = oracle.tpd_budget(nb, 1.0)
        assert k == [i + 1 for i in range(nb)]
        assert t == nb * (nb + 1) // 2


def test_tpd_headline_shape():
    """128K tokens in 128-token blocks at density 1/4: T = 131200 and the
    first 36 rows are dense (closed form: for alpha=1/2 a row is dense while
    (I+2)/sqrt(I+1) stays below the final threshold)."""
    k, t = oracle.tpd_budget(1024, 0.25)
    assert t == 131200
    assert k[:36] == list(range(1, 37)) and k[36] < 37
    assert max(k) == k[-1]


def test_tpd_rejects_bad_args():
    with pytest.raises(ValueError):
        oracle.tpd_budget(8, 0.0)
    with pytest.raises(ValueError):
        oracle.tpd_budget(8, 1.5)
    with pytest.raises(ValueError):
        oracle.tpd_budget(8, 0.5, 0.3)


# --------------------------------------------------------------------------
# Selection
# --------------------------------------------------------------------------

def test_select_golden(golden_dir):
    for ln in _lines(os.path.join(golden_dir, "select_worked.txt")):
        head, sc, kept = [p.strip() for p in ln.split("|")]
        i, budget = (int(x) for x in head.split())
        scores = np.array([_num(x) for x in sc.split()])
        assert oracle.select_row(scores, i, budget) == [int(x) for x in kept.split()]


def _select_bruteforce_row(scores, i, budget):
    cands = list(range(1, i))

    def key(j):
        s = scores[j]
        return (1 if math.isnan(s) else 0, -s if not math.isnan(s) else 0.0, j)
    cands.sort(key=key)
    keep = {0, i}
    keep.update(cands[: budget - len(keep)])
    return sorted(keep)


def test_select_equals_bruteforce_and_invariants():
    rng = np.random.default_rng(2)
    nb = 40
    # coarse values so that ties are frequent
    scores = np.round(rng.standard_normal((1, 3, nb, nb)), 1)
    scores[0, 1, :, 5] = np.nan
    budget, t = oracle.tpd_budget(nb, 0.3)
    mask = oracle.select_blocks(scores, budget)
    for h in range(3):
        assert mask[0, h].sum() == t
        for i in range(nb):
            row = np.nonzero(mask[0, h, i])[0].tolist()
            assert row == _select_bruteforce_row(scores[0, h, i], i, budget[i])
            assert len(row) == budget[i]
            assert mask[0, h, i, 0] and mask[0, h, i, i]
            assert not mask[0, h, i, i + 1:].any()


def test_pack_mask_bit_order():
    m = np.zeros((1, 1, 40, 40), dtype=bool)
    m[0, 0, 39, [0, 1, 31, 32, 39]] = True
    w = oracle.pack_block_mask(m)
    assert w.shape == (1, 1, 40, 2)
    assert w[0, 0, 39, 0] == (1 | 2 | (1 << 31))
    assert w[0, 0, 39, 1] == (1 | (1 << 7))
    assert np.array_equal(oracle.unpack_block_mask(w, 40), m)


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------

def test_attention_golden(golden_dir):
    q = np.ones((1, 4, 1, 1))
    k = np.log(np.arange(1, 5, dtype=np.float64)).reshape(1, 4, 1, 1)
    v = np.arange(1, 5, dtype=np.float64).reshape(1, 4, 1, 1)
    for ln in _lines(os.path.join(golden_dir, "attention_worked.txt")):
        name, mrows, os_, ls_ = [p.strip() for p in ln.split("|")]
        rows = [[int(x) for x in r.split()] for r in mrows.split(";")]
        mask = np.array(rows, dtype=bool).reshape(1, 1, 2, 2)
        o, lse = oracle.block_sparse_attention(q, k, v, mask, 2, softmax_scale=1.0)
        want_o = [_num(x) for x in os_.split()]
        want_l = [_num(x) for x in ls_.split()]
        assert np.allclose(o[0, :, 0, 0], want_o, atol=1e-14), name
        for got, want in zip(lse[0, 0], want_l):
            assert (got == want) if math.isinf(want) else abs(got - want) < 1e-14, name


def _sdpa(q, k, v, attn_mask=None, causal=False):
    """torch's textbook attention in fp64 on the CPU; GQA by repeating KV heads."""
    G = q.shape[2] // k.shape[2]
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    vt = torch.from_numpy(v).repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=attn_mask, is_causal=causal)
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("shape", [(1, 64, 2, 2, 8, 16), (2, 96, 4, 2, 16, 32), (1, 128, 3, 1, 32, 64)])
def test_density_one_equals_dense_and_sdpa(shape):
    b, S, hq, hkv, d, B = shape
    q, k, v = _rand_qkv(21, b, S, hq, hkv, d)
    nb = S // B
    full = np.broadcast_to(np.tril(np.ones((nb, nb), dtype=bool)), (b, hq, nb, nb))
    o1, l1 = oracle.block_sparse_attention(q, k, v, full, B)
    o2, l2 = oracle.dense_causal_attention(q, k, v)
    o3 = _sdpa(q, k, v, causal=True)
    assert np.max(np.abs(o1 - o2)) < 1e-12
    assert np.max(np.abs(l1 - l2)) < 1e-12
    assert np.max(np.abs(o1 - o3)) < 1e-12
    # the same through the whole pipeline at density 1
    _, budget, mask, o4, _ = oracle.stem_pipeline(q, k, v, B, 1.0)
    assert mask.sum() == b * hq * nb * (nb + 1) // 2
    assert np.max(np.abs(o4 - o2)) < 1e-12


def _additive_mask(block_mask, S, B):
    """-inf on every skipped B x B tile and above the diagonal, 0 elsewhere."""
    b, hq, nb, _ = block_mask.shape
    tok = np.repeat(np.repeat(block_mask, B, axis=2), B, axis=3)          # [b,hq,S,S]
    causal = np.tril(np.ones((S, S), dtype=bool))
    allowed = tok & causal
    return np.where(allowed, 0.0, -np.inf), allowed


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_skipped_block_equals_minus_inf_logits(seed):
    b, S, hq, hkv, d, B = 1, 128, 4, 2, 16, 16
    q, k, v = _rand_qkv(seed, b, S, hq, hkv, d)
    nb = S // B
    rng = np.random.default_rng(seed + 100)
    bm = rng.random((b, hq, nb, nb)) < 0.4
    idx = np.arange(nb)
    bm[..., idx, idx] = True                                    # keep rows non-empty
    o, lse = oracle.block_sparse_attention(q, k, v, bm, B)
    add, allowed = _additive_mask(bm, S, B)
    o_ref = _sdpa(q, k, v, attn_mask=torch.from_numpy(add))
    assert np.max(np.abs(o - o_ref)) < 1e-12
    # LSE is the log-sum-exp of the visible logits
    G = hq // hkv
    for h in range(hq):
        L = q[0, :, h] @ k[0, :, h // G].T / math.sqrt(d)
        L = np.where(allowed[0, h], L, -np.inf)
        want = torch.logsumexp(torch.from_numpy(L), dim=1).numpy()
        assert np.max(np.abs(lse[0, h] - want)) < 1e-12
    # every output row is a convex combination of V rows
    assert np.all(np.abs(o) <= np.abs(v).max() + 1e-12)


def test_empty_row_gives_zero_and_minus_inf():
    q, k, v = _rand_qkv(4, 1, 32, 1, 1, 4)
    bm = np.tril(np.ones((1, 1, 4, 4), dtype=bool))
    bm[0, 0, 2] = False
    o, lse = oracle.block_sparse_attention(q, k, v, bm, 8)
    assert np.all(o[0, 16:24] == 0) and np.all(lse[0, 0, 16:24] == -np.inf)
    assert np.all(np.isfinite(lse[0, 0, :16]))


def test_blocks_above_diagonal_are_ignored():
    q, k, v = _rand_qkv(6, 1, 64, 2, 1, 8)
    nb, B = 4, 16
    low = np.tril(np.ones((1, 2, nb, nb), dtype=bool))
    o1, l1 = oracle.block_sparse_attention(q, k, v, low, B)
    o2, l2 = oracle.block_sparse_attention(q, k, v, np.ones_like(low), B)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_attention_rows_matches_full():
    b, S, hq, hkv, d, B = 2, 96, 4, 2, 8, 16
    q, k, v = _rand_qkv(8, b, S, hq, hkv, d)
    nb = S // B
    rng = np.random.default_rng(8)
    bm = rng.random((b, hq, nb, nb)) < 0.5
    o, lse = oracle.block_sparse_attention(q, k, v, bm, B)
    rows = [(0, 0, 0), (1, 3, 95), (0, 2, 40), (1, 1, 17), (0, 3, 63)]
    orow, lrow = oracle.attention_rows(q, k, v, bm, B, rows)
    for n, (bi, h, i) in enumerate(rows):
        assert np.max(np.abs(orow[n] - o[bi, i, h])) < 1e-13
        assert (lrow[n] == lse[bi, h, i]) or abs(lrow[n] - lse[bi, h, i]) < 1e-13
    od, ld = oracle.attention_rows(q, k, v, None, B, rows)
    o2, l2 = oracle.dense_causal_attention(q, k, v)
    for n, (bi, h, i) in enumerate(rows):
        assert np.max(np.abs(od[n] - o2[bi, i, h])) < 1e-13


def test_value_width_is_free_and_weights_sum_to_one():
    """The attention output has V's width, column by column: with V widened
    by an all-ones column, that column is exactly the sum of the softmax
    weights, 1 (0 on a row that sees no key), and the other columns equal the
    output for V alone.  Holds for the full and the row-sampled oracle, with
    and without the online skip."""
    b, S, hq, hkv, d, B = 1, 96, 4, 2, 8, 16
    q, k, v = _rand_qkv(12, b, S, hq, hkv, d)
    k[:, :2] *= 3.0
    nb = S // B
    rng = np.random.default_rng(12)
    bm = rng.random((b, hq, nb, nb)) < 0.6
    bm[0, 1, 3] = False                                   # query block 3 of head 1 sees nothing
    v1 = np.concatenate([v, np.ones(v.shape[:-1] + (1,))], axis=-1)
    rows = [(0, 0, 0), (0, 3, 95), (0, 1, 50), (0, 2, 63), (0, 1, 3 * B + 5)]
    for lam in (None, 0.1):
        if lam is None:
            o, lse = oracle.block_sparse_attention(q, k, v, bm, B)
            o1, _ = oracle.block_sparse_attention(q, k, v1, bm, B)
            r, rl = oracle.attention_rows(q, k, v, bm, B, rows)
            r1, _ = oracle.attention_rows(q, k, v1, bm, B, rows)
        else:
            o, lse = oracle.blasst_attention(q, k, v, bm, B, lam)[:2]
            o1 = oracle.blasst_attention(q, k, v1, bm, B, lam)[0]
            r, rl = oracle.blasst_attention_rows(q, k, v, bm, B, lam, rows)[:2]
            r1 = oracle.blasst_attention_rows(q, k, v1, bm, B, lam, rows)[0]
        assert o1.shape == (b, S, hq, d + 1) and r1.shape == (len(rows), d + 1)
        assert np.array_equal(o1[..., :d], o) and np.array_equal(r1[:, :d], r)
        empty = np.isneginf(lse).transpose(0, 2, 1)            # [b, S, Hq]: rows that see no key
        assert empty[0, 3 * B:4 * B, 1].all() and not empty.all()
        assert np.all(o1[..., d][empty] == 0.0)
        assert np.max(np.abs(o1[..., d][~empty] - 1.0)) < 1e-14
        r_empty = np.isneginf(rl)
        assert r_empty[-1] and not r_empty.all()
        assert np.all(r1[r_empty, d] == 0.0)
        assert np.max(np.abs(r1[~r_empty, d] - 1.0)) < 1e-14


# --------------------------------------------------------------------------
# Decode
# --------------------------------------------------------------------------

def test_dense_decode_equals_sdpa_and_ignores_tokens_past_the_end():
    rng = np.random.default_rng(21)
    b, S, hq, hkv, d, B = 2, 96, 4, 2, 16, 16
    q = rng.standard_normal((b, hq, d))
    k = rng.standard_normal((b, S, hkv, d))
    v = rng.standard_normal((b, S, hkv, d))
    lens = [37, 96]
    k2, v2 = k.copy(), v.copy()
    k2[0, 37:] = 1e6                               # past the end of sequence 0
    v2[0, 37:] = -1e6
    o, lse, kept = oracle.decode_step(q, k2, v2, lens, B)
    tau = 1 / math.sqrt(d)
    for bi in range(b):
        n = lens[bi]
        assert kept[bi][0] == list(range((n - 1) // B + 1))
        for h in range(hq):
            g = h // (hq // hkv)
            qt = torch.from_numpy(q[bi, h]).view(1, 1, 1, d)
            kt = torch.from_numpy(k[bi, :n, g]).view(1, 1, n, d)
            vt = torch.from_numpy(v[bi, :n, g]).view(1, 1, n, d)
            want = F.scaled_dot_product_attention(qt, kt, vt, scale=tau).view(d).numpy()
            assert np.max(np.abs(o[bi, h] - want)) < 1e-12
            want_lse = torch.logsumexp(tau * (kt.view(n, d) @ qt.view(d)), 0).item()
            assert abs(lse[bi, h] - want_lse) < 1e-12


@pytest.mark.parametrize("t,keep", [(16 * 5 + 3, 3), (16 * 6 - 1, 4), (16 * 7, 2), (16 * 6 + 8, 7), (5, 3)])
def test_decode_equals_prefill_row_of_a_constant_query_block(t, keep):
    """A query block made of B copies of the new token has the token as its
    mean, so the prefill path (OAM scores, select_row, block-sparse attention)
    must keep the same blocks for that row and give the same output at t."""
    rng = np.random.default_rng(t)
    b, hq, hkv, d, B = 1, 4, 2, 8, 16
    I = t // B
    S = (I + 1) * B
    k = rng.standard_normal((b, S, hkv, d))
    v = rng.standard_normal((b, S, hkv, d)) * np.exp(rng.standard_normal((b, S, 1, 1)))
    q_full = rng.standard_normal((b, S, hq, d))
    qt = rng.standard_normal((b, hq, d))
    q_full[0, I * B:(I + 1) * B] = qt[0]
    o, lse, kept = oracle.decode_step(qt, k, v, [t + 1], B, keep=[keep])
    s = oracle.oam_scores(q_full, k, v, B)
    budget = [1] + [2] * I
    budget[I] = min(max(keep, 1 if I == 0 else 2), I + 1)
    mask = oracle.select_blocks(s, budget)
    o_p, lse_p = oracle.block_sparse_attention(q_full, k, v, mask, B)
    for h in range(hq):
        assert kept[0][h] == list(np.nonzero(mask[0, h, I])[0])
        assert np.max(np.abs(o[0, h] - o_p[0, t, h])) < 1e-12
        assert abs(lse[0, h] - lse_p[0, h, t]) < 1e-12


@pytest.mark.parametrize("t,keep,lam", [(16 * 5 + 3, 3, 0.05), (16 * 6 - 1, 4, 0.5), (16 * 7, None, 0.3),
                                        (16 * 6 + 8, 7, 1.0), (5, 3, 0.5), (16 * 8 - 1, None, 1e-3)])
def test_decode_blasst_equals_prefill_row_of_a_constant_query_block(t, keep, lam):
    """As for decode_step: a query block of copies of the new token makes the
    prefill row at t keep the same blocks, and the online skip then drops the
    same blocks there (it depends only on that row's logits)."""
    rng = np.random.default_rng(t + 100)
    b, hq, hkv, d, B = 1, 4, 2, 8, 16
    I = t // B
    S = (I + 1) * B
    k = rng.standard_normal((b, S, hkv, d))
    k[:, :2] *= 3.0
    v = rng.standard_normal((b, S, hkv, d)) * np.exp(rng.standard_normal((b, S, 1, 1)))
    q_full = rng.standard_normal((b, S, hq, d))
    qt = rng.standard_normal((b, hq, d))
    q_full[0, I * B:(I + 1) * B] = qt[0]
    o, lse, kept, dropped, _ = oracle.decode_step_blasst(qt, k, v, [t + 1], B, lam,
                                                         keep=None if keep is None else [keep])
    nb = I + 1
    if keep is None:
        mask = np.tril(np.ones((b, hq, nb, nb), dtype=bool))
    else:
        s = oracle.oam_scores(q_full, k, v, B)
        budget = [1] + [2] * I
        budget[I] = min(max(keep, 1 if I == 0 else 2), I + 1)
        mask = oracle.select_blocks(s, budget)
    o_p, lse_p, d_p, _ = oracle.blasst_attention(q_full, k, v, mask, B, lam)
    for h in range(hq):
        assert kept[0][h] == list(np.nonzero(mask[0, h, I])[0])
        assert dropped[0, h] == d_p[0, h, t]
        assert np.max(np.abs(o[0, h] - o_p[0, t, h])) < 1e-12
        assert abs(lse[0, h] - lse_p[0, h, t]) < 1e-12


def test_decode_blasst_lambda_zero_is_decode_step():
    rng = np.random.default_rng(9)
    b, hq, hkv, d, B, S = 2, 4, 2, 8, 16, 16 * 9
    k = rng.standard_normal((b, S, hkv, d))
    v = rng.standard_normal((b, S, hkv, d))
    qt = rng.standard_normal((b, hq, d))
    lens = [S, 16 * 5 + 7]
    o, lse, kept = oracle.decode_step(qt, k, v, lens, B, keep=[4, 3])
    o2, lse2, kept2, dropped, _ = oracle.decode_step_blasst(qt, k, v, lens, B, 0.0, keep=[4, 3])
    assert kept == kept2 and not dropped.any()
    assert np.max(np.abs(o - o2)) < 1e-12 and np.max(np.abs(lse - lse2)) < 1e-12


# --------------------------------------------------------------------------
# FP8 E4M3 rounding
# --------------------------------------------------------------------------

def test_e4m3_closed_form_values():
    cases = {448.0: 448.0, 460.0: 448.0, 1e6: 448.0, 2.0 ** -9: 2.0 ** -9,
             2.0 ** -10: 0.0,                 # half of the smallest subnormal ties to even (0)
             3 * 2.0 ** -10: 2.0 ** -8,       # 1.5 subnormal quanta ties to even (2)
             1.0625: 1.0,                     # halfway between 1 and 1.125 -> even mantissa
             1.1875: 1.25, 240.0: 240.0, 248.0: 256.0, -0.3: -0.3125, 0.0: 0.0}
    for x, want in cases.items():
        assert float(oracle.e4m3fn_round(x)) == want, x


def test_e4m3_matches_torch_cast_on_every_bf16():
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    x = bits.view(torch.bfloat16).float()
    ok = torch.isfinite(x) & (x.abs() <= 448.0)
    x = x[ok]
    want = x.to(torch.float8_e4m3fn).double().numpy()
    got = oracle.e4m3fn_round(x.double().numpy())
    assert np.array_equal(got, want)


# --------------------------------------------------------------------------
# Planted mistakes: copies of oracle functions with one plausible error each
# must fail the pins above.
# --------------------------------------------------------------------------

def _oam_no_v(q, k, v, B, softmax_scale=None):
    s = ostem.oam_scores(q, k, v, B, softmax_scale)
    _, _, lvn = ostem.pool_blocks(q, k, v, B)
    return s - lvn[:, np.repeat(np.arange(lvn.shape[1]), q.shape[2] // k.shape[2])][:, :, None, :]


def _oam_transposed(q, k, v, B, softmax_scale=None):
    s = ostem.oam_scores(q, k, v, B, softmax_scale)
    _, _, lvn = ostem.pool_blocks(q, k, v, B)
    G = q.shape[2] // k.shape[2]
    qk = s - lvn[:, np.repeat(np.arange(lvn.shape[1]), G)][:, :, None, :]
    qk = np.swapaxes(qk, 2, 3)
    out = qk + lvn[:, np.repeat(np.arange(lvn.shape[1]), G)][:, :, None, :]
    nb = s.shape[2]
    out[..., np.triu(np.ones((nb, nb), dtype=bool), 1)] = -np.inf
    return out


def _oam_wrong_group(q, k, v, B, softmax_scale=None):
    # head h paired with KV head h % Hkv instead of h // G
    hq, hkv = q.shape[2], k.shape[2]
    perm = [h % hkv for h in range(hq)]
    kk = k[:, :, perm]
    vv = v[:, :, perm]
    return ostem.oam_scores(q, kk, vv, B, softmax_scale)


@pytest.mark.parametrize("mutant", [_oam_no_v, _oam_transposed, _oam_wrong_group])
def test_planted_oam_mistakes_are_caught(mutant):
    b, S, hq, hkv, d, B = 1, 96, 4, 2, 16, 32
    q, k, v = _rand_qkv(11, b, S, hq, hkv, d)
    got = mutant(q, k, v, B)
    want = _oam_bruteforce(q, k, v, B, 1 / math.sqrt(d))
    fin = np.isfinite(want)
    assert np.max(np.abs(got[fin] - want[fin])) > 1e-3


def test_planted_tpd_mistakes_are_caught(monkeypatch):
    def wrong_tie(alpha, i, n):                    # ties to the larger I
        return (ostem.Fraction(n * n, i + 1), -i) if alpha == 0.5 else ostem.Fraction(n, i + 1)

    def growth(alpha, i, n):                       # favours late rows
        return ostem.Fraction(n * n * (i + 1))

    for bad in (wrong_tie, growth):
        monkeypatch.setattr(ostem, "_tpd_key", bad)
        mismatches = 0
        for nb, dens in itertools.product((8, 16, 33), (0.25, 0.5, 0.6)):
            if ostem.tpd_budget(nb, dens, 0.5) != _tpd_bruteforce(nb, dens, 0.5):
                mismatches += 1
        assert mismatches > 0
    monkeypatch.undo()


def test_planted_attention_mistakes_are_caught(monkeypatch):
    b, S, hq, hkv, d, B = 1, 64, 2, 1, 8, 16
    q, k, v = _rand_qkv(5, b, S, hq, hkv, d)
    nb = S // B
    full = np.broadcast_to(np.tril(np.ones((nb, nb), dtype=bool)), (b, hq, nb, nb))
    ref = _sdpa(q, k, v, causal=True)

    orig = ostem._attend

    def no_causal(qrows, pos, keys_idx, diag_kept, i_blk, block, k_h, v_h, tau):
        return orig(qrows, pos, keys_idx, False, i_blk, block, k_h, v_h, tau)

    def no_scale(qrows, pos, keys_idx, diag_kept, i_blk, block, k_h, v_h, tau):
        return orig(qrows, pos, keys_idx, diag_kept, i_blk, block, k_h, v_h, 1.0)

    for bad in (no_causal, no_scale):
        monkeypatch.setattr(ostem, "_attend", bad)
        o, _ = ostem.block_sparse_attention(q, k, v, full, B)
        assert np.max(np.abs(o - ref)) > 1e-3
    monkeypatch.undo()


# --------------------------------------------------------------------------
# Online skip on top of the mask (BLASST summary §2.1)
# --------------------------------------------------------------------------

def _blasst_hand_case():
    """d = 1, softmax scale 1, q = 1 on every row, so a key's logit is its K
    value.  Blocks of 4 tokens: J0 logits 5, J1 0, J2 6, J3 -2, J4
    [1.5, 1.5, 9, 9]; V is 10, 20, 30, 40 per block and 50, 60, 70, 80 in J4."""
    B, nb = 4, 5
    logit = np.array([5.0] * 4 + [0.0] * 4 + [6.0] * 4 + [-2.0] * 4 + [1.5, 1.5, 9.0, 9.0])
    val = np.array([10.0] * 4 + [20.0] * 4 + [30.0] * 4 + [40.0] * 4 + [50.0, 60.0, 70.0, 80.0])
    q = np.ones((1, B * nb, 1, 1))
    k = logit.reshape(1, -1, 1, 1)
    v = val.reshape(1, -1, 1, 1)
    return q, k, v, B, nb


def _weighted(pairs):
    """O and LSE of explicit (count, logit, value) terms."""
    w = np.array([c * math.exp(x) for c, x, _ in pairs])
    vals = np.array([val for _, _, val in pairs])
    return float(w @ vals / w.sum()), math.log(w.sum())


def test_blasst_hand_worked_case():
    """ln(lam) = -4, worked by hand from the rule: a block is dropped when its
    largest visible logit is more than 4 below the running maximum."""
    q, k, v, B, nb = _blasst_hand_case()
    lam = math.exp(-4.0)
    o, lse, dropped, _ = oracle.blasst_attention(q, k, v, None, B, lam, softmax_scale=1.0)
    e5, e6 = (4, 5.0, 10.0), (4, 6.0, 30.0)
    want = {}
    for i in range(4):                                        # J0 only (diagonal, first): kept
        want[i] = (_weighted([(i + 1, 5.0, 10.0)]), 0)
    for i in range(4, 8):                                     # J1 (0 - 5 = -5): dropped
        want[i] = (_weighted([e5]), 1)
    for i in range(8, 12):                                    # J2 (6 - 5 = 1): kept
        want[i] = (_weighted([e5, (i - 7, 6.0, 30.0)]), 1)
    for i in range(12, 16):                                   # J3 (-2 - 6 = -8): dropped
        want[i] = (_weighted([e5, e6]), 2)
    for i in (16, 17):                                        # J4 sees only 1.5: 1.5 - 6 < -4
        want[i] = (_weighted([e5, e6]), 3)
    want[18] = (_weighted([e5, e6, (1, 1.5, 50.0), (1, 1.5, 60.0), (1, 9.0, 70.0)]), 2)
    want[19] = (_weighted([e5, e6, (1, 1.5, 50.0), (1, 1.5, 60.0), (1, 9.0, 70.0), (1, 9.0, 80.0)]), 2)
    for i, ((oi, li), di) in want.items():
        assert abs(o[0, i, 0, 0] - oi) < 1e-12 * abs(oi), i
        assert abs(lse[0, 0, i] - li) < 1e-12, i
        assert dropped[0, 0, i] == di, i

    # the running maximum covers the mask's kept blocks only: without J2 in
    # row I = 4, J4's 1.5 is 3.5 below J0's 5 and is kept
    mask = np.tril(np.ones((1, 1, nb, nb), dtype=bool))
    mask[0, 0, 4, 2] = False
    o2, _, d2, _ = oracle.blasst_attention(q, k, v, mask, B, lam, softmax_scale=1.0)
    for i in (16, 17):
        terms = [e5] + [(1, 1.5, 50.0 + 10 * t) for t in range(i - 15)]
        assert abs(o2[0, i, 0, 0] - _weighted(terms)[0]) < 1e-12 * 60, i
        assert d2[0, 0, i] == 2, i                            # J1 and J3


def _blasst_by_prefix_max(q, k, v, mask, B, lam, tau):
    """The rule restated without a sequential loop: a dropped block never
    raises the running maximum, so block J is dropped exactly when its local
    maximum lies more than ln(1/lam) below the largest local maximum of the
    row's earlier kept blocks.  Attention over the rest comes from torch's
    SDPA with a boolean mask."""
    b, S, hq, d = q.shape
    G = hq // k.shape[2]
    nb = S // B
    o = np.zeros_like(q)
    dropped = np.zeros((b, hq, S), dtype=np.int64)
    causal = np.tril(np.ones((S, S), dtype=bool))
    for bi in range(b):
        for h in range(hq):
            g = h // G
            logits = tau * q[bi, :, h] @ k[bi, :, g].T
            allowed = np.zeros((S, S), dtype=bool)
            for i in range(S):
                I = i // B
                kept = [J for J in range(I + 1) if mask[bi, h, I, J]]
                local = np.array([logits[i, J * B:min((J + 1) * B, i + 1)].max() for J in kept])
                before = np.concatenate([[-np.inf], np.maximum.accumulate(local)[:-1]])
                for J, mt, pm in zip(kept, local, before):
                    if lam > 0 and mt - pm < math.log(lam):
                        dropped[bi, h, i] += 1
                    else:
                        allowed[i, J * B:(J + 1) * B] = True
            allowed &= causal
            qt = torch.from_numpy(q[bi, :, h][None, None])
            kt = torch.from_numpy(np.ascontiguousarray(k[bi, :, g])[None, None])
            vt = torch.from_numpy(np.ascontiguousarray(v[bi, :, g])[None, None])
            out = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(allowed), scale=tau)
            o[bi, :, h] = out[0, 0].numpy()
    return o, dropped


@pytest.mark.parametrize("lam", [1e-3, 0.05, 0.3, 1.0])
def test_blasst_equals_prefix_max_rule_with_sdpa(lam):
    b, S, hq, hkv, d, B = 1, 96, 4, 2, 8, 16
    q, k, v = _rand_qkv(21, b, S, hq, hkv, d)
    k[:, :2] *= 3.0                                           # a sink, so that drops happen
    nb = S // B
    rng = np.random.default_rng(3)
    mask = np.tril(rng.random((b, hq, nb, nb)) < 0.6)
    mask[..., 0] = True
    mask[:, :, np.arange(nb), np.arange(nb)] = True
    tau = 1 / math.sqrt(d)
    o, _, dropped, _ = oracle.blasst_attention(q, k, v, mask, B, lam)
    o_ref, d_ref = _blasst_by_prefix_max(q, k, v, mask, B, lam, tau)
    assert np.array_equal(dropped, d_ref)
    assert np.max(np.abs(o - o_ref)) < 1e-12
    if lam >= 0.05:
        assert dropped.sum() > 0


def test_blasst_lambda_zero_is_plain_attention():
    b, S, hq, hkv, d, B = 2, 64, 2, 1, 8, 16
    q, k, v = _rand_qkv(8, b, S, hq, hkv, d)
    nb = S // B
    mask = np.tril(np.random.default_rng(1).random((b, hq, nb, nb)) < 0.5)
    mask[..., 0] = True
    mask[:, :, np.arange(nb), np.arange(nb)] = True
    o, lse, dropped, closest = oracle.blasst_attention(q, k, v, mask, B, 0.0)
    o_ref, lse_ref = oracle.block_sparse_attention(q, k, v, mask, B)
    assert not dropped.any() and np.all(np.isinf(closest))
    assert np.max(np.abs(o - o_ref)) < 1e-12 and np.max(np.abs(lse - lse_ref)) < 1e-12


@pytest.mark.parametrize("lam", [1e-4, 1e-2])
def test_blasst_error_bound(lam):
    """Every dropped key's weight is below lam relative to the row maximum,
    which a kept block holds, so O moves by at most 2 lam B n_dropped max|v|."""
    b, S, hq, hkv, d, B = 1, 128, 2, 2, 16, 16
    q, k, v = _rand_qkv(4, b, S, hq, hkv, d)
    k[:, :4] *= 4.0
    o, _, dropped, _ = oracle.blasst_attention(q, k, v, None, B, lam)
    o_full, _ = oracle.dense_causal_attention(q, k, v)
    vmax = np.abs(v).max()
    bound = 2 * lam * B * dropped * vmax                       # [b, hq, S]
    err = np.abs(o - o_full).max(axis=3).transpose(0, 2, 1)    # [b, hq, S]
    assert np.all(err <= bound + 1e-12)
    assert dropped.sum() > 0


def test_blasst_rows_match_full():
    b, S, hq, hkv, d, B = 1, 96, 4, 2, 8, 16
    q, k, v = _rand_qkv(6, b, S, hq, hkv, d)
    k[:, :2] *= 3.0
    nb = S // B
    mask = np.tril(np.ones((b, hq, nb, nb), dtype=bool))
    o, lse, dropped, closest = oracle.blasst_attention(q, k, v, mask, B, 0.1)
    rows = [(0, 1, 5), (0, 3, 95), (0, 0, 40), (0, 2, 63)]
    ro, rl, rd, rc = oracle.blasst_attention_rows(q, k, v, mask, B, 0.1, rows)
    for n, (bi, h, i) in enumerate(rows):
        assert np.allclose(ro[n], o[bi, i, h], atol=1e-13)
        assert abs(rl[n] - lse[bi, h, i]) < 1e-13
        assert rd[n] == dropped[bi, h, i]
        assert rc[n] == closest[bi, h, i] or abs(rc[n] - closest[bi, h, i]) < 1e-12


def test_blasst_rejects_bad_lambda():
    q, k, v, B, nb = _blasst_hand_case()
    for lam in (-0.1, 1.5, float("nan")):
        with pytest.raises(ValueError):
            oracle.blasst_attention(q, k, v, None, B, lam)


def test_planted_blasst_mistakes_are_caught(monkeypatch):
    q, k, v, B, nb = _blasst_hand_case()
    lam = math.exp(-4.0)
    want_dropped = np.array([0] * 4 + [1] * 4 + [1] * 4 + [2] * 4 + [3, 3, 2, 2])

    def flipped(gap, log_lam):                      # running max minus block max
        return -gap < log_lam

    def log2_threshold(gap, log_lam):               # threshold taken in log2 units
        return gap < log_lam / math.log(2.0)

    for bad in (flipped, log2_threshold):
        monkeypatch.setattr(ostem, "_blasst_drops", bad)
        with np.errstate(invalid="ignore"):                 # a mutant may drop a row's every block
            _, _, dropped, _ = oracle.blasst_attention(q, k, v, None, B, lam, softmax_scale=1.0)
        assert not np.array_equal(dropped[0, 0], want_dropped)
    monkeypatch.undo()
    _, _, dropped, _ = oracle.blasst_attention(q, k, v, None, B, lam, softmax_scale=1.0)
    assert np.array_equal(dropped[0, 0], want_dropped)
