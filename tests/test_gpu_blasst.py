"""GPU parity of bsa_prefill_blasst, the attention with BLASST's online skip
on top of the mask, through the C ABI, against the oracle's blasst_attention:

  * O within the attention tolerance of the dtype, LSE within TOL_LSE, and the
    blocks each row dropped exactly equal to the oracle's count;
  * rows where some block's decision lies within SKIP_TIE (natural-log units)
    of the threshold in the oracle's fp64 logits are left out of those three
    checks (the kernel takes the same decision on fp32 logits); their share
    is printed and must stay below 2%;
  * lambda = 0 gives bsa_prefill's output bit for bit and no dropped block;
  * a workload with a dominant sink makes most rows drop most blocks, so that
    whole wavefronts take the branch without the softmax.
Every case prints its name before it touches the GPU."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import block_sparse_attention_24_amd as sb
import oracle
import workloads as wl
from gpu_common import (TOL_LSE, TOL_O, kv_args, mask_bits, oracle_qkv, output_error, problem, split_magnitude,
                        with_scale_column)

pytestmark = pytest.mark.gpu

DEV = "cuda"
SKIP_TIE = 1e-3


def _announce(name):
    print(f"\n[case] {name}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sb.lib()
    yield


def _stem_mask(w, q, k, v):
    s = oracle.oam_scores(q, k, v, w.block)
    budget, _ = oracle.tpd_budget(w.num_blocks, w.density, w.alpha)
    return oracle.select_blocks(s, budget)


def _words(m):
    return torch.from_numpy(oracle.pack_block_mask(m).view(np.int32)).to(DEV)


def _compare(w, o, lse, skipped, o_aug, l_ref, d_ref, closest):
    """O, LSE and dropped counts on the rows whose decisions are clear of the
    threshold; returns the share of rows left out.  o_aug: the oracle's O over
    V with the V-row scale column (the row magnitudes of the fp8 bar)."""
    o_ref, mag = split_magnitude(w, o_aug)
    keep = closest >= SKIP_TIE                                  # [b, Hq, S]
    share = 1.0 - keep.mean()
    print(f"  rows near the threshold: {share:.4%}; dropped per row: mean {d_ref.mean():.2f}", flush=True)
    assert share < 0.02
    b_i, h_i, t_i = np.nonzero(keep)
    og = o[b_i, t_i, h_i]
    err = output_error(og, o_ref[b_i, t_i, h_i], mag[b_i, t_i, h_i])
    print(f"  O error / row magnitude: {err:.4f} (bar {TOL_O[w.dtype]})", flush=True)
    assert err < TOL_O[w.dtype]
    lg = lse.cpu().double().numpy()[b_i, h_i, t_i]
    assert np.max(np.abs(lg - l_ref[b_i, h_i, t_i])) < TOL_LSE[w.dtype]
    sg = skipped.cpu().numpy()
    assert np.array_equal(sg[b_i, h_i, t_i], d_ref[b_i, h_i, t_i])
    return share


# (workload, lambdas, mask): "stem" = the oracle's Stem selection, "dense" = every causal block
CASES = [
    (wl.Workload("bl-bf16-gqa-nb13", 1, 128 * 13, 4, 2, 128, 128, "bf16", density=0.5),
     [1e-3, 0.1, 0.5, 1.0], "stem"),
    (wl.Workload("bl-fp8-paged64-nb14", 1, 128 * 14, 4, 1, 128, 128, "fp8", density=0.4, sink=False,
                 v_sigma=0.0, paged=True, page_size=64), [1e-3, 0.2, 1.0], "stem"),
    (wl.Workload("bl-bf16-dense-b2-nb9", 2, 128 * 9, 2, 1, 128, 128, "bf16"), [0.05, 1.0], "dense"),
    (wl.Workload("bl-fp8-dense-nb10", 1, 128 * 10, 2, 2, 128, 128, "fp8", sink=False, v_sigma=0.0),
     [0.01, 0.5], "dense"),
    (wl.Workload("bl-fp8-sink-contig-nb11", 1, 128 * 11, 4, 2, 128, 128, "fp8", density=0.6, sink=False,
                 v_sigma=0.0, sink_logit=16.0), [1e-3], "stem"),
    (wl.Workload("bl-bf16-sink-paged16-nb10", 1, 128 * 10, 2, 2, 128, 128, "bf16", sink=False,
                 sink_logit=16.0, paged=True, page_size=16), [1e-3, 1e-2], "dense"),
    (wl.Workload("bl-fp8-gqa3-hq12-b2-paged32", 2, 128 * 10, 12, 4, 128, 128, "fp8", density=0.5,
                 paged=True, page_size=32), [0.1], "stem"),
    # the remaining (dtype, mask, layout) instantiations: fp8 dense paged, bf16 sparse paged
    (wl.Workload("bl-fp8-dense-paged32-nb9", 1, 128 * 9, 4, 2, 128, 128, "fp8", sink=False, v_sigma=0.0,
                 paged=True, page_size=32), [0.05, 0.8], "dense"),
    (wl.Workload("bl-bf16-stem-paged64-b2-nb11", 2, 128 * 11, 4, 2, 128, 128, "bf16", density=0.5,
                 paged=True, page_size=64), [0.02, 0.3], "stem"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0].name)
def test_blasst_equals_oracle(case):
    w, lams, kind = case
    inp = wl.make_inputs(w, device=DEV)
    p = problem(w, inp)
    k, v, table, page = kv_args(w, inp)
    q64, k64, v64 = oracle_qkv(inp)
    m_ref = _stem_mask(w, q64, k64, v64) if kind == "stem" else None
    words = _words(m_ref) if m_ref is not None else None
    for lam in lams:
        _announce(f"blasst {w.name} lambda={lam}")
        o, lse, skipped = sb.attention_blasst(p, inp["q"], k, v, lam, words, table, page)
        torch.cuda.synchronize()
        o_aug, l_ref, d_ref, closest = oracle.blasst_attention(q64, k64, with_scale_column(w, v64), m_ref,
                                                               w.block, lam)
        _compare(w, o, lse, skipped, o_aug, l_ref, d_ref, closest)
        if w.sink_logit > 0:
            kept = (np.tril(np.ones((w.num_blocks,) * 2, dtype=bool)) if m_ref is None
                    else m_ref[0, 0]).sum(axis=1)
            # a row's first block is never dropped
            share = d_ref.sum() / ((kept[np.arange(w.seq) // w.block] - 1).sum() * w.batch * w.hq)
            print(f"  droppable blocks dropped: {share:.1%}", flush=True)
            assert share > 0.9                                  # whole wavefronts skip


@pytest.mark.parametrize("case", [CASES[0], CASES[1], CASES[3]], ids=lambda c: c[0].name)
def test_lambda_zero_is_bsa_prefill(case):
    w, _, kind = case
    _announce(f"blasst lambda=0 {w.name}")
    inp = wl.make_inputs(w, device=DEV)
    p = problem(w, inp)
    k, v, table, page = kv_args(w, inp)
    words = None
    if kind == "stem":
        s, _ = sb.score(p, inp["q"], k, v, table, page)
        words, _, _ = sb.select(p, s, w.density, w.alpha)
    o0, l0 = sb.attention(p, inp["q"], k, v, words, table, page)
    o1, l1, skipped = sb.attention_blasst(p, inp["q"], k, v, 0.0, words, table, page)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    assert int(skipped.abs().sum()) == 0


def test_blasst_run_twice_bit_identical():
    w = CASES[1][0]
    _announce(f"blasst twice {w.name}")
    inp = wl.make_inputs(w, device=DEV)
    p = problem(w, inp)
    k, v, table, page = kv_args(w, inp)
    s, _ = sb.score(p, inp["q"], k, v, table, page)
    words, _, _ = sb.select(p, s, w.density, w.alpha)
    r1 = sb.attention_blasst(p, inp["q"], k, v, 0.2, words, table, page)
    r2 = sb.attention_blasst(p, inp["q"], k, v, 0.2, words, table, page)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(r1, r2))


def test_blasst_empty_rows_and_null_outputs():
    """A user mask with empty rows: O = 0, LSE = -inf, nothing dropped; the
    optional outputs may be NULL."""
    w = wl.Workload("bl-edge-bf16", 1, 128 * 6, 2, 1, 128, 128, "bf16")
    _announce(f"blasst edge {w.name}")
    inp = wl.make_inputs(w, device=DEV)
    p = problem(w, inp)
    nb = w.num_blocks
    m = np.tril(np.ones((1, 2, nb, nb), dtype=bool))
    m[0, 0, 3, :] = False                                     # query block 3 of head 0 sees nothing
    m[0, 1, 5, 1:5] = False                                   # sink and diagonal only
    words = _words(m)
    o, lse, skipped = sb.attention_blasst(p, inp["q"], inp["k"], inp["v"], 0.3, words)
    o2 = torch.empty_like(o)
    sb.bsa_prefill_blasst(p, inp["q"], inp["k"], inp["v"], words, 0.3, o2)   # lse, skipped NULL
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    rows = slice(3 * 128, 4 * 128)
    assert torch.all(o[0, rows, 0] == 0)
    assert torch.all(torch.isneginf(lse[0, 0, rows]))
    assert torch.all(skipped[0, 0, rows] == 0)
    q64, k64, v64 = oracle_qkv(inp)
    o_aug, l_ref, d_ref, closest = oracle.blasst_attention(q64, k64, with_scale_column(w, v64), m, w.block, 0.3)
    o_ref, mag = split_magnitude(w, o_aug)
    fin = np.isfinite(l_ref)
    keep = (closest >= SKIP_TIE) & fin
    b_i, h_i, t_i = np.nonzero(keep)
    assert output_error(o[b_i, t_i, h_i], o_ref[b_i, t_i, h_i], mag[b_i, t_i, h_i]) < TOL_O[w.dtype]
    assert np.array_equal(skipped.cpu().numpy()[keep], d_ref[keep])


def test_blasst_full_128k_sampled():
    """The 128K fp8 paged configuration at full size with the GPU's own Stem
    mask, lambda = 1e-3: sampled rows of sampled heads against the oracle."""
    w = wl.GQA_128K_FP8_PAGED
    _announce(f"blasst full {w.name}")
    inp = wl.make_inputs(w, device=DEV, gen_device=DEV)
    p = problem(w, inp)
    k, v, table, page = kv_args(w, inp)
    s, _ = sb.score(p, inp["q"], k, v, table, page)
    words, _, _ = sb.select(p, s, w.density, w.alpha)
    lam = 1e-3
    o, lse, skipped = sb.attention_blasst(p, inp["q"], k, v, lam, words, table, page)
    torch.cuda.synchronize()
    nb = w.num_blocks
    G = w.hq // w.hkv
    rng = np.random.default_rng(7)
    checked = near = 0
    for h in (0, 21, w.hq - 1):
        g = h // G
        qh = oracle.dequantize(wl.to_float64(inp["q"][:, :, h:h + 1]), inp["q_scale"])
        kh = oracle.dequantize(wl.to_float64(inp["k"][:, :, g:g + 1]), inp["k_scale"])
        vh = oracle.dequantize(wl.to_float64(inp["v"][:, :, g:g + 1]), inp["v_scale"])
        m_h = mask_bits(words[:, h:h + 1], nb)
        toks = sorted({0, 5, 127, 128, w.seq - 1} | set(int(x) for x in rng.integers(0, w.seq, 16)))
        o_aug, l_ref, d_ref, closest = oracle.blasst_attention_rows(
            qh, kh, with_scale_column(w, vh, DEV), m_h, w.block, lam, [(0, 0, t) for t in toks])
        o_ref, mag = split_magnitude(w, o_aug)
        keep = closest >= SKIP_TIE
        near += int((~keep).sum())
        checked += len(toks)
        t_k = [t for t, kk in zip(toks, keep) if kk]
        assert output_error(o[0, t_k, h], o_ref[keep], mag[keep]) < TOL_O[w.dtype], h
        assert np.max(np.abs(lse[0, h, t_k].cpu().double().numpy() - l_ref[keep])) < TOL_LSE[w.dtype], h
        assert np.array_equal(skipped[0, h, t_k].cpu().numpy(), d_ref[keep]), h
    print(f"  rows near the threshold: {near} of {checked}", flush=True)
    assert near <= checked // 10
