"""GPU parity of the entry points around the path, through the C ABI:

  * stem_score_sam against the oracle's score-only metric (|delta| < 1e-4,
    -inf above the diagonal), and selection on those scores;
  * stem_score_pooled: bit-identical to stem_score (and to stem_score_sam
    without lvn) given the representations stem_score pooled;
  * stem_cache_write: stored E4M3 codes bit-exact against the oracle's
    quantisation (fp32 quotient, ties to even, saturation), copies exact for
    bf16/fp32 caches, kbar/lvn within 1e-5 of the oracle, and bit-identical to
    what stem_score pools back from the written cache.
Every case prints its name before it touches the GPU."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import block_sparse_attention_24_amd as sb
import oracle
import workloads as wl
from gpu_common import TOL_SCORE, mask_bits, oracle_qkv, problem, kv_args, workspace_views

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _announce(name):
    print(f"\n[case] {name}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sb.lib()
    yield


SAM_CASES = [
    wl.Workload("sam-bf16-gqa-ragged-b2", 2, 128 * 70, 8, 2, 128, 128, "bf16"),
    wl.Workload("sam-fp8-paged", 1, 128 * 40, 8, 1, 128, 128, "fp8", paged=True, page_size=64),
    wl.Workload("sam-f32-b64-d64", 1, 64 * 33, 2, 2, 64, 64, "f32"),
    wl.Workload("sam-bf16-single-block", 1, 128, 2, 1, 128, 128, "bf16"),
    wl.Workload("sam-bf16-nb130", 1, 64 * 130, 2, 1, 128, 64, "bf16"),
]


@pytest.mark.parametrize("w", SAM_CASES, ids=lambda w: w.name)
def test_sam_scores_and_selection(w):
    _announce(f"sam {w.name}")
    inp = wl.make_inputs(w, device=DEV)
    p = problem(w, inp)
    k, v, table, page = kv_args(w, inp)
    s_sam, _ = sb.score(p, inp["q"], k, v, table, page, sam=True)
    mask, _, _ = sb.select(p, s_sam, w.density, w.alpha)
    torch.cuda.synchronize()
    q, kk, _ = oracle_qkv(inp)
    ref = oracle.sam_scores(q, kk, w.block)
    got = s_sam.cpu().double().numpy()
    nb = w.num_blocks
    low = np.tril(np.ones((nb, nb), dtype=bool))
    assert np.all(got[..., ~low] == -np.inf)
    assert np.max(np.abs(got[..., low] - ref[..., low])) < TOL_SCORE
    budget, _ = oracle.tpd_budget(nb, w.density, w.alpha)
    assert np.array_equal(mask_bits(mask, nb), oracle.select_blocks(got, budget))


@pytest.mark.parametrize("w", [SAM_CASES[0], SAM_CASES[1], SAM_CASES[2]], ids=lambda w: w.name)
def test_score_pooled_is_bit_identical_to_score(w):
    _announce(f"pooled {w.name}")
    inp = wl.make_inputs(w, device=DEV)
    p = problem(w, inp)
    k, v, table, page = kv_args(w, inp)
    s_oam, ws = sb.score(p, inp["q"], k, v, table, page)
    s_sam, _ = sb.score(p, inp["q"], k, v, table, page, sam=True)
    _, kbar, lvn = workspace_views(p, ws)
    kbar, lvn = kbar.clone(), lvn.clone()
    s_p, _ = sb.score_pooled(p, inp["q"], kbar, lvn)
    s_ps, _ = sb.score_pooled(p, inp["q"], kbar, None)
    torch.cuda.synchronize()
    assert torch.equal(s_p, s_oam)
    assert torch.equal(s_ps, s_sam)


# Cache writes: (workload, fixed FP8 scale or None for amax / 448, inject extremes)
CACHE_CASES = [
    (wl.Workload("cw-fp8-paged64", 1, 128 * 9, 2, 2, 128, 128, "fp8", paged=True, page_size=64), None, False),
    (wl.Workload("cw-fp8-paged16-b2-pow2scale", 2, 128 * 5, 4, 2, 128, 128, "fp8", paged=True,
                 page_size=16), 0.25, True),
    (wl.Workload("cw-fp8-contig-d64-b64", 1, 64 * 11, 2, 2, 64, 64, "fp8"), 0.0123, True),
    (wl.Workload("cw-bf16-paged128", 1, 128 * 6, 2, 2, 128, 128, "bf16", paged=True, page_size=128), None, False),
    (wl.Workload("cw-bf16-d64-b64", 1, 64 * 7, 2, 1, 64, 64, "bf16"), None, False),
    (wl.Workload("cw-f32-mha", 1, 64 * 8, 2, 2, 64, 64, "f32"), None, False),
]


def _inject_extremes(x: torch.Tensor, scale: float, seed: int):
    """Overwrite a few token rows with values that saturate, fall into the
    E4M3 subnormal range or round to zero, and exact halfway cases."""
    g = torch.Generator().manual_seed(seed)
    b, S, H, d = x.shape
    n = H * d
    expo = torch.randint(-16, 12, (n,), generator=g).float()
    sign = torch.where(torch.rand(n, generator=g) < 0.5, -1.0, 1.0)
    spread = (sign * torch.exp2(expo) * scale).view(H, d)
    x[0, 5] = spread.to(x.dtype)
    x[0, S - 1] = (torch.full((H, d), 1000.0) * scale).to(x.dtype)          # saturates
    ties = torch.tensor([1.0625, 1.1875, 2.125, 2.375, -3.125, 17.0, -0.59375, 2.0 ** -10 * 3])
    x[b - 1, S // 2] = (ties.repeat(n // len(ties) + 1)[:n].view(H, d) * scale).to(x.dtype)


@pytest.mark.parametrize("case", CACHE_CASES, ids=lambda c: c[0].name)
def test_cache_write(case):
    w, fixed_scale, extremes = case
    _announce(f"cache write {w.name}")
    src = wl.make_cache_inputs(w, device="cpu", fp8_scale=fixed_scale)
    if extremes:
        _inject_extremes(src["k"], src["k_scale"], 1)
        _inject_extremes(src["v"], src["v_scale"], 2)
    k_in, v_in = src["k"].to(DEV), src["v"].to(DEV)
    p = sb.Problem(w.batch, w.seq, w.hq, w.hkv, w.head_dim, w.block, w.dtype, 1.0,
                   float(src["k_scale"]), float(src["v_scale"]))
    cdt = {"fp8": torch.float8_e4m3fn, "bf16": torch.bfloat16, "f32": torch.float32}[w.dtype]
    if w.paged:
        table = src["block_table"].to(DEV)
        shape = (src["num_pages"], w.page_size, w.hkv, w.head_dim)
    else:
        table = None
        shape = (w.batch, w.seq, w.hkv, w.head_dim)
    # fill the cache with a pattern first, so stale bytes would show
    if w.dtype == "fp8":
        k_c = torch.full(shape, 7, dtype=torch.uint8, device=DEV).view(cdt)
    else:
        k_c = torch.full(shape, 7.0, dtype=cdt, device=DEV)
    v_c = k_c.clone()
    kbar, lvn = sb.cache_write(p, k_in, v_in, k_c, v_c, table, w.page_size if w.paged else 0)
    torch.cuda.synchronize()

    # stored values, in token order
    k_tok = wl.gather_pages(k_c, table) if w.paged else k_c
    v_tok = wl.gather_pages(v_c, table) if w.paged else v_c
    ks_ref, vs_ref, kbar_ref, lvn_ref = oracle.cache_write(
        wl.to_float64(src["k"]), wl.to_float64(src["v"]), w.block, fp8=w.dtype == "fp8",
        k_scale=src["k_scale"], v_scale=src["v_scale"])
    assert np.array_equal(wl.to_float64(k_tok), ks_ref)
    assert np.array_equal(wl.to_float64(v_tok), vs_ref)
    if w.dtype != "fp8":
        assert torch.equal(k_tok.cpu(), src["k"]) and torch.equal(v_tok.cpu(), src["v"])
    assert np.max(np.abs(kbar.cpu().double().numpy() - kbar_ref)) < 1e-5
    assert np.max(np.abs(lvn.cpu().double().numpy() - lvn_ref)) < 1e-5

    # pooling the written cache again gives the same bits, and so do the scores
    gq = torch.Generator(device="cpu").manual_seed(9)
    q32 = torch.randn((w.batch, w.seq, w.hq, w.head_dim), generator=gq)
    if w.dtype == "fp8":
        q, q_scale = wl.quantize_fp8(q32)
        p.q_scale = float(q_scale)
    elif w.dtype == "bf16":
        q = q32.to(torch.bfloat16)
    else:
        q = q32
    q = q.to(DEV)
    s_ref, ws = sb.score(p, q, k_c, v_c, table, w.page_size if w.paged else 0)
    s_p, _ = sb.score_pooled(p, q, kbar, lvn)
    torch.cuda.synchronize()
    _, kb2, lv2 = workspace_views(p, ws)
    assert torch.equal(kb2, kbar)
    assert torch.equal(lv2, lvn)
    assert torch.equal(s_p, s_ref)


def test_cache_write_full_128k_sampled():
    """The 128K fp8 paged configuration (8 KV heads, 64-token pages): a cache
    write at full size, checked on sampled blocks against the oracle."""
    w = wl.GQA_128K_FP8_PAGED
    _announce(f"cache write full {w.name}")
    src = wl.make_cache_inputs(w, device=DEV, gen_device=DEV)
    p = sb.Problem(w.batch, w.seq, w.hq, w.hkv, w.head_dim, w.block, w.dtype, 1.0,
                   float(src["k_scale"]), float(src["v_scale"]))
    shape = (src["num_pages"], w.page_size, w.hkv, w.head_dim)
    k_c = torch.empty(shape, dtype=torch.float8_e4m3fn, device=DEV)
    v_c = torch.empty_like(k_c)
    table = src["block_table"]
    kbar, lvn = sb.cache_write(p, src["k"], src["v"], k_c, v_c, table, w.page_size)
    torch.cuda.synchronize()
    k_tok = wl.gather_pages(k_c, table)
    v_tok = wl.gather_pages(v_c, table)
    g = torch.Generator().manual_seed(5)
    blocks = sorted({0, w.num_blocks - 1} | set(torch.randint(w.num_blocks, (6,), generator=g).tolist()))
    for J in blocks:
        sl = slice(J * w.block, (J + 1) * w.block)
        ks_ref, vs_ref, kb_ref, lv_ref = oracle.cache_write(
            wl.to_float64(src["k"][:, sl]), wl.to_float64(src["v"][:, sl]), w.block, fp8=True,
            k_scale=src["k_scale"], v_scale=src["v_scale"])
        assert np.array_equal(wl.to_float64(k_tok[:, sl]), ks_ref), J
        assert np.array_equal(wl.to_float64(v_tok[:, sl]), vs_ref), J
        assert np.max(np.abs(kbar[:, :, J].cpu().double().numpy() - kb_ref[:, :, 0])) < 1e-5
        assert np.max(np.abs(lvn[:, :, J].cpu().double().numpy() - lv_ref[:, :, 0])) < 1e-5
