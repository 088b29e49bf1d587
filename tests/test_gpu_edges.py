"""GPU checks at the edges of the API:

  * the Python binding rejects, before any C call, tensors the C ABI would
    read wrongly: strided views, a wrong element type (an int64 block table),
    CPU tensors and buffers smaller than the call writes;
  * the attention kernels at the largest block count the API takes
    (Nb = 4096, 512K tokens): with every causal block kept, the last query
    block's rows visit 4096 blocks, the longest kept-block list; sampled
    rows against the oracle, and the density-1 sparse kernel bit for bit
    against the dense one.
Every case prints its name before it touches the GPU."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import block_sparse_attention_24_amd as sb
import oracle
import workloads as wl
from gpu_common import TOL_LSE, TOL_O, kv_args, output_error, problem, split_magnitude, with_scale_column

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _announce(name):
    print(f"\n[case] {name}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sb.lib()
    yield


def test_binding_rejects_tensors_the_abi_would_misread():
    _announce("binding checks")
    w = wl.Workload("binding", 1, 128 * 4, 4, 2, 128, 128, "bf16", paged=True, page_size=64)
    inp = wl.make_inputs(w, device=DEV)
    p = problem(w, inp)
    q, k, v = inp["q"], inp["k"], inp["v"]
    o = torch.empty((1, w.seq, w.hq, w.head_dim), dtype=torch.bfloat16, device=DEV)
    # a [b, h, S, d] transpose of Q is a strided view
    qt = q.transpose(1, 2).contiguous().transpose(1, 2)
    assert not qt.is_contiguous()
    with pytest.raises(ValueError, match="contiguous"):
        sb.bsa_prefill(p, qt, k, v, None, o)
    with pytest.raises(ValueError, match="dtype"):
        sb.bsa_prefill(p, q.float(), k, v, None, o)
    with pytest.raises(ValueError, match="dtype"):                      # int64, as torch.randperm gives
        sb.bsa_prefill(p, q, inp["k_pages"], inp["v_pages"], None, o, None, inp["block_table"].long(), 64)
    with pytest.raises(ValueError, match="elements"):
        sb.bsa_prefill(p, q, k, v, None, o[:, :-1].contiguous())
    with pytest.raises(ValueError, match="GPU"):
        sb.bsa_prefill(p, q.cpu(), k, v, None, o)
    scores = torch.empty((1, w.hq, 4, 3), dtype=torch.float32, device=DEV)
    ws = torch.empty(sb.stem_score_workspace_size(p), dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError, match="elements"):
        sb.stem_score(p, q, k, v, scores, ws)
    mask = torch.empty((1, w.hq, 4, 1), dtype=torch.int64, device=DEV)
    with pytest.raises(ValueError, match="dtype"):
        sb.stem_select(p, torch.zeros((1, w.hq, 4, 4), device=DEV), 0.5, 0.5, mask)
    # the same calls with correct tensors go through
    sb.bsa_prefill(p, q, k, v, None, o)
    sb.bsa_prefill(p, q, inp["k_pages"], inp["v_pages"], None, o, None, inp["block_table"], 64)
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["fp8", "bf16"])
def test_attention_at_4096_blocks(dtype):
    w = wl.Workload(f"nb4096-{dtype}", 1, 128 * 4096, 1, 1, 128, 128, dtype, paged=dtype == "fp8",
                    page_size=64, density=0.02)
    _announce(f"attention at 4096 blocks {w.name}")
    inp = wl.make_inputs(w, device=DEV, gen_device=DEV)
    p = problem(w, inp)
    k, v, table, page = kv_args(w, inp)
    nb = w.num_blocks
    full = torch.full((1, 1, nb, p.mask_words), -1, dtype=torch.int32, device=DEV)   # every causal block
    o_s, l_s = sb.attention(p, inp["q"], k, v, full, table, page)
    o_d, l_d = sb.attention(p, inp["q"], k, v, None, table, page)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_d) and torch.equal(l_s, l_d)
    q64 = oracle.dequantize(wl.to_float64(inp["q"]), inp["q_scale"])
    k64 = oracle.dequantize(wl.to_float64(inp["k"]), inp["k_scale"])
    v64 = oracle.dequantize(wl.to_float64(inp["v"]), inp["v_scale"])
    toks = [0, 127, 2048 * 128 + 7, w.seq - 128, w.seq - 65, w.seq - 1]      # the last three keep 4096 blocks
    o_aug, l_ref = oracle.attention_rows(q64, k64, with_scale_column(w, v64, DEV), None, w.block,
                                         [(0, 0, t) for t in toks])
    o_ref, mag = split_magnitude(w, o_aug)
    err = output_error(o_d[0, toks, 0], o_ref, mag)
    print(f"  O error / row magnitude {err:.4f} (bar {TOL_O[dtype]})", flush=True)
    assert err < TOL_O[dtype]
    assert np.max(np.abs(l_d[0, 0, toks].cpu().double().numpy() - l_ref)) < TOL_LSE[dtype]
    # a Stem mask at 4096 blocks: scoring, selection and the sparse kernel
    s, _ = sb.score(p, inp["q"], k, v, table, page)
    words, _, _ = sb.select(p, s, w.density, w.alpha)
    o_m, l_m = sb.attention(p, inp["q"], k, v, words, table, page)
    torch.cuda.synchronize()
    budget, total = oracle.tpd_budget(nb, w.density, w.alpha)
    m = oracle.unpack_block_mask(words[:, :, -2:].cpu().numpy().view(np.uint32), nb)   # rows 4094, 4095
    assert m.sum() == budget[-2] + budget[-1]
    mask_rows = lambda bi, h, i: m[bi, h, i - (nb - 2)]
    toks = [w.seq - 200, w.seq - 1]
    o_aug, l_ref = oracle.attention_rows(q64, k64, with_scale_column(w, v64, DEV), mask_rows, w.block,
                                         [(0, 0, t) for t in toks])
    o_ref, mag = split_magnitude(w, o_aug)
    assert output_error(o_m[0, toks, 0], o_ref, mag) < TOL_O[dtype]
    assert np.max(np.abs(l_m[0, 0, toks].cpu().double().numpy() - l_ref)) < TOL_LSE[dtype]


def test_debug_mode_rejects_bad_block_table_before_launch(monkeypatch):
    """With STEM_DEBUG set, an entry point that reads a block table checks it
    on the host: an entry outside [0, num_pages) gives STEM_EINVAL and nothing
    runs; the same call without the bad entry runs and matches debug-off."""
    _announce("STEM_DEBUG block table")
    w = wl.Workload("debug-table", 1, 128 * 6, 4, 2, 128, 128, "fp8", paged=True, page_size=64)
    inp = wl.make_inputs(w, device=DEV)
    p = problem(w, inp)
    k, v, table, page = kv_args(w, inp)
    # K/V pages in the first half of allocations twice that size, so that the
    # page one past the last still lies in allocated memory
    npg = k.shape[0]
    kb, vb = torch.cat([k, k]), torch.cat([v, v])
    k, v = kb[:npg], vb[:npg]
    o_ref, l_ref = sb.attention(p, inp["q"], k, v, None, table, page)
    monkeypatch.setenv("STEM_DEBUG", "1")
    o, l = sb.attention(p, inp["q"], k, v, None, table, page)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)
    bad = table.clone()
    bad[0, 5] = npg                                           # one past the last page
    o2 = torch.zeros_like(o)
    with pytest.raises(sb.StemError, match=r"block_table\[0\]\[5\]"):
        sb.bsa_prefill(p, inp["q"], k, v, None, o2, None, bad, page)
    with pytest.raises(sb.StemError, match="block_table"):
        sb.score(p, inp["q"], k, v, bad, page)
    torch.cuda.synchronize()
    assert int(o2.abs().sum()) == 0                           # nothing was launched
    # stem_select's lists are checked after its kernel (they are valid here)
    s, _ = sb.score(p, inp["q"], k, v, table, page)
    sb.select(p, s, w.density, w.alpha, with_list=True)
    torch.cuda.synchronize()
