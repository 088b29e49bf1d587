"""GPU parity at a softmax scale other than 1/sqrt(head_dim) (the
descriptor's softmax_scale), through the C ABI, against the oracle with the
same scale: OAM and SAM scores (within TOL_SCORE), the selection on the
GPU's own scores (exact), attention on the oracle's mask for every kernel
family (fp8 and bf16 pipelined kernels, the generic kernel), the online skip
(rows near the threshold left out, as in test_gpu_blasst), and the decode
step with and without the skip.  Every case prints its name before it
touches the GPU."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import block_sparse_attention_24_amd as sb
import oracle
import workloads as wl
from gpu_common import (TOL_LSE, TOL_O, TOL_SCORE, kv_args, mask_bits, oracle_qkv, output_error, problem,
                        split_magnitude, with_scale_column)

pytestmark = pytest.mark.gpu

DEV = "cuda"
SCALES = [0.05, 0.2]
SKIP_TIE = 1e-3


def _announce(name):
    print(f"\n[case] {name}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sb.lib()
    yield


def _tol_lse(w, scale):
    """TOL_LSE holds at the default scale.  The fp8 MFMA's dot products carry
    an error of about 2^-16 of tau * sum |q_i k_i| (measured: the LSE error
    grows with the scale, and tenfold with the x4 sink keys), so for fp8 the
    bound grows with tau / tau_default."""
    if w.dtype != "fp8":
        return TOL_LSE[w.dtype]
    return TOL_LSE["fp8"] * max(1.0, scale * math.sqrt(w.head_dim))


def _tol_o(w, v):
    """TOL_O (fp8: per row magnitude, see split_magnitude), and for bf16 at
    least the bound of rounding P to bf16: with p~ = p (1 + e), |e| <= 2^-9,
    the normalised weights move by at most 2^-8 in total, so O moves by at
    most 2^-8 max |V|.  A larger scale makes the softmax sharper; fewer keys
    then carry O and their rounding errors average out less than at the
    default scale."""
    if w.dtype != "bf16":
        return TOL_O[w.dtype]
    return max(TOL_O[w.dtype], 2.0 ** -8 * float(v.float().abs().max()))


PREFILL = [
    wl.Workload("ss-fp8-paged64", 1, 128 * 12, 4, 2, 128, 128, "fp8", density=0.4, paged=True, page_size=64),
    wl.Workload("ss-bf16-gqa", 1, 128 * 10, 4, 1, 128, 128, "bf16", density=0.5, v_sigma=0.0),
    wl.Workload("ss-f32-d64-b64", 1, 64 * 12, 2, 2, 64, 64, "f32", density=0.5, sink=False),
]


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("w", PREFILL, ids=lambda w: w.name)
def test_prefill_path_at_softmax_scale(w, scale):
    _announce(f"softmax scale {scale} {w.name}")
    inp = wl.make_inputs(w, device=DEV)
    p = problem(w, inp)
    p.softmax_scale = scale
    k, v, table, page = kv_args(w, inp)
    q64, k64, v64 = oracle_qkv(inp)
    nb = w.num_blocks
    low = np.tril(np.ones((nb, nb), dtype=bool))
    budget, _ = oracle.tpd_budget(nb, w.density, w.alpha)
    for sam in (False, True):
        s, _ = sb.score(p, inp["q"], k, v, table, page, sam=sam)
        torch.cuda.synchronize()
        ref = (oracle.sam_scores(q64, k64, w.block, softmax_scale=scale) if sam
               else oracle.oam_scores(q64, k64, v64, w.block, softmax_scale=scale))
        got = s.cpu().double().numpy()
        assert np.max(np.abs(got[..., low] - ref[..., low])) < TOL_SCORE, sam
        mask, _, _ = sb.select(p, s, w.density, w.alpha)
        torch.cuda.synchronize()
        assert np.array_equal(mask_bits(mask, nb), oracle.select_blocks(got, budget)), sam
    m_ref = oracle.select_blocks(oracle.oam_scores(q64, k64, v64, w.block, softmax_scale=scale), budget)
    words = torch.from_numpy(oracle.pack_block_mask(m_ref).view(np.int32)).to(DEV)
    o, lse = sb.attention(p, inp["q"], k, v, words, table, page)
    torch.cuda.synchronize()
    o_aug, l_ref = oracle.block_sparse_attention(q64, k64, with_scale_column(w, v64), m_ref, w.block,
                                                 softmax_scale=scale)
    o_ref, mag = split_magnitude(w, o_aug)
    err = output_error(o, o_ref, mag)
    print(f"  O error / row magnitude: {err:.4f} (bar {_tol_o(w, inp['v']):.4f})", flush=True)
    assert err < _tol_o(w, inp["v"])
    assert np.max(np.abs(lse.cpu().double().numpy() - l_ref)) < _tol_lse(w, scale)
    if (w.head_dim, w.block) == (128, 128):
        lam = 0.2
        o, lse, skipped = sb.attention_blasst(p, inp["q"], k, v, lam, words, table, page)
        torch.cuda.synchronize()
        o_aug, l_ref, d_ref, closest = oracle.blasst_attention(q64, k64, with_scale_column(w, v64), m_ref,
                                                               w.block, lam, softmax_scale=scale)
        o_ref, mag = split_magnitude(w, o_aug)
        keep = closest >= SKIP_TIE
        assert keep.mean() > 0.98
        b_i, h_i, t_i = np.nonzero(keep)
        assert output_error(o[b_i, t_i, h_i], o_ref[b_i, t_i, h_i], mag[b_i, t_i, h_i]) < _tol_o(w, inp["v"])
        assert np.max(np.abs(lse.cpu().double().numpy()[b_i, h_i, t_i] - l_ref[b_i, h_i, t_i])) < _tol_lse(w, scale)
        assert np.array_equal(skipped.cpu().numpy()[b_i, h_i, t_i], d_ref[b_i, h_i, t_i])


DECODE = [
    wl.Workload("ssd-fp8-paged64-b2", 2, 128 * 12, 8, 2, 128, 128, "fp8", density=0.5, paged=True, page_size=64),
    wl.Workload("ssd-bf16-d64-b64", 1, 64 * 14, 4, 2, 64, 64, "bf16", density=0.5),
]


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("w", DECODE, ids=lambda w: w.name)
def test_decode_at_softmax_scale(w, scale):
    _announce(f"decode softmax scale {scale} {w.name}")
    src = wl.make_cache_inputs(w, device="cpu")
    p = sb.Problem(w.batch, w.seq, w.hq, w.hkv, w.head_dim, w.block, w.dtype, 1.0,
                   float(src["k_scale"]), float(src["v_scale"]), scale)
    cdt = {"fp8": torch.float8_e4m3fn, "bf16": torch.bfloat16}[w.dtype]
    table = src["block_table"].to(DEV) if w.paged else None
    shape = (src["num_pages"], w.page_size, w.hkv, w.head_dim) if w.paged else (w.batch, w.seq, w.hkv, w.head_dim)
    page = w.page_size if w.paged else 0
    kc = torch.empty(shape, dtype=cdt, device=DEV)
    vc = torch.empty_like(kc)
    kbar, lvn = sb.cache_write(p, src["k"].to(DEV), src["v"].to(DEV), kc, vc, table, page)
    q, q_scale = wl.make_decode_query(w, 3, DEV)
    p.q_scale = q_scale
    lens = [w.seq, w.seq - 77][:w.batch]
    keepv = []
    for n in lens:
        I = (n - 1) // w.block
        budget, _ = sb.stem_tpd_budget(I + 1, w.density, w.alpha)
        keepv.append(budget[I])
    lens_t = torch.tensor(lens, dtype=torch.int32, device=DEV)
    keep_t = torch.tensor(keepv, dtype=torch.int32, device=DEV)
    o, lse = sb.decode(p, q, kc, vc, lens_t, keep_t, kbar, lvn, table, page)
    o2, lse2, skipped = sb.decode_blasst(p, q, kc, vc, lens_t, 0.3, keep_t, kbar, lvn, table, page)
    torch.cuda.synchronize()
    k_tok = wl.gather_pages(kc, table) if w.paged else kc
    v_tok = wl.gather_pages(vc, table) if w.paged else vc
    kd = oracle.dequantize(wl.to_float64(k_tok), p.k_scale)
    vd = oracle.dequantize(wl.to_float64(v_tok), p.v_scale)
    qd = oracle.dequantize(wl.to_float64(q), q_scale)
    o_ref, l_ref, _ = oracle.decode_step(qd, kd, vd, lens, w.block, keep=keepv, softmax_scale=scale)
    assert output_error(o, o_ref) < 2e-4
    assert np.max(np.abs(lse.cpu().double().numpy() - l_ref)) < 1e-4
    o_ref, l_ref, _, d_ref, closest = oracle.decode_step_blasst(qd, kd, vd, lens, w.block, 0.3, keep=keepv,
                                                                softmax_scale=scale)
    keep = closest >= SKIP_TIE
    assert keep.mean() > 0.9
    b_i, h_i = np.nonzero(keep)
    assert output_error(o2[b_i, h_i], o_ref[b_i, h_i]) < 2e-4
    assert np.max(np.abs(lse2.cpu().double().numpy()[b_i, h_i] - l_ref[b_i, h_i])) < 1e-4
    assert np.array_equal(skipped.cpu().numpy()[b_i, h_i], d_ref[b_i, h_i])
