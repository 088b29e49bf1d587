"""GPU parity of stem_decode (through the C ABI) against the oracle's
decode_step: kept blocks bit-exact except at near-ties (|delta score| < 1e-4,
the rule of the prefill selection), and O / LSE of the kept blocks within
2e-4 beyond the output's rounding (the decode path is fp32 end to end) and
1e-4.  The cache is written by stem_cache_write over its whole capacity, so
tokens past each sequence's end hold data that must not be read.  Every case
prints its name before it touches the GPU."""

from __future__ import annotations

import dataclasses
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_24_amd as sb
import oracle
import workloads as wl
from gpu_common import output_error

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL_DEC_O = 2e-4
TOL_DEC_LSE = 1e-4


def _announce(name):
    print(f"\n[case] {name}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sb.lib()
    yield


@dataclasses.dataclass
class Case:
    w: wl.Workload            # the cache: seq = capacity
    lens: list
    keep: str = "tpd"         # "tpd" (prefill budget of the row), "none" (dense) or "fixed:<n>"
    sam: bool = False


CASES = [
    Case(wl.Workload("dec-fp8-paged64-b2", 2, 128 * 12, 8, 2, 128, 128, "fp8", paged=True, page_size=64),
         [128 * 12, 128 * 7 + 37]),
    Case(wl.Workload("dec-bf16-mha-d64-b64", 3, 64 * 12, 4, 4, 64, 64, "bf16"),
         [1, 64, 64 * 9 + 1]),
    Case(wl.Workload("dec-f32-paged16-d128-b64", 1, 64 * 20, 2, 1, 128, 64, "f32", paged=True, page_size=16),
         [64 * 20 - 5]),
    Case(wl.Workload("dec-fp8-dense", 1, 128 * 9, 4, 1, 128, 128, "fp8", paged=True, page_size=128),
         [128 * 8 + 100], keep="none"),
    Case(wl.Workload("dec-bf16-sam", 2, 128 * 10, 4, 2, 128, 128, "bf16"), [128 * 10, 128 * 5 + 1], sam=True),
    Case(wl.Workload("dec-fp8-d64-keep-clamped", 2, 64 * 40, 4, 2, 64, 64, "fp8"), [64 * 40, 64 * 31 + 7],
         keep="fixed:1000"),
    Case(wl.Workload("dec-bf16-keep-zero", 1, 128 * 8, 2, 1, 128, 128, "bf16"), [128 * 8 - 1], keep="fixed:0"),
    Case(wl.Workload("dec-bf16-len-clamped", 2, 128 * 4, 2, 1, 128, 128, "bf16"), [0, 10 ** 6]),
    # a GQA group of 3 with batch 3 and 32-token pages; a group of 80 query
    # heads, more than the scoring kernel stages at a time
    Case(wl.Workload("dec-fp8-gqa3-hq12-b3-paged32", 3, 128 * 10, 12, 4, 128, 128, "fp8", paged=True,
                     page_size=32), [128 * 10, 128 * 6 + 5, 77]),
    Case(wl.Workload("dec-bf16-g80-d64-b64", 1, 64 * 16, 80, 1, 64, 64, "bf16"), [64 * 16 - 9]),
    # the remaining (dtype, head_dim, block) instantiations of the decode kernels
    Case(wl.Workload("dec-fp8-d128-b64", 1, 64 * 20, 4, 2, 128, 64, "fp8"), [64 * 20 - 1]),
    Case(wl.Workload("dec-fp8-d64-b128-paged32", 1, 128 * 9, 2, 1, 64, 128, "fp8", paged=True, page_size=32),
         [128 * 9 - 40]),
    Case(wl.Workload("dec-bf16-d128-b64-paged16", 2, 64 * 18, 4, 1, 128, 64, "bf16", paged=True, page_size=16),
         [64 * 18, 64 * 7 + 3]),
    Case(wl.Workload("dec-bf16-d64-b128", 1, 128 * 10, 2, 2, 64, 128, "bf16"), [128 * 10 - 2]),
    Case(wl.Workload("dec-f32-d64-b64", 1, 64 * 15, 2, 1, 64, 64, "f32"), [64 * 15 - 1]),
    Case(wl.Workload("dec-f32-d64-b128-paged64", 1, 128 * 8, 2, 1, 64, 128, "f32", paged=True, page_size=64),
         [128 * 8 - 17]),
    Case(wl.Workload("dec-f32-d128-b128", 1, 128 * 8, 2, 1, 128, 128, "f32"), [128 * 8 - 5]),
    # 1,500 and 3,000 key blocks: the 32- and 64-chunk selection instantiations
    Case(wl.Workload("dec-bf16-nb1500-d64-b64", 1, 64 * 1500, 2, 1, 64, 64, "bf16"), [64 * 1500 - 3],
         keep="fixed:150"),
    Case(wl.Workload("dec-fp8-nb3000-d64-b64-paged16", 2, 64 * 3000, 2, 1, 64, 64, "fp8", paged=True,
                     page_size=16), [64 * 3000, 64 * 2222 + 9], keep="fixed:300"),
]


def _keep_values(case: Case, lens):
    if case.keep == "none":
        return None
    out = []
    for n in lens:
        n = min(max(n, 1), case.w.seq)
        I = (n - 1) // case.w.block
        if case.keep == "tpd":
            budget, _ = sb.stem_tpd_budget(I + 1, case.w.density, case.w.alpha)
            out.append(budget[I])
        else:
            out.append(int(case.keep.split(":")[1]))
    return out


def _query(w: wl.Workload, seed: int):
    g = torch.Generator().manual_seed(seed)
    q32 = torch.randn((w.batch, w.hq, w.head_dim), generator=g)
    if w.dtype == "fp8":
        codes, scale = wl.quantize_fp8(q32)
        return codes, float(scale)
    return (q32.to(torch.bfloat16) if w.dtype == "bf16" else q32), 1.0


def _run(case: Case, seed: int = 11):
    w = case.w
    src = wl.make_cache_inputs(w, device="cpu")
    p = sb.Problem(w.batch, w.seq, w.hq, w.hkv, w.head_dim, w.block, w.dtype, 1.0,
                   float(src["k_scale"]), float(src["v_scale"]))
    cdt = {"fp8": torch.float8_e4m3fn, "bf16": torch.bfloat16, "f32": torch.float32}[w.dtype]
    if w.paged:
        table = src["block_table"].to(DEV)
        shape = (src["num_pages"], w.page_size, w.hkv, w.head_dim)
    else:
        table = None
        shape = (w.batch, w.seq, w.hkv, w.head_dim)
    page = w.page_size if w.paged else 0
    kc = torch.empty(shape, dtype=cdt, device=DEV)
    vc = torch.empty_like(kc)
    kbar, lvn = sb.cache_write(p, src["k"].to(DEV), src["v"].to(DEV), kc, vc, table, page)
    q, q_scale = _query(w, seed)
    p.q_scale = q_scale
    q = q.to(DEV)
    lens = torch.tensor(case.lens, dtype=torch.int32, device=DEV)
    keepv = _keep_values(case, case.lens)
    keep = None if keepv is None else torch.tensor(keepv, dtype=torch.int32, device=DEV)
    odt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    o = torch.empty((w.batch, w.hq, w.head_dim), dtype=odt, device=DEV)
    lse = torch.empty((w.batch, w.hq), dtype=torch.float32, device=DEV)
    ws = torch.empty(sb.stem_decode_workspace_size(p), dtype=torch.uint8, device=DEV)
    sb.stem_decode(p, q, kc, vc, lens, keep, kbar, None if case.sam else lvn, o, lse, ws, table, page)
    torch.cuda.synchronize()
    nb = w.num_blocks
    bh = w.batch * w.hq
    lists = ws[:bh * nb * 4].view(torch.int32).view(w.batch, w.hq, nb).cpu().numpy()
    off = (bh * nb * 4 + 255) // 256 * 256
    counts = ws[off:off + bh * 4].view(torch.int32).view(w.batch, w.hq).cpu().numpy()
    # the oracle sees exactly the stored cache, in token order, dequantised
    k_tok = wl.gather_pages(kc, table) if w.paged else kc
    v_tok = wl.gather_pages(vc, table) if w.paged else vc
    kd = oracle.dequantize(wl.to_float64(k_tok), p.k_scale)
    vd = oracle.dequantize(wl.to_float64(v_tok), p.v_scale)
    qd = oracle.dequantize(wl.to_float64(q), q_scale)
    return dict(p=p, o=o, lse=lse, lists=lists, counts=counts, q=qd, k=kd, v=vd, keep=keepv)


def _check(case: Case, r):
    w = case.w
    lens = [min(max(n, 1), w.seq) for n in case.lens]
    o_ref, lse_ref, kept = oracle.decode_step(r["q"], r["k"], r["v"], lens, w.block, keep=r["keep"],
                                              value_term=not case.sam)
    tau = 1 / math.sqrt(w.head_dim)
    group = w.hq // w.hkv
    near = 0
    for bi in range(w.batch):
        t = lens[bi] - 1
        I = t // w.block
        for h in range(w.hq):
            want = kept[bi][h]
            got = list(r["lists"][bi, h, :r["counts"][bi, h]])
            assert r["counts"][bi, h] == len(want), (bi, h)
            if got != want:
                # near-tie rule: every differing block scores within 1e-4 of the
                # oracle's lowest kept candidate
                near += 1
                g = h // group
                done = slice(bi, bi + 1), slice(0, I * w.block)
                _, kbar, lvn = oracle.pool_blocks(r["k"][done], r["k"][done], r["v"][done], w.block)
                s = tau * (kbar[0, g] @ r["q"][bi, h]) + (0 if case.sam else lvn[0, g])
                cands = [j for j in want if 0 < j < I]
                theta = min(s[j] for j in cands)
                for j in set(got) ^ set(want):
                    assert abs(s[j] - theta) < 1e-4, (bi, h, j)
                # compare the output on the GPU's own selection
                q_full = np.zeros((1, (I + 1) * w.block, w.hq, w.head_dim))
                q_full[0, t] = r["q"][bi]
                mrow = np.zeros(I + 1, dtype=bool)
                mrow[got] = True
                oo, ll = oracle.attention_rows(q_full, r["k"][bi:bi + 1, :(I + 1) * w.block],
                                               r["v"][bi:bi + 1, :(I + 1) * w.block],
                                               lambda *_: mrow, w.block, [(0, h, t)])
                o_ref[bi, h], lse_ref[bi, h] = oo[0], ll[0]
    assert output_error(r["o"], o_ref) < TOL_DEC_O
    assert np.max(np.abs(r["lse"].cpu().double().numpy() - lse_ref)) < TOL_DEC_LSE
    return near


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.w.name)
def test_decode_small(case):
    _announce(f"decode {case.w.name}")
    r = _run(case)
    near = _check(case, r)
    print(f"[case] rows decided at near-ties: {near}", flush=True)


def test_decode_run_twice_bit_identical():
    case = CASES[0]
    _announce(f"decode twice {case.w.name}")
    r1 = _run(case)
    r2 = _run(case)
    assert torch.equal(r1["o"], r2["o"]) and torch.equal(r1["lse"], r2["lse"])
    assert np.array_equal(r1["counts"], r2["counts"])
    for bi in range(case.w.batch):
        for h in range(case.w.hq):
            n = r1["counts"][bi, h]                # entries past the count are undefined
            assert np.array_equal(r1["lists"][bi, h, :n], r2["lists"][bi, h, :n])


def test_decode_full_128k_sampled_heads():
    """128K tokens, 64/8 heads, fp8 paged (64-token pages), density 1/4: the
    new token at the last position of a full cache; two KV groups (16 query
    heads) checked against the oracle under the near-tie rule."""
    w = wl.GQA_128K_FP8_PAGED
    _announce(f"decode full {w.name}")
    src = wl.make_cache_inputs(w, device=DEV, gen_device=DEV)
    p = sb.Problem(w.batch, w.seq, w.hq, w.hkv, w.head_dim, w.block, w.dtype, 1.0,
                   float(src["k_scale"]), float(src["v_scale"]))
    shape = (src["num_pages"], w.page_size, w.hkv, w.head_dim)
    kc = torch.empty(shape, dtype=torch.float8_e4m3fn, device=DEV)
    vc = torch.empty_like(kc)
    table = src["block_table"]
    kbar, lvn = sb.cache_write(p, src["k"], src["v"], kc, vc, table, w.page_size)
    del src
    q, q_scale = _query(w, 5)
    p.q_scale = q_scale
    nb = w.num_blocks
    budget, _ = sb.stem_tpd_budget(nb, w.density, w.alpha)
    lens = torch.tensor([w.seq], dtype=torch.int32, device=DEV)
    keep = torch.tensor([budget[nb - 1]], dtype=torch.int32, device=DEV)
    o = torch.empty((1, w.hq, w.head_dim), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((1, w.hq), dtype=torch.float32, device=DEV)
    ws = torch.empty(sb.stem_decode_workspace_size(p), dtype=torch.uint8, device=DEV)
    sb.stem_decode(p, q.to(DEV), kc, vc, lens, keep, kbar, lvn, o, lse, ws, table, w.page_size)
    torch.cuda.synchronize()
    lists = ws[:w.hq * nb * 4].view(torch.int32).view(w.hq, nb).cpu().numpy()
    k_tok = wl.gather_pages(kc, table)
    v_tok = wl.gather_pages(vc, table)
    qd = oracle.dequantize(wl.to_float64(q), q_scale)
    group = w.hq // w.hkv
    for g in (0, w.hkv - 1):
        kd = oracle.dequantize(wl.to_float64(k_tok[:, :, g:g + 1]), p.k_scale)
        vd = oracle.dequantize(wl.to_float64(v_tok[:, :, g:g + 1]), p.v_scale)
        hs = list(range(g * group, (g + 1) * group))
        sub = Case(dataclasses.replace(w, hq=group, hkv=1), [w.seq])
        r = dict(q=qd[:, hs], k=kd, v=vd, keep=[budget[nb - 1]], o=o[:, hs], lse=lse[:, hs],
                 lists=lists[hs][None], counts=np.full((1, group), budget[nb - 1]))
        _check(sub, r)


def test_decode_cache_beyond_4gib():
    """A paged FP8 cache of more than 4 GiB per tensor, with the sequence's pages
    placed past the 4 GiB mark: the decode step takes its 64-bit-offset kernels
    (below 4 GiB it uses 32-bit offsets) and returns, bit for bit, what the same
    pages give in a small cache."""
    case = Case(wl.Workload("dec-fp8-paged64-beyond4g", 1, 128 * 12, 4, 1, 128, 128, "fp8", paged=True,
                            page_size=64), [128 * 12 - 3])
    w = case.w
    _announce(f"decode {w.name}")
    src = wl.make_cache_inputs(w, device="cpu")
    p = sb.Problem(w.batch, w.seq, w.hq, w.hkv, w.head_dim, w.block, w.dtype, 1.0,
                   float(src["k_scale"]), float(src["v_scale"]))
    table = src["block_table"].to(DEV)
    small = (src["num_pages"], w.page_size, w.hkv, w.head_dim)
    kc = torch.empty(small, dtype=torch.float8_e4m3fn, device=DEV)
    vc = torch.empty_like(kc)
    kbar, lvn = sb.cache_write(p, src["k"].to(DEV), src["v"].to(DEV), kc, vc, table, w.page_size)
    page_bytes = w.page_size * w.hkv * w.head_dim                 # one byte per element
    shift = (1 << 32) // page_bytes                                # pages below the 4 GiB mark
    big = (shift + src["num_pages"], w.page_size, w.hkv, w.head_dim)
    kb = torch.empty(big, dtype=torch.float8_e4m3fn, device=DEV)   # 4 GiB and more, left unwritten below
    vb = torch.empty_like(kb)
    kb[shift:] = kc
    vb[shift:] = vc
    table_big = (table + shift).contiguous()
    q, q_scale = _query(w, 11)
    p.q_scale = q_scale
    q = q.to(DEV)
    lens = torch.tensor(case.lens, dtype=torch.int32, device=DEV)
    keep = torch.tensor(_keep_values(case, case.lens), dtype=torch.int32, device=DEV)
    outs = []
    for k_, v_, t_ in ((kc, vc, table), (kb, vb, table_big)):
        o = torch.empty((w.batch, w.hq, w.head_dim), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((w.batch, w.hq), dtype=torch.float32, device=DEV)
        ws = torch.empty(sb.stem_decode_workspace_size(p), dtype=torch.uint8, device=DEV)
        sb.stem_decode(p, q, k_, v_, lens, keep, kbar, lvn, o, lse, ws, t_, w.page_size)
        outs.append((o, lse))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    del kb, vb
    torch.cuda.empty_cache()
