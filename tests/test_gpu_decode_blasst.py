"""GPU parity of stem_decode_blasst (the decode step with BLASST's online
skip) through the C ABI, against the oracle's decode_step_blasst:

  * the kept lists as for stem_decode (bit-exact, or a near-tie under the
    selection's rule, whose rows are then left out);
  * rows where a skip decision lies within SKIP_TIE (natural-log units) of
    the threshold in the oracle's fp64 logits are left out (the kernels decide
    on fp32 logits); their share is printed and stays small;
  * on the other rows: the dropped-block counts exact, O within 2e-4 beyond
    the output's rounding and LSE within 1e-4 (fp32 end to end, as stem_decode);
  * lambda = 0 gives stem_decode's output bit for bit.
The cache is written by stem_cache_write over its whole capacity.  Every case
prints its name before it touches the GPU."""

from __future__ import annotations

import dataclasses

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
SKIP_TIE = 1e-3


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
    lams: list
    keep: str = "tpd"         # "tpd" (the prefill budget of the row) or "none" (dense)


CASES = [
    Case(wl.Workload("dbl-fp8-paged64-b2", 2, 128 * 12, 8, 2, 128, 128, "fp8", density=0.6, paged=True,
                     page_size=64),
         [128 * 12, 128 * 7 + 37], [1e-3, 0.3, 1.0]),
    Case(wl.Workload("dbl-bf16-d64-b64-dense", 2, 64 * 14, 4, 2, 64, 64, "bf16"), [64 * 14, 64 * 5 + 3],
         [0.05, 1.0], keep="none"),
    Case(wl.Workload("dbl-f32-paged16-d128-b64", 1, 64 * 20, 2, 1, 128, 64, "f32", paged=True, page_size=16),
         [64 * 20 - 5], [0.5]),
    Case(wl.Workload("dbl-bf16-sink-dense", 2, 128 * 16, 4, 1, 128, 128, "bf16", sink=False, sink_logit=12.0),
         [128 * 16, 128 * 11 + 90], [1e-3, 1e-2], keep="none"),
    Case(wl.Workload("dbl-fp8-sink-tpd", 1, 128 * 20, 8, 2, 128, 128, "fp8", sink=False, sink_logit=12.0),
         [128 * 20 - 1], [1e-3]),
    Case(wl.Workload("dbl-fp8-gqa3-hq12-paged32", 2, 128 * 12, 12, 4, 128, 128, "fp8", paged=True, page_size=32),
         [128 * 12, 128 * 8 + 3], [0.1]),
    # the remaining (dtype, head_dim, block) instantiations of the two passes
    Case(wl.Workload("dbl-fp8-d128-b64", 1, 64 * 20, 4, 2, 128, 64, "fp8"), [64 * 20 - 1], [0.2]),
    Case(wl.Workload("dbl-fp8-d64-b64-paged16", 1, 64 * 16, 2, 1, 64, 64, "fp8", paged=True, page_size=16),
         [64 * 16 - 7], [0.2]),
    Case(wl.Workload("dbl-fp8-d64-b128", 1, 128 * 9, 2, 1, 64, 128, "fp8"), [128 * 9 - 40], [0.2]),
    Case(wl.Workload("dbl-bf16-d128-b64-paged32", 1, 64 * 18, 4, 1, 128, 64, "bf16", paged=True, page_size=32),
         [64 * 18 - 2], [0.2]),
    Case(wl.Workload("dbl-bf16-d64-b128", 1, 128 * 10, 2, 2, 64, 128, "bf16"), [128 * 10 - 2], [0.2]),
    Case(wl.Workload("dbl-f32-d64-b64", 1, 64 * 15, 2, 1, 64, 64, "f32"), [64 * 15 - 1], [0.2]),
    Case(wl.Workload("dbl-f32-d64-b128", 1, 128 * 8, 2, 1, 64, 128, "f32"), [128 * 8 - 17], [0.2]),
    Case(wl.Workload("dbl-f32-d128-b128", 1, 128 * 8, 2, 1, 128, 128, "f32"), [128 * 8 - 5], [0.2]),
]


def _setup(w: wl.Workload, lens, keep_kind, seed=11, device_gen=None):
    src = wl.make_cache_inputs(w, device=DEV if device_gen else "cpu", gen_device=device_gen)
    p = sb.Problem(w.batch, w.seq, w.hq, w.hkv, w.head_dim, w.block, w.dtype, 1.0,
                   float(src["k_scale"]), float(src["v_scale"]))
    cdt = {"fp8": torch.float8_e4m3fn, "bf16": torch.bfloat16, "f32": torch.float32}[w.dtype]
    table = src["block_table"].to(DEV) if w.paged else None
    shape = (src["num_pages"], w.page_size, w.hkv, w.head_dim) if w.paged else (w.batch, w.seq, w.hkv, w.head_dim)
    page = w.page_size if w.paged else 0
    kc = torch.empty(shape, dtype=cdt, device=DEV)
    vc = torch.empty_like(kc)
    kbar, lvn = sb.cache_write(p, src["k"].to(DEV), src["v"].to(DEV), kc, vc, table, page)
    del src
    q, q_scale = wl.make_decode_query(w, seed, DEV)
    p.q_scale = q_scale
    lens_c = [min(max(n, 1), w.seq) for n in lens]
    keepv = None
    if keep_kind == "tpd":
        keepv = []
        for n in lens_c:
            I = (n - 1) // w.block
            budget, _ = sb.stem_tpd_budget(I + 1, w.density, w.alpha)
            keepv.append(budget[I])
    return dict(p=p, q=q, q_scale=q_scale, kc=kc, vc=vc, table=table, page=page, kbar=kbar, lvn=lvn,
                lens=torch.tensor(lens, dtype=torch.int32, device=DEV), lens_c=lens_c, keepv=keepv,
                keep=None if keepv is None else torch.tensor(keepv, dtype=torch.int32, device=DEV))


def _decode(w, s, lam):
    p = s["p"]
    o = torch.empty((w.batch, w.hq, w.head_dim), dtype=torch.float32 if w.dtype == "f32" else torch.bfloat16,
                    device=DEV)
    lse = torch.empty((w.batch, w.hq), dtype=torch.float32, device=DEV)
    skipped = torch.empty((w.batch, w.hq), dtype=torch.int32, device=DEV)
    ws = torch.empty(sb.stem_decode_blasst_workspace_size(p), dtype=torch.uint8, device=DEV)
    sb.stem_decode_blasst(p, s["q"], s["kc"], s["vc"], s["lens"], s["keep"], s["kbar"], s["lvn"], lam, o, lse,
                          skipped, ws, s["table"], s["page"])
    torch.cuda.synchronize()
    nb = w.num_blocks
    bh = w.batch * w.hq
    lists = ws[:bh * nb * 4].view(torch.int32).view(w.batch, w.hq, nb).cpu().numpy()
    off = (bh * nb * 4 + 255) // 256 * 256
    counts = ws[off:off + bh * 4].view(torch.int32).view(w.batch, w.hq).cpu().numpy()
    return o, lse, skipped, lists, counts


def _oracle_inputs(w, s, heads=None, g=None):
    k_tok = wl.gather_pages(s["kc"], s["table"]) if w.paged else s["kc"]
    v_tok = wl.gather_pages(s["vc"], s["table"]) if w.paged else s["vc"]
    if g is not None:
        k_tok, v_tok = k_tok[:, :, g:g + 1], v_tok[:, :, g:g + 1]
    kd = oracle.dequantize(wl.to_float64(k_tok), s["p"].k_scale)
    vd = oracle.dequantize(wl.to_float64(v_tok), s["p"].v_scale)
    qd = oracle.dequantize(wl.to_float64(s["q"]), s["q_scale"])
    if heads is not None:
        qd = qd[:, heads]
    return qd, kd, vd


def _compare(w, lens_c, keepv, lam, got, qd, kd, vd, heads=None):
    """Returns (rows compared, rows left out)."""
    o, lse, skipped, lists, counts = got
    hs = list(range(qd.shape[1])) if heads is None else heads
    o_ref, l_ref, kept, d_ref, closest = oracle.decode_step_blasst(qd, kd, vd, lens_c, w.block, lam, keep=keepv)
    og = o[:, hs]
    lg = lse[:, hs].cpu().double().numpy()
    sg = skipped[:, hs].cpu().numpy()
    rows = []
    out = 0
    for bi in range(qd.shape[0]):
        for j, h in enumerate(hs):
            same_list = list(lists[bi, h, :counts[bi, h]]) == kept[bi][j]
            if not same_list or closest[bi, j] < SKIP_TIE:
                out += 1
                continue
            rows.append((bi, j))
    assert out <= max(1, len(rows) // 10), (out, len(rows))
    b_i = [r[0] for r in rows]
    j_i = [r[1] for r in rows]
    assert output_error(og[b_i, j_i], o_ref[b_i, j_i]) < TOL_DEC_O
    assert np.max(np.abs(lg[b_i, j_i] - l_ref[b_i, j_i])) < TOL_DEC_LSE
    assert np.array_equal(sg[b_i, j_i], d_ref[b_i, j_i])
    return len(rows), out, float(d_ref.sum())


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.w.name)
def test_decode_blasst_equals_oracle(case):
    w = case.w
    s = _setup(w, case.lens, case.keep)
    qd, kd, vd = _oracle_inputs(w, s)
    for lam in case.lams:
        _announce(f"decode blasst {w.name} lambda={lam}")
        got = _decode(w, s, lam)
        n, out, dropped = _compare(w, s["lens_c"], s["keepv"], lam, got, qd, kd, vd)
        print(f"  rows compared {n}, left out {out}, blocks dropped {dropped:.0f}", flush=True)
        if w.sink_logit > 0:
            assert dropped > 0


@pytest.mark.parametrize("case", [CASES[0], CASES[1], CASES[2]], ids=lambda c: c.w.name)
def test_decode_blasst_lambda_zero_is_stem_decode(case):
    w = case.w
    _announce(f"decode blasst lambda=0 {w.name}")
    s = _setup(w, case.lens, case.keep)
    o1, l1, skipped, _, _ = _decode(w, s, 0.0)
    o0 = torch.empty_like(o1)
    l0 = torch.empty_like(l1)
    ws = torch.empty(sb.stem_decode_workspace_size(s["p"]), dtype=torch.uint8, device=DEV)
    sb.stem_decode(s["p"], s["q"], s["kc"], s["vc"], s["lens"], s["keep"], s["kbar"], s["lvn"], o0, l0, ws,
                   s["table"], s["page"])
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    assert int(skipped.abs().sum()) == 0


def test_decode_blasst_run_twice_bit_identical():
    case = CASES[3]
    w = case.w
    _announce(f"decode blasst twice {w.name}")
    s = _setup(w, case.lens, case.keep)
    r1 = _decode(w, s, 1e-3)
    r2 = _decode(w, s, 1e-3)
    assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1]) and torch.equal(r1[2], r2[2])


def test_decode_blasst_full_128k_sampled_groups():
    """128K tokens, 64/8 heads, fp8 paged: the new token at the last position
    of a full cache, the TPD budget, lambda = 1e-3; two KV groups against the
    oracle, on the default recipe and with a dominant sink."""
    base = wl.GQA_128K_FP8_PAGED
    for w in (base, dataclasses.replace(base, name=base.name + "-sink12", sink=False, sink_logit=12.0)):
        _announce(f"decode blasst full {w.name}")
        s = _setup(w, [w.seq], "tpd", seed=5, device_gen=DEV)
        got = _decode(w, s, 1e-3)
        group = w.hq // w.hkv
        total_dropped = 0
        for g in (0, w.hkv - 1):
            hs = list(range(g * group, (g + 1) * group))
            qd, kd, vd = _oracle_inputs(w, s, heads=hs, g=g)
            wg = dataclasses.replace(w, hq=group, hkv=1)
            n, out, dropped = _compare(wg, s["lens_c"], s["keepv"], 1e-3, got, qd, kd, vd, heads=hs)
            total_dropped += dropped
            print(f"  group {g}: rows compared {n}, left out {out}, blocks dropped {dropped:.0f}", flush=True)
        if w.sink_logit > 0:
            assert total_dropped > 0
