"""Benchmark of the Stem prefill path on one MI355X.

One step = the whole hot path over one batch: OAM scoring (pool + score
GEMM), the fused TPD budget + top-k selection, and causal block-sparse
attention over the kept blocks.  Inputs are resident in HBM before the timed
region.  The dense causal kernel (the same attention kernel without mask
logic) is timed separately as the denominator of the density ratio.

Prints one JSON line.  Default workload: 131072 tokens, 64 query / 8 KV heads,
head_dim 128, 128-token blocks, OCP FP8 E4M3 Q/K/V with per-tensor scales,
paged K/V (64-token pages, random page order), TPD density 1/4.
"""

from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import re
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import block_sparse_attention_24_amd as sb  # noqa: E402
import workloads as wl  # noqa: E402

METRIC = "BSA prefill ms + kept-block TFLOP/s at 25% density, 128K; ratio vs dense"
PEAK_TFLOPS = {"fp8": 5000.0, "bf16": 2500.0, "f32": 157.3}   # MI355X dense MFMA peaks
HBM_PEAK_GBS = 8000.0

WORKLOADS = {w.name: w for w in wl.ALL}
# the attention kernels and the launcher that runs them on the measured path
ATTN_SRC = [os.path.join(ROOT, "block_sparse_attention_24_amd", "csrc", f) for f in ("bsa_kernels.h", "bsa.hip")]
PROFILES = os.path.join(ROOT, "profiles")


def attn_kernel_name(w: wl.Workload) -> str:
    return "bsa_fp8_kernel" if (w.dtype, w.head_dim, w.block) == ("fp8", 128, 128) else "bsa_kernel"


def attn_source_hash() -> str:
    """sha256 of the attention source with comments and whitespace removed, so
    that only a change of the code itself retires a recorded measurement."""
    code = ""
    for path in ATTN_SRC:
        with open(path, encoding="utf-8") as f:
            code += "".join(line.split("//", 1)[0] for line in f)
    return hashlib.sha256("".join(code.split()).encode()).hexdigest()


def measured_traffic(w: wl.Workload, kernel: str):
    """HBM bytes per launch of the sparse attention kernel on workload w, from
    the rocprofv3 FETCH_SIZE/WRITE_SIZE summaries under profiles/ (a line
    `traffic: <kernel> <workload> density=<d> bytes=<n> source_sha256=<h>`,
    h = attn_source_hash() when the counters were taken).  None if no summary
    covers this kernel and workload, or if the attention code has changed since.
    Run `python bench.py --source-hash` to print the current hash."""
    sha = attn_source_hash()
    pat = re.compile(r"traffic: (\S+) (\S+) density=(\S+) bytes=(\d+) source_sha256=([0-9a-f]+)")
    for name in sorted(os.listdir(PROFILES)) if os.path.isdir(PROFILES) else []:
        with open(os.path.join(PROFILES, name), encoding="utf-8") as f:
            for m in pat.finditer(f.read()):
                if (m.group(1), m.group(2), float(m.group(3))) == (kernel, w.name, w.density) and m.group(5) == sha:
                    return int(m.group(4))
    return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def visible_pairs(nb: int, block: int, kept_blocks: int) -> int:
    """(query, key) pairs attended per head: full B x B tiles for the kept
    blocks off the diagonal, the causal triangle for each diagonal block."""
    return block * block * (kept_blocks - nb) + nb * block * (block + 1) // 2


def attn_flops(w: wl.Workload, kept_blocks_per_head: int) -> float:
    """Algorithmic FLOPs: 2*d for q.k plus 2*d for p*v per visible pair."""
    return 4.0 * w.head_dim * w.hq * w.batch * visible_pairs(w.num_blocks, w.block, kept_blocks_per_head)


def score_bytes(w: wl.Workload) -> float:
    """Algorithmic HBM bytes of the scoring pass: read Q, K, V once, write the
    pooled representations and the scores on and below the diagonal (the GEMM
    re-reads the pooled rows, a few MiB, not counted)."""
    es = {"f32": 4, "bf16": 2, "fp8": 1}[w.dtype]
    nb = w.num_blocks
    read = w.batch * w.seq * (w.hq + 2 * w.hkv) * w.head_dim * es
    write = 4 * w.batch * nb * ((w.hq + w.hkv) * w.head_dim + w.hkv) + 4 * w.batch * w.hq * nb * (nb + 1) // 2
    return float(read + write)


def cache_write_bytes(w: wl.Workload) -> float:
    """Algorithmic HBM bytes of a KV-cache write: read the new K and V (bf16,
    or fp32 for an fp32 cache), write them in the cache type, write kbar and
    lvn."""
    es_out = {"f32": 4, "bf16": 2, "fp8": 1}[w.dtype]
    es_in = 4 if w.dtype == "f32" else 2
    n = w.batch * w.seq * w.hkv * w.head_dim
    return float(2 * n * (es_in + es_out) + 4 * w.batch * w.hkv * w.num_blocks * (w.head_dim + 1))


def pooled_score_bytes(w: wl.Workload) -> float:
    """Algorithmic HBM bytes of scoring from precomputed kbar/lvn: read Q,
    kbar and lvn, write qbar and the scores on and below the diagonal."""
    es = {"f32": 4, "bf16": 2, "fp8": 1}[w.dtype]
    nb = w.num_blocks
    read = w.batch * w.seq * w.hq * w.head_dim * es + 4 * w.batch * w.hkv * nb * (w.head_dim + 1)
    write = 4 * w.batch * w.hq * nb * w.head_dim + 4 * w.batch * w.hq * nb * (nb + 1) // 2
    return float(read + write)


def time_cache_write(w: wl.Workload, p, q, runs: int):
    """The step before the path, timed on its own: the fused KV-cache write
    (new bf16/fp32 K and V -> cache + kbar + lvn), then scoring from those
    representations (Q pooled, score GEMM)."""
    dev = "cuda"
    src = wl.make_cache_inputs(w, device=dev, gen_device=dev)
    pc = dataclasses.replace(p, k_scale=float(src["k_scale"]), v_scale=float(src["v_scale"]))
    cdt = {"fp8": torch.float8_e4m3fn, "bf16": torch.bfloat16, "f32": torch.float32}[w.dtype]
    if w.paged:
        shape, table, page = (src["num_pages"], w.page_size, w.hkv, w.head_dim), src["block_table"], w.page_size
    else:
        shape, table, page = (w.batch, w.seq, w.hkv, w.head_dim), None, 0
    kc = torch.empty(shape, dtype=cdt, device=dev)
    vc = torch.empty_like(kc)
    nb = w.num_blocks
    kbar = torch.empty((w.batch, w.hkv, nb, w.head_dim), dtype=torch.float32, device=dev)
    lvn = torch.empty((w.batch, w.hkv, nb), dtype=torch.float32, device=dev)
    scores = torch.empty((w.batch, w.hq, nb, nb), dtype=torch.float32, device=dev)
    ws = torch.empty(sb.stem_score_workspace_size(pc), dtype=torch.uint8, device=dev)
    t_cw, t_sp = Timer(), Timer()
    sb.stem_cache_write(pc, src["k"], src["v"], kc, vc, kbar, lvn, table, page)
    sb.stem_score_pooled(pc, q, kbar, lvn, scores, ws)
    for _ in range(runs):
        with t_cw:
            sb.stem_cache_write(pc, src["k"], src["v"], kc, vc, kbar, lvn, table, page)
        with t_sp:
            sb.stem_score_pooled(pc, q, kbar, lvn, scores, ws)
    torch.cuda.synchronize()
    cw_ms = sum(t_cw.ms()) / runs
    sp_ms = sum(t_sp.ms()) / runs
    del src, kc, vc, scores
    return {
        "cache_write_ms": cw_ms,
        "cache_write_gbs": cache_write_bytes(w) / (cw_ms * 1e-3) / 1e9,
        "cache_write_hbm_frac": cache_write_bytes(w) / (cw_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "score_pooled_ms": sp_ms,
        "score_pooled_gbs": pooled_score_bytes(w) / (sp_ms * 1e-3) / 1e9,
    }


def time_decode(w: wl.Workload, p, k, v, table, page, ws_score, runs: int):
    """One decode step over the full cache of the workload (the new token at
    position seq_len - 1, keeping the TPD budget of the last row), with the
    block representations stem_score left in its workspace.  Reports the step
    time and the HBM bytes of the kept K/V blocks: summed over query heads
    (what a per-head kernel requests) and as the union over each KV group's
    heads (the least any kernel must read)."""
    dev = "cuda"
    nb = w.num_blocks
    g = torch.Generator(device=dev).manual_seed(w.seed + 7)
    q32 = torch.randn((w.batch, w.hq, w.head_dim), generator=g, device=dev)
    pd = dataclasses.replace(p)
    if w.dtype == "fp8":
        q, qs = wl.quantize_fp8(q32)
        pd.q_scale = float(qs)
    else:
        q = q32.to(torch.bfloat16 if w.dtype == "bf16" else torch.float32)
    budget, _ = sb.stem_tpd_budget(nb, w.density, w.alpha)
    lens = torch.full((w.batch,), w.seq, dtype=torch.int32, device=dev)
    keep = torch.full((w.batch,), budget[nb - 1], dtype=torch.int32, device=dev)
    al = lambda x: (x + 255) // 256 * 256
    nq = w.batch * w.hq * nb * w.head_dim * 4
    nk = w.batch * w.hkv * nb * w.head_dim * 4
    kbar = ws_score[al(nq):al(nq) + nk].view(torch.float32).view(w.batch, w.hkv, nb, w.head_dim)
    lvn = ws_score[al(nq) + al(nk):al(nq) + al(nk) + w.batch * w.hkv * nb * 4].view(torch.float32)
    odt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    o = torch.empty((w.batch, w.hq, w.head_dim), dtype=odt, device=dev)
    lse = torch.empty((w.batch, w.hq), dtype=torch.float32, device=dev)
    ws = torch.empty(sb.stem_decode_workspace_size(pd), dtype=torch.uint8, device=dev)
    t = Timer()
    sb.stem_decode(pd, q, k, v, lens, keep, kbar, lvn, o, lse, ws, table, page)
    for _ in range(runs):
        with t:
            sb.stem_decode(pd, q, k, v, lens, keep, kbar, lvn, o, lse, ws, table, page)
    torch.cuda.synchronize()
    st = t.stats()
    ms = st["mean"]
    es = {"f32": 4, "bf16": 2, "fp8": 1}[w.dtype]
    block_bytes = 2 * w.block * w.head_dim * es           # K and V of one block, one KV head
    lists = ws[:w.batch * w.hq * nb * 4].view(torch.int32).view(w.batch, w.hq, nb)
    kept = budget[nb - 1]
    per_head = w.batch * w.hq * kept * block_bytes
    group = w.hq // w.hkv
    union = 0
    for bi in range(w.batch):
        for gg in range(w.hkv):
            union += int(torch.unique(lists[bi, gg * group:(gg + 1) * group, :kept]).numel())
    union *= block_bytes
    return {
        "decode_ms": ms,
        "decode_ms_stats": st,
        "kept_blocks_per_head": kept,
        "kv_bytes_group_union": union,
        "kv_bytes_requested_per_head_sum": per_head,
        "gbs_group_union": union / (ms * 1e-3) / 1e9,
        "hbm_frac_group_union": union / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "gbs_requested_per_head_sum": per_head / (ms * 1e-3) / 1e9,
    }


def time_decode_pair(w: wl.Workload, p, q, k, v, table, page, kbar, lvn, lam: float, runs: int):
    """One decode step over the full cache (the new token at the last
    position, row Nb-1's TPD budget) with and without the online skip: ms of
    each, the blocks dropped per row, and the V bytes the dropped blocks
    did not read."""
    dev = "cuda"
    nb = w.num_blocks
    budget, _ = sb.stem_tpd_budget(nb, w.density, w.alpha)
    lens = torch.full((w.batch,), w.seq, dtype=torch.int32, device=dev)
    keep = torch.full((w.batch,), budget[nb - 1], dtype=torch.int32, device=dev)
    o = torch.empty((w.batch, w.hq, w.head_dim), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.batch, w.hq), dtype=torch.float32, device=dev)
    skipped = torch.empty((w.batch, w.hq), dtype=torch.int32, device=dev)
    ws0 = torch.empty(sb.stem_decode_workspace_size(p), dtype=torch.uint8, device=dev)
    ws1 = torch.empty(sb.stem_decode_blasst_workspace_size(p), dtype=torch.uint8, device=dev)
    plain = lambda: sb.stem_decode(p, q, k, v, lens, keep, kbar, lvn, o, lse, ws0, table, page)
    skip = lambda: sb.stem_decode_blasst(p, q, k, v, lens, keep, kbar, lvn, lam, o, lse, skipped, ws1,
                                         table, page)
    res = {}
    for name, fn in (("decode_ms", plain), ("decode_skip_ms", skip)):
        t = Timer()
        fn()
        for _ in range(runs):
            with t:
                fn()
        torch.cuda.synchronize()
        res[name] = sum(t.ms()) / runs
    es = {"bf16": 2, "fp8": 1}[w.dtype]
    dropped = float(skipped.to(torch.float64).mean())
    res.update({"lambda": lam, "kept_blocks_per_row": budget[nb - 1], "dropped_blocks_per_row": dropped,
                "v_bytes_not_read": int(skipped.to(torch.int64).sum()) * w.block * w.head_dim * es,
                "speedup": res["decode_ms"] / res["decode_skip_ms"]})
    return res


def _droppable(w: wl.Workload, mask: torch.Tensor) -> int:
    """(row, block) pairs the online skip could drop: every kept block of a
    row except its first (never dropped), summed over rows."""
    bits = torch.zeros((), dtype=torch.int64, device=mask.device)
    words = mask.view(torch.int32)
    for i in range(words.shape[-1]):
        x = words[..., i].to(torch.int64) & 0xFFFFFFFF
        for _ in range(32):
            bits = bits + (x & 1).sum()
            x = x >> 1
    return int(bits) * w.block - w.batch * w.hq * w.seq          # bits above the diagonal are zero


def time_blasst(w: wl.Workload, p, q, k, v, table, page, mask, plain_ms: float, lam: float, runs: int):
    """The attention with BLASST's online skip at threshold lam on top of the
    mask (None: every causal block): time per launch, its ratio to the same
    launch without the skip, and the share of droppable (row, block) pairs
    the rows dropped."""
    dev = "cuda"
    o = torch.empty((w.batch, w.seq, w.hq, w.head_dim), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.batch, w.hq, w.seq), dtype=torch.float32, device=dev)
    skipped = torch.empty((w.batch, w.hq, w.seq), dtype=torch.int32, device=dev)
    t = Timer()
    sb.bsa_prefill_blasst(p, q, k, v, mask, lam, o, lse, skipped, table, page)
    for _ in range(runs):
        with t:
            sb.bsa_prefill_blasst(p, q, k, v, mask, lam, o, lse, skipped, table, page)
    torch.cuda.synchronize()
    ms = sum(t.ms()) / runs
    dropped = int(skipped.to(torch.int64).sum())
    nb = w.num_blocks
    droppable = (_droppable(w, mask) if mask is not None
                 else w.batch * w.hq * w.block * (nb * (nb + 1) // 2 - nb))
    return {"lambda": lam, "ms": ms, "without_skip_ms": plain_ms, "speedup": plain_ms / ms,
            "dropped_share": dropped / max(droppable, 1)}


def blasst_report(w: wl.Workload, p, q, k, v, table, page, mask, plain_ms: float, runs: int, ws_score=None):
    """The online skip on the bench workload's Stem mask, and on the same
    shapes with a sink that every query attends to (sink_logit 12: the
    situation the skip is made for; the default recipe's random sink is
    rarely dominant), there both on the Stem mask and inside dense causal
    attention (the pages' own setting of the skip).  Also a decode step over
    each cache with and without the skip (ws_score: the workspace stem_score
    left, whose block representations the decode step scores with)."""
    dev = "cuda"
    rep = {"recipe": [time_blasst(w, p, q, k, v, table, page, mask, plain_ms, lam, runs)
                      for lam in (1e-3, 1e-2)]}
    if ws_score is not None:
        al = lambda x: (x + 255) // 256 * 256
        nb = w.num_blocks
        nq = w.batch * w.hq * nb * w.head_dim * 4
        nk = w.batch * w.hkv * nb * w.head_dim * 4
        kbar = ws_score[al(nq):al(nq) + nk].view(torch.float32).view(w.batch, w.hkv, nb, w.head_dim)
        lvn = ws_score[al(nq) + al(nk):al(nq) + al(nk) + w.batch * w.hkv * nb * 4].view(torch.float32)
        qd, qds = wl.make_decode_query(w, w.seed + 7, dev)
        pd = dataclasses.replace(p, q_scale=qds)
        rep["decode_recipe"] = time_decode_pair(w, pd, qd, k, v, table, page, kbar, lvn, 1e-3, runs * 10)
    ws_ = dataclasses.replace(w, name=w.name + "-sink12", sink=False, sink_logit=12.0)
    inp = wl.make_inputs(ws_, device=dev, gen_device=dev)
    ps = sb.Problem(w.batch, w.seq, w.hq, w.hkv, w.head_dim, w.block, w.dtype,
                    float(inp["q_scale"]), float(inp["k_scale"]), float(inp["v_scale"]))
    ks, vs = (inp["k_pages"], inp["v_pages"]) if w.paged else (inp["k"], inp["v"])
    nb = w.num_blocks
    scores = torch.empty((w.batch, w.hq, nb, nb), dtype=torch.float32, device=dev)
    wsb = torch.empty(sb.stem_score_workspace_size(ps), dtype=torch.uint8, device=dev)
    ms_ = torch.empty_like(mask)
    sb.stem_score(ps, inp["q"], ks, vs, scores, wsb, table, page)
    sb.stem_select(ps, scores, w.density, w.alpha, ms_)
    del scores
    # decode over this cache, with the block representations stem_score pooled
    al = lambda x: (x + 255) // 256 * 256
    nq = w.batch * w.hq * nb * w.head_dim * 4
    nk = w.batch * w.hkv * nb * w.head_dim * 4
    kbar = wsb[al(nq):al(nq) + nk].view(torch.float32).view(w.batch, w.hkv, nb, w.head_dim)
    lvn = wsb[al(nq) + al(nk):al(nq) + al(nk) + w.batch * w.hkv * nb * 4].view(torch.float32)
    qd, qds = wl.make_decode_query(ws_, w.seed + 7, dev)
    pd = dataclasses.replace(ps, q_scale=qds)
    rep["decode_sink_logit_12"] = time_decode_pair(ws_, pd, qd, ks, vs, table, page, kbar, lvn, 1e-3, runs * 10)
    o = torch.empty((w.batch, w.seq, w.hq, w.head_dim), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.batch, w.hq, w.seq), dtype=torch.float32, device=dev)
    t = Timer()
    sb.bsa_prefill(ps, inp["q"], ks, vs, ms_, o, lse, table, page)
    for _ in range(runs):
        with t:
            sb.bsa_prefill(ps, inp["q"], ks, vs, ms_, o, lse, table, page)
    torch.cuda.synchronize()
    sink_plain = sum(t.ms()) / runs
    t = Timer()
    sb.bsa_prefill(ps, inp["q"], ks, vs, None, o, lse, table, page)
    for _ in range(runs):
        with t:
            sb.bsa_prefill(ps, inp["q"], ks, vs, None, o, lse, table, page)
    torch.cuda.synchronize()
    sink_dense = sum(t.ms()) / runs
    del o, lse
    rep["sink_logit_12"] = [time_blasst(ws_, ps, inp["q"], ks, vs, table, page, ms_, sink_plain, lam, runs)
                            for lam in (1e-3, 1e-2)]
    rep["sink_logit_12_dense"] = [time_blasst(ws_, ps, inp["q"], ks, vs, table, page, None, sink_dense, lam, runs)
                                  for lam in (1e-3, 1e-2)]
    return rep


class Timer:
    """HIP events on the stream the library launches on (torch's current stream)."""

    def __init__(self):
        self.pairs = []

    def __enter__(self):
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)
        self.a.record()
        return self

    def __exit__(self, *exc):
        self.b.record()
        self.pairs.append((self.a, self.b))

    def ms(self):
        return [a.elapsed_time(b) for a, b in self.pairs]

    def stats(self):
        """min, median and mean of the event-timed durations (ms)."""
        x = sorted(self.ms())
        n = len(x)
        med = x[n // 2] if n % 2 else 0.5 * (x[n // 2 - 1] + x[n // 2])
        return {"min": x[0], "median": med, "mean": sum(x) / n, "runs": n}


def cpu_baseline(w: wl.Workload, inp, budget, seconds: float = 15.0):
    """The oracle, untuned, on the host cores: OAM scores of head 0, the TPD
    budget, the selection of head 0 and block-sparse attention of head 0 on
    query blocks sampled evenly over the sequence until about `seconds` of
    work, reported as kept-block FLOP/s."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    G = w.hq // w.hkv
    t0 = time.perf_counter()
    qh = oracle.dequantize(wl.to_float64(inp["q"][:1, :, 0:1]), inp["q_scale"])
    kh = oracle.dequantize(wl.to_float64(inp["k"][:1, :, 0:1]), inp["k_scale"])
    vh = oracle.dequantize(wl.to_float64(inp["v"][:1, :, 0:1]), inp["v_scale"])
    t_conv = time.perf_counter() - t0
    t0 = time.perf_counter()
    s = oracle.oam_scores(qh, kh, vh, w.block)
    k_budget, _ = oracle.tpd_budget(w.num_blocks, w.density, w.alpha)
    mask = oracle.select_blocks(s, k_budget)
    t_sel = time.perf_counter() - t0
    nb = w.num_blocks
    order = []
    stride = max(1, nb // 64)
    for start in range(stride):
        order.extend(range(nb - 1 - start, -1, -stride))
    flops = 0.0
    done = 0
    t_attn = 0.0
    for i_blk in order:
        t0 = time.perf_counter()
        rows = [(0, 0, t) for t in range(i_blk * w.block, (i_blk + 1) * w.block)]
        oracle.attention_rows(qh, kh, vh, mask, w.block, rows)
        t_attn += time.perf_counter() - t0
        kept = int(mask[0, 0, i_blk, :i_blk + 1].sum())
        flops += 4.0 * w.head_dim * (w.block * w.block * (kept - 1) + w.block * (w.block + 1) // 2)
        done += 1
        if t_attn + t_sel > seconds:
            break
    # whole-head selection cost is charged pro rata to the sampled blocks
    t_total = t_attn + t_sel * done / nb
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": (f"head 0 (KV head {0 // G}): OAM scores, TPD budget and selection of all "
                       f"{nb} rows (time charged pro rata), then block-sparse attention of "
                       f"{done} of {nb} query blocks spread over the sequence; "
                       f"{flops / 1e9:.2f} GFLOP in {t_total:.1f} s (+{t_conv:.1f} s fp64 upcast, not charged)")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=wl.GQA_128K_FP8_PAGED.name, choices=sorted(WORKLOADS))
    ap.add_argument("--density", type=float, default=None)
    ap.add_argument("--dense-steps", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip timing one decode step over the full cache")
    ap.add_argument("--no-cache-write", action="store_true",
                    help="skip timing the fused KV-cache write and scoring from its output")
    ap.add_argument("--no-blasst", action="store_true",
                    help="skip timing the attention with BLASST's online skip")
    ap.add_argument("--source-hash", action="store_true",
                    help="print the attention source hash recorded next to measured traffic, and exit")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one 1 GiB device copy first (a known-size reference for HBM byte counters)")
    args = ap.parse_args()
    if args.source_hash:
        print(attn_source_hash())
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    w = WORKLOADS[args.workload]
    if args.density is not None:
        w = dataclasses.replace(w, density=args.density)
    dev = "cuda"
    torch.cuda.init()
    log(f"[bench] workload {w.name} density {w.density}: generating inputs", )
    inp = wl.make_inputs(w, device=dev, gen_device=dev)
    p = sb.Problem(w.batch, w.seq, w.hq, w.hkv, w.head_dim, w.block, w.dtype,
                   float(inp["q_scale"]), float(inp["k_scale"]), float(inp["v_scale"]))
    if w.paged:
        k, v, table, page = inp["k_pages"], inp["v_pages"], inp["block_table"], w.page_size
    else:
        k, v, table, page = inp["k"], inp["v"], None, 0
    q = inp["q"]
    nb = w.num_blocks
    budget, total = sb.stem_tpd_budget(nb, w.density, w.alpha)
    kept_flops = attn_flops(w, total)
    dense_flops = attn_flops(w, nb * (nb + 1) // 2)

    # buffers (allocated once, outside the timed region)
    scores = torch.empty((w.batch, w.hq, nb, nb), dtype=torch.float32, device=dev)
    ws = torch.empty(sb.stem_score_workspace_size(p), dtype=torch.uint8, device=dev)
    mask = torch.empty((w.batch, w.hq, nb, p.mask_words), dtype=torch.int32, device=dev)
    odt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    o = torch.empty((w.batch, w.seq, w.hq, w.head_dim), dtype=odt, device=dev)
    lse = torch.empty((w.batch, w.hq, w.seq), dtype=torch.float32, device=dev)

    t_score, t_select, t_bsa = Timer(), Timer(), Timer()

    def step(timed: bool):
        if timed:
            with t_score:
                sb.stem_score(p, q, k, v, scores, ws, table, page)
            with t_select:
                sb.stem_select(p, scores, w.density, w.alpha, mask)
            with t_bsa:
                sb.bsa_prefill(p, q, k, v, mask, o, lse, table, page)
        else:
            sb.stem_score(p, q, k, v, scores, ws, table, page)
            sb.stem_select(p, scores, w.density, w.alpha, mask)
            sb.bsa_prefill(p, q, k, v, mask, o, lse, table, page)

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("[bench] copied 1 GiB (counter calibration)")
    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = 1e3 * wall / args.steps
    st_score, st_select, st_bsa = (t.stats() for t in (t_score, t_select, t_bsa))
    sc_ms, se_ms, bsa_ms = st_score["mean"], st_select["mean"], st_bsa["mean"]
    log(f"[bench] step {ms_step:.3f} ms: score {sc_ms:.3f} select {se_ms:.3f} bsa {bsa_ms:.3f} "
        f"(min {st_bsa['min']:.3f}, median {st_bsa['median']:.3f})")

    result = {
        "metric": METRIC,
        "value": kept_flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": w.describe(),
        "stages_ms": {"score": sc_ms, "select": se_ms, "bsa": bsa_ms},
        "stages_ms_stats": {"score": st_score, "select": st_select, "bsa": st_bsa},
        "bsa_ms": bsa_ms,
        "bsa_ms_min": st_bsa["min"],
        "bsa_ms_median": st_bsa["median"],
        "bsa_kept_tflops": kept_flops / (bsa_ms * 1e-3) / 1e12,
        "kept_tflop_per_step": kept_flops / 1e12,
        "score_gbs": score_bytes(w) / (sc_ms * 1e-3) / 1e9,
        "score_hbm_frac": score_bytes(w) / (sc_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
    }
    peak = PEAK_TFLOPS[w.dtype]
    kname = attn_kernel_name(w)
    traffic = measured_traffic(w, kname)
    result["roofline"] = {"bound": "mfma", "kernel": kname + " (sparse)",
                          "achieved": result["bsa_kept_tflops"], "peak": peak, "unit": "TFLOP/s",
                          "frac": result["bsa_kept_tflops"] / peak, "traffic": traffic,
                          "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                          "traffic_source": ("the summary under profiles/ taken on this attention source "
                                             "(not measured in this run); null once the source changed"),
                          "achieved_from": "mean of the HIP-event durations of the timed launches"}

    if not args.no_dense:
        log(f"[bench] dense baseline and density-1 sparse run, {args.dense_steps} each")
        full = torch.empty_like(mask)
        sb.stem_select(p, scores, 1.0, w.alpha, full)
        t_dense, t_full = Timer(), Timer()
        sb.bsa_prefill(p, q, k, v, None, o, lse, table, page)
        for _ in range(args.dense_steps):
            with t_dense:
                sb.bsa_prefill(p, q, k, v, None, o, lse, table, page)
        sb.bsa_prefill(p, q, k, v, full, o, lse, table, page)
        for _ in range(args.dense_steps):
            with t_full:
                sb.bsa_prefill(p, q, k, v, full, o, lse, table, page)
        torch.cuda.synchronize()
        st_dense, st_full = t_dense.stats(), t_full.stats()
        dense_ms, full_ms = st_dense["mean"], st_full["mean"]
        rho = kept_flops / dense_flops
        result.update({
            "dense_ms": dense_ms,
            "dense_tflops": dense_flops / (dense_ms * 1e-3) / 1e12,
            "ratio_vs_dense": bsa_ms / (w.density * dense_ms),
            "ratio_vs_dense_rho": bsa_ms / (rho * dense_ms),
            "skip_overhead_density1": full_ms / dense_ms - 1.0,
            "density1_sparse_ms": full_ms,
            "dense_ms_stats": st_dense,
            "density1_sparse_ms_stats": st_full,
            "ratio_vs_dense_median": st_bsa["median"] / (w.density * st_dense["median"]),
        })
        log(f"[bench] dense {dense_ms:.3f} ms, density-1 sparse {full_ms:.3f} ms, "
            f"R {result['ratio_vs_dense']:.3f}")

    if not args.no_decode:
        log(f"[bench] decode step over the full cache, {args.dense_steps * 10} runs")
        result["decode"] = time_decode(w, p, k, v, table, page, ws, args.dense_steps * 10)

    if not args.no_blasst and (w.head_dim, w.block) == (128, 128) and w.dtype != "f32":
        log(f"[bench] online skip (BLASST) on the Stem mask, {args.dense_steps} runs each")
        result["blasst"] = blasst_report(w, p, q, k, v, table, page, mask, bsa_ms, args.dense_steps, ws)

    if not args.no_cache_write:
        log(f"[bench] fused KV-cache write and pooled scoring, {args.dense_steps} runs each")
        result["before_the_path"] = time_cache_write(w, p, q, args.dense_steps)

    if not args.no_cpu_baseline:
        log("[bench] oracle CPU baseline (bounded sample)")
        result["cpu_baseline"] = cpu_baseline(w, inp, budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
