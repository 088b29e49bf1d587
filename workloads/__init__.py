"""Seeded synthetic inputs for the Stem prefill path.

This module is shared by the tests, the bench and the smoke check.  It holds
shapes, value distributions and memory layouts only, and none of the method's
arithmetic (no pooling, scoring, budget, selection or attention), so that the
oracle and the HIP path both consume it without sharing any of the
computation they are compared on.

Value recipe (standing in for model activations, which the pages measure on
but which are not available here): Q, K ~ N(0, 1); the first four tokens' K
rows scaled by 4 (an attention-sink stand-in) where asked; V ~ N(0, 1) with
every token's V row scaled by exp(N(0, 0.5^2)), one factor per token shared
by all KV heads.  Cast to the working dtype with round-to-nearest-even; FP8
inputs are quantised per tensor with scale = amax / 448 (OCP E4M3 range).

A sink that every query attends to (what trained models show at the first
tokens) is an option: with sink_logit = L > 0, every Q row gains 8 u, with
u = (1, ..., 1) / sqrt(d), and the first four K rows gain L sqrt(d) / 8 u,
so that (q . k) / sqrt(d) on those keys is L (1 + N(0, 1) / 8) plus the
keys' own N(0, 1 + 64 / d) term, while the logits on other keys widen from
N(0, 1) to N(0, 1 + 64 / d).
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import torch

FP8_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seq: int
    hq: int
    hkv: int
    head_dim: int
    block: int
    dtype: str                  # "f32" | "bf16" | "fp8"
    density: float = 0.25
    alpha: float = 0.5
    sink: bool = True           # scale K of the first 4 tokens by 4
    paged: bool = False
    page_size: int = 64
    seed: int = 0
    v_sigma: float = 0.5        # V row scale ~ LogNormal(0, v_sigma); 0 gives unit-variance V
    sink_logit: float = 0.0     # > 0: every query's logit on the first 4 tokens is about this

    @property
    def num_blocks(self) -> int:
        return self.seq // self.block

    def describe(self) -> dict:
        return {"workload": self.name, "batch": self.batch, "seq_len": self.seq,
                "q_heads": self.hq, "kv_heads": self.hkv, "head_dim": self.head_dim,
                "block": self.block, "dtype": self.dtype, "density": self.density,
                "alpha": self.alpha, "paged_kv": self.paged,
                "page_size": self.page_size if self.paged else None, "v_sigma": self.v_sigma,
                "sink_logit": self.sink_logit}


# The five workloads of the measurement plan, smallest first.
TINY_2K = Workload("tiny-2k-f32-mha", 1, 2048, 2, 2, 64, 64, "f32", sink=False)
GQA_8K = Workload("8k-bf16-gqa32x8", 1, 8192, 32, 8, 128, 128, "bf16")
GQA_64K = Workload("64k-bf16-gqa32x8", 1, 65536, 32, 8, 128, 128, "bf16")
GQA_128K_FP8_PAGED = Workload("128k-fp8-paged-gqa64x8", 1, 131072, 64, 8, 128, 128,
                              "fp8", paged=True, page_size=64)
GQA_256K = Workload("256k-bf16-gqa32x8", 1, 262144, 32, 8, 128, 128, "bf16")

ALL = [TINY_2K, GQA_8K, GQA_64K, GQA_128K_FP8_PAGED, GQA_256K]


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, seed, device):
    return torch.randn(shape, generator=_gen(seed, device), device=device, dtype=torch.float32)


def quantize_fp8(x: torch.Tensor):
    """Per-tensor OCP E4M3 quantisation: scale = amax / 448, codes = cast(x / scale)."""
    amax = float(x.abs().max())
    scale = amax / FP8_MAX if amax > 0 else 1.0
    codes = (x / scale).to(torch.float8_e4m3fn)
    return codes, scale


def _add_sink_direction(q: Optional[torch.Tensor], k: torch.Tensor, sink_logit: float):
    """q += 8 u on every row, k[:, :4] += sink_logit * sqrt(d) / 8 * u, with
    u = (1, ..., 1) / sqrt(d) (in place)."""
    d = k.shape[-1]
    u = 1.0 / d ** 0.5
    if q is not None:
        q.add_(8.0 * u)
    k[:, :4].add_(sink_logit * d ** 0.5 / 8.0 * u)


def v_row_scale(w: Workload, gen_device: Optional[str] = None) -> torch.Tensor:
    """The per-token V row scales ([b, S], on gen_device) that make_inputs
    applies: exp(v_sigma * N(0, 1)) from seed + 3."""
    return torch.exp(w.v_sigma * _randn((w.batch, w.seq), w.seed + 3, gen_device or "cpu"))


def make_inputs(w: Workload, device="cpu", gen_device: Optional[str] = None):
    """Returns a dict with
      q [b, S, Hq, d], k/v [b, S, Hkv, d]      working dtype (fp8: E4M3 codes)
      q_scale, k_scale, v_scale                 per-tensor scales (1.0 unless fp8)
      and, when paged: k_pages/v_pages [num_pages, page_size, Hkv, d] and
      block_table [b, S/page_size] int32 (a random page permutation).
    Seeds: Q = seed, K = seed+1, V = seed+2, V token scales = seed+3,
    page permutation = seed+4.  Values are drawn on `gen_device` (CPU by
    default; the large workloads draw on the GPU) and moved to `device`."""
    gd = gen_device or "cpu"
    b, S, hq, hkv, d = w.batch, w.seq, w.hq, w.hkv, w.head_dim
    q = _randn((b, S, hq, d), w.seed, gd)
    k = _randn((b, S, hkv, d), w.seed + 1, gd)
    v = _randn((b, S, hkv, d), w.seed + 2, gd)
    v.mul_(v_row_scale(w, gd)[:, :, None, None])
    if w.sink:
        k[:, :4].mul_(4.0)
    if w.sink_logit > 0:
        _add_sink_direction(q, k, w.sink_logit)
    out = {"q_scale": 1.0, "k_scale": 1.0, "v_scale": 1.0}
    if w.dtype == "f32":
        out.update(q=q, k=k, v=v)
    elif w.dtype == "bf16":
        out.update(q=q.to(torch.bfloat16), k=k.to(torch.bfloat16), v=v.to(torch.bfloat16))
    elif w.dtype == "fp8":
        for name, x in (("q", q), ("k", k), ("v", v)):
            codes, scale = quantize_fp8(x)
            out[name] = codes
            out[name + "_scale"] = scale
    else:
        raise ValueError(w.dtype)
    del q, k, v
    for name in ("q", "k", "v"):
        out[name] = out[name].to(device).contiguous()
    if w.paged:
        pages_per_seq = S // w.page_size
        num_pages = b * pages_per_seq
        perm = torch.randperm(num_pages, generator=_gen(w.seed + 4, "cpu"))
        table = perm.view(b, pages_per_seq).to(torch.int32)
        out["block_table"] = table.to(device)
        for name in ("k", "v"):
            x = out[name]
            pages = torch.empty((num_pages, w.page_size, hkv, d), dtype=x.dtype, device=device)
            pages[table.to(device).long().view(-1)] = x.view(num_pages, w.page_size, hkv, d)
            out[name + "_pages"] = pages
    return out


def make_cache_inputs(w: Workload, device="cpu", gen_device: Optional[str] = None,
                      fp8_scale: Optional[float] = None):
    """Inputs of a KV-cache write for workload w: the new K and V ([b, S, Hkv,
    d], drawn as make_inputs draws them) in the type the write reads (bf16 for
    an FP8 or bf16 cache, fp32 for an fp32 cache); k_scale / v_scale (for an
    FP8 cache amax / 448 of those values, or fp8_scale for both when given;
    else 1.0); and, when paged, the block table of make_inputs and num_pages."""
    gd = gen_device or "cpu"
    b, S, hkv, d = w.batch, w.seq, w.hkv, w.head_dim
    k = _randn((b, S, hkv, d), w.seed + 1, gd)
    v = _randn((b, S, hkv, d), w.seed + 2, gd)
    v.mul_(v_row_scale(w, gd)[:, :, None, None])
    if w.sink:
        k[:, :4].mul_(4.0)
    if w.sink_logit > 0:
        _add_sink_direction(None, k, w.sink_logit)
    out = {"k_scale": 1.0, "v_scale": 1.0}
    if w.dtype == "f32":
        out.update(k=k, v=v)
    else:
        out.update(k=k.to(torch.bfloat16), v=v.to(torch.bfloat16))
        if w.dtype == "fp8":
            for name in ("k", "v"):
                amax = float(out[name].float().abs().max())
                out[name + "_scale"] = fp8_scale if fp8_scale else (amax / FP8_MAX if amax > 0 else 1.0)
    del k, v
    for name in ("k", "v"):
        out[name] = out[name].to(device).contiguous()
    if w.paged:
        pages_per_seq = S // w.page_size
        num_pages = b * pages_per_seq
        perm = torch.randperm(num_pages, generator=_gen(w.seed + 4, "cpu"))
        out["block_table"] = perm.view(b, pages_per_seq).to(torch.int32).to(device)
        out["num_pages"] = num_pages
    return out


def make_decode_query(w: Workload, seed: int, device="cpu"):
    """The new token's query of a decode step over workload w's cache:
    q [b, Hq, d] ~ N(0, 1) from `seed` (plus the sink direction 8 u when
    sink_logit > 0), in the working dtype; returns (q, q_scale)."""
    q = torch.randn((w.batch, w.hq, w.head_dim), generator=_gen(seed, "cpu"), dtype=torch.float32)
    if w.sink_logit > 0:
        q.add_(8.0 / w.head_dim ** 0.5)
    if w.dtype == "fp8":
        codes, scale = quantize_fp8(q)
        return codes.to(device), float(scale)
    return (q.to(torch.bfloat16) if w.dtype == "bf16" else q).to(device), 1.0


def to_float64(x: torch.Tensor):
    """Exact upcast of a working-dtype tensor (fp8 codes included) to a float64
    numpy array.  Per-tensor scales are applied by the consumer."""
    return x.detach().to("cpu").to(torch.float64).numpy()


def gather_pages(pages: torch.Tensor, table: torch.Tensor):
    """Inverse of the paged layout: [num_pages, P, H, d] + [b, S/P] -> [b, S, H, d]."""
    b, n = table.shape
    x = pages[table.long().view(-1)]
    return x.view(b, n * pages.shape[1], *pages.shape[2:])


def sample_rows(w: Workload, count: int, seed: int = 1234):
    """(batch, head, token) triples for sampled checks: the first and last
    token, the first and last token of the middle block, plus `count` random
    ones."""
    g = torch.Generator().manual_seed(seed)
    rows = {(0, 0, 0), (w.batch - 1, w.hq - 1, w.seq - 1),
            (0, w.hq // 2, (w.num_blocks // 2) * w.block),
            (0, w.hq // 2, (w.num_blocks // 2) * w.block + w.block - 1)}
    while len(rows) < count + 4:
        rows.add((int(torch.randint(w.batch, (1,), generator=g)),
                  int(torch.randint(w.hq, (1,), generator=g)),
                  int(torch.randint(w.seq, (1,), generator=g))))
    return sorted(rows)
