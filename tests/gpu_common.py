"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
binding, and bring the same inputs to the oracle as fp64 arrays."""

from __future__ import annotations

import math

import numpy as np
import torch

import block_sparse_attention_24_amd as sb
import oracle
import workloads as wl


def problem(w: wl.Workload, inp) -> sb.Problem:
    return sb.Problem(w.batch, w.seq, w.hq, w.hkv, w.head_dim, w.block, w.dtype,
                      float(inp["q_scale"]), float(inp["k_scale"]), float(inp["v_scale"]))


def kv_args(w: wl.Workload, inp, paged=None):
    paged = w.paged if paged is None else paged
    if paged:
        return inp["k_pages"], inp["v_pages"], inp["block_table"], w.page_size
    return inp["k"], inp["v"], None, 0


def run_path(w: wl.Workload, inp, density=None, alpha=None, paged=None, mask=None):
    """score -> select -> BSA on the GPU; returns a dict of device tensors.
    If `mask` is given it replaces the selected mask for the attention."""
    p = problem(w, inp)
    k, v, table, page = kv_args(w, inp, paged)
    density = w.density if density is None else density
    alpha = w.alpha if alpha is None else alpha
    scores, ws = sb.score(p, inp["q"], k, v, table, page)
    sel_mask, lst, cnt = sb.select(p, scores, density, alpha, with_list=True)
    o, lse = sb.attention(p, inp["q"], k, v, sel_mask if mask is None else mask, table, page)
    torch.cuda.synchronize()
    return dict(p=p, scores=scores, ws=ws, mask=sel_mask, list=lst, count=cnt, o=o, lse=lse)


def workspace_views(p: sb.Problem, ws: torch.Tensor):
    """qbar, kbar, lvn from the documented workspace layout."""
    nb = p.num_blocks
    al = lambda x: (x + 255) // 256 * 256
    nq = p.batch * p.num_q_heads * nb * p.head_dim * 4
    nk = p.batch * p.num_kv_heads * nb * p.head_dim * 4
    f = ws.view(torch.uint8)
    qbar = f[:nq].view(torch.float32).view(p.batch, p.num_q_heads, nb, p.head_dim)
    kbar = f[al(nq):al(nq) + nk].view(torch.float32).view(p.batch, p.num_kv_heads, nb, p.head_dim)
    off = al(nq) + al(nk)
    lvn = f[off:off + p.batch * p.num_kv_heads * nb * 4].view(torch.float32).view(p.batch, p.num_kv_heads, nb)
    return qbar, kbar, lvn


def oracle_qkv(inp, paged_w: wl.Workload | None = None):
    """fp64 dequantised Q, K, V exactly as the GPU consumed them."""
    q = oracle.dequantize(wl.to_float64(inp["q"]), inp["q_scale"])
    k = oracle.dequantize(wl.to_float64(inp["k"]), inp["k_scale"])
    v = oracle.dequantize(wl.to_float64(inp["v"]), inp["v_scale"])
    return q, k, v


def mask_bits(mask_words: torch.Tensor, nb: int) -> np.ndarray:
    return oracle.unpack_block_mask(mask_words.cpu().numpy().view(np.uint32), nb)


def near_tie_diff(gpu_mask, oracle_scores, budget, tol=1e-4):
    """Compare masks row by row under the near-tie rule: a GPU/oracle
    difference at J is allowed only if |s_oracle(J) - theta| < tol, theta the
    oracle's lowest kept candidate score of the row; the row counts must match.
    Returns (rows differing, rows with a difference outside the rule)."""
    b, hq, nb, _ = gpu_mask.shape
    want = oracle.select_blocks(oracle_scores, budget)
    differing, bad = 0, []
    for bi in range(b):
        for h in range(hq):
            for i in range(nb):
                g_row, o_row = gpu_mask[bi, h, i], want[bi, h, i]
                if g_row.sum() != o_row.sum():
                    bad.append((bi, h, i, "count"))
                    continue
                if np.array_equal(g_row, o_row):
                    continue
                differing += 1
                cands = [j for j in range(1, i) if o_row[j]]
                theta = min(oracle_scores[bi, h, i, j] for j in cands) if cands else math.inf
                for j in np.nonzero(g_row != o_row)[0]:
                    if not abs(oracle_scores[bi, h, i, j] - theta) < tol:
                        bad.append((bi, h, i, int(j)))
    return differing, bad


def output_error(o_gpu: torch.Tensor, o_ref: np.ndarray, magnitude=None):
    """Max |O_gpu - O_ref| after allowing for the output's own rounding to its
    storage type (half a bf16 ulp of the reference value), each row divided by
    its magnitude (see split_magnitude) when one is given."""
    og = o_gpu.float().cpu().numpy().astype(np.float64)
    err = np.abs(og - o_ref)
    if o_gpu.dtype == torch.bfloat16:
        mag = np.maximum(np.abs(o_ref), 2.0 ** -126)
        half_ulp = np.ldexp(1.0, np.floor(np.log2(mag)).astype(np.int64) - 8)
        err = np.maximum(err - half_ulp, 0.0)
    if magnitude is not None:
        err = err / np.asarray(magnitude, dtype=np.float64)[..., None]
    return float(err.max()) if err.size else 0.0


# Max-abs output tolerances at unit-variance inputs.
TOL_O = {"f32": 1e-4, "bf16": 1e-2, "fp8": 6e-2}
TOL_LSE = {"f32": 1e-4, "bf16": 1e-3, "fp8": 1e-3}
TOL_SCORE = 1e-4


def with_scale_column(w: wl.Workload, v64: np.ndarray, gen_device=None) -> np.ndarray:
    """The oracle's V ([b, S, H, d] fp64) with one more column: the per-token
    V-row scale s_t the inputs were drawn with (1 for every token when
    v_sigma = 0).  Attention over it returns in that column each row's
    softmax-weighted mean of the scales of the V rows it attends to."""
    sc = wl.v_row_scale(w, gen_device).cpu().double().numpy()           # [b, S]
    col = np.broadcast_to(sc[:, :, None, None], v64.shape[:-1] + (1,))
    return np.concatenate([v64, col], axis=-1)


def split_magnitude(w: wl.Workload, o_aug: np.ndarray):
    """(O, magnitude) from attention over with_scale_column's V.  The fp8 bar
    is stated for unit-variance V.  O is linear in V, and the error of rounding
    P is a weighted sum over the V rows a row attends to, so with V rows scaled
    by s_j a row's bound scales by its weighted mean scale S_i = sum_j w_ij s_j:
    the magnitude is max(1, S_i) for fp8, and 1 otherwise (bf16 and fp32 keep
    their bars unscaled)."""
    o, s = o_aug[..., :-1], o_aug[..., -1]
    if w.dtype == "fp8":
        return o, np.maximum(1.0, s)
    return o, np.ones_like(s)
