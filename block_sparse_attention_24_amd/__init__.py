"""Python binding of the Stem block-sparse prefill-attention library (gfx950).

Argument marshalling only: every step of the path runs in the HIP kernels of
``libstem_bsa.so`` (C ABI in ``include/stem_bsa.h``).  PyTorch supplies device
memory and the current HIP stream.  There is no fallback: if the library is
missing, every call raises.

Entry points mirror the C names:
  stem_score_workspace_size, stem_score, stem_score_noalloc, stem_score_sam, stem_score_pooled,
  stem_cache_write, stem_tpd_budget, stem_select, bsa_prefill,
  bsa_prefill_blasst, stem_decode_workspace_size, stem_decode,
  stem_decode_blasst_workspace_size, stem_decode_blasst, stem_validate_block_table,
  stem_validate_lists, stem_last_error
plus allocating conveniences ``score``, ``score_pooled``, ``cache_write``,
``select``, ``attention``, ``attention_blasst``, ``decode`` and ``decode_blasst``.
"""

from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libstem_bsa.so")

STEM_OK, STEM_EINVAL, STEM_EUNSUPPORTED, STEM_EHIP, STEM_EWORKSPACE = 0, -1, -2, -3, -4
STEM_NOALLOC_SCRATCH_BYTES = 64 << 20          # include/stem_bsa.h
STEM_F32, STEM_BF16, STEM_FP8_E4M3 = 0, 1, 2
_DTYPES = {"f32": STEM_F32, "bf16": STEM_BF16, "fp8": STEM_FP8_E4M3}
_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}
# the block mask is 32-bit words: int32 tensors (torch's usual) or uint32
_MASK = (torch.int32, torch.uint32)

EXPORTS = ("stem_score_workspace_size", "stem_score", "stem_score_noalloc", "stem_score_sam", "stem_score_pooled",
           "stem_cache_write", "stem_tpd_budget", "stem_select", "bsa_prefill", "bsa_prefill_blasst",
           "stem_decode_workspace_size", "stem_decode", "stem_decode_blasst_workspace_size",
           "stem_decode_blasst", "stem_validate_block_table", "stem_validate_lists", "stem_last_error")


class StemError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"stem error {code}: {message}")
        self.code = code


class AttnDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("q_scale", ctypes.c_float),
                ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
                ("softmax_scale", ctypes.c_float)]


class KvDesc(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("page_size", ctypes.c_int32),
                ("pages_per_seq", ctypes.c_int32), ("num_pages", ctypes.c_int32)]


_lib_handle = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m block_sparse_attention_24_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        P, I32, I64, D, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_size_t
        h.stem_score_workspace_size.argtypes = [ctypes.POINTER(AttnDesc), ctypes.POINTER(SZ)]
        h.stem_score.argtypes = [ctypes.POINTER(AttnDesc), P, ctypes.POINTER(KvDesc), P, P, SZ, P]
        h.stem_score_noalloc.argtypes = [ctypes.POINTER(AttnDesc), P, ctypes.POINTER(KvDesc), P, P]
        h.stem_score_sam.argtypes = h.stem_score.argtypes
        h.stem_score_pooled.argtypes = [ctypes.POINTER(AttnDesc), P, P, P, P, P, SZ, P]
        h.stem_cache_write.argtypes = [ctypes.POINTER(AttnDesc), P, P, ctypes.POINTER(KvDesc), P, P, P]
        h.stem_tpd_budget.argtypes = [I32, D, D, P, ctypes.POINTER(I64)]
        h.stem_select.argtypes = [ctypes.POINTER(AttnDesc), P, D, D, P, P, I32, P, P]
        h.bsa_prefill.argtypes = [ctypes.POINTER(AttnDesc), P, ctypes.POINTER(KvDesc), P, P, P, P]
        h.bsa_prefill_blasst.argtypes = [ctypes.POINTER(AttnDesc), P, ctypes.POINTER(KvDesc), P, D, P, P, P, P]
        h.stem_decode_workspace_size.argtypes = [ctypes.POINTER(AttnDesc), ctypes.POINTER(SZ)]
        h.stem_decode.argtypes = [ctypes.POINTER(AttnDesc), P, ctypes.POINTER(KvDesc), P, P, P, P,
                                  P, P, P, SZ, P]
        h.stem_decode_blasst_workspace_size.argtypes = [ctypes.POINTER(AttnDesc), ctypes.POINTER(SZ)]
        h.stem_decode_blasst.argtypes = [ctypes.POINTER(AttnDesc), P, ctypes.POINTER(KvDesc), P, P, P, P, D,
                                         P, P, P, P, SZ, P]
        h.stem_validate_block_table.argtypes = [P, I32, I32, I32, I32, I32]
        h.stem_validate_lists.argtypes = [P, P, I32, I32, I32]
        h.stem_last_error.argtypes = []
        h.stem_last_error.restype = ctypes.c_char_p
        for name in EXPORTS[:-1]:
            getattr(h, name).restype = ctypes.c_int
        _lib_handle = h
    return _lib_handle


def _check(rc: int):
    if rc != STEM_OK:
        raise StemError(rc, lib().stem_last_error().decode())


@dataclasses.dataclass
class Problem:
    """Shape and element type of one prefill problem."""
    batch: int
    seq_len: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str = "bf16"                 # "f32" | "bf16" | "fp8"
    q_scale: float = 1.0
    k_scale: float = 1.0
    v_scale: float = 1.0
    softmax_scale: float = 0.0          # 0: 1/sqrt(head_dim)

    @property
    def num_blocks(self) -> int:
        return self.seq_len // self.block_size

    @property
    def mask_words(self) -> int:
        return (self.num_blocks + 31) // 32

    def desc(self) -> AttnDesc:
        return AttnDesc(self.batch, self.seq_len, self.num_q_heads, self.num_kv_heads,
                        self.head_dim, self.block_size, _DTYPES[self.dtype], self.q_scale,
                        self.k_scale, self.v_scale, self.softmax_scale)


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None, numel: int = 0, required: bool = True):
    """Device address of tensor t, after checking what the C call reads from
    it: a contiguous GPU tensor of the given dtype(s) with at least `numel`
    elements.  None passes through as NULL unless the argument is required."""
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a tensor in GPU memory")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (a strided view would be read as if it were)")
    if dtype is not None:
        allowed = dtype if isinstance(dtype, tuple) else (dtype,)
        if t.dtype not in allowed:
            raise ValueError(f"{name} has dtype {t.dtype}, expected {' or '.join(str(x) for x in allowed)}")
    if t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, the call reads or writes {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _elem(p: Problem):
    """torch dtype of Q, K and V for the problem's element type."""
    return _TORCH[p.dtype]


def _out_dtype(p: Problem):
    return torch.float32 if p.dtype == "f32" else torch.bfloat16


def _kv(p: Problem, k, v, block_table=None, page_size=0, dtype=None):
    """stem_kv_desc for contiguous [b, S, Hkv, d] K/V, or paged
    [num_pages, page_size, Hkv, d] K/V with an int32 [b, pages_per_seq] table."""
    dt = _elem(p) if dtype is None else dtype
    row = p.num_kv_heads * p.head_dim
    if block_table is None:
        n = p.batch * p.seq_len * row
        return KvDesc(_ptr(k, "k", dt, n).value, _ptr(v, "v", dt, n).value, None, 0, 0, 0)
    if block_table.dim() != 2 or block_table.shape[0] != p.batch:
        raise ValueError("block_table must be [batch, pages_per_seq]")
    if k.dim() != 4 or k.shape[1] != page_size or v.shape != k.shape:
        raise ValueError("paged k and v must be [num_pages, page_size, num_kv_heads, head_dim]")
    n = k.shape[0] * page_size * row
    tbl = _ptr(block_table, "block_table", torch.int32, block_table.numel())
    return KvDesc(_ptr(k, "k", dt, n).value, _ptr(v, "v", dt, n).value, tbl.value, page_size,
                  block_table.shape[1], k.shape[0])


def _sizes(p: Problem):
    """Element counts of the tensors the entry points read or write."""
    b, S, hq, hkv, d, nb = p.batch, p.seq_len, p.num_q_heads, p.num_kv_heads, p.head_dim, p.num_blocks
    return dict(q=b * S * hq * d, o=b * S * hq * d, lse=b * hq * S, scores=b * hq * nb * nb,
                mask=b * hq * nb * p.mask_words, count=b * hq * nb, kbar=b * hkv * nb * d, lvn=b * hkv * nb,
                kv_in=b * S * hkv * d, dq=b * hq * d, drow=b * hq)


# ---- C entry points --------------------------------------------------------

def stem_score_workspace_size(p: Problem) -> int:
    n = ctypes.c_size_t(0)
    d = p.desc()
    _check(lib().stem_score_workspace_size(ctypes.byref(d), ctypes.byref(n)))
    return n.value


def stem_score(p: Problem, q, k, v, scores, workspace, block_table=None, page_size=0, stream=None):
    d = p.desc()
    n = _sizes(p)
    kv = _kv(p, k, v, block_table, page_size)
    _check(lib().stem_score(ctypes.byref(d), _ptr(q, "q", _elem(p), n["q"]), ctypes.byref(kv),
                            _ptr(scores, "scores", torch.float32, n["scores"]), _ptr(workspace, "workspace"),
                            workspace.numel() * workspace.element_size(), _stream(stream)))


def stem_score_noalloc(p: Problem, q, k, v, scores, block_table=None, page_size=0, stream=None):
    d = p.desc()
    n = _sizes(p)
    kv = _kv(p, k, v, block_table, page_size)
    _check(lib().stem_score_noalloc(ctypes.byref(d), _ptr(q, "q", _elem(p), n["q"]), ctypes.byref(kv),
                                    _ptr(scores, "scores", torch.float32, n["scores"]), _stream(stream)))


def stem_score_sam(p: Problem, q, k, v, scores, workspace, block_table=None, page_size=0,
                   stream=None):
    d = p.desc()
    n = _sizes(p)
    kv = _kv(p, k, v, block_table, page_size)
    _check(lib().stem_score_sam(ctypes.byref(d), _ptr(q, "q", _elem(p), n["q"]), ctypes.byref(kv),
                                _ptr(scores, "scores", torch.float32, n["scores"]), _ptr(workspace, "workspace"),
                                workspace.numel() * workspace.element_size(), _stream(stream)))


def stem_score_pooled(p: Problem, q, kbar, lvn, scores, workspace, stream=None):
    d = p.desc()
    n = _sizes(p)
    _check(lib().stem_score_pooled(ctypes.byref(d), _ptr(q, "q", _elem(p), n["q"]),
                                   _ptr(kbar, "kbar", torch.float32, n["kbar"]),
                                   _ptr(lvn, "lvn", torch.float32, n["lvn"], required=False),
                                   _ptr(scores, "scores", torch.float32, n["scores"]), _ptr(workspace, "workspace"),
                                   workspace.numel() * workspace.element_size(), _stream(stream)))


def stem_cache_write(p: Problem, k_in, v_in, k_cache, v_cache, kbar, lvn, block_table=None,
                     page_size=0, stream=None):
    d = p.desc()
    n = _sizes(p)
    in_t = torch.float32 if p.dtype == "f32" else torch.bfloat16
    kv = _kv(p, k_cache, v_cache, block_table, page_size)
    _check(lib().stem_cache_write(ctypes.byref(d), _ptr(k_in, "k_in", in_t, n["kv_in"]),
                                  _ptr(v_in, "v_in", in_t, n["kv_in"]), ctypes.byref(kv),
                                  _ptr(kbar, "kbar", torch.float32, n["kbar"]),
                                  _ptr(lvn, "lvn", torch.float32, n["lvn"]), _stream(stream)))


def stem_tpd_budget(num_blocks: int, density: float, alpha: float = 0.5):
    buf = (ctypes.c_int32 * max(num_blocks, 1))()
    total = ctypes.c_int64(0)
    _check(lib().stem_tpd_budget(num_blocks, density, alpha, ctypes.cast(buf, ctypes.c_void_p),
                                 ctypes.byref(total)))
    return [int(x) for x in buf[:num_blocks]], int(total.value)


def stem_select(p: Problem, scores, density, alpha, mask, list_out=None, list_stride=0,
                count=None, stream=None):
    d = p.desc()
    n = _sizes(p)
    _check(lib().stem_select(ctypes.byref(d), _ptr(scores, "scores", torch.float32, n["scores"]), density, alpha,
                             _ptr(mask, "mask", _MASK, n["mask"]),
                             _ptr(list_out, "list", torch.int32, n["count"] * max(list_stride, 0), required=False),
                             list_stride, _ptr(count, "count", torch.int32, n["count"], required=False),
                             _stream(stream)))


def bsa_prefill(p: Problem, q, k, v, mask, o, lse=None, block_table=None, page_size=0, stream=None):
    d = p.desc()
    n = _sizes(p)
    kv = _kv(p, k, v, block_table, page_size)
    _check(lib().bsa_prefill(ctypes.byref(d), _ptr(q, "q", _elem(p), n["q"]), ctypes.byref(kv),
                             _ptr(mask, "mask", _MASK, n["mask"], required=False),
                             _ptr(o, "o", _out_dtype(p), n["o"]),
                             _ptr(lse, "lse", torch.float32, n["lse"], required=False), _stream(stream)))


def bsa_prefill_blasst(p: Problem, q, k, v, mask, lam, o, lse=None, skipped=None, block_table=None,
                       page_size=0, stream=None):
    d = p.desc()
    n = _sizes(p)
    kv = _kv(p, k, v, block_table, page_size)
    _check(lib().bsa_prefill_blasst(ctypes.byref(d), _ptr(q, "q", _elem(p), n["q"]), ctypes.byref(kv),
                                    _ptr(mask, "mask", _MASK, n["mask"], required=False), float(lam),
                                    _ptr(o, "o", _out_dtype(p), n["o"]),
                                    _ptr(lse, "lse", torch.float32, n["lse"], required=False),
                                    _ptr(skipped, "skipped", torch.int32, n["lse"], required=False),
                                    _stream(stream)))


def stem_decode_workspace_size(p: Problem) -> int:
    n = ctypes.c_size_t(0)
    d = p.desc()
    _check(lib().stem_decode_workspace_size(ctypes.byref(d), ctypes.byref(n)))
    return n.value


def _decode_args(p: Problem, q, seq_lens, keep, kbar, lvn, o, lse):
    n = _sizes(p)
    return (_ptr(q, "q", _elem(p), n["dq"]), _ptr(seq_lens, "seq_lens", torch.int32, p.batch),
            _ptr(keep, "keep", torch.int32, p.batch, required=False),
            _ptr(kbar, "kbar", torch.float32, n["kbar"], required=False),
            _ptr(lvn, "lvn", torch.float32, n["lvn"], required=False),
            _ptr(o, "o", _out_dtype(p), n["dq"]), _ptr(lse, "lse", torch.float32, n["drow"], required=False))


def stem_decode(p: Problem, q, k, v, seq_lens, keep, kbar, lvn, o, lse, workspace,
                block_table=None, page_size=0, stream=None):
    d = p.desc()
    kv = _kv(p, k, v, block_table, page_size)
    qa, sl, kp, kb, lv, oa, la = _decode_args(p, q, seq_lens, keep, kbar, lvn, o, lse)
    _check(lib().stem_decode(ctypes.byref(d), qa, ctypes.byref(kv), sl, kp, kb, lv, oa, la,
                             _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                             _stream(stream)))


def stem_decode_blasst_workspace_size(p: Problem) -> int:
    n = ctypes.c_size_t(0)
    d = p.desc()
    _check(lib().stem_decode_blasst_workspace_size(ctypes.byref(d), ctypes.byref(n)))
    return n.value


def stem_decode_blasst(p: Problem, q, k, v, seq_lens, keep, kbar, lvn, lam, o, lse, skipped, workspace,
                       block_table=None, page_size=0, stream=None):
    d = p.desc()
    kv = _kv(p, k, v, block_table, page_size)
    qa, sl, kp, kb, lv, oa, la = _decode_args(p, q, seq_lens, keep, kbar, lvn, o, lse)
    _check(lib().stem_decode_blasst(ctypes.byref(d), qa, ctypes.byref(kv), sl, kp, kb, lv, float(lam), oa, la,
                                    _ptr(skipped, "skipped", torch.int32, _sizes(p)["drow"], required=False),
                                    _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                                    _stream(stream)))


def stem_validate_block_table(table, batch: int, pages_per_seq: int, num_pages: int, seq_len: int,
                              page_size: int) -> None:
    """Host-side check of a block table (a CPU int32 tensor or array);
    raises StemError naming the first entry outside [0, num_pages)."""
    t = torch.as_tensor(table, dtype=torch.int32).contiguous()
    _check(lib().stem_validate_block_table(ctypes.c_void_p(t.data_ptr()), batch, pages_per_seq, num_pages,
                                           seq_len, page_size))


def stem_validate_lists(lists, counts, rows: int, num_blocks: int, list_stride: int) -> None:
    """Host-side check of kept lists and counts in stem_select's layout."""
    l = torch.as_tensor(lists, dtype=torch.int32).contiguous()
    c = torch.as_tensor(counts, dtype=torch.int32).contiguous()
    if l.numel() < rows * num_blocks * list_stride or c.numel() < rows * num_blocks:
        raise ValueError("lists or counts smaller than rows * num_blocks (* list_stride)")
    _check(lib().stem_validate_lists(ctypes.c_void_p(l.data_ptr()), ctypes.c_void_p(c.data_ptr()), rows,
                                     num_blocks, list_stride))


def stem_last_error() -> str:
    return lib().stem_last_error().decode()


# ---- allocating conveniences -------------------------------------------------

def score(p: Problem, q, k, v, block_table=None, page_size=0, stream=None, sam=False):
    """Returns (scores [b,Hq,Nb,Nb] fp32, workspace bytes as uint8).  sam=True
    leaves the value term out.  The library writes J <= I only; the returned
    tensor is filled with -inf above the diagonal."""
    nb = p.num_blocks
    scores = torch.full((p.batch, p.num_q_heads, nb, nb), float("-inf"), dtype=torch.float32, device=q.device)
    ws = torch.empty(stem_score_workspace_size(p), dtype=torch.uint8, device=q.device)
    (stem_score_sam if sam else stem_score)(p, q, k, v, scores, ws, block_table, page_size, stream)
    return scores, ws


def score_pooled(p: Problem, q, kbar, lvn=None, stream=None):
    """Scores from precomputed kbar/lvn (lvn None: SAM).  Returns (scores,
    workspace); -inf above the diagonal, as score() gives."""
    nb = p.num_blocks
    scores = torch.full((p.batch, p.num_q_heads, nb, nb), float("-inf"), dtype=torch.float32, device=q.device)
    ws = torch.empty(stem_score_workspace_size(p), dtype=torch.uint8, device=q.device)
    stem_score_pooled(p, q, kbar, lvn, scores, ws, stream)
    return scores, ws


def cache_write(p: Problem, k_in, v_in, k_cache, v_cache, block_table=None, page_size=0,
                stream=None):
    """Writes K/V into the given cache tensors; returns (kbar, lvn)."""
    nb = p.num_blocks
    dev = k_in.device
    kbar = torch.empty((p.batch, p.num_kv_heads, nb, p.head_dim), dtype=torch.float32, device=dev)
    lvn = torch.empty((p.batch, p.num_kv_heads, nb), dtype=torch.float32, device=dev)
    stem_cache_write(p, k_in, v_in, k_cache, v_cache, kbar, lvn, block_table, page_size, stream)
    return kbar, lvn


def select(p: Problem, scores, density, alpha=0.5, with_list=False, stream=None):
    """Returns (mask words, list or None, count or None)."""
    nb = p.num_blocks
    dev = scores.device
    mask = torch.empty((p.batch, p.num_q_heads, nb, p.mask_words), dtype=torch.int32, device=dev)
    lst = cnt = None
    stride = 0
    if with_list:
        budget, _ = stem_tpd_budget(nb, density, alpha)
        stride = max(budget)
        lst = torch.empty((p.batch, p.num_q_heads, nb, stride), dtype=torch.int32, device=dev)
        cnt = torch.empty((p.batch, p.num_q_heads, nb), dtype=torch.int32, device=dev)
    stem_select(p, scores, density, alpha, mask, lst, stride, cnt, stream)
    return mask, lst, cnt


def attention(p: Problem, q, k, v, mask=None, block_table=None, page_size=0, with_lse=True,
              stream=None):
    """Returns (O [b,S,Hq,d], LSE [b,Hq,S] or None).  mask None = dense causal."""
    odt = torch.float32 if p.dtype == "f32" else torch.bfloat16
    o = torch.empty((p.batch, p.seq_len, p.num_q_heads, p.head_dim), dtype=odt, device=q.device)
    lse = (torch.empty((p.batch, p.num_q_heads, p.seq_len), dtype=torch.float32, device=q.device)
           if with_lse else None)
    bsa_prefill(p, q, k, v, mask, o, lse, block_table, page_size, stream)
    return o, lse


def attention_blasst(p: Problem, q, k, v, lam, mask=None, block_table=None, page_size=0,
                     with_lse=True, stream=None):
    """Attention with the online skip at threshold lam.  Returns (O, LSE or
    None, skipped [b, Hq, S] int32: blocks each row dropped)."""
    odt = torch.bfloat16
    o = torch.empty((p.batch, p.seq_len, p.num_q_heads, p.head_dim), dtype=odt, device=q.device)
    lse = (torch.empty((p.batch, p.num_q_heads, p.seq_len), dtype=torch.float32, device=q.device)
           if with_lse else None)
    skipped = torch.empty((p.batch, p.num_q_heads, p.seq_len), dtype=torch.int32, device=q.device)
    bsa_prefill_blasst(p, q, k, v, mask, lam, o, lse, skipped, block_table, page_size, stream)
    return o, lse, skipped


def decode(p: Problem, q, k, v, seq_lens, keep=None, kbar=None, lvn=None, block_table=None,
           page_size=0, stream=None):
    """One decode step.  p describes the cache (seq_len = capacity).  Returns
    (O [b, Hq, d], LSE [b, Hq])."""
    odt = torch.float32 if p.dtype == "f32" else torch.bfloat16
    o = torch.empty((p.batch, p.num_q_heads, p.head_dim), dtype=odt, device=q.device)
    lse = torch.empty((p.batch, p.num_q_heads), dtype=torch.float32, device=q.device)
    ws = torch.empty(stem_decode_workspace_size(p), dtype=torch.uint8, device=q.device)
    stem_decode(p, q, k, v, seq_lens, keep, kbar, lvn, o, lse, ws, block_table, page_size, stream)
    return o, lse


def decode_blasst(p: Problem, q, k, v, seq_lens, lam, keep=None, kbar=None, lvn=None, block_table=None,
                  page_size=0, stream=None):
    """One decode step with the online skip at threshold lam.  Returns
    (O [b, Hq, d], LSE [b, Hq], skipped [b, Hq] int32)."""
    odt = torch.float32 if p.dtype == "f32" else torch.bfloat16
    o = torch.empty((p.batch, p.num_q_heads, p.head_dim), dtype=odt, device=q.device)
    lse = torch.empty((p.batch, p.num_q_heads), dtype=torch.float32, device=q.device)
    skipped = torch.empty((p.batch, p.num_q_heads), dtype=torch.int32, device=q.device)
    ws = torch.empty(stem_decode_blasst_workspace_size(p), dtype=torch.uint8, device=q.device)
    stem_decode_blasst(p, q, k, v, seq_lens, keep, kbar, lvn, lam, o, lse, skipped, ws, block_table, page_size,
                       stream)
    return o, lse, skipped
