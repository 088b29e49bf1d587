"""stem_score_noalloc, the allocation-free variant of stem_score, through the
C ABI: its scores must equal stem_score's bit for bit (the same kernels on
the same inputs), on two calls in a row, the second with a smaller problem
than the first (the scratch keeps the first call's contents).  The argument
checks run on the CPU."""

from __future__ import annotations

import ctypes

import pytest
import torch

import block_sparse_attention_24_amd as sb
import workloads as wl

FAKE = ctypes.c_void_p(0x1000)           # never dereferenced: validation fails first


def test_noalloc_rejects_oversized_problems_and_nulls():
    L = sb.lib()
    kv = sb.KvDesc(0x1000, 0x1000, None, 0, 0, 0)
    big = sb.Problem(1, 262144, 64, 8, 128, 128, "bf16")        # qbar alone is 64 MiB
    assert sb.stem_score_workspace_size(big) > sb.STEM_NOALLOC_SCRATCH_BYTES
    d = big.desc()
    assert L.stem_score_noalloc(ctypes.byref(d), FAKE, ctypes.byref(kv), FAKE, None) == sb.STEM_EWORKSPACE
    assert "scratch" in sb.stem_last_error()
    ok = sb.Problem(1, 131072, 64, 8, 128, 128, "fp8", 0.01, 0.01, 0.01)
    assert sb.stem_score_workspace_size(ok) <= sb.STEM_NOALLOC_SCRATCH_BYTES
    d = ok.desc()
    assert L.stem_score_noalloc(ctypes.byref(d), None, ctypes.byref(kv), FAKE, None) == sb.STEM_EINVAL
    assert L.stem_score_noalloc(ctypes.byref(d), FAKE, ctypes.byref(kv), None, None) == sb.STEM_EINVAL
    assert L.stem_score_noalloc(ctypes.byref(d), FAKE, None, FAKE, None) == sb.STEM_EINVAL


@pytest.mark.gpu
def test_noalloc_equals_stem_score_twice_second_smaller():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    cases = [wl.GQA_128K_FP8_PAGED,                                   # 36 MiB of scratch
             wl.Workload("noalloc-small-bf16", 1, 128 * 21, 8, 2, 128, 128, "bf16")]
    for w in cases:
        print(f"\n[case] stem_score_noalloc {w.name}", flush=True)
        gd = "cuda" if w.seq > 65536 else None
        inp = wl.make_inputs(w, device="cuda", gen_device=gd)
        p = sb.Problem(w.batch, w.seq, w.hq, w.hkv, w.head_dim, w.block, w.dtype,
                       float(inp["q_scale"]), float(inp["k_scale"]), float(inp["v_scale"]))
        if w.paged:
            k, v, table, page = inp["k_pages"], inp["v_pages"], inp["block_table"], w.page_size
        else:
            k, v, table, page = inp["k"], inp["v"], None, 0
        nb = w.num_blocks
        s_na = torch.full((w.batch, w.hq, nb, nb), float("nan"), dtype=torch.float32, device="cuda")
        sb.stem_score_noalloc(p, inp["q"], k, v, s_na, table, page)
        s_ref, _ = sb.score(p, inp["q"], k, v, table, page)
        torch.cuda.synchronize()
        # scores on and below the diagonal; nothing is written above it
        low = torch.tril(torch.ones((nb, nb), dtype=torch.bool, device="cuda"))
        assert torch.equal(s_na[..., low], s_ref[..., low]), w.name
        assert bool(torch.isnan(s_na[..., ~low]).all()), w.name
