"""CPU-side checks of the C ABI: the library loads and exports every entry
point include/stem_bsa.h declares, argument checks fail before anything is
enqueued, and the host TPD budget equals the oracle's.  No GPU is used: the
calls below either never reach HIP (invalid arguments) or are host-only
(stem_tpd_budget)."""

import math
import ctypes
import os
import re

import pytest

import block_sparse_attention_24_amd as sb
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x1000)           # never dereferenced: validation fails first


def _header_functions():
    with open(os.path.join(ROOT, "include", "stem_bsa.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_entry_points_are_exported():
    names = _header_functions()
    assert set(names) == set(sb.EXPORTS), names
    h = sb.lib()
    for n in names:
        assert hasattr(h, n), n


def _desc(**kw):
    p = dict(batch=1, seq_len=1024, num_q_heads=4, num_kv_heads=2, head_dim=128, block_size=128,
             dtype="bf16")
    p.update(kw)
    return sb.Problem(**p).desc()


def _rc_score(d, kv=None, ws_bytes=1 << 30, scores=FAKE, q=FAKE, ws=FAKE):
    kv = kv or sb.KvDesc(0x1000, 0x1000, None, 0, 0, 0)
    return sb.lib().stem_score(ctypes.byref(d), q, ctypes.byref(kv), scores, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(seq_len=1000), sb.STEM_EINVAL),               # not a multiple of the block
    (dict(num_q_heads=3), sb.STEM_EINVAL),              # not a multiple of kv heads
    (dict(head_dim=96), sb.STEM_EUNSUPPORTED),
    (dict(block_size=32), sb.STEM_EUNSUPPORTED),
    (dict(seq_len=128 * 4097), sb.STEM_EUNSUPPORTED),   # too many blocks
    (dict(batch=0), sb.STEM_EINVAL),
    (dict(q_scale=2.0), sb.STEM_EINVAL),                # scales only for fp8
    (dict(dtype="fp8", k_scale=0.0), sb.STEM_EINVAL),
    (dict(softmax_scale=-1.0), sb.STEM_EINVAL),
])
def test_bad_shapes_rejected_everywhere(kw, code):
    d = _desc(**kw)
    assert _rc_score(d) == code
    assert sb.lib().stem_select(ctypes.byref(d), FAKE, 0.25, 0.5, FAKE, None, 0, None, None) == code
    kv = sb.KvDesc(0x1000, 0x1000, None, 0, 0, 0)
    assert sb.lib().bsa_prefill(ctypes.byref(d), FAKE, ctypes.byref(kv), None, FAKE, None, None) == code
    L = sb.lib()
    assert L.stem_score_sam(ctypes.byref(d), FAKE, ctypes.byref(kv), FAKE, FAKE, 1 << 30, None) == code
    assert L.stem_score_pooled(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == code
    assert L.stem_cache_write(ctypes.byref(d), FAKE, FAKE, ctypes.byref(kv), FAKE, FAKE, None) == code
    assert L.bsa_prefill_blasst(ctypes.byref(d), FAKE, ctypes.byref(kv), None, 0.1, FAKE, None, None,
                                None) == code
    assert sb.stem_last_error() != ""


def test_bad_dtype_code():
    d = _desc()
    d.dtype = 7
    assert _rc_score(d) == sb.STEM_EINVAL


def test_null_pointers_rejected():
    d = _desc()
    assert _rc_score(d, q=None) == sb.STEM_EINVAL
    assert _rc_score(d, scores=None) == sb.STEM_EINVAL
    assert _rc_score(d, ws=None) == sb.STEM_EINVAL
    kv = sb.KvDesc(None, 0x1000, None, 0, 0, 0)
    assert _rc_score(d, kv=kv) == sb.STEM_EINVAL
    assert sb.lib().stem_score(ctypes.byref(d), FAKE, None, FAKE, FAKE, 1 << 30, None) == sb.STEM_EINVAL
    assert sb.lib().stem_score(None, FAKE, ctypes.byref(kv), FAKE, FAKE, 1 << 30, None) == sb.STEM_EINVAL
    assert sb.lib().stem_select(ctypes.byref(d), None, 0.25, 0.5, FAKE, None, 0, None, None) == sb.STEM_EINVAL
    assert sb.lib().stem_select(ctypes.byref(d), FAKE, 0.25, 0.5, None, None, 0, None, None) == sb.STEM_EINVAL
    kv = sb.KvDesc(0x1000, 0x1000, None, 0, 0, 0)
    assert sb.lib().bsa_prefill(ctypes.byref(d), None, ctypes.byref(kv), None, FAKE, None, None) == sb.STEM_EINVAL
    assert sb.lib().bsa_prefill(ctypes.byref(d), FAKE, ctypes.byref(kv), None, None, None, None) == sb.STEM_EINVAL


def test_new_entry_points_reject_nulls_and_small_workspace():
    d = _desc()
    L = sb.lib()
    kv = sb.KvDesc(0x1000, 0x1000, None, 0, 0, 0)
    n = sb.stem_score_workspace_size(sb.Problem(1, 1024, 4, 2, 128, 128, "bf16"))
    assert L.stem_score_sam(ctypes.byref(d), None, ctypes.byref(kv), FAKE, FAKE, n, None) == sb.STEM_EINVAL
    assert L.stem_score_sam(ctypes.byref(d), FAKE, ctypes.byref(kv), FAKE, FAKE, n - 1, None) == sb.STEM_EWORKSPACE
    for args in ((None, FAKE, FAKE, FAKE), (FAKE, None, FAKE, FAKE), (FAKE, FAKE, None, FAKE),
                 (FAKE, FAKE, FAKE, None)):
        q, kbar, scores, ws = args
        assert L.stem_score_pooled(ctypes.byref(d), q, kbar, FAKE, scores, ws, n, None) == sb.STEM_EINVAL
    assert L.stem_score_pooled(ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, n - 1, None) == sb.STEM_EWORKSPACE
    for args in ((None, FAKE, FAKE, FAKE), (FAKE, None, FAKE, FAKE), (FAKE, FAKE, None, FAKE),
                 (FAKE, FAKE, FAKE, None)):
        k_in, v_in, kbar, lvn = args
        assert L.stem_cache_write(ctypes.byref(d), k_in, v_in, ctypes.byref(kv), kbar, lvn, None) == sb.STEM_EINVAL
    assert L.stem_cache_write(ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, None) == sb.STEM_EINVAL
    bad_page = sb.KvDesc(0x1000, 0x1000, 0x2000, 48, 32, 64)
    assert L.stem_cache_write(ctypes.byref(d), FAKE, FAKE, ctypes.byref(bad_page), FAKE, FAKE, None) == sb.STEM_EINVAL


def test_decode_rejects_nulls_and_small_workspace():
    d = _desc()
    L = sb.lib()
    kv = sb.KvDesc(0x1000, 0x1000, None, 0, 0, 0)
    n = sb.stem_decode_workspace_size(sb.Problem(1, 1024, 4, 2, 128, 128, "bf16"))
    ok = dict(q=FAKE, seq=FAKE, keep=FAKE, kbar=FAKE, lvn=FAKE, o=FAKE, ws=FAKE)

    def rc(**kw):
        a = dict(ok, **kw)
        return L.stem_decode(ctypes.byref(d), a["q"], ctypes.byref(kv), a["seq"], a["keep"], a["kbar"],
                             a["lvn"], a["o"], None, a["ws"], kw.get("n", n), None)
    for name in ("q", "seq", "o", "ws"):
        assert rc(**{name: None}) == sb.STEM_EINVAL, name
    assert rc(kbar=None) == sb.STEM_EINVAL                     # keep given without kbar
    assert rc(n=n - 1) == sb.STEM_EWORKSPACE
    assert L.stem_decode(ctypes.byref(d), FAKE, None, FAKE, None, None, None, FAKE, None, FAKE, n,
                         None) == sb.STEM_EINVAL
    bad = _desc(head_dim=96)
    assert L.stem_decode(ctypes.byref(bad), FAKE, ctypes.byref(kv), FAKE, None, None, None, FAKE, None,
                         FAKE, n, None) == sb.STEM_EUNSUPPORTED


def test_workspace_size_and_too_small_workspace():
    p = sb.Problem(2, 1024, 4, 2, 128, 128, "bf16")
    n = sb.stem_score_workspace_size(p)
    nb = 8
    want = 0
    for x in (2 * 4 * nb * 128 * 4, 2 * 2 * nb * 128 * 4, 2 * 2 * nb * 4):
        want += (x + 255) // 256 * 256
    assert n == want
    assert _rc_score(p.desc(), ws_bytes=n - 1) == sb.STEM_EWORKSPACE


def test_paged_kv_checks():
    d = _desc()
    bad_page = sb.KvDesc(0x1000, 0x1000, 0x2000, 48, 32, 64)
    assert _rc_score(d, kv=bad_page) == sb.STEM_EINVAL
    short = sb.KvDesc(0x1000, 0x1000, 0x2000, 64, 8, 64)      # 8 * 64 < 1024 tokens
    assert _rc_score(d, kv=short) == sb.STEM_EINVAL
    nopages = sb.KvDesc(0x1000, 0x1000, 0x2000, 64, 16, 0)
    assert _rc_score(d, kv=nopages) == sb.STEM_EINVAL


def test_select_rejects_bad_density_alpha_and_list_stride():
    d = _desc()
    L = sb.lib()
    assert L.stem_select(ctypes.byref(d), FAKE, 0.0, 0.5, FAKE, None, 0, None, None) == sb.STEM_EINVAL
    assert L.stem_select(ctypes.byref(d), FAKE, 1.01, 0.5, FAKE, None, 0, None, None) == sb.STEM_EINVAL
    assert L.stem_select(ctypes.byref(d), FAKE, 0.5, 0.3, FAKE, None, 0, None, None) == sb.STEM_EUNSUPPORTED
    budget, _ = sb.stem_tpd_budget(8, 0.5, 0.5)
    assert L.stem_select(ctypes.byref(d), FAKE, 0.5, 0.5, FAKE, FAKE, max(budget) - 1, None, None) == sb.STEM_EINVAL


@pytest.mark.parametrize("alpha", [0.0, 0.5, 1.0])
def test_host_tpd_budget_equals_oracle(alpha):
    for nb in list(range(1, 40)) + [63, 64, 65, 100, 127, 256, 511, 512]:
        for dens in (0.01, 0.05, 0.1, 0.2, 0.25, 1 / 3, 0.5, 0.75, 0.8, 0.99, 1.0):
            got = sb.stem_tpd_budget(nb, dens, alpha)
            want = oracle.tpd_budget(nb, dens, alpha)
            assert got == (want[0], want[1]), (nb, dens, alpha)


@pytest.mark.parametrize("nb,dens", [(1024, 0.25), (2048, 0.25), (512, 0.2), (4096, 0.1)])
def test_host_tpd_budget_equals_oracle_large(nb, dens):
    assert sb.stem_tpd_budget(nb, dens, 0.5) == oracle.tpd_budget(nb, dens, 0.5)


def test_tpd_budget_repeated_and_interleaved_calls():
    """The host keeps recent plans: more distinct (num_blocks, density, alpha)
    than it keeps, called twice in interleaved order, each equal to the oracle."""
    combos = [(nb, dens, alpha) for nb in (33, 70, 200) for dens in (0.1, 0.4) for alpha in (0.0, 0.5)]
    want = {c: oracle.tpd_budget(*c) for c in combos}
    for _ in range(2):
        for c in combos + combos[::-1]:
            assert sb.stem_tpd_budget(*c) == want[c], c


def test_tpd_budget_concurrent_callers():
    """Threads calling with different parameters at once (ctypes releases the
    GIL during the call, so the library's plan cache is shared for real):
    every result equals the oracle's."""
    import concurrent.futures as cf
    combos = [(nb, dens, alpha) for nb in (150, 301, 512) for dens in (0.07, 0.3, 0.6) for alpha in (0.0, 0.5, 1.0)]
    want = {c: oracle.tpd_budget(*c) for c in combos}
    jobs = combos * 4
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        got = list(ex.map(lambda c: sb.stem_tpd_budget(*c), jobs))
    for c, g in zip(jobs, got):
        assert g == want[c], c


@pytest.mark.parametrize("alpha", [0.0, 0.5, 1.0])
def test_tpd_budget_max_blocks_properties(alpha):
    """At the largest block count the API takes (65,536) the oracle's
    one-grant-at-a-time simulation is too slow, so the budget is pinned by the
    properties that define water-filling: the total, the forced rows, the
    bounds, and that no grant was given out of order.  The last grant a row
    received, (I, k_I), comes no later than the next grant any row with room
    could take, (I', k_I' + 1), in the order of key (n / (I+1)^(1-alpha),
    compared exactly in integers) and then row."""
    nb, dens = 65536, 0.25
    k, total = sb.stem_tpd_budget(nb, dens, alpha)
    c = nb * (nb + 1) // 2
    assert total == max(2 * nb - 1, min(c, math.floor(dens * c + 0.5)))
    assert sum(k) == total
    assert k[0] == 1 and all(2 <= k[i] <= i + 1 for i in range(1, nb))
    p = {0.0: 1, 0.5: 2, 1.0: 0}[alpha]      # key n^p / (I+1), or n alone for alpha = 1

    def key(row, n):                          # (numerator, denominator) of the key, and the row
        return (n, 1, row) if p == 0 else (n ** p, row + 1, row)

    def before(a, b):                         # grant a strictly before grant b
        l, r = a[0] * b[1], b[0] * a[1]
        return l < r or (l == r and a[2] < b[2])

    last = None                               # the latest grant given
    for i in range(1, nb):
        if k[i] > 2:
            g = key(i, k[i])
            if last is None or before(last, g):
                last = g
    nxt = None                                # the earliest grant still open
    for i in range(1, nb):
        if k[i] < i + 1:
            g = key(i, k[i] + 1)
            if nxt is None or before(g, nxt):
                nxt = g
    assert last is not None and nxt is not None
    assert before(last, nxt)


def test_tpd_budget_errors():
    with pytest.raises(sb.StemError):
        sb.stem_tpd_budget(0, 0.5)
    with pytest.raises(sb.StemError):
        sb.stem_tpd_budget(8, -0.1)
    with pytest.raises(sb.StemError) as e:
        sb.stem_tpd_budget(8, 0.5, 0.25)
    assert e.value.code == sb.STEM_EUNSUPPORTED


def test_blasst_rejects_bad_lambda_unsupported_shapes_and_nulls():
    L = sb.lib()
    kv = sb.KvDesc(0x1000, 0x1000, None, 0, 0, 0)
    d = _desc()
    for lam in (-0.1, 1.01, float("nan"), float("inf")):
        assert L.bsa_prefill_blasst(ctypes.byref(d), FAKE, ctypes.byref(kv), FAKE, lam, FAKE, None, None,
                                    None) == sb.STEM_EINVAL
        assert "lambda" in sb.stem_last_error()
    for kw in (dict(head_dim=64), dict(block_size=64), dict(dtype="f32")):
        dd = _desc(**kw)
        assert L.bsa_prefill_blasst(ctypes.byref(dd), FAKE, ctypes.byref(kv), FAKE, 0.1, FAKE, None, None,
                                    None) == sb.STEM_EUNSUPPORTED
    assert L.bsa_prefill_blasst(ctypes.byref(d), None, ctypes.byref(kv), FAKE, 0.1, FAKE, None, None,
                                None) == sb.STEM_EINVAL
    assert L.bsa_prefill_blasst(ctypes.byref(d), FAKE, ctypes.byref(kv), FAKE, 0.1, None, None, None,
                                None) == sb.STEM_EINVAL


def test_decode_blasst_checks():
    L = sb.lib()
    kv = sb.KvDesc(0x1000, 0x1000, None, 0, 0, 0)
    p = sb.Problem(1, 1024, 4, 2, 128, 128, "bf16")
    d = p.desc()
    n = sb.stem_decode_blasst_workspace_size(p)
    assert n > sb.stem_decode_workspace_size(p)
    args = lambda q=FAKE, lens=FAKE, keep=None, kbar=None, lam=0.1, o=FAKE, ws=FAKE, nbytes=n: (
        ctypes.byref(d), q, ctypes.byref(kv), lens, keep, kbar, None, lam, o, None, None, ws, nbytes, None)
    for kw in (dict(q=None), dict(lens=None), dict(o=None), dict(ws=None), dict(keep=FAKE)):
        assert L.stem_decode_blasst(*args(**kw)) == sb.STEM_EINVAL, kw
    for lam in (-1e-3, 1.5, float("nan")):
        assert L.stem_decode_blasst(*args(lam=lam)) == sb.STEM_EINVAL
        assert "lambda" in sb.stem_last_error()
    assert L.stem_decode_blasst(*args(nbytes=n - 1)) == sb.STEM_EWORKSPACE


@pytest.mark.parametrize("page", [1, 2, 8])
def test_decode_rejects_pages_below_16_tokens(page):
    """The decode kernels hand a block's page entries to its rows one per lane
    of a wave; pages of fewer than 16 tokens are rejected before any launch,
    as for the attention entry points."""
    L = sb.lib()
    p = sb.Problem(1, 1024, 4, 2, 128, 128, "bf16")
    d = p.desc()
    kv = sb.KvDesc(0x1000, 0x1000, 0x2000, page, 1024 // page, 1024 // page)
    n = sb.stem_decode_blasst_workspace_size(p)
    assert L.stem_decode(ctypes.byref(d), FAKE, ctypes.byref(kv), FAKE, None, None, None, FAKE, None, FAKE,
                         n, None) == sb.STEM_EUNSUPPORTED
    assert "page_size" in sb.stem_last_error()
    assert L.stem_decode_blasst(ctypes.byref(d), FAKE, ctypes.byref(kv), FAKE, None, None, None, 0.1, FAKE,
                                None, None, FAKE, n, None) == sb.STEM_EUNSUPPORTED
    assert L.bsa_prefill(ctypes.byref(d), FAKE, ctypes.byref(kv), None, FAKE, None, None) == sb.STEM_EUNSUPPORTED


def test_validate_block_table():
    """The debug-mode check of a block table, on host arrays: every page the
    batch's seq_len tokens use must name a page in [0, num_pages)."""
    import numpy as np
    t = np.arange(2 * 8, dtype=np.int32).reshape(2, 8)            # 2 sequences, 8 pages each
    sb.stem_validate_block_table(t, 2, 8, 16, 512, 64)
    sb.stem_validate_block_table(t, 2, 8, 16, 500, 64)             # a partial last page
    for bad_at, val in (((0, 3), 16), ((1, 7), -1), ((1, 0), 1 << 30)):
        u = t.copy()
        u[bad_at] = val
        with pytest.raises(sb.StemError, match=rf"block_table\[{bad_at[0]}\]\[{bad_at[1]}\]"):
            sb.stem_validate_block_table(u, 2, 8, 16, 512, 64)
    u = t.copy()
    u[1, 7] = 99                                                    # a page no token uses
    sb.stem_validate_block_table(u, 2, 8, 16, 448, 64)
    with pytest.raises(sb.StemError):
        sb.stem_validate_block_table(t, 2, 8, 16, 513, 64)         # more tokens than pages
    with pytest.raises(sb.StemError):
        sb.stem_validate_block_table(t, 2, 8, 16, 512, 48)         # not a power of two


def test_validate_lists():
    """The debug-mode check of stem_select's lists and counts: counts in
    [0, min(I + 1, stride)], entries strictly ascending in [0, I]."""
    import numpy as np
    nb, stride, rows = 6, 3, 2
    budget, _ = oracle.tpd_budget(nb, 0.5)
    scores = np.random.default_rng(3).standard_normal((1, rows, nb, nb))
    m = oracle.select_blocks(scores, budget)
    lists = np.full((rows, nb, stride), -7, dtype=np.int32)
    counts = np.zeros((rows, nb), dtype=np.int32)
    for h in range(rows):
        for i in range(nb):
            js = np.nonzero(m[0, h, i])[0]
            counts[h, i] = len(js)
            lists[h, i, :len(js)] = js
    assert counts.max() <= stride
    sb.stem_validate_lists(lists, counts, rows, nb, stride)
    for mutate, what in ((lambda l, c: c.__setitem__((1, 2), 4), "count"),
                         (lambda l, c: c.__setitem__((0, 0), -1), "count"),
                         (lambda l, c: l.__setitem__((1, 5, 0), 6), "entry"),
                         (lambda l, c: l.__setitem__((0, 3, 1), l[0, 3, 0]), "ascending")):
        l2, c2 = lists.copy(), counts.copy()
        mutate(l2, c2)
        with pytest.raises(sb.StemError, match=what):
            sb.stem_validate_lists(l2, c2, rows, nb, stride)
