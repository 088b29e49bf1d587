"""Plain CPU fp64 oracle of Stem block-sparse prefill attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only the tests, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may call it.  It shares no code with the HIP library
(no kernels, headers, helpers, tables or constant generators); the only thing
both sides see is the seeded input generator in ``workloads``, which holds
none of the method's arithmetic.

Every function follows the method as the pages describe it (cited per
function) and is written for a reader to check by eye: fp64 NumPy, library
primitives (mean, matmul, log, sort) and plain loops, with no blocking,
fusion or reordering beyond what the definition states.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(brute force, closed forms, library routines, hand-worked fixtures under
``tests/golden/``).  Where the pages leave a formula out (the OAM formula,
the TPD budget shape) the oracle is the definition of record of the reading
it implements; those readings cannot be checked against the authors and are
"parity unpinned against the authors", which the module docstrings state.
"""

from .stem import (  # noqa: F401
    E4M3_MAX,
    attention_rows,
    blasst_attention,
    blasst_attention_rows,
    block_sparse_attention,
    cache_write,
    causal_block_count,
    decode_step,
    decode_step_blasst,
    dense_causal_attention,
    dequantize,
    e4m3fn_round,
    oam_scores,
    pack_block_mask,
    pool_blocks,
    quantize_e4m3,
    sam_scores,
    select_blocks,
    select_row,
    stem_pipeline,
    tpd_budget,
    tpd_total,
    unpack_block_mask,
)
