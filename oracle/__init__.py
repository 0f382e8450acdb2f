"""fp64 CPU oracle for sliding-window FlashAttention (TND varlen, sparse_mode 0/2/3/4).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The HIP product path
never imports, calls or links it, and this package imports nothing from the
product.

Parity status: every function here is pinned by CPU tests (finite differences,
an independent library routine, closed forms derived from the pages' worked
examples, brute-force mask enumeration, invariants).  See ``tests/test_oracle_*``.
"""
from .attention import (  # noqa: F401
    INT_MAX,
    SPARSE_MODES,
    sequences,
    allowed_mask,
    forward,
    backward,
    forward_rows,
    backward_rows,
    backward_keys,
    drop_mask_bits,
    unpack_drop_mask,
)
from .tiles import enumerate_tiles, count_pairs  # noqa: F401
