"""CPU oracle for paged attention (decode and chunked prefill).

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package. The product path (the HIP library and
its Python binding) never calls it, and this package imports nothing from the
product path.

See :mod:`oracle.paged` for the definitions and their sources.
"""

from .paged import (  # noqa: F401
    append_kv,
    attention_rows,
    combine_splits_lse,
    gather_history,
    paged_attention,
    paged_attention_blockwise,
    split_partials,
)
