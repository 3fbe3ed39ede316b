"""Plain fp64 CPU oracle for GQLA decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the test suite, the smoke check and the
CPU-baseline leg of the benchmark use it.  It depends on numpy alone and shares
no code with the HIP library or its Python binding.
"""
from .gqla import (  # noqa: F401
    absorb_decode,
    append_rows,
    expand_groups,
    gqa_decode,
    group_of_head,
    lse_merge,
    rope_rotate,
    sparse_gqa_decode,
    split_partials,
    textbook_decode,
    visible_rows,
)
