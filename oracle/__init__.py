"""CPU oracle for tree-attention verification.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU-baseline leg may
import it; the product path never does.  See ``tree_oracle.c`` for what it computes.
"""
from .oracle import (  # noqa: F401
    ORC_BAD_LEN,
    ORC_BAD_PATH,
    ORC_BAD_TREE,
    ORC_OVERFLOW,
    accept,
    attention,
    build,
    build_mask,
    compact,
    lib_path,
    tree_paths,
)
