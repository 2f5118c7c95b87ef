"""Float64 CPU oracle for tree-verification attention -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package.  The GPU library never imports, links or calls it.
"""
from .oracle import (  # noqa: F401
    Oracle, SRC, build, compile_oracle, default, lib_path, lse_merge, mask_build, tree_attn,
    ORACLE_OK, ORACLE_EBADTREE, ORACLE_EINVAL,
)
