"""Tree-verification attention for AMD MI355X (gfx950).

TokenSwift verifies a 3-ary tree of drafted tokens in one forward pass with
tree-structured attention over the full KV cache, and drafts with the same
model over a partial cache.  This package is the attention step of both
passes, plus the greedy acceptance of the verified tree, the compaction of
the accepted path's K/V rows and the selection of the next draft pass's
partial cache: a C-ABI library of hand-written HIP kernels
(include/tsw.h, libtsw.so) and this thin Python binding.  PyTorch supplies
device memory and streams only.
"""
from ._binding import (  # noqa: F401
    DTYPE_BF16, DTYPE_F32, IMPL, LIB_PATH, AttnDesc, TswError, declared_functions, lib, lse_merge,
    make_desc, plan_splits, status_str, tree_attn_partial, tree_attn_split, tree_attn_verify,
    tree_mask, workspace_size, PreparedCall, prepare_merge, prepare_split, prepare_verify,
    accept_workspace_size, accept_greedy, prepare_accept, kv_compact, prepare_compact,
    context_penalty, prepare_penalty, accept_greedy_penalized, prepare_accept_penalized,
    PagedDesc, make_paged_desc, paged_workspace_size, tree_attn_verify_paged, prepare_verify_paged,
    paged_partial_workspace_size, tree_attn_partial_paged, prepare_partial_paged,
    select_workspace_size, select_partial, prepare_select,
    verify_select_workspace_size, tree_attn_verify_select, prepare_verify_select,
    read_stream, prepare_read_stream, prepare_launch_floor, noalloc_scratch_bytes, tree_attn_verify_noalloc,
)
