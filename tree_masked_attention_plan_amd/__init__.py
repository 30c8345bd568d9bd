"""Tree-causal paged attention for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libtree_attn.so`` (C ABI in ``include/tree_attn.h``).
It only marshals arguments: torch tensors supply device memory and the
current HIP stream, every step of the computation runs in the library's HIP
kernels.  There is no fallback: if the library is not built, importing the
binding's entry points raises.

    plan(parent, tree_off, prefix_len)   -> anc_mask, depth, pos_id, status
    fwd(q, k_tree, v_tree, k_cache, v_cache, block_table, prefix_len,
        tree_off, anc_mask)               -> out, lse
    plan_fwd(q, k_tree, v_tree, k_cache, v_cache, block_table, prefix_len,
             tree_off, parent)            -> plan, out, lse  (one call)
    build_tree(logp, T)                 -> parent, choice, score
    commit(anc_mask, depth, tree_off, prefix_len, accepted, k_tree, v_tree,
           k_cache, v_cache, block_table)  -> new_prefix_len, status
    plan_dfs(parent, tree_off, prefix_len) -> perm, inv_perm, parent_new, plan
    gather_rows(src, index)              -> src[index]
    fwd_noalloc(..., out=, lse=)         -> out, lse  (no allocation; fixed
                                            per-device split workspace)
"""
from ._binding import (MASK_WORDS, MAX_TREE, NOALLOC_SCRATCH_BYTES, FwdCall, PlanDfsResult, PlanFwdCall, PlanResult,
                       TreeAttnError, abi_version, build_tree, check_status, commit, fwd, fwd_noalloc,
                       gather_rows, library_path, load_library, num_splits, plan, plan_dfs, plan_fwd, prepare_fwd,
                       prepare_plan_fwd, workspace_bytes)

__all__ = ["MASK_WORDS", "MAX_TREE", "NOALLOC_SCRATCH_BYTES", "FwdCall", "PlanDfsResult", "PlanFwdCall", "PlanResult",
           "TreeAttnError", "abi_version", "build_tree", "check_status", "commit", "fwd", "fwd_noalloc",
           "gather_rows",
           "library_path", "load_library", "num_splits", "plan", "plan_dfs", "plan_fwd", "prepare_fwd",
           "prepare_plan_fwd", "workspace_bytes"]
