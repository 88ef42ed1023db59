"""Tree-verify MLA-absorb attention for AMD MI355X (gfx950).

The work runs in libkdt.so (hand-written HIP kernels behind the C ABI of include/kdt.h);
this package is its Python binding.  Build the library with
``python -m tree_verify_mla_02_amd.build``.
"""
from ._lib import (KdtError, VerifyDesc, alloc_workspace, attend, build_tree, build_visibility, combine, kv_compact,
                   load, make_desc, num_splits, plan, prepare, prepare_attend, prepare_attend_launches, tree_accept,
                   tree_verify_attn, tree_verify_attn_noalloc, workspace_size)

__all__ = ["KdtError", "VerifyDesc", "alloc_workspace", "attend", "build_tree", "build_visibility", "combine", "kv_compact",
           "load", "make_desc", "num_splits", "plan", "prepare", "prepare_attend", "prepare_attend_launches", "tree_accept",
           "tree_verify_attn", "tree_verify_attn_noalloc", "workspace_size"]
