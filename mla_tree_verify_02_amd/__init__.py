"""MI355X-native absorbed-MLA tree-verify attention.

The computation lives in libmla_tree_verify.so (hand-written gfx950 HIP kernels
behind a C ABI, declared in include/mla_tree_verify.h). This package holds the
kernel sources (csrc/), the in-tree build (build.py), the ctypes binding
(_lib.py) and the seeded synthetic workloads (inputs.py). Importing it loads
nothing; the library is opened on first use.
"""
from ._lib import (MtvError, MtvShape, PreparedCall, PreparedPagedCall, check_inputs, kv_commit, kv_defrag, load,  # noqa: F401
                   make_shape, mla_tree_verify, mla_tree_verify_noalloc, mla_tree_verify_paged,
                   plan_query, prepare_workload, status_string, tree_mask_build, verify_workload,
                   workspace_size)

__all__ = ["mla_tree_verify", "verify_workload", "workspace_size", "plan_query", "make_shape",
           "status_string", "load", "MtvError", "MtvShape", "PreparedCall", "PreparedPagedCall",
           "prepare_workload",
           "tree_mask_build", "kv_commit", "kv_defrag", "mla_tree_verify_paged", "check_inputs",
           "mla_tree_verify_noalloc"]
