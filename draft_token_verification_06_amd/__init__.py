"""MI355X (gfx950) speculative-decoding verification.

The work runs in libspecverify.so (hand-written HIP kernels behind the C ABI
of include/sv.h); this package is its Python binding plus the seeded input
generators (``synth``).  The library is loaded on first use and a missing
build raises: there is no CPU path.
"""
from .api import (  # noqa: F401
    SvError,
    WindowResult,
    TreeResult,
    workspace_size,
    workspace,
    verify_window,
    verify_window_noalloc,
    verify_window_lmhead,
    verify_greedy,
    verify_tree,
    tree_max_depth,
    rollback,
    probe_read,
    SV_OP_WINDOW,
    SV_OP_GREEDY,
    SV_OP_TREE,
    SV_OP_LMHEAD,
)

__all__ = [
    "SvError", "WindowResult", "TreeResult", "workspace_size", "workspace",
    "verify_window", "verify_window_noalloc", "verify_window_lmhead", "verify_greedy", "verify_tree", "tree_max_depth", "rollback",
    "probe_read",
]
