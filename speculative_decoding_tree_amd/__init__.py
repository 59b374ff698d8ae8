"""Tree-structured speculative verification for Gated DeltaNet layers on MI355X.

The compute lives in libgdn_tree.so (hand-written gfx950 HIP kernels behind the
C ABI in include/gdn_tree.h); ``gdn_tree`` is its thin ctypes binding.
"""
from . import gdn_tree  # noqa: F401
from .gdn_tree import (  # noqa: F401
    GdnTreeError, accepted_path, commit, commit_storeall, verify, verify_storeall,
)
