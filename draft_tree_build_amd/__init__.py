"""DDTree per-round hot path on MI355X (gfx950).

The work runs in hand-written HIP kernels behind the C ABI declared in
``include/ddtree.h`` (``libddtree.so``); this package is the thin Python
binding over it (argument marshalling only) plus the seeded input
generators in ``synth``.
"""

from . import synth  # noqa: F401  (seeded inputs; no method arithmetic)
from .api import (  # noqa: F401
    DDTreeError, Round, ddtree_accept, ddtree_accept_sample, ddtree_accept_workspace_size,
    ddtree_build, ddtree_build_noalloc, ddtree_commit_kv,
    ddtree_build_workspace_size, ddtree_mask, ddtree_verify_attn, ddtree_verify_workspace_size,
    lib, new_workspace, strerror, version,
)
