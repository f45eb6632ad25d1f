"""DDTree per-round hot path on MI355X (gfx950).

The work runs in hand-written HIP kernels behind the C ABI declared in
``include/ddtree.h`` (``libddtree.so``); this package is the thin Python
binding over it (argument marshalling only) plus the seeded input
generators in ``synth``.
"""
