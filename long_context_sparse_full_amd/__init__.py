"""MI355X-native HySparse2 cross-decoder attention hot path.

``long_context_sparse_full_amd.hs2`` is the Python binding of the C-ABI library
``libhs2.so`` (hand-written HIP kernels for gfx950); importing it loads the
library and fails loudly when it has not been built.
``long_context_sparse_full_amd.synth`` draws the seeded synthetic workloads.
"""
__all__ = ["hs2", "synth"]
