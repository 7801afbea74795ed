"""DSA sparse-attention hot path (indexer -> top-k -> sparse MLA) for AMD MI355X.

The computation lives in libdsa.so (hand-written HIP kernels for gfx950, C ABI
in include/dsa.h); ``long_context_sparse_index_amd.dsa`` is its Python binding
and ``long_context_sparse_index_amd.synth`` draws seeded synthetic inputs.
Importing the package does not load the library.
"""
__all__ = ["dsa", "synth"]
