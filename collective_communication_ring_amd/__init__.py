"""MI355X-native ring / double-binary-tree all-reduce over logical ranks.

The collective runs in ``libar.so`` (hand-written HIP kernels for gfx950
behind a C ABI, ``include/ar.h``); this package is the thin Python binding.
Importing the package does not load the library: ``api`` does, and fails
loudly when it has not been built.
"""

__all__ = ["api", "inputs"]
