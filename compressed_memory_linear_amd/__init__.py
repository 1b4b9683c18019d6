"""MI355X-native Orthogonal State Recurrence (OSR) forward and decode.

The compute path is the C-ABI library ``liblattice_osr.so`` (hand-written HIP
kernels for gfx950, see ``include/lattice_osr.h``); ``osr`` holds the thin
Python binding with the same entry-point names.  Importing this package does
not load the library; the first call through ``osr`` does, and raises if the
library was not built.
"""
__all__ = ["osr", "synth"]
