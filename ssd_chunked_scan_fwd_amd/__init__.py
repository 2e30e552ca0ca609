"""MI355X-native chunked SSD forward pass (the Mamba-2 layer's scan).

The compute path is a C-ABI shared library of hand-written HIP kernels for
gfx950 (``libssd_mi355x.so``, built in-tree); this package is a thin ctypes
binding over it. Importing the package does not load the library: the first
call does, and it raises if the library is missing.
"""
from . import synth  # noqa: F401

__all__ = ["synth"]
