"""MI355X-native chunked SSD forward pass (the Mamba-2 layer's scan).

The compute path is a C-ABI shared library of hand-written HIP kernels for
gfx950 (``libssd_mi355x.so``, built in-tree by ``build.py``); ``binding`` is a
thin ctypes layer over it. Importing the package does not load the library:
the first call does, and it raises if the library is missing.
"""
from . import synth  # noqa: F401
from .binding import (  # noqa: F401
    SSDError,
    Shape,
    Workspace,
    bwd,
    bwd_mamba2,
    bwd_mamba2_workspace_bytes,
    bwd_workspace_bytes,
    chunk_cumsum,
    chunk_scan,
    chunk_state,
    default_state_block,
    fwd,
    fwd_mamba2,
    fwd_noalloc,
    layout,
    lib,
    make_shape,
    set_state_chain,
    state_chain_cooperative,
    chunk_scan_kernel,
    state_passing,
    step,
    step_mamba2,
    workspace_bytes,
)

__all__ = [
    "synth",
    "fwd", "step", "fwd_mamba2", "step_mamba2", "fwd_noalloc",
    "bwd", "bwd_workspace_bytes", "bwd_mamba2", "bwd_mamba2_workspace_bytes",
    "chunk_cumsum", "chunk_state", "state_passing", "chunk_scan",
    "set_state_chain", "state_chain_cooperative", "chunk_scan_kernel", "Workspace", "Shape", "SSDError", "layout", "workspace_bytes", "make_shape", "lib",
    "default_state_block",
]
