"""ctypes binding of libssd_mi355x.so (the C ABI in include/ssd.h).

Argument marshalling only: every step of the forward pass and of the decode
step runs in the library's HIP kernels. torch provides device memory and the
current stream. The library is loaded on first use; a missing library raises
(there is no CPU fallback).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_LIB_NAME = "libssd_mi355x.so"
# SSD_MI355X_LIBRARY names another build of the same library (the sanitizer
# build the CPU checks load); by default the in-tree one.
_LIB_PATH = os.environ.get("SSD_MI355X_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), _LIB_NAME)
_lib = None

SSD_OK = 0
STATUS = {0: "SSD_OK", 1: "SSD_ERR_INVALID_ARGUMENT", 2: "SSD_ERR_UNSUPPORTED",
          3: "SSD_ERR_WORKSPACE_TOO_SMALL", 4: "SSD_ERR_HIP"}
DTYPE_F32, DTYPE_BF16 = 0, 1

# Every symbol include/ssd.h declares.
EXPORTS = ("ssd_abi_version", "ssd_status_string", "ssd_default_state_block", "ssd_fwd_layout",
           "ssd_fwd_workspace_bytes", "ssd_fwd", "ssd_fwd_ex", "ssd_chunk_cumsum", "ssd_chunk_state",
           "ssd_state_passing", "ssd_chunk_scan", "ssd_step", "ssd_fwd_mamba2", "ssd_step_mamba2",
           "ssd_bwd_workspace_bytes", "ssd_bwd", "ssd_set_state_chain", "ssd_state_chain_cooperative",
           "ssd_chunk_scan_kernel", "ssd_bwd_mamba2_workspace_bytes", "ssd_bwd_mamba2", "ssd_fwd_noalloc")


class SSDError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} returned {STATUS.get(status, status)}")


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32), ("nheads", ctypes.c_int32),
                ("ngroups", ctypes.c_int32), ("headdim", ctypes.c_int32), ("dstate", ctypes.c_int32),
                ("num_seqs", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class Layout(ctypes.Structure):
    _fields_ = [("slots_per_row", ctypes.c_int64), ("nslots", ctypes.c_int64), ("blocks_per_row", ctypes.c_int64),
                ("nblocks", ctypes.c_int64), ("table_offset", ctypes.c_size_t),
                ("block_table_offset", ctypes.c_size_t), ("cumsum_offset", ctypes.c_size_t),
                ("key_cumsum_offset", ctypes.c_size_t), ("block_decay_offset", ctypes.c_size_t), ("block_states_offset", ctypes.c_size_t),
                ("start_states_offset", ctypes.c_size_t), ("total_bytes", ctypes.c_size_t)]


def library_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded library; raises when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_NAME} is not built (python -m ssd_chunked_scan_fwd_amd.build)")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        shp = ctypes.POINTER(Shape)
        L.ssd_abi_version.restype = i32
        L.ssd_abi_version.argtypes = []
        L.ssd_status_string.restype = ctypes.c_char_p
        L.ssd_status_string.argtypes = [ctypes.c_int]
        L.ssd_default_state_block.restype = i32
        L.ssd_default_state_block.argtypes = [shp, i32]
        L.ssd_fwd_layout.restype = ctypes.c_int
        L.ssd_fwd_layout.argtypes = [shp, i32, i32, ctypes.POINTER(Layout)]
        L.ssd_fwd_workspace_bytes.restype = ctypes.c_int
        L.ssd_fwd_workspace_bytes.argtypes = [shp, i32, i32, ctypes.POINTER(sz)]
        L.ssd_fwd.restype = ctypes.c_int
        L.ssd_fwd.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, shp, vp, sz, vp]
        L.ssd_fwd_noalloc.restype = ctypes.c_int
        L.ssd_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, shp, vp]
        L.ssd_fwd_ex.restype = ctypes.c_int
        L.ssd_fwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, shp, vp, sz, vp]
        L.ssd_chunk_cumsum.restype = ctypes.c_int
        L.ssd_chunk_cumsum.argtypes = [vp, vp, i32, i32, shp, vp, sz, vp]
        L.ssd_chunk_state.restype = ctypes.c_int
        L.ssd_chunk_state.argtypes = [vp, vp, vp, i32, i32, shp, vp, sz, vp]
        L.ssd_state_passing.restype = ctypes.c_int
        L.ssd_state_passing.argtypes = [vp, vp, i32, i32, vp, shp, vp, sz, vp]
        L.ssd_chunk_scan.restype = ctypes.c_int
        L.ssd_chunk_scan.argtypes = [vp, vp, vp, vp, i32, i32, vp, shp, vp, sz, vp]
        L.ssd_step.restype = ctypes.c_int
        L.ssd_step.argtypes = [vp, vp, vp, vp, vp, vp, shp, vp]
        L.ssd_fwd_mamba2.restype = ctypes.c_int
        L.ssd_fwd_mamba2.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, shp, vp, sz, vp]
        L.ssd_bwd_workspace_bytes.restype = ctypes.c_int
        L.ssd_bwd_workspace_bytes.argtypes = [shp, i32, i32, ctypes.POINTER(sz)]
        L.ssd_bwd.restype = ctypes.c_int
        L.ssd_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, shp, vp, sz, vp]
        L.ssd_step_mamba2.restype = ctypes.c_int
        L.ssd_step_mamba2.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, shp, vp]
        L.ssd_set_state_chain.restype = i32
        L.ssd_set_state_chain.argtypes = [i32]
        L.ssd_state_chain_cooperative.restype = ctypes.c_int
        L.ssd_state_chain_cooperative.argtypes = [shp, i32, i32, ctypes.POINTER(i32)]
        L.ssd_chunk_scan_kernel.restype = ctypes.c_int
        L.ssd_chunk_scan_kernel.argtypes = [shp, i32, i32, ctypes.POINTER(i32)]
        L.ssd_bwd_mamba2_workspace_bytes.restype = ctypes.c_int
        L.ssd_bwd_mamba2_workspace_bytes.argtypes = [shp, i32, i32, ctypes.POINTER(sz)]
        L.ssd_bwd_mamba2.restype = ctypes.c_int
        L.ssd_bwd_mamba2.argtypes = [vp] * 12 + [i32, i32] + [vp] * 9 + [shp, vp, sz, vp]
        _lib = L
    return _lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return DTYPE_BF16
    if dt == torch.float32:
        return DTYPE_F32
    raise TypeError(f"unsupported dtype {dt}")


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _call(fn: str, *args):
    st = getattr(lib(), fn)(*args)
    if st != SSD_OK:
        raise SSDError(fn, st)


def make_shape(X: torch.Tensor, B: torch.Tensor, cu_seqlens: Optional[torch.Tensor] = None) -> Shape:
    b, T, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    S = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    return Shape(b, T, H, G, P, N, S, _dtype_code(X.dtype))


def default_state_block(shape: Shape, chunk: int) -> int:
    return int(lib().ssd_default_state_block(ctypes.byref(shape), int(chunk)))


def layout(shape: Shape, chunk: int, state_block: int = 0) -> Layout:
    L = Layout()
    _call("ssd_fwd_layout", ctypes.byref(shape), int(chunk), int(state_block), ctypes.byref(L))
    return L


def workspace_bytes(shape: Shape, chunk: int, state_block: int = 0) -> int:
    n = ctypes.c_size_t(0)
    _call("ssd_fwd_workspace_bytes", ctypes.byref(shape), int(chunk), int(state_block), ctypes.byref(n))
    return int(n.value)


class Workspace:
    """A caller-owned workspace for one shape, chunk length and state block, with
    typed views of the stages' intermediate results (for inspection and tests)."""

    def __init__(self, shape: Shape, chunk: int, device, state_block: int = 0):
        self.shape = shape
        self.chunk = int(chunk)
        self.state_block = int(state_block) if state_block > 0 else default_state_block(shape, chunk)
        self.layout = layout(shape, chunk, self.state_block)
        self.buffer = torch.empty(self.layout.total_bytes, dtype=torch.uint8, device=device)

    @property
    def nbytes(self) -> int:
        return self.buffer.numel()

    def _view(self, off: int, count: int, dtype: torch.dtype, shape):
        esz = torch.empty((), dtype=dtype).element_size()
        return self.buffer[off:off + count * esz].view(dtype).view(*shape)

    def table(self) -> torch.Tensor:
        n = self.layout.nslots
        return self._view(self.layout.table_offset, n * 4, torch.int32, (n, 4))

    def block_table(self) -> torch.Tensor:
        n = self.layout.nblocks
        return self._view(self.layout.block_table_offset, n * 4, torch.int32, (n, 4))

    def cumsum(self) -> torch.Tensor:
        s, n = self.shape, self.layout.nslots
        return self._view(self.layout.cumsum_offset, n * s.nheads * self.chunk, torch.float32,
                          (n, s.nheads, self.chunk))

    def key_cumsum(self) -> torch.Tensor:
        s, n = self.shape, self.layout.nslots
        return self._view(self.layout.key_cumsum_offset, n * s.nheads * self.chunk, torch.float32,
                          (n, s.nheads, self.chunk))

    def block_decay(self) -> torch.Tensor:
        s, n = self.shape, self.layout.nblocks
        return self._view(self.layout.block_decay_offset, n * s.nheads, torch.float32, (n, s.nheads))

    def block_states(self) -> torch.Tensor:
        s, n = self.shape, self.layout.nblocks
        return self._view(self.layout.block_states_offset, n * s.nheads * s.headdim * s.dstate, torch.float32,
                          (n, s.nheads, s.headdim, s.dstate))

    def start_states(self) -> torch.Tensor:
        s, n = self.shape, self.layout.nblocks
        dt = torch.bfloat16 if s.dtype == DTYPE_BF16 else torch.float32
        return self._view(self.layout.start_states_offset, n * s.nheads * s.headdim * s.dstate, dt,
                          (n, s.nheads, s.headdim, s.dstate))


def _expect(t: Optional[torch.Tensor], name: str, shape=None, dtype=None, device=None, align: int = 0):
    """Raise ValueError unless `t` (None passes) has the given shape, dtype,
    contiguity and device."""
    _expect_all([(t, name, shape, dtype, align)], device)


def _expect_all(specs, device=None):
    """Check every (tensor, name, shape, dtype, align) in `specs`: first the
    structure of all of them (shape, dtype, contiguity), then their device and
    alignment, so a mismatched tensor is reported as such wherever it lives."""
    specs = [sp for sp in specs if sp[0] is not None]
    for t, name, shape, dtype, _ in specs:
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a torch tensor")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if dtype is not None and t.dtype != dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    for t, name, _, _, align in specs:
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if device is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")
        if align and t.data_ptr() % align:
            raise ValueError(f"{name} must be {align}-byte aligned")


def _check_inputs(X, log_a, B, C, cu_seqlens):
    """The forward inputs against one another: X [b, T, H, P], log_a [b, T, H]
    fp32, B and C [b, T, G, N] of X's dtype with H % G == 0, cu_seqlens int32
    [S + 1] with b == 1. Returns their specs for _expect_all."""
    if not isinstance(X, torch.Tensor) or X.dim() != 4:
        raise ValueError("X must be a 4-d tensor [batch, seqlen, nheads, headdim]")
    if X.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"X has dtype {X.dtype}; bfloat16 and float32 are supported")
    b, T, H, P = X.shape
    if not isinstance(B, torch.Tensor) or B.dim() != 4 or tuple(B.shape[:2]) != (b, T):
        raise ValueError(f"B must be a 4-d tensor [{b}, {T}, ngroups, dstate]")
    G, N = B.shape[2], B.shape[3]
    if G < 1 or H % G:
        raise ValueError(f"nheads {H} must be a multiple of ngroups {G}")
    if cu_seqlens is not None:
        if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
            raise ValueError("cu_seqlens must be a 1-d tensor of num_seqs + 1 >= 2 entries")
        if b != 1:
            raise ValueError("packed sequences (cu_seqlens) need batch 1")
    return [(X, "X", None, None, 0), (B, "B", (b, T, G, N), X.dtype, 0), (C, "C", (b, T, G, N), X.dtype, 0),
            (log_a, "log_a", (b, T, H), torch.float32, 0), (cu_seqlens, "cu_seqlens", None, torch.int32, 0)]


def _nseq(shape: Shape) -> int:
    return shape.num_seqs if shape.num_seqs > 0 else shape.batch


def _state_spec(t: Optional[torch.Tensor], shape: Shape, name: str):
    """A state tensor: fp32 [rows or sequences, H, P, N], 16-byte aligned."""
    return (t, name, (_nseq(shape), shape.nheads, shape.headdim, shape.dstate), torch.float32, 16)


def _check_state(t: Optional[torch.Tensor], shape: Shape, name: str, device=None):
    _expect_all([_state_spec(t, shape, name)], device)


def _check_workspace(ws: "Workspace", shape: Shape, chunk: int):
    if not isinstance(ws, Workspace):
        raise ValueError("workspace must be a Workspace")
    mine = tuple(getattr(ws.shape, f) for f, _ in Shape._fields_)
    theirs = tuple(getattr(shape, f) for f, _ in Shape._fields_)
    if mine != theirs or ws.chunk != int(chunk):
        raise ValueError("the workspace was made for another shape or chunk length")


def fwd(X: torch.Tensor, log_a: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
        cu_seqlens: Optional[torch.Tensor] = None, chunk: int = 128, state_block: int = 0,
        Y: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None, want_final: bool = True,
        workspace: Optional[Workspace] = None,
        initial_state: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked SSD forward pass (ssd_fwd_ex). Returns (Y, final_state or None).

    state_block <= 0 uses the library's default (the workspace's, when one is given).
    initial_state: fp32 [rows or sequences, H, P, N] the state each row (each
    packed sequence) starts from; None for zero states.
    """
    specs = _check_inputs(X, log_a, B, C, cu_seqlens)
    shape = make_shape(X, B, cu_seqlens)
    if workspace is not None:
        _check_workspace(workspace, shape, chunk)
        if state_block > 0 and state_block != workspace.state_block:
            raise ValueError("state_block differs from the workspace's")
    _expect_all(specs + [_state_spec(initial_state, shape, "initial_state"), (Y, "Y", tuple(X.shape), X.dtype, 0),
                         _state_spec(final_state, shape, "final_state")], X.device)
    if Y is None:
        Y = torch.empty_like(X)
    if final_state is None and want_final:
        final_state = torch.empty(_nseq(shape), X.shape[2], X.shape[3], B.shape[3], dtype=torch.float32,
                                  device=X.device)
    if workspace is None:
        workspace = Workspace(shape, chunk, X.device, state_block)
    _call("ssd_fwd_ex", _ptr(X), _ptr(log_a), _ptr(B), _ptr(C), _ptr(cu_seqlens), _ptr(initial_state), int(chunk),
          workspace.state_block,
          _ptr(Y), _ptr(final_state), ctypes.byref(shape), _ptr(workspace.buffer), workspace.nbytes,
          _stream(X.device))
    return Y, final_state


def _stage_check(shape: Shape, ws: Workspace, X=None, log_a=None, B=None, C=None, Y=None, cu_seqlens=None):
    """Tensors handed to a single stage against the shape its workspace was made for."""
    _check_workspace(ws, shape, ws.chunk)
    dt = torch.bfloat16 if shape.dtype == DTYPE_BF16 else torch.float32
    b, T, H, G, P, N = shape.batch, shape.seqlen, shape.nheads, shape.ngroups, shape.headdim, shape.dstate
    want_cu = shape.num_seqs + 1 if shape.num_seqs > 0 else None
    if (cu_seqlens is None) != (want_cu is None):
        raise ValueError("cu_seqlens must be given exactly when the shape is packed (num_seqs > 0)")
    _expect_all([(X, "X", (b, T, H, P), dt, 0), (Y, "Y", (b, T, H, P), dt, 0), (B, "B", (b, T, G, N), dt, 0),
                 (C, "C", (b, T, G, N), dt, 0), (log_a, "log_a", (b, T, H), torch.float32, 0),
                 (cu_seqlens, "cu_seqlens", (want_cu,) if want_cu else None, torch.int32, 0)], ws.buffer.device)


NOALLOC_SCRATCH_BYTES = 64 << 20   # SSD_NOALLOC_SCRATCH_BYTES


def fwd_noalloc(X: torch.Tensor, log_a: torch.Tensor, B: torch.Tensor, C: torch.Tensor, Y: torch.Tensor,
                final_state: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None,
                chunk: int = 128) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """ssd_fwd_noalloc: the forward pass in the library's static per-GPU scratch (no
    workspace; nothing allocated here either, so Y, and final_state when wanted,
    are the caller's). Calls that overlap on one GPU race on that scratch."""
    specs = _check_inputs(X, log_a, B, C, cu_seqlens)
    shape = make_shape(X, B, cu_seqlens)
    if Y is None:
        raise ValueError("Y is required")
    _expect_all(specs + [(Y, "Y", tuple(X.shape), X.dtype, 0), _state_spec(final_state, shape, "final_state")],
                X.device)
    _call("ssd_fwd_noalloc", _ptr(X), _ptr(log_a), _ptr(B), _ptr(C), _ptr(cu_seqlens), int(chunk), _ptr(Y),
          _ptr(final_state), ctypes.byref(shape), _stream(X.device))
    return Y, final_state


def chunk_cumsum(log_a, cu_seqlens, shape: Shape, ws: Workspace):
    _stage_check(shape, ws, log_a=log_a, cu_seqlens=cu_seqlens)
    _call("ssd_chunk_cumsum", _ptr(log_a), _ptr(cu_seqlens), ws.chunk, ws.state_block, ctypes.byref(shape),
          _ptr(ws.buffer), ws.nbytes, _stream(ws.buffer.device))


def chunk_state(X, B, cu_seqlens, shape: Shape, ws: Workspace):
    _stage_check(shape, ws, X=X, B=B, cu_seqlens=cu_seqlens)
    _call("ssd_chunk_state", _ptr(X), _ptr(B), _ptr(cu_seqlens), ws.chunk, ws.state_block, ctypes.byref(shape),
          _ptr(ws.buffer), ws.nbytes, _stream(ws.buffer.device))


def state_passing(cu_seqlens, final_state, shape: Shape, ws: Workspace, initial_state=None):
    _stage_check(shape, ws, cu_seqlens=cu_seqlens)
    _expect_all([_state_spec(initial_state, shape, "initial_state"), _state_spec(final_state, shape, "final_state")],
                ws.buffer.device)
    _call("ssd_state_passing", _ptr(cu_seqlens), _ptr(initial_state), ws.chunk, ws.state_block, _ptr(final_state),
          ctypes.byref(shape), _ptr(ws.buffer), ws.nbytes, _stream(ws.buffer.device))


def chunk_scan(X, B, C, cu_seqlens, Y, shape: Shape, ws: Workspace):
    _stage_check(shape, ws, X=X, B=B, C=C, Y=Y, cu_seqlens=cu_seqlens)
    _call("ssd_chunk_scan", _ptr(X), _ptr(B), _ptr(C), _ptr(cu_seqlens), ws.chunk, ws.state_block, _ptr(Y),
          ctypes.byref(shape), _ptr(ws.buffer), ws.nbytes, _stream(ws.buffer.device))


def _check_step(state, x, B, C, y, log_a=None):
    """Decode-step tensors: x [b, H, P], state fp32 [b, H, P, N] (16-byte aligned),
    B and C [b, G, N] of x's dtype, log_a fp32 [b, H], y like x."""
    if not isinstance(x, torch.Tensor) or x.dim() != 3:
        raise ValueError("x must be a 3-d tensor [batch, nheads, headdim]")
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"x has dtype {x.dtype}; bfloat16 and float32 are supported")
    b, H, P = x.shape
    if not isinstance(B, torch.Tensor) or B.dim() != 3 or B.shape[0] != b:
        raise ValueError(f"B must be a 3-d tensor [{b}, ngroups, dstate]")
    G, N = B.shape[1], B.shape[2]
    if G < 1 or H % G:
        raise ValueError(f"nheads {H} must be a multiple of ngroups {G}")
    if state is None:
        raise ValueError("state is required")
    specs = [(x, "x", None, None, 0), (B, "B", (b, G, N), x.dtype, 0), (C, "C", (b, G, N), x.dtype, 0),
             (state, "state", (b, H, P, N), torch.float32, 16), (log_a, "log_a", (b, H), torch.float32, 0),
             (y, "y", (b, H, P), x.dtype, 0)]
    return Shape(b, 1, H, G, P, N, 0, _dtype_code(x.dtype)), specs


def step(state: torch.Tensor, x: torch.Tensor, log_a: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
         y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode step (ssd_step): updates `state` in place and returns y."""
    if log_a is None:
        raise ValueError("log_a is required")
    shape, specs = _check_step(state, x, B, C, y, log_a)
    _expect_all(specs, x.device)
    if y is None:
        y = torch.empty_like(x)
    _call("ssd_step", _ptr(state), _ptr(x), _ptr(log_a), _ptr(B), _ptr(C), _ptr(y), ctypes.byref(shape),
          _stream(x.device))
    return y


def _check_mamba2(X, dt, dt_bias, A_log, D, z, H: int):
    """Specs of the Mamba-2 call's extra tensors: dt [*X.shape[:-1]] fp32, dt_bias,
    A_log, D [H] fp32, z like X."""
    if dt is None or A_log is None:
        raise ValueError("dt and A_log are required")
    return [(dt, "dt", tuple(X.shape[:-1]), torch.float32, 0), (dt_bias, "dt_bias", (H,), torch.float32, 0),
            (A_log, "A_log", (H,), torch.float32, 0), (D, "D", (H,), torch.float32, 0),
            (z, "z", tuple(X.shape), X.dtype, 0)]


def fwd_mamba2(X: torch.Tensor, dt: torch.Tensor, A_log: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
               dt_bias: Optional[torch.Tensor] = None, D: Optional[torch.Tensor] = None,
               z: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None, chunk: int = 128,
               state_block: int = 0, Y: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
               want_final: bool = True, workspace: Optional[Workspace] = None,
               initial_state: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """The Mamba-2 block's SSD call (ssd_fwd_mamba2). Returns (Y, final_state or None).

    X is the block's x (unscaled), dt the raw step sizes [b, T, H] fp32; dt_bias,
    A_log and D are fp32 [H]; z (the gate) has X's shape and dtype. The other
    arguments are those of fwd().
    """
    specs = _check_inputs(X, None, B, C, cu_seqlens) + _check_mamba2(X, dt, dt_bias, A_log, D, z, X.shape[2])
    shape = make_shape(X, B, cu_seqlens)
    if workspace is not None:
        _check_workspace(workspace, shape, chunk)
        if state_block > 0 and state_block != workspace.state_block:
            raise ValueError("state_block differs from the workspace's")
    _expect_all(specs + [_state_spec(initial_state, shape, "initial_state"), (Y, "Y", tuple(X.shape), X.dtype, 0),
                         _state_spec(final_state, shape, "final_state")], X.device)
    if Y is None:
        Y = torch.empty_like(X)
    if final_state is None and want_final:
        final_state = torch.empty(_nseq(shape), X.shape[2], X.shape[3], B.shape[3], dtype=torch.float32,
                                  device=X.device)
    if workspace is None:
        workspace = Workspace(shape, chunk, X.device, state_block)
    _call("ssd_fwd_mamba2", _ptr(X), _ptr(dt), _ptr(dt_bias), _ptr(A_log), _ptr(D), _ptr(z), _ptr(B), _ptr(C),
          _ptr(cu_seqlens), _ptr(initial_state), int(chunk), workspace.state_block, _ptr(Y), _ptr(final_state),
          ctypes.byref(shape), _ptr(workspace.buffer), workspace.nbytes, _stream(X.device))
    return Y, final_state


def step_mamba2(state: torch.Tensor, x: torch.Tensor, dt: torch.Tensor, A_log: torch.Tensor, B: torch.Tensor,
                C: torch.Tensor, dt_bias: Optional[torch.Tensor] = None, D: Optional[torch.Tensor] = None,
                z: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One Mamba-2 decode step (ssd_step_mamba2): updates `state` in place and returns y."""
    shape, specs = _check_step(state, x, B, C, y)
    _expect_all(specs + _check_mamba2(x, dt, dt_bias, A_log, D, z, x.shape[1]), x.device)
    if y is None:
        y = torch.empty_like(x)
    _call("ssd_step_mamba2", _ptr(state), _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A_log), _ptr(D), _ptr(z),
          _ptr(B), _ptr(C), _ptr(y), ctypes.byref(shape), _stream(x.device))
    return y


def set_state_chain(mode: int) -> int:
    """ssd_set_state_chain: 1 runs the state chain as one cooperative launch when
    it fits, 0 (the default) always as two launches. Returns the previous mode."""
    return int(lib().ssd_set_state_chain(int(mode)))


def state_chain_cooperative(shape: Shape, chunk: int, state_block: int = 0) -> bool:
    """ssd_state_chain_cooperative: whether mode 1 runs this shape's state chain as
    the cooperative launch on the current device (uncaptured stream)."""
    r = ctypes.c_int32(0)
    _call("ssd_state_chain_cooperative", ctypes.byref(shape), int(chunk), int(state_block), ctypes.byref(r))
    return bool(r.value)


SCAN_KERNELS = ("f32", "single", "pair", "half_pair", "half_pair_wide")


def chunk_scan_kernel(shape: Shape, chunk: int, state_block: int = 0) -> str:
    """ssd_chunk_scan_kernel: the chunk_scan kernel a forward call with this shape
    runs: "f32", "single" (one head per workgroup), "pair" (two heads, whole
    chunks, one workgroup per CU), "half_pair" (two heads, chunks in halves of
    64 tokens, two workgroups per CU) or "half_pair_wide" (the same walk at
    dstate 256, one workgroup per CU)."""
    r = ctypes.c_int32(-1)
    _call("ssd_chunk_scan_kernel", ctypes.byref(shape), int(chunk), int(state_block), ctypes.byref(r))
    return SCAN_KERNELS[r.value]


def bwd_workspace_bytes(shape: Shape, chunk: int, state_block: int = 0) -> int:
    n = ctypes.c_size_t(0)
    _call("ssd_bwd_workspace_bytes", ctypes.byref(shape), int(chunk), int(state_block), ctypes.byref(n))
    return int(n.value)


def bwd(X: torch.Tensor, log_a: torch.Tensor, B: torch.Tensor, C: torch.Tensor, dY: torch.Tensor,
        cu_seqlens: Optional[torch.Tensor] = None, chunk: int = 128, state_block: int = 0,
        initial_state: Optional[torch.Tensor] = None, dfinal_state: Optional[torch.Tensor] = None,
        want_dinit: bool = False, workspace: Optional[torch.Tensor] = None):
    """Backward pass (ssd_bwd): gradients of <dY, Y> + <dfinal_state, final_state>
    for the forward pass with these inputs. Returns dict(dX, dlog_a, dB, dC, dinit or None)."""
    specs = _check_inputs(X, log_a, B, C, cu_seqlens)
    if dY is None:
        raise ValueError("dY is required")
    shape = make_shape(X, B, cu_seqlens)
    _expect_all(specs + [(dY, "dY", tuple(X.shape), X.dtype, 0), _state_spec(initial_state, shape, "initial_state"),
                         _state_spec(dfinal_state, shape, "dfinal_state")], X.device)
    nbytes = bwd_workspace_bytes(shape, chunk, state_block)
    _expect(workspace, "workspace", dtype=torch.uint8, device=X.device, align=256)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=X.device)
    dX = torch.empty_like(X)
    dla = torch.empty_like(log_a)
    dB = torch.empty_like(B)
    dC = torch.empty_like(C)
    dinit = None
    if want_dinit:
        nseq = X.shape[0] if cu_seqlens is None else cu_seqlens.numel() - 1
        dinit = torch.empty(nseq, X.shape[2], X.shape[3], B.shape[3], dtype=torch.float32, device=X.device)
    _call("ssd_bwd", _ptr(X), _ptr(log_a), _ptr(B), _ptr(C), _ptr(cu_seqlens), _ptr(initial_state), _ptr(dY),
          _ptr(dfinal_state), int(chunk), int(state_block), _ptr(dX), _ptr(dla), _ptr(dB), _ptr(dC), _ptr(dinit),
          ctypes.byref(shape), _ptr(workspace), workspace.numel(), _stream(X.device))
    return dict(dX=dX, dlog_a=dla, dB=dB, dC=dC, dinit=dinit)


def bwd_mamba2_workspace_bytes(shape: Shape, chunk: int, state_block: int = 0) -> int:
    n = ctypes.c_size_t(0)
    _call("ssd_bwd_mamba2_workspace_bytes", ctypes.byref(shape), int(chunk), int(state_block), ctypes.byref(n))
    return int(n.value)


def bwd_mamba2(X: torch.Tensor, dt: torch.Tensor, A_log: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
               dY: torch.Tensor, dt_bias: Optional[torch.Tensor] = None, D: Optional[torch.Tensor] = None,
               z: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None, chunk: int = 128,
               state_block: int = 0, initial_state: Optional[torch.Tensor] = None,
               dfinal_state: Optional[torch.Tensor] = None, want_dinit: bool = False,
               workspace: Optional[torch.Tensor] = None):
    """Backward pass of the Mamba-2 call (ssd_bwd_mamba2). Returns dict(dX, ddt, ddt_bias,
    dA_log, dD or None, dz or None, dB, dC, dinit or None)."""
    specs = _check_inputs(X, None, B, C, cu_seqlens) + _check_mamba2(X, dt, dt_bias, A_log, D, z, X.shape[2])
    if dY is None:
        raise ValueError("dY is required")
    shape = make_shape(X, B, cu_seqlens)
    _expect_all(specs + [(dY, "dY", tuple(X.shape), X.dtype, 0), _state_spec(initial_state, shape, "initial_state"),
                         _state_spec(dfinal_state, shape, "dfinal_state")], X.device)
    nbytes = bwd_mamba2_workspace_bytes(shape, chunk, state_block)
    _expect(workspace, "workspace", dtype=torch.uint8, device=X.device, align=256)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=X.device)
    H = X.shape[2]
    out = dict(dX=torch.empty_like(X), ddt=torch.empty_like(dt),
               ddt_bias=torch.empty(H, dtype=torch.float32, device=X.device),
               dA_log=torch.empty(H, dtype=torch.float32, device=X.device),
               dD=None if D is None else torch.empty(H, dtype=torch.float32, device=X.device),
               dz=None if z is None else torch.empty_like(z), dB=torch.empty_like(B), dC=torch.empty_like(C),
               dinit=None)
    if want_dinit:
        nseq = X.shape[0] if cu_seqlens is None else cu_seqlens.numel() - 1
        out["dinit"] = torch.empty(nseq, H, X.shape[3], B.shape[3], dtype=torch.float32, device=X.device)
    _call("ssd_bwd_mamba2", _ptr(X), _ptr(dt), _ptr(dt_bias), _ptr(A_log), _ptr(D), _ptr(z), _ptr(B), _ptr(C),
          _ptr(cu_seqlens), _ptr(initial_state), _ptr(dY), _ptr(dfinal_state), int(chunk), int(state_block),
          _ptr(out["dX"]), _ptr(out["ddt"]), _ptr(out["ddt_bias"]), _ptr(out["dA_log"]), _ptr(out["dD"]),
          _ptr(out["dz"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dinit"]), ctypes.byref(shape),
          _ptr(workspace), workspace.numel(), _stream(X.device))
    return out
