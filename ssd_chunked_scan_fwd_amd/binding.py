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
_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), _LIB_NAME)
_lib = None

SSD_OK = 0
STATUS = {0: "SSD_OK", 1: "SSD_ERR_INVALID_ARGUMENT", 2: "SSD_ERR_UNSUPPORTED",
          3: "SSD_ERR_WORKSPACE_TOO_SMALL", 4: "SSD_ERR_HIP"}
DTYPE_F32, DTYPE_BF16 = 0, 1

# Every symbol include/ssd.h declares.
EXPORTS = ("ssd_abi_version", "ssd_status_string", "ssd_default_state_block", "ssd_fwd_layout",
           "ssd_fwd_workspace_bytes", "ssd_fwd", "ssd_fwd_ex", "ssd_chunk_cumsum", "ssd_chunk_state",
           "ssd_state_passing", "ssd_chunk_scan", "ssd_step", "ssd_fwd_mamba2", "ssd_step_mamba2",
           "ssd_bwd_workspace_bytes", "ssd_bwd", "ssd_set_state_chain", "ssd_bwd_mamba2_workspace_bytes",
           "ssd_bwd_mamba2")


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


def _check_inputs(X, log_a, B, C, cu_seqlens):
    for name, t in (("X", X), ("B", B), ("C", C)):
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous device tensor")
    if log_a is not None and (log_a.dtype != torch.float32 or not log_a.is_contiguous() or not log_a.is_cuda):
        raise ValueError("log_a must be a contiguous fp32 device tensor")
    if cu_seqlens is not None and (cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda):
        raise ValueError("cu_seqlens must be an int32 device tensor")
    if X is not None and B is not None and (X.dtype != B.dtype or (C is not None and C.dtype != X.dtype)):
        raise ValueError("X, B and C must share one dtype")


def _check_state(t: Optional[torch.Tensor], shape: Shape, name: str):
    if t is None:
        return
    nseq = shape.num_seqs if shape.num_seqs > 0 else shape.batch
    want = (nseq, shape.nheads, shape.headdim, shape.dstate)
    if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != want:
        raise ValueError(f"{name} must be a contiguous fp32 device tensor of shape {want}")


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
    _check_inputs(X, log_a, B, C, cu_seqlens)
    shape = make_shape(X, B, cu_seqlens)
    _check_state(initial_state, shape, "initial_state")
    if Y is None:
        Y = torch.empty_like(X)
    if final_state is None and want_final:
        nseq = X.shape[0] if cu_seqlens is None else cu_seqlens.numel() - 1
        final_state = torch.empty(nseq, X.shape[2], X.shape[3], B.shape[3], dtype=torch.float32, device=X.device)
    if workspace is None:
        workspace = Workspace(shape, chunk, X.device, state_block)
    elif state_block > 0 and state_block != workspace.state_block:
        raise ValueError("state_block differs from the workspace's")
    _call("ssd_fwd_ex", _ptr(X), _ptr(log_a), _ptr(B), _ptr(C), _ptr(cu_seqlens), _ptr(initial_state), int(chunk),
          workspace.state_block,
          _ptr(Y), _ptr(final_state), ctypes.byref(shape), _ptr(workspace.buffer), workspace.nbytes,
          _stream(X.device))
    return Y, final_state


def chunk_cumsum(log_a, cu_seqlens, shape: Shape, ws: Workspace):
    _call("ssd_chunk_cumsum", _ptr(log_a), _ptr(cu_seqlens), ws.chunk, ws.state_block, ctypes.byref(shape),
          _ptr(ws.buffer), ws.nbytes, _stream(ws.buffer.device))


def chunk_state(X, B, cu_seqlens, shape: Shape, ws: Workspace):
    _call("ssd_chunk_state", _ptr(X), _ptr(B), _ptr(cu_seqlens), ws.chunk, ws.state_block, ctypes.byref(shape),
          _ptr(ws.buffer), ws.nbytes, _stream(ws.buffer.device))


def state_passing(cu_seqlens, final_state, shape: Shape, ws: Workspace, initial_state=None):
    _check_state(initial_state, shape, "initial_state")
    _call("ssd_state_passing", _ptr(cu_seqlens), _ptr(initial_state), ws.chunk, ws.state_block, _ptr(final_state),
          ctypes.byref(shape), _ptr(ws.buffer), ws.nbytes, _stream(ws.buffer.device))


def chunk_scan(X, B, C, cu_seqlens, Y, shape: Shape, ws: Workspace):
    _call("ssd_chunk_scan", _ptr(X), _ptr(B), _ptr(C), _ptr(cu_seqlens), ws.chunk, ws.state_block, _ptr(Y),
          ctypes.byref(shape), _ptr(ws.buffer), ws.nbytes, _stream(ws.buffer.device))


def step(state: torch.Tensor, x: torch.Tensor, log_a: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
         y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode step (ssd_step): updates `state` in place and returns y."""
    for name, t in (("state", state), ("x", x), ("B", B), ("C", C)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if state.dtype != torch.float32 or log_a.dtype != torch.float32:
        raise ValueError("state and log_a must be fp32")
    b, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    shape = Shape(b, 1, H, G, P, N, 0, _dtype_code(x.dtype))
    if y is None:
        y = torch.empty_like(x)
    _call("ssd_step", _ptr(state), _ptr(x), _ptr(log_a), _ptr(B), _ptr(C), _ptr(y), ctypes.byref(shape),
          _stream(x.device))
    return y


def _check_mamba2(X, dt, dt_bias, A_log, D, z, H: int):
    lead = tuple(X.shape[:-1])
    if dt.dtype != torch.float32 or not dt.is_cuda or not dt.is_contiguous() or tuple(dt.shape) != lead:
        raise ValueError(f"dt must be a contiguous fp32 device tensor of shape {lead}")
    for name, t, need in (("dt_bias", dt_bias, False), ("A_log", A_log, True), ("D", D, False)):
        if t is None:
            if need:
                raise ValueError(f"{name} is required")
            continue
        if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != (H,):
            raise ValueError(f"{name} must be a contiguous fp32 device tensor of shape ({H},)")
    if z is not None and (z.dtype != X.dtype or not z.is_cuda or not z.is_contiguous() or z.shape != X.shape):
        raise ValueError("z must be a contiguous device tensor of X's shape and dtype")


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
    _check_inputs(X, None, B, C, cu_seqlens)
    _check_mamba2(X, dt, dt_bias, A_log, D, z, X.shape[2])
    shape = make_shape(X, B, cu_seqlens)
    _check_state(initial_state, shape, "initial_state")
    if Y is None:
        Y = torch.empty_like(X)
    if final_state is None and want_final:
        nseq = X.shape[0] if cu_seqlens is None else cu_seqlens.numel() - 1
        final_state = torch.empty(nseq, X.shape[2], X.shape[3], B.shape[3], dtype=torch.float32, device=X.device)
    if workspace is None:
        workspace = Workspace(shape, chunk, X.device, state_block)
    elif state_block > 0 and state_block != workspace.state_block:
        raise ValueError("state_block differs from the workspace's")
    _call("ssd_fwd_mamba2", _ptr(X), _ptr(dt), _ptr(dt_bias), _ptr(A_log), _ptr(D), _ptr(z), _ptr(B), _ptr(C),
          _ptr(cu_seqlens), _ptr(initial_state), int(chunk), workspace.state_block, _ptr(Y), _ptr(final_state),
          ctypes.byref(shape), _ptr(workspace.buffer), workspace.nbytes, _stream(X.device))
    return Y, final_state


def step_mamba2(state: torch.Tensor, x: torch.Tensor, dt: torch.Tensor, A_log: torch.Tensor, B: torch.Tensor,
                C: torch.Tensor, dt_bias: Optional[torch.Tensor] = None, D: Optional[torch.Tensor] = None,
                z: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One Mamba-2 decode step (ssd_step_mamba2): updates `state` in place and returns y."""
    for name, t in (("state", state), ("x", x), ("B", B), ("C", C)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if state.dtype != torch.float32:
        raise ValueError("state must be fp32")
    b, H, P = x.shape
    _check_mamba2(x, dt, dt_bias, A_log, D, z, H)
    G, N = B.shape[1], B.shape[2]
    if tuple(state.shape) != (b, H, P, N):
        raise ValueError(f"state must have shape {(b, H, P, N)}")
    shape = Shape(b, 1, H, G, P, N, 0, _dtype_code(x.dtype))
    if y is None:
        y = torch.empty_like(x)
    _call("ssd_step_mamba2", _ptr(state), _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A_log), _ptr(D), _ptr(z),
          _ptr(B), _ptr(C), _ptr(y), ctypes.byref(shape), _stream(x.device))
    return y


def set_state_chain(mode: int) -> int:
    """ssd_set_state_chain: 1 runs the state chain as one cooperative launch when
    it fits (the default), 0 always as two launches. Returns the previous mode."""
    return int(lib().ssd_set_state_chain(int(mode)))


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
    _check_inputs(X, log_a, B, C, cu_seqlens)
    if dY.dtype != X.dtype or not dY.is_cuda or not dY.is_contiguous() or dY.shape != X.shape:
        raise ValueError("dY must be a contiguous device tensor of X's shape and dtype")
    shape = make_shape(X, B, cu_seqlens)
    _check_state(initial_state, shape, "initial_state")
    _check_state(dfinal_state, shape, "dfinal_state")
    nbytes = bwd_workspace_bytes(shape, chunk, state_block)
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
    _check_inputs(X, None, B, C, cu_seqlens)
    _check_mamba2(X, dt, dt_bias, A_log, D, z, X.shape[2])
    if dY.dtype != X.dtype or not dY.is_cuda or not dY.is_contiguous() or dY.shape != X.shape:
        raise ValueError("dY must be a contiguous device tensor of X's shape and dtype")
    shape = make_shape(X, B, cu_seqlens)
    _check_state(initial_state, shape, "initial_state")
    _check_state(dfinal_state, shape, "dfinal_state")
    nbytes = bwd_mamba2_workspace_bytes(shape, chunk, state_block)
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
