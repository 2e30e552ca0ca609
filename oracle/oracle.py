"""fp64 CPU oracle for the scalar-decay SSM forward pass (test infrastructure).

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg are the only callers. The HIP library never
imports, links or runs anything in this directory, and this directory imports
nothing from the HIP library.

The oracle is the plain definition of the layer, run token by token in fp64:

    h_t = a_t h_{t-1} + B_t x_t^T,    y_t = C_t^T h_t,    a_t = exp(log_a_t)

("Transformers are SSMs" paper card, wikillm.com/papers/2405.21060: Method 1,
selective SSM as a matrix, paper sections 2-3; Method 2, scalar-identity case,
paper section 5.1). The chunked SSD algorithm (paper card Method 5, paper
section 6) is an exact rewrite of this recurrence, so the recurrence is the
reference and not an approximation of it.

Helpers here that are not the recurrence:
  * ``chunk_segments`` -- the chunk grid used to read intermediate results
    (chunks restart at every sequence start; the last chunk of a sequence may
    be short).
  * ``chunk_cumsum`` -- the cumulative log decay restarted in every chunk
    (paper card Method 5, the within-chunk cumulative decay), a plain fp64 cumsum.

The Mamba-2 functions (``softplus``, ``silu``, ``mamba2_discretize``,
``mamba2_forward``, ``mamba2_step``) put the block's discretisation, skip and
gate around that recurrence (paper card Method 6, Paper vs code 3, 7, 8).

``backward`` is reverse mode through the same recurrence (its adjoint), the
plain definition of the gradients; the pages give no backward algorithm.
``mamba2_backward`` applies the chain rule through the Mamba-2 gate, skip and
discretisation around it.

Every function in this file is pinned by ``tests/test_oracle.py`` against the
quadratic dual form, closed forms, causal linear attention, packing,
continuation, hand-worked examples and invariants; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Iterable, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libssd_oracle.so")
# SSD_ORACLE_LIBRARY names a prebuilt oracle library to load instead (the
# sanitizer build, build_sanitized()).
_LIB_OVERRIDE = os.environ.get("SSD_ORACLE_LIBRARY")
_lib = None

# Mutant codes (see ssd_oracle.c); used only by the pin-strength tests.
MUTANTS = {
    "decay_after_input": 1,
    "output_before_update": 2,
    "swap_b_c": 3,
    "decay_sign": 4,
    "no_decay": 5,
    "group_mod": 6,
    "decay_next_token": 7,
    "state_transpose": 8,
}


def build(force: bool = True) -> str:
    """Compile ssd_oracle.c with gcc (fp64, OpenMP, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def build_sanitized(out_path: str) -> str:
    """The same oracle built with clang, AddressSanitizer and
    UndefinedBehaviorSanitizer (one ASan runtime with the HIP library's
    checking build), for the CPU sanitizer run."""
    clang = "/opt/rocm/llvm/bin/clang"
    cmd = [clang, "-O1", "-g", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-Wall",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
           "-shared-libasan", "-o", out_path, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return out_path


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB_PATH):
                build(force=True)
            lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int)
        lib.ssd_oracle_scan.restype = ctypes.c_int
        lib.ssd_oracle_scan.argtypes = [ctypes.c_int] * 6 + [dp] * 4 + [ctypes.c_int, ip, dp, dp, dp, ip, dp,
                                                                       ctypes.c_int, ctypes.c_int]
        lib.ssd_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().ssd_oracle_max_threads())


def _dptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _iptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int))


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def sequence_segments(rows: int, T: int, cu_seqlens: Optional[Sequence[int]] = None):
    """(row, begin, end) triples of the independent sequences.

    Without cu_seqlens every row is one sequence [0, T). With cu_seqlens (one
    packed row) sequence s is [cu[s], cu[s+1]) of row 0 and starts from a zero
    state: a packed batch behaves as separate runs (the pages' variable-length
    training without padding, read as a reset at every boundary).
    """
    if cu_seqlens is None:
        return [(r, 0, T) for r in range(rows)]
    cu = [int(v) for v in cu_seqlens]
    if rows != 1:
        raise ValueError("packed sequences need a single row")
    return [(0, cu[s], cu[s + 1]) for s in range(len(cu) - 1)]


def chunk_segments(rows: int, T: int, Q: int, cu_seqlens: Optional[Sequence[int]] = None):
    """Chunk grid: every sequence cut into chunks of Q tokens from its start.

    Returns (row, begin, end) per chunk in sequence order, chunk order. The
    last chunk of a sequence holds the remainder (paper card Method 5 cuts
    the sequence into T/Q blocks; a short last chunk is the reading for
    lengths that Q does not divide).
    """
    out = []
    for (r, b, e) in sequence_segments(rows, T, cu_seqlens):
        t = b
        while t < e:
            out.append((r, t, min(t + Q, e)))
            t += Q
    return out


def scan(X, la, B, C, segments: Optional[Iterable] = None, init=None, want_y: bool = True,
         want_final: bool = True, snap_slot=None, nsnaps: int = 0, threads: int = 0,
         mutant: int = 0):
    """Run the fp64 recurrence.

    X [rows,T,H,P], la [rows,T,H], B and C [rows,T,G,N] (any float dtype; upcast
    to fp64 exactly). ``segments`` defaults to one segment per row. ``init``
    [nseg,H,P,N] is the starting state of each segment (zero when None).
    Returns (Y [rows,T,H,P] or None, final [nseg,H,P,N] or None, snaps or None).
    """
    X = _f64(X)
    la = _f64(la)
    B = _f64(B)
    C = _f64(C)
    rows, T, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    if la.shape != (rows, T, H) or B.shape != (rows, T, G, N) or C.shape != B.shape:
        raise ValueError("shape mismatch")
    if segments is None:
        segments = [(r, 0, T) for r in range(rows)]
    seg = np.ascontiguousarray(np.asarray(list(segments), dtype=np.int32).reshape(-1, 3))
    nseg = seg.shape[0]
    Y = np.zeros((rows, T, H, P), np.float64) if want_y else None
    fin = np.zeros((nseg, H, P, N), np.float64) if want_final else None
    ini = None
    if init is not None:
        ini = _f64(init)
        if ini.shape != (nseg, H, P, N):
            raise ValueError("init must be [nseg,H,P,N]")
    ss = None
    snaps = None
    if snap_slot is not None:
        ss = np.ascontiguousarray(np.asarray(snap_slot, dtype=np.int32).reshape(rows * T))
        snaps = np.zeros((max(nsnaps, 1), H, P, N), np.float64)
    rc = _load().ssd_oracle_scan(rows, T, H, G, P, N, _dptr(X), _dptr(la), _dptr(B), _dptr(C), nseg,
                                 _iptr(seg), _dptr(ini), _dptr(Y), _dptr(fin), _iptr(ss), _dptr(snaps),
                                 int(threads), int(mutant))
    if rc != 0:
        raise ValueError("ssd_oracle_scan rejected its arguments")
    return Y, fin, snaps


def forward(X, la, B, C, cu_seqlens=None, threads: int = 0, mutant: int = 0, init=None):
    """Y and final states of the layer, from zero initial states or ``init``.

    final (and init) is [rows,H,P,N] without cu_seqlens and [S,H,P,N] with it.
    """
    X = _f64(X)
    rows, T = X.shape[0], X.shape[1]
    segs = sequence_segments(rows, T, cu_seqlens)
    Y, fin, _ = scan(X, la, B, C, segments=segs, init=init, threads=threads, mutant=mutant)
    return Y, fin


def step(state, x, la, B, C):
    """One recurrent step (the loop body of the recurrence) from ``state``.

    state [b,H,P,N], x [b,H,P], la [b,H], B and C [b,G,N]. Returns (y [b,H,P],
    new_state [b,H,P,N]); y is read from the updated state.
    """
    x = _f64(x)
    b, H, P = x.shape
    Y, fin, _ = scan(x[:, None], _f64(la)[:, None], _f64(B)[:, None], _f64(C)[:, None],
                     segments=[(r, 0, 1) for r in range(b)], init=_f64(state))
    return Y[:, 0], fin


# ---------------------------------------------------------------------------
# The Mamba-2 block's SSD call ("Transformers are SSMs" paper card,
# wikillm.com/papers/2405.21060: Method 6, the block sketch; Paper vs code
# items 3, 7 and 8; Pitfalls, "Discretisation is missing from the paper").
# The block does not hand the layer log a and a scaled input; it hands raw
# step sizes and per-head parameters, and finishes the output itself:
#
#   dt'  = softplus(dt + dt_bias)              per (row, token, head)
#   log a = dt' * A,  A = -exp(A_log)          per head
#   y    = SSM(a, B, C)(x * dt') + D * x       the skip uses the unscaled x
#   y    = y * silu(z),  silu(v) = v / (1 + exp(-v))   the gate, when z is given
#
# Readings where the pages leave a step open: softplus is log(1 + e^v) with no
# threshold; there is no clamp on dt'; the gate multiplies after the skip and
# before any normalisation (the block sketch gates first, then normalises).
# ---------------------------------------------------------------------------
# Planted mistakes of the Mamba-2 arithmetic, used only by the pin-strength tests.
MAMBA2_MUTANTS = {
    "skip_uses_scaled_x": 1,
    "gate_before_skip": 2,
    "bias_ignored": 3,
    "decay_rate_positive": 4,
    "input_not_scaled": 5,
    "gate_sigmoid": 6,
    "decay_uses_raw_dt": 7,
}


def softplus(v) -> np.ndarray:
    """log(1 + e^v) in fp64, evaluated without overflow (numpy's logaddexp(0, v))."""
    return np.logaddexp(0.0, _f64(v))


def silu(v) -> np.ndarray:
    """v / (1 + e^-v) in fp64, written as v * sigmoid(v) with a stable sigmoid."""
    v = _f64(v)
    return v * (0.5 * (1.0 + np.tanh(0.5 * v)))


def mamba2_discretize(dt, dt_bias, A_log, mutant: int = 0):
    """Step sizes dt' = softplus(dt + dt_bias) and log decays dt' * A, A = -exp(A_log).

    dt [..., H] (raw), dt_bias [H] or None (zero), A_log [H]. Returns (dt', log_a),
    both fp64 with the shape of dt.
    """
    dt = _f64(dt)
    bias = np.zeros(dt.shape[-1]) if dt_bias is None else _f64(dt_bias)
    v = dt if mutant == MAMBA2_MUTANTS["bias_ignored"] else dt + bias
    dtp = softplus(v)
    A = np.exp(_f64(A_log))
    A = A if mutant == MAMBA2_MUTANTS["decay_rate_positive"] else -A
    la = (v if mutant == MAMBA2_MUTANTS["decay_uses_raw_dt"] else dtp) * A
    return dtp, la


def _mamba2_epilogue(Y, x, D, z, mutant):
    if mutant == MAMBA2_MUTANTS["gate_before_skip"]:
        if z is not None:
            Y = Y * silu(z)
        return Y + (0.0 if D is None else _f64(D)[None, None, :, None] * x)
    if D is not None:
        Y = Y + _f64(D)[None, None, :, None] * x
    if z is not None:
        g = _f64(z)
        Y = Y * (0.5 * (1.0 + np.tanh(0.5 * g)) if mutant == MAMBA2_MUTANTS["gate_sigmoid"] else silu(g))
    return Y


def mamba2_forward(X, dt, dt_bias, A_log, D, z, B, C, cu_seqlens=None, init=None, threads: int = 0,
                   mutant: int = 0):
    """Y and final states of the Mamba-2 block's SSD call.

    X [rows,T,H,P] (the block's x, unscaled), dt [rows,T,H] raw step sizes,
    dt_bias [H] or None, A_log [H], D [H] or None (no skip), z [rows,T,H,P] or
    None (no gate), B and C [rows,T,G,N]; cu_seqlens and init as in forward().
    The recurrence itself is forward()'s, run on x * dt' with log a = dt' * A.
    """
    x = _f64(X)
    dtp, la = mamba2_discretize(dt, dt_bias, A_log, mutant)
    Xs = x if mutant == MAMBA2_MUTANTS["input_not_scaled"] else x * dtp[..., None]
    Y, fin = forward(Xs, la, B, C, cu_seqlens=cu_seqlens, threads=threads, init=init)
    if mutant == MAMBA2_MUTANTS["skip_uses_scaled_x"]:
        x = x * dtp[..., None]
    return _mamba2_epilogue(Y, x, D, z, mutant), fin


def mamba2_step(state, x, dt, dt_bias, A_log, D, z, B, C):
    """One Mamba-2 decode step from ``state``.

    state [b,H,P,N], x [b,H,P], dt [b,H] raw, dt_bias/A_log/D [H] (D may be
    None), z [b,H,P] or None, B and C [b,G,N]. Returns (y [b,H,P], new_state).
    """
    x = _f64(x)
    Y, fin = mamba2_forward(x[:, None], _f64(dt)[:, None], dt_bias, A_log, D,
                            None if z is None else _f64(z)[:, None], _f64(B)[:, None], _f64(C)[:, None],
                            init=_f64(state))
    return Y[:, 0], fin


# ---------------------------------------------------------------------------
# Backward pass (reverse mode through the recurrence). The pages motivate the
# layer by training but give no backward algorithm; the plain definition of
# the gradient is the adjoint of the recurrence h_t = a_t h_{t-1} + B_t x_t^T,
# y_t = C_t^T h_t (paper card Method 1; Method 2 for the scalar a_t). For
# L = <dY, Y> + <dfinal, h_last>, with lam_t = dL/dh_t:
#   lam_last = dfinal + C_last dY_last^T,  lam_t = a_{t+1} lam_{t+1} + C_t dY_t^T
#   dx_t = lam_t^T B_t,  dB_t = lam_t x_t,  dC_t = h_t dY_t,
#   d log a_t = a_t <lam_t, h_{t-1}>,  d h_init = a_first lam_first.
# ---------------------------------------------------------------------------
BACKWARD_MUTANTS = {
    "decay_before_input": 1,    # lam decayed before C_t dY_t^T is added
    "log_a_uses_h_t": 2,        # <lam_t, h_t> in place of <lam_t, h_{t-1}>
    "final_ignored": 3,         # dfinal dropped
    "dC_previous_state": 4,     # dC_t from h_{t-1}
    "dx_reads_C": 5,            # dx_t = lam_t^T C_t
}


def backward(X, la, B, C, dY, dfinal=None, cu_seqlens=None, init=None, mutant: int = 0):
    """Gradients of L = <dY, Y> + <dfinal, final> through the layer.

    X [rows,T,H,P], la [rows,T,H], B and C [rows,T,G,N], dY like X; dfinal and
    init [rows or S,H,P,N] (the final-state layout, element (p, n) = h[n][p]) or
    None. Returns dict(dX, dlog_a, dB, dC, dinit), fp64, dB and dC summed over
    the heads of each group. Keeps every state in memory: small cases only.
    """
    X, la, B, C, dY = (_f64(a) for a in (X, la, B, C, dY))
    rows, T, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    grp = np.arange(H) // (H // G)
    segs = sequence_segments(rows, T, cu_seqlens)
    dX = np.zeros_like(X)
    dla = np.zeros_like(la)
    dB = np.zeros_like(B)
    dC = np.zeros_like(C)
    dinit = np.zeros((len(segs), H, P, N))
    for si, (r, b, e) in enumerate(segs):
        # forward, keeping h_t for every t of the sequence: hs[k] = h_{b+k-1}
        hs = np.zeros((e - b + 1, H, N, P))
        if init is not None:
            hs[0] = np.transpose(_f64(init)[si], (0, 2, 1))
        for t in range(b, e):
            a = np.exp(la[r, t])[:, None, None]
            hs[t - b + 1] = a * hs[t - b] + np.einsum("hn,hp->hnp", B[r, t, grp], X[r, t])
        lam = np.zeros((H, N, P))
        if dfinal is not None and mutant != BACKWARD_MUTANTS["final_ignored"]:
            lam = np.transpose(_f64(dfinal)[si], (0, 2, 1)).copy()
        for t in range(e - 1, b - 1, -1):
            a = np.exp(la[r, t])[:, None, None]
            h_prev, h_t = hs[t - b], hs[t - b + 1]
            if mutant == BACKWARD_MUTANTS["decay_before_input"]:
                lam = a * lam
            lam = lam + np.einsum("hn,hp->hnp", C[r, t, grp], dY[r, t])
            Bt = C[r, t, grp] if mutant == BACKWARD_MUTANTS["dx_reads_C"] else B[r, t, grp]
            dX[r, t] = np.einsum("hnp,hn->hp", lam, Bt)
            np.add.at(dB[r, t], grp, np.einsum("hnp,hp->hn", lam, X[r, t]))
            hc = h_prev if mutant == BACKWARD_MUTANTS["dC_previous_state"] else h_t
            np.add.at(dC[r, t], grp, np.einsum("hnp,hp->hn", hc, dY[r, t]))
            hl = h_t if mutant == BACKWARD_MUTANTS["log_a_uses_h_t"] else h_prev
            dla[r, t] = a[:, 0, 0] * np.einsum("hnp,hnp->h", lam, hl)
            if mutant != BACKWARD_MUTANTS["decay_before_input"]:
                lam = a * lam
        dinit[si] = np.transpose(lam, (0, 2, 1))
    return dict(dX=dX, dlog_a=dla, dB=dB, dC=dC, dinit=dinit)


# ---------------------------------------------------------------------------
# Backward of the Mamba-2 block's call (mamba2_forward): the chain rule through
# the gate, the skip and the discretisation around the recurrence's backward.
# With dt' = softplus(dt + dt_bias), A = -exp(A_log), x~ = x dt', v = SSM(x~) +
# D x and y = v silu(z):
#   dz = dY v silu'(z),  silu'(g) = sig(g) (1 + g (1 - sig(g))),  dv = dY silu(z)
#   (dx~, d log a, dB, dC, d h_init) = backward of the recurrence for cotangent dv
#   dx = dx~ dt' + D dv,   dD = sum_{t,p} dv x
#   d dt' = sum_p dx~ x + A d log a,   d dt = d dt' sig(dt + dt_bias)
#   d dt_bias = sum_t d dt,   d A_log = A sum_t dt' d log a
# (softplus' = sig; dA / dA_log = A).
# ---------------------------------------------------------------------------
MAMBA2_BACKWARD_MUTANTS = {
    "gate_derivative_sigmoid": 1,   # dz with sig(z) in place of silu'(z)
    "skip_grad_scaled": 2,          # the skip's dx multiplied by dt'
    "softplus_derivative_dropped": 3,  # d dt = d dt'
    "A_log_chain_dropped": 4,       # d A_log = sum_t dt' d log a (factor A dropped)
}


def _sigmoid(v):
    return 0.5 * (1.0 + np.tanh(0.5 * _f64(v)))


def mamba2_backward(X, dt, dt_bias, A_log, D, z, B, C, dY, dfinal=None, cu_seqlens=None, init=None,
                    mutant: int = 0):
    """Gradients of L = <dY, y> + <dfinal, final> for mamba2_forward with the same inputs.

    Returns dict(dX, ddt, ddt_bias, dA_log, dD, dz, dB, dC, dinit, dxs), fp64; dD is
    None without a skip, dz None without a gate; ddt_bias is returned whether or not
    a bias was given (the gradient with respect to a zero bias); dxs is the
    recurrence's gradient of its input x dt'.
    """
    x, dY = _f64(X), _f64(dY)
    dtp, la = mamba2_discretize(dt, dt_bias, A_log)
    A = -np.exp(_f64(A_log))
    xs = x * dtp[..., None]
    dz = None
    dv = dY
    if z is not None:
        g = _f64(z)
        sg = _sigmoid(g)
        u, _ = forward(xs, la, B, C, cu_seqlens=cu_seqlens, init=init)
        v = u + (0.0 if D is None else _f64(D)[None, None, :, None] * x)
        dsilu = sg if mutant == MAMBA2_BACKWARD_MUTANTS["gate_derivative_sigmoid"] else sg * (1.0 + g * (1.0 - sg))
        dz = dY * v * dsilu
        dv = dY * (g * sg)
    gs = backward(xs, la, B, C, dv, dfinal=dfinal, cu_seqlens=cu_seqlens, init=init)
    dxs, dla = gs["dX"], gs["dlog_a"]
    dX = dxs * dtp[..., None]
    if D is not None:
        skip = _f64(D)[None, None, :, None] * dv
        if mutant == MAMBA2_BACKWARD_MUTANTS["skip_grad_scaled"]:
            skip = skip * dtp[..., None]
        dX = dX + skip
    ddtp = np.sum(dxs * x, axis=-1) + A * dla
    bias = np.zeros(dtp.shape[-1]) if dt_bias is None else _f64(dt_bias)
    ddt = ddtp if mutant == MAMBA2_BACKWARD_MUTANTS["softplus_derivative_dropped"] else \
        ddtp * _sigmoid(_f64(dt) + bias)
    dA = np.sum(dla * dtp, axis=(0, 1))
    dA_log = dA if mutant == MAMBA2_BACKWARD_MUTANTS["A_log_chain_dropped"] else dA * A
    dD = None if D is None else np.sum(dv * x, axis=(0, 1, 3))
    return dict(dX=dX, ddt=ddt, ddt_bias=np.sum(ddt, axis=(0, 1)), dA_log=dA_log, dD=dD, dz=dz,
                dB=gs["dB"], dC=gs["dC"], dinit=gs["dinit"], dxs=dxs)


def chunk_cumsum(la, segments) -> np.ndarray:
    """Cumulative log decay restarted at the start of every segment (fp64).

    Same layout as la [rows,T,H]; tokens outside every segment are 0.
    """
    la = _f64(la)
    out = np.zeros_like(la)
    for (r, b, e) in segments:
        out[r, b:e] = np.cumsum(la[r, b:e], axis=0)
    return out
