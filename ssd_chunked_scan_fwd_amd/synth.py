"""Seeded synthetic inputs for the SSD forward pass and the decode step.

This module only draws random numbers and builds the shapes of the named
workloads; it holds none of the layer's arithmetic, and both the HIP path's
tests and the CPU oracle's tests take their inputs from it.

Value recipe (same for every workload): X ~ N(0, 1); dt ~ U(0.001, 0.1) per
(row, token, head); A_h ~ U(1, 16) per head; log_a = -dt * A_h (the product
taken in fp64, stored fp32); B, C ~ N(0, 1) / sqrt(N). The decay recipe mirrors
the discretisation the "Transformers are SSMs" paper card describes in its
"Paper vs code" items 7-8 (a = exp(dt * A) with A < 0, A initialised in [1, 16],
dt in [0.001, 0.1]); X is not scaled by dt. Draw order: sequence lengths
(packed workloads only), X, dt, A, B, C. X, B and C are drawn in fp32 and
rounded to the workload dtype (bf16: round-to-nearest-even).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                 # "fp32" or "bf16": dtype of X, B, C, Y
    batch: int
    T: int                     # tokens per row (packed: total tokens)
    H: int
    P: int
    N: int
    G: int
    Q: int                     # chunk length
    seed: int
    varlen: Optional[Tuple[int, int]] = None   # (min, max) sequence length for packed rows
    steps: int = 0             # decode workloads: number of single-token steps

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16


WORKLOADS: Dict[str, Workload] = {
    "tiny-fp32-T256": Workload("tiny-fp32-T256", "fp32", 1, 256, 2, 16, 16, 1, 32, seed=0),
    "b2-T2048-H24-N64": Workload("b2-T2048-H24-N64", "bf16", 2, 2048, 24, 64, 64, 1, 64, seed=1),
    "long-T16384-H32-N128": Workload("long-T16384-H32-N128", "bf16", 1, 16384, 32, 64, 128, 1, 128, seed=2),
    "sweep-b8-T4096-N64": Workload("sweep-b8-T4096-N64", "bf16", 8, 4096, 32, 64, 64, 1, 128, seed=30),
    "sweep-b8-T4096-N128": Workload("sweep-b8-T4096-N128", "bf16", 8, 4096, 32, 64, 128, 1, 128, seed=31),
    "sweep-b8-T4096-N256": Workload("sweep-b8-T4096-N256", "bf16", 8, 4096, 32, 64, 256, 1, 128, seed=32),
    "packed-T32768-H80-N128": Workload("packed-T32768-H80-N128", "bf16", 1, 32768, 80, 64, 128, 1, 128, seed=4,
                                       varlen=(512, 8192)),
    "decode-b64-H80-N128": Workload("decode-b64-H80-N128", "bf16", 64, 1, 80, 64, 128, 1, 0, seed=40, steps=4096),
}

# The headline workload: one long sequence, T = 16384, H = 32, P = 64, N = 128, Q = 128.
HEADLINE = "long-T16384-H32-N128"


def draw_lengths(rng: np.random.Generator, total: int, lo: int, hi: int) -> List[int]:
    """Lengths ~ U{lo..hi} (both ends included) until `total` is filled; the last one truncated."""
    out: List[int] = []
    filled = 0
    while filled < total:
        n = int(rng.integers(lo, hi, endpoint=True))
        n = min(n, total - filled)
        out.append(n)
        filled += n
    return out


def _to_dtype(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(dtype) if dtype != torch.float32 else t


def make_forward_inputs(batch: int, T: int, H: int, P: int, N: int, G: int = 1, dtype=torch.bfloat16,
                        seed: int = 0, varlen: Optional[Tuple[int, int]] = None,
                        lengths: Optional[List[int]] = None, dt_range=(0.001, 0.1), A_range=(1.0, 16.0)):
    """Inputs of one forward call as CPU tensors.

    Returns dict(X [b,T,H,P], log_a [b,T,H] fp32, B [b,T,G,N], C [b,T,G,N],
    cu_seqlens int32 [S+1] or None, lengths list or None).
    """
    rng = np.random.default_rng(seed)
    cu = None
    if varlen is not None or lengths is not None:
        if batch != 1:
            raise ValueError("packed sequences use a single row")
        if lengths is None:
            lengths = draw_lengths(rng, T, varlen[0], varlen[1])
        if sum(lengths) != T:
            raise ValueError("lengths must add up to T")
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32))
    X = rng.standard_normal((batch, T, H, P), dtype=np.float32)
    dt = rng.uniform(dt_range[0], dt_range[1], size=(batch, T, H))
    A = rng.uniform(A_range[0], A_range[1], size=(H,))
    inv = np.float32(1.0 / math.sqrt(N))
    Bm = rng.standard_normal((batch, T, G, N), dtype=np.float32) * inv
    Cm = rng.standard_normal((batch, T, G, N), dtype=np.float32) * inv
    la = (-dt * A[None, None, :]).astype(np.float32)
    return dict(X=_to_dtype(X, dtype), log_a=torch.from_numpy(la), B=_to_dtype(Bm, dtype),
                C=_to_dtype(Cm, dtype), cu_seqlens=cu, lengths=lengths)


def make_decode_inputs(batch: int, steps: int, H: int, P: int, N: int, G: int = 1, dtype=torch.bfloat16,
                       seed: int = 0):
    """Per-step decode inputs, stacked over steps, as CPU tensors.

    Returns dict(x [steps,b,H,P], log_a [steps,b,H] fp32, B [steps,b,G,N], C [steps,b,G,N]).
    """
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((steps, batch, H, P), dtype=np.float32)
    dt = rng.uniform(0.001, 0.1, size=(steps, batch, H))
    A = rng.uniform(1.0, 16.0, size=(H,))
    inv = np.float32(1.0 / math.sqrt(N))
    Bm = rng.standard_normal((steps, batch, G, N), dtype=np.float32) * inv
    Cm = rng.standard_normal((steps, batch, G, N), dtype=np.float32) * inv
    la = (-dt * A[None, None, :]).astype(np.float32)
    return dict(x=_to_dtype(X, dtype), log_a=torch.from_numpy(la), B=_to_dtype(Bm, dtype),
                C=_to_dtype(Cm, dtype))


def workload_inputs(w: Workload, seed: Optional[int] = None):
    """Inputs of a named workload (seeded by the workload unless `seed` is given)."""
    s = w.seed if seed is None else seed
    if w.steps:
        return make_decode_inputs(w.batch, w.steps, w.H, w.P, w.N, w.G, w.torch_dtype, s)
    return make_forward_inputs(w.batch, w.T, w.H, w.P, w.N, w.G, w.torch_dtype, s, varlen=w.varlen)


# ---------------------------------------------------------------------------
# Mamba-2 block inputs: the SSD call as the block makes it, with the raw step
# sizes, the per-head parameters and the gate instead of a precomputed log a.
#
# Value recipe: x ~ N(0, 1); dt (raw, per row, token and head) ~ N(0, 0.5^2);
# dt_bias = ln(u) with u log-uniform in [0.001, 0.1], so that the step sizes
# land around the [0.001, 0.1] range of the pages' initialisation;
# A_log = ln(U(1, 16)) (A initialised uniformly in [1, 16] and stored as its
# log); D ~ U(0.5, 1.5); z ~ N(0, 1); B, C ~ N(0, 1) / sqrt(N). Draw order:
# sequence lengths (packed only), x, dt, dt_bias, A_log, D, z, B, C. x, z, B
# and C are drawn in fp32 and rounded to the workload dtype; dt, dt_bias, A_log
# and D stay fp32.
# ---------------------------------------------------------------------------
def make_mamba2_inputs(batch: int, T: int, H: int, P: int, N: int, G: int = 1, dtype=torch.bfloat16,
                       seed: int = 0, varlen: Optional[Tuple[int, int]] = None,
                       lengths: Optional[List[int]] = None):
    """Inputs of one Mamba-2 SSD call as CPU tensors.

    Returns dict(X [b,T,H,P], dt [b,T,H] fp32, dt_bias [H], A_log [H], D [H]
    (fp32), z [b,T,H,P], B [b,T,G,N], C [b,T,G,N], cu_seqlens int32 [S+1] or
    None, lengths list or None).
    """
    rng = np.random.default_rng(seed)
    cu = None
    if varlen is not None or lengths is not None:
        if batch != 1:
            raise ValueError("packed sequences use a single row")
        if lengths is None:
            lengths = draw_lengths(rng, T, varlen[0], varlen[1])
        if sum(lengths) != T:
            raise ValueError("lengths must add up to T")
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32))
    X = rng.standard_normal((batch, T, H, P), dtype=np.float32)
    dt = rng.standard_normal((batch, T, H), dtype=np.float32) * np.float32(0.5)
    dt_bias = rng.uniform(math.log(0.001), math.log(0.1), size=(H,)).astype(np.float32)
    A_log = np.log(rng.uniform(1.0, 16.0, size=(H,))).astype(np.float32)
    D = rng.uniform(0.5, 1.5, size=(H,)).astype(np.float32)
    z = rng.standard_normal((batch, T, H, P), dtype=np.float32)
    inv = np.float32(1.0 / math.sqrt(N))
    Bm = rng.standard_normal((batch, T, G, N), dtype=np.float32) * inv
    Cm = rng.standard_normal((batch, T, G, N), dtype=np.float32) * inv
    return dict(X=_to_dtype(X, dtype), dt=torch.from_numpy(dt), dt_bias=torch.from_numpy(dt_bias),
                A_log=torch.from_numpy(A_log), D=torch.from_numpy(D), z=_to_dtype(z, dtype),
                B=_to_dtype(Bm, dtype), C=_to_dtype(Cm, dtype), cu_seqlens=cu, lengths=lengths)


def make_mamba2_decode_inputs(batch: int, steps: int, H: int, P: int, N: int, G: int = 1,
                              dtype=torch.bfloat16, seed: int = 0):
    """Per-step inputs of the Mamba-2 decode step, stacked over steps (same recipe).

    Returns dict(x [steps,b,H,P], dt [steps,b,H] fp32, dt_bias [H], A_log [H],
    D [H], z [steps,b,H,P], B [steps,b,G,N], C [steps,b,G,N]).
    """
    d = make_mamba2_inputs(steps, batch, H, P, N, G, dtype, seed)
    return dict(x=d["X"], dt=d["dt"], dt_bias=d["dt_bias"], A_log=d["A_log"], D=d["D"], z=d["z"],
                B=d["B"], C=d["C"])


def make_cotangents(batch: int, T: int, H: int, P: int, N: int, nseq: int, dtype=torch.bfloat16, seed: int = 0):
    """Seeded output gradients for a backward call: dY [b,T,H,P] ~ N(0, 1) in the
    workload dtype and dfinal [nseq,H,P,N] ~ N(0, 1) fp32 (the final-state layout)."""
    rng = np.random.default_rng(seed)
    dY = rng.standard_normal((batch, T, H, P), dtype=np.float32)
    dfin = rng.standard_normal((nseq, H, P, N), dtype=np.float32)
    return dict(dY=_to_dtype(dY, dtype), dfinal=torch.from_numpy(dfin))
