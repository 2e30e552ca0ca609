"""Shared helpers of the GPU parity tests: tolerance functionals, oracle runs.

Tolerances (written here once, used by every parity test):
  * fp32 inputs: max_i |d_i| / max(|ref_i|, rms(ref)) <= 1e-4.
  * bf16 inputs with fp32 accumulation: ||d||_2 / ||ref||_2 <= 2e-2 and
    max_i |d_i| / rms(ref) <= 5e-2 (the per-element bound on unit-scale output,
    with the output scaled by its RMS).
Both are applied separately to Y and to the final states.
"""
from __future__ import annotations

import numpy as np
import torch

FP32_MAXREL = 1e-4
BF16_RELL2 = 2e-2
BF16_MAXABS_UNIT = 5e-2


def errors(gpu, ref):
    g = np.asarray(gpu, np.float64).ravel()
    r = np.asarray(ref, np.float64).ravel()
    d = np.abs(g - r)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    rms = max(rms, 1e-30)
    return dict(
        rel_l2=float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)),
        max_unit=float(d.max() / rms) if d.size else 0.0,
        max_rel=float(np.max(d / np.maximum(np.abs(r), rms))) if d.size else 0.0,
        finite=bool(np.all(np.isfinite(g))),
    )


def assert_close(gpu, ref, dtype: str, what: str = ""):
    e = errors(gpu, ref)
    assert e["finite"], f"{what}: non-finite values"
    if dtype == "fp32":
        assert e["max_rel"] <= FP32_MAXREL, f"{what}: {e}"
    else:
        assert e["rel_l2"] <= BF16_RELL2 and e["max_unit"] <= BF16_MAXABS_UNIT, f"{what}: {e}"
    return e


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").double().numpy()


def dtype_name(t: torch.Tensor) -> str:
    return "fp32" if t.dtype == torch.float32 else "bf16"
