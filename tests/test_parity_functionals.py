"""CPU checks of the tolerance functionals the GPU parity tests apply."""
import numpy as np
import pytest
import torch

from parity import assert_close, assert_close_gated, errors, gated_errors


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).double().numpy()


def test_bf16_rounding_alone_passes_the_bars():
    rng = np.random.default_rng(0)
    u = rng.standard_normal(200_000)
    assert_close(_bf16(u), u, "bf16")
    # gated: heavy tails, where the plain max|d|/rms bar is met by the rounding alone only barely or not at all
    z = rng.standard_normal(200_000) * 2.0
    s = z / (1.0 + np.exp(-z))
    y = u * s
    assert_close_gated(_bf16(y), y, u, s, "bf16")


def test_gated_bar_reduces_to_unit_scale_and_catches_errors():
    rng = np.random.default_rng(1)
    u = rng.standard_normal(10_000)
    s = np.ones_like(u)
    y = u.copy()
    bad = y.copy()
    i = int(np.argmin(np.abs(u)))           # an element far below unit scale
    bad[i] += 0.06                          # 6 % of rms(u): over the 5e-2 bar
    with pytest.raises(AssertionError):
        assert_close_gated(bad, y, u, s, "bf16")
    ok = y.copy()
    ok[i] += 0.04
    assert_close_gated(ok, y, u, s, "bf16")
    # a wrong gate on 1 % of the elements fails
    g = rng.standard_normal(10_000)
    sg = g / (1.0 + np.exp(-g))
    wrong = u * sg
    wrong[:100] = u[:100] / (1.0 + np.exp(-g[:100]))   # sigmoid instead of silu
    with pytest.raises(AssertionError):
        assert_close_gated(wrong, u * sg, u, sg, "bf16")


def test_functionals_report_non_finite():
    assert not errors([np.nan, 1.0], [1.0, 1.0])["finite"]
    assert not gated_errors([np.inf], [1.0], [1.0], [1.0])["finite"]
