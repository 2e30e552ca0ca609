"""CPU checks of the tolerance functionals the GPU parity tests apply."""
import numpy as np
import pytest
import torch

from parity import assert_close, assert_close_gated, assert_close_rounded, errors, gated_errors


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


def test_gated_bar_catches_relative_errors_on_large_elements():
    """The allowance relative to |ref_i| is the output's own rounding (2^-8), not
    a fraction of the bar: 5 % of the value on the largest gated elements fails,
    and so does 1 % where the unit-scale term is small."""
    rng = np.random.default_rng(2)
    u = rng.standard_normal(50_000)
    z = rng.standard_normal(50_000) * 2.0
    s = z / (1.0 + np.exp(-z))
    y = u * s
    big = np.argsort(-np.abs(y))[:20]
    bad = y.copy()
    bad[big] *= 1.05
    with pytest.raises(AssertionError):
        assert_close_gated(bad, y, u, s, "bf16")
    k = int(np.argmax(np.abs(u) / (np.abs(s) + 1e-3) * (np.abs(s) < 0.05)))   # large u, tiny gate
    bad = y.copy()
    bad[k] += 0.06 * abs(s[k]) * np.sqrt(np.mean(u * u)) + 0.01 * abs(y[k])
    with pytest.raises(AssertionError):
        assert_close_gated(bad, y, u, s, "bf16")
    # the old allowance (5e-2 (|s_i| r + |ref_i|)) would have passed the 5 % error
    r = np.sqrt(np.mean(u * u))
    bad = y.copy()
    bad[big] *= 1.05
    assert np.all(np.abs(bad - y) <= 5e-2 * (np.abs(s) * r + np.abs(y)))


def test_gated_bar_fp32():
    rng = np.random.default_rng(3)
    u = rng.standard_normal(10_000)
    z = rng.standard_normal(10_000)
    s = z / (1.0 + np.exp(-z))
    y = u * s
    assert_close_gated(y * (1 + 5e-5), y, u, s, "fp32")
    with pytest.raises(AssertionError):
        assert_close_gated(y * (1 + 2e-4), y, u, s, "fp32")


def test_functionals_report_non_finite():
    assert not errors([np.nan, 1.0], [1.0, 1.0])["finite"]
    assert not gated_errors([np.inf], [1.0], [1.0], [1.0])["finite"]


def test_rounded_bar_admits_exact_rounding_only():
    """A heavy-tailed output (a few elements at ~17 rms, as the Mamba-2 backward's dB):
    the exact values rounded to bf16 once fail the plain max-abs bar but pass the bar
    with the rounding allowance; 5 % errors on the large elements, or 6 % of rms on a
    small one, fail it."""
    rng = np.random.default_rng(4)
    ref = rng.standard_normal(100_000) * np.exp(rng.standard_normal(100_000))   # log-normal scales
    r = np.sqrt(np.mean(ref * ref))
    # 20 elements just under half a bf16 ulp above a power of two near 17 rms: rounding
    # moves each by almost 2^-8 of its value
    p2 = 2.0 ** np.round(np.log2(17.0 * r))
    ref[:20] = p2 * (1 + 0.99 * 2.0 ** -8) * np.sign(rng.standard_normal(20))
    rnd = _bf16(ref)
    assert errors(rnd, ref)["max_unit"] > 5e-2     # the plain bar fails on rounding alone
    assert_close_rounded(rnd, ref, "bf16")
    big = np.argsort(-np.abs(ref))[:10]
    bad = ref.copy()
    bad[big] *= 1.05
    with pytest.raises(AssertionError):
        assert_close_rounded(bad, ref, "bf16")
    i = int(np.argmin(np.abs(ref)))
    bad = ref.copy()
    bad[i] += 0.06 * r
    with pytest.raises(AssertionError):
        assert_close_rounded(bad, ref, "bf16")
