"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Every check here compares the oracle's token-by-token recurrence with
something other than itself: hand-worked examples, the brute-force quadratic
dual form, the chunked block decomposition at many chunk lengths, scalar closed
forms, causal linear attention, packing/reset, continuation and invariants.
``test_mutants_are_caught`` plants plausible mistakes in the oracle (on the CPU)
and shows that each one fails at least one pin.
"""
import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import oracle
from ssd_forms import chunked_form, dual_form
from ssd_chunked_scan_fwd_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _rand(T, H, P, N, G=1, seed=0, rows=1, la_scale=1.0):
    d = synth.make_forward_inputs(rows, T, H, P, N, G, dtype=__import__("torch").float32, seed=seed)
    X = d["X"].double().numpy()
    la = d["log_a"].double().numpy() * la_scale
    B = d["B"].double().numpy()
    C = d["C"].double().numpy()
    return X, la, B, C


def _relmax(a, b):
    scale = max(np.max(np.abs(b)), 1e-300)
    return np.max(np.abs(a - b)) / scale


# ---------------------------------------------------------------- hand worked

def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_hand_worked(case):
    x = np.array(case["x"])[None]
    a = np.array(case["a"])
    with np.errstate(divide="ignore"):
        la = np.log(a)[None]
    B = np.array(case["B"])[None]
    C = np.array(case["C"])[None]
    Y, fin = oracle.forward(x, la, B, C)
    np.testing.assert_allclose(Y[0], np.array(case["y"]), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(fin[0], np.array(case["final"]), rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------- dual form

@settings(max_examples=25, deadline=None)
@given(T=st.integers(1, 24), H=st.integers(1, 3), P=st.integers(1, 5), N=st.integers(1, 5),
       gsel=st.integers(0, 2), seed=st.integers(0, 2 ** 31 - 1))
def test_dual_form_bruteforce(T, H, P, N, gsel, seed):
    G = [1, H, 1 if H % 2 else max(H // 2, 1)][gsel]
    X, la, B, C = _rand(T, H, P, N, G, seed)
    Y, fin = oracle.forward(X, la, B, C)
    Yd, fd = dual_form(X[0], la[0], B[0], C[0])
    assert _relmax(Y[0], Yd) <= 1e-12
    assert _relmax(fin[0], fd) <= 1e-12


def test_dual_form_multi_group():
    # G = 2 groups of 2 heads: head h reads group h // 2
    X, la, B, C = _rand(40, 4, 3, 4, G=2, seed=11)
    Y, fin = oracle.forward(X, la, B, C)
    Yd, fd = dual_form(X[0], la[0], B[0], C[0])
    assert _relmax(Y[0], Yd) <= 1e-12
    assert _relmax(fin[0], fd) <= 1e-12


# ---------------------------------------------------------------- chunked form

@pytest.mark.parametrize("Q", [1, 2, 3, 5, 16, 64])
def test_chunked_form_every_chunk_length(Q):
    T = 64
    X, la, B, C = _rand(T, 3, 4, 6, seed=5)
    Y, fin = oracle.forward(X, la, B, C)
    Yc, fc, _, _ = chunked_form(X[0], la[0], B[0], C[0], Q)
    assert _relmax(Y[0], Yc) <= 1e-12
    assert _relmax(fin[0], fc) <= 1e-12


@pytest.mark.parametrize("Q", [1, 7, 16])
def test_chunked_form_from_an_initial_state(Q):
    """The chunk-pair form with an entering state equals the oracle continued from it
    (outputs, final state, and the state entering every chunk)."""
    T, H, P, N = 40, 2, 3, 5
    X, la, B, C = _rand(T, H, P, N, seed=12)
    h0 = np.random.default_rng(3).standard_normal((1, H, P, N))
    Y, fin, _ = oracle.scan(X, la, B, C, init=h0)
    Yc, fc, starts, _ = chunked_form(X[0], la[0], B[0], C[0], Q, init=h0[0])
    assert _relmax(Y[0], Yc) <= 1e-12
    assert _relmax(fin[0], fc) <= 1e-12
    assert _relmax(starts[0], h0[0]) <= 1e-15
    segs = oracle.chunk_segments(1, T, Q)
    snap = -np.ones(T, np.int32)
    for k, (_, b, e) in enumerate(segs[:-1]):
        snap[e - 1] = k + 1
    _, _, snaps = oracle.scan(X, la, B, C, init=h0, want_y=False, snap_slot=snap, nsnaps=len(segs))
    assert _relmax(snaps[1:], starts[1:]) <= 1e-12


def test_chunked_intermediates_match_oracle_snapshots():
    """Chunk states = oracle restarted per chunk; start states = oracle state at chunk ends."""
    T, Q, H, P, N = 50, 16, 2, 3, 4
    X, la, B, C = _rand(T, H, P, N, seed=9)
    _, _, starts, chunk_states = chunked_form(X[0], la[0], B[0], C[0], Q)
    segs = oracle.chunk_segments(1, T, Q)
    _, fin_restart, _ = oracle.scan(X, la, B, C, segments=segs, want_y=False)
    assert _relmax(fin_restart, chunk_states) <= 1e-12
    snap = -np.ones(T, np.int32)
    for k, (_, b, e) in enumerate(segs[:-1]):
        snap[e - 1] = k + 1
    _, _, snaps = oracle.scan(X, la, B, C, want_y=False, snap_slot=snap, nsnaps=len(segs))
    assert np.all(snaps[0] == 0)
    assert _relmax(snaps[1:], starts[1:]) <= 1e-12


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("a", [0.3, 0.9, 0.999])
def test_scalar_geometric_closed_form(a):
    T = 200
    x = np.ones((1, T, 1, 1))
    la = np.full((1, T, 1), math.log(a))
    one = np.ones((1, T, 1, 1))
    Y, fin = oracle.forward(x, la, one, one)
    t = np.arange(T)
    expect = (1 - a ** (t + 1)) / (1 - a)
    np.testing.assert_allclose(Y[0, :, 0, 0], expect, rtol=1e-13)
    assert abs(fin[0, 0, 0, 0] - expect[-1]) <= 1e-13 * expect[-1]


def test_scalar_no_decay_counts():
    T = 300
    one = np.ones((1, T, 1, 1))
    Y, _ = oracle.forward(one, np.zeros((1, T, 1)), one, one)
    np.testing.assert_array_equal(Y[0, :, 0, 0], np.arange(1, T + 1))


def test_scalar_full_reset_passes_input():
    T = 50
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, T, 1, 1))
    one = np.ones((1, T, 1, 1))
    Y, _ = oracle.forward(x, np.full((1, T, 1), -np.inf), one, one)
    np.testing.assert_array_equal(Y, x)


def test_scalar_recurrence_random_decays():
    T = 100
    rng = np.random.default_rng(4)
    x = rng.standard_normal((1, T, 1, 1))
    la = -rng.uniform(0, 2, (1, T, 1))
    one = np.ones((1, T, 1, 1))
    Y, _ = oracle.forward(x, la, one, one)
    y = 0.0
    for t in range(T):  # y_t = a_t y_{t-1} + x_t (1-SS multiplication)
        y = math.exp(la[0, t, 0]) * y + x[0, t, 0, 0]
        assert abs(Y[0, t, 0, 0] - y) <= 1e-13 * max(1.0, abs(y))


# ---------------------------------------------------------------- linear attention

def test_causal_linear_attention():
    T, H, P, N = 37, 2, 5, 7
    X, la, B, C = _rand(T, H, P, N, seed=21)
    la[:] = 0.0
    Y, _ = oracle.forward(X, la, B, C)
    for h in range(H):
        A = np.tril(C[0, :, 0, :] @ B[0, :, 0, :].T)
        assert _relmax(Y[0, :, h, :], A @ X[0, :, h, :]) <= 1e-12


# ---------------------------------------------------------------- packing / resets

def test_packing_equals_separate_runs_and_resets():
    lengths = [5, 17, 1, 9, 32]
    T = sum(lengths)
    H, P, N = 3, 4, 5
    X, la, B, C = _rand(T, H, P, N, seed=8)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    Y, fin = oracle.forward(X, la, B, C, cu_seqlens=cu)
    for s in range(len(lengths)):
        b, e = cu[s], cu[s + 1]
        Ys, fs = oracle.forward(X[:, b:e], la[:, b:e], B[:, b:e], C[:, b:e])
        np.testing.assert_array_equal(Y[0, b:e], Ys[0])
        np.testing.assert_array_equal(fin[s], fs[0])
    # an unpacked run with a = 0 at every sequence start gives the same result
    la_reset = la.copy()
    la_reset[0, cu[1:-1]] = -np.inf
    Yr, fr = oracle.forward(X, la_reset, B, C)
    np.testing.assert_array_equal(Yr, Y)
    np.testing.assert_array_equal(fr[0], fin[-1])


def test_rows_are_independent():
    X, la, B, C = _rand(20, 2, 3, 4, seed=12, rows=3)
    Y, fin = oracle.forward(X, la, B, C)
    for r in range(3):
        Yr, fr = oracle.forward(X[r:r + 1], la[r:r + 1], B[r:r + 1], C[r:r + 1])
        np.testing.assert_array_equal(Y[r], Yr[0])
        np.testing.assert_array_equal(fin[r], fr[0])


# ---------------------------------------------------------------- continuation / step

def test_continuation_from_state():
    T, T1 = 60, 23
    X, la, B, C = _rand(T, 2, 4, 6, seed=13)
    Y, fin = oracle.forward(X, la, B, C)
    Y1, f1 = oracle.forward(X[:, :T1], la[:, :T1], B[:, :T1], C[:, :T1])
    Y2, f2, _ = oracle.scan(X[:, T1:], la[:, T1:], B[:, T1:], C[:, T1:], init=f1)
    np.testing.assert_array_equal(Y[0, :T1], Y1[0])
    np.testing.assert_array_equal(Y[0, T1:], Y2[0])
    np.testing.assert_array_equal(fin, f2)


def test_step_matches_scan():
    T = 12
    X, la, B, C = _rand(T, 2, 3, 4, seed=14, rows=2)
    Y, fin = oracle.forward(X, la, B, C)
    state = np.zeros((2, 2, 3, 4))
    for t in range(T):
        y, state = oracle.step(state, X[:, t], la[:, t], B[:, t], C[:, t])
        np.testing.assert_array_equal(y, Y[:, t])
    np.testing.assert_array_equal(state, fin)


# ---------------------------------------------------------------- invariants

def test_linearity_in_x():
    X, la, B, C = _rand(33, 2, 3, 4, seed=15)
    X2, _, _, _ = _rand(33, 2, 3, 4, seed=16)
    Y1, f1 = oracle.forward(X, la, B, C)
    Y2, f2 = oracle.forward(X2, la, B, C)
    Y3, f3 = oracle.forward(2.5 * X - 0.75 * X2, la, B, C)
    assert _relmax(Y3, 2.5 * Y1 - 0.75 * Y2) <= 1e-12
    assert _relmax(f3, 2.5 * f1 - 0.75 * f2) <= 1e-12


def test_head_permutation_equivariance():
    H = 5
    X, la, B, C = _rand(29, H, 3, 4, seed=17)
    perm = np.array([3, 0, 4, 1, 2])
    Y, fin = oracle.forward(X, la, B, C)
    Yp, fp = oracle.forward(X[:, :, perm], la[:, :, perm], B, C)
    np.testing.assert_array_equal(Yp, Y[:, :, perm])
    np.testing.assert_array_equal(fp, fin[:, perm])


def test_gauge_b_scaled_c_unscaled():
    X, la, B, C = _rand(31, 2, 3, 4, seed=18)
    alpha = 3.0
    Y, fin = oracle.forward(X, la, B, C)
    Yg, fg = oracle.forward(X, la, alpha * B, C / alpha)
    assert _relmax(Yg, Y) <= 1e-12
    assert _relmax(fg, alpha * fin) <= 1e-12


# ---------------------------------------------------------------- helpers

def test_chunk_segments_cover_sequences():
    cu = [0, 5, 300, 301, 517]
    segs = oracle.chunk_segments(1, 517, 128, cu)
    covered = np.zeros(517, int)
    for (r, b, e) in segs:
        assert r == 0 and 0 < e - b <= 128
        covered[b:e] += 1
        s = np.searchsorted(cu, b, side="right") - 1
        assert e <= cu[s + 1] and (b - cu[s]) % 128 == 0
    assert np.all(covered == 1)
    assert len(segs) == sum(-(-(cu[i + 1] - cu[i]) // 128) for i in range(4))


def test_chunk_cumsum_restarts():
    la = -np.arange(1, 11, dtype=np.float64).reshape(1, 10, 1)
    cs = oracle.chunk_cumsum(la, oracle.chunk_segments(1, 10, 4))
    np.testing.assert_array_equal(cs[0, :, 0], [-1, -3, -6, -10, -5, -11, -18, -26, -9, -19])


# ---------------------------------------------------------------- pin strength

def _pins(mutant):
    """Run the pins against a (possibly mutated) oracle; returns the names that fail."""
    failed = []
    m = mutant

    def fwd(X, la, B, C, **kw):
        return oracle.forward(X, la, B, C, mutant=m, **kw)

    # hand-worked
    for case in _golden_cases():
        x = np.array(case["x"])[None]
        with np.errstate(divide="ignore"):
            la = np.log(np.array(case["a"]))[None]
        Y, fin = fwd(x, la, np.array(case["B"])[None], np.array(case["C"])[None])
        if not (np.allclose(Y[0], case["y"], atol=1e-12) and np.allclose(fin[0], case["final"], atol=1e-12)):
            failed.append("hand:" + case["name"])
    # dual form, including two groups of heads, P == N
    X, la, B, C = _rand(17, 4, 4, 4, G=2, seed=99)
    Y, fin = fwd(X, la, B, C)
    Yd, fd = dual_form(X[0], la[0], B[0], C[0])
    if _relmax(Y[0], Yd) > 1e-12 or _relmax(fin[0], fd) > 1e-12:
        failed.append("dual")
    return failed


@pytest.mark.parametrize("name", sorted(oracle.MUTANTS))
def test_mutants_are_caught(name):
    assert _pins(0) == []
    assert _pins(oracle.MUTANTS[name]), f"mutant {name} passed every pin"


# ---------------------------------------------------------------- Mamba-2 block call

GOLDEN_M2 = os.path.join(os.path.dirname(__file__), "golden", "mamba2_hand_worked.json")


def _m2_cases():
    with open(GOLDEN_M2) as f:
        return json.load(f)["cases"]


def _m2_case_inputs(case):
    x = np.array(case["x"])[None]
    dt = np.array(case["dt"])[None]
    bias = np.log(np.array(case["dt_bias_exp"]))
    A_log = np.log(np.array(case["A_mag"]))
    D = None if case["D"] is None else np.array(case["D"])
    z = None if case["z_ln3"] is None else np.array(case["z_ln3"])[None] * math.log(3.0)
    return x, dt, bias, A_log, D, z, np.array(case["B"])[None], np.array(case["C"])[None]


def _m2_case_expected(case):
    y = np.array(case["y_ln2"]) * math.log(2.0) + np.array(case["y_const"])
    if case["gate_ln3"] is not None:
        y = y * np.array(case["gate_ln3"]) * math.log(3.0)
    return y, np.array(case["final_ln2"]) * math.log(2.0)


def _m2_rand(T, H, P, N, G=1, seed=0, rows=1):
    d = synth.make_mamba2_inputs(rows, T, H, P, N, G, dtype=__import__("torch").float32, seed=seed)
    return {k: (v.double().numpy() if hasattr(v, "double") else v) for k, v in d.items()}


@pytest.mark.parametrize("case", _m2_cases(), ids=lambda c: c["name"])
def test_mamba2_hand_worked(case):
    Y, fin = oracle.mamba2_forward(*_m2_case_inputs(case))
    y, f = _m2_case_expected(case)
    np.testing.assert_allclose(Y[0], y, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(fin[0], f, rtol=1e-14, atol=1e-14)


def test_softplus_and_silu_closed_forms():
    ln2 = math.log(2.0)
    assert oracle.softplus(0.0)[0] == pytest.approx(ln2, rel=1e-15)
    assert oracle.softplus(math.log(3.0))[0] == pytest.approx(2 * ln2, rel=1e-15)
    v = np.linspace(-30, 30, 121)
    np.testing.assert_allclose(oracle.softplus(v) - oracle.softplus(-v), v, atol=1e-13)  # softplus(v) - softplus(-v) = v
    assert oracle.softplus(800.0)[0] == 800.0                      # no overflow at large v
    assert oracle.softplus(-60.0)[0] == pytest.approx(math.exp(-60.0), rel=1e-14)
    np.testing.assert_allclose(oracle.silu([0.0, math.log(3.0), -math.log(3.0)]),
                               [0.0, 0.75 * math.log(3.0), -0.25 * math.log(3.0)], rtol=1e-15, atol=1e-300)
    assert oracle.silu(-800.0)[0] == 0.0 and oracle.silu(800.0)[0] == 800.0


def test_mamba2_discretize_closed_forms():
    # raw + bias = 0 -> dt' = ln 2; A_log = ln 3 -> A = -3, log a = -3 ln 2.
    dtp, la = oracle.mamba2_discretize(np.array([[1.0, 0.0]]), np.array([-1.0, 0.0]),
                                       np.array([0.0, math.log(3.0)]))
    np.testing.assert_allclose(dtp, [[math.log(2.0)] * 2], rtol=1e-15)
    np.testing.assert_allclose(la, [[-math.log(2.0), -3 * math.log(2.0)]], rtol=1e-15)
    dtp, la = oracle.mamba2_discretize(np.zeros((1, 1)), None, np.zeros(1))
    assert dtp[0, 0] == pytest.approx(math.log(2.0)) and la[0, 0] == pytest.approx(-math.log(2.0))


def test_mamba2_no_input_path_is_skip_times_gate():
    # B = 0: the SSM contributes nothing, so y = D x silu(z) exactly, whatever dt and A.
    d = _m2_rand(37, 3, 5, 4, seed=3)
    Y, fin = oracle.mamba2_forward(d["X"], d["dt"], d["dt_bias"], d["A_log"], d["D"], d["z"],
                                   np.zeros_like(d["B"]), d["C"])
    ref = d["D"][None, None, :, None] * d["X"] * d["z"] / (1.0 + np.exp(-d["z"]))
    np.testing.assert_allclose(Y, ref, rtol=1e-14, atol=1e-15)
    assert not fin.any()


def test_mamba2_first_token_closed_form():
    # T = 1 from zero: h = dt' x B^T, y = (dt' (C . B) + D) x silu(z) per head.
    d = _m2_rand(1, 4, 3, 6, G=2, seed=4)
    Y, fin = oracle.mamba2_forward(d["X"], d["dt"], d["dt_bias"], d["A_log"], d["D"], d["z"], d["B"], d["C"])
    dtp = np.log1p(np.exp(d["dt"][0, 0] + d["dt_bias"]))
    for h in range(4):
        g = h // 2
        cb = float(np.dot(d["C"][0, 0, g], d["B"][0, 0, g]))
        x = d["X"][0, 0, h]
        zz = d["z"][0, 0, h]
        want = (dtp[h] * cb + d["D"][h]) * x * zz / (1.0 + np.exp(-zz))
        np.testing.assert_allclose(Y[0, 0, h], want, rtol=1e-13)
        np.testing.assert_allclose(fin[0, h], dtp[h] * np.outer(x, d["B"][0, 0, g]), rtol=1e-13)


def test_mamba2_vanishing_step_size():
    # dt' -> 0 (raw step sizes far below zero): no state update and no decay, y = D x silu(z).
    d = _m2_rand(20, 2, 4, 4, seed=5)
    Y, fin = oracle.mamba2_forward(d["X"], np.full_like(d["dt"], -80.0), d["dt_bias"], d["A_log"], d["D"],
                                   d["z"], d["B"], d["C"])
    ref = d["D"][None, None, :, None] * d["X"] * d["z"] / (1.0 + np.exp(-d["z"]))
    np.testing.assert_allclose(Y, ref, rtol=1e-12, atol=1e-30)
    assert np.abs(fin).max() < 1e-30


def test_mamba2_dual_form():
    # The quadratic dual form on x * dt' with log a = dt' A, plus the skip and the gate.
    d = _m2_rand(19, 4, 3, 5, G=2, seed=6)
    Y, fin = oracle.mamba2_forward(d["X"], d["dt"], d["dt_bias"], d["A_log"], d["D"], d["z"], d["B"], d["C"])
    dtp = np.log1p(np.exp(d["dt"][0] + d["dt_bias"][None]))
    Yd, fd = dual_form(d["X"][0] * dtp[..., None], dtp * -np.exp(d["A_log"])[None], d["B"][0], d["C"][0])
    zz = d["z"][0]
    Yd = (Yd + d["D"][None, :, None] * d["X"][0]) * zz / (1.0 + np.exp(-zz))
    assert _relmax(Y[0], Yd) < 1e-12 and _relmax(fin[0], fd) < 1e-12


def test_mamba2_steps_continue_the_forward_pass():
    # A prompt through the forward pass, then decode steps, equals the longer prompt at once.
    d = _m2_rand(12, 2, 3, 4, seed=7)
    T0 = 8
    Y, fin = oracle.mamba2_forward(d["X"], d["dt"], d["dt_bias"], d["A_log"], d["D"], d["z"], d["B"], d["C"])
    _, st = oracle.mamba2_forward(d["X"][:, :T0], d["dt"][:, :T0], d["dt_bias"], d["A_log"], d["D"],
                                  d["z"][:, :T0], d["B"][:, :T0], d["C"][:, :T0])
    for t in range(T0, 12):
        y, st = oracle.mamba2_step(st, d["X"][:, t], d["dt"][:, t], d["dt_bias"], d["A_log"], d["D"],
                                   d["z"][:, t], d["B"][:, t], d["C"][:, t])
        assert _relmax(y, Y[:, t]) < 1e-13
    assert _relmax(st, fin) < 1e-13


def _m2_pins(mutant):
    failed = []
    for case in _m2_cases():
        Y, fin = oracle.mamba2_forward(*_m2_case_inputs(case), mutant=mutant)
        y, f = _m2_case_expected(case)
        if not (np.allclose(Y[0], y, atol=1e-12) and np.allclose(fin[0], f, atol=1e-12)):
            failed.append("hand:" + case["name"])
    d = _m2_rand(9, 2, 3, 4, seed=8)
    Y, _ = oracle.mamba2_forward(d["X"], d["dt"], d["dt_bias"], d["A_log"], d["D"], d["z"],
                                 np.zeros_like(d["B"]), d["C"], mutant=mutant)
    ref = d["D"][None, None, :, None] * d["X"] * d["z"] / (1.0 + np.exp(-d["z"]))
    if not np.allclose(Y, ref, rtol=1e-12, atol=1e-15):
        failed.append("no_input_path")
    return failed


@pytest.mark.parametrize("name", sorted(oracle.MAMBA2_MUTANTS))
def test_mamba2_mutants_are_caught(name):
    assert _m2_pins(0) == []
    assert _m2_pins(oracle.MAMBA2_MUTANTS[name]), f"mutant {name} passed every pin"


# ---------------------------------------------------------------- backward (reverse mode)

def _bwd_case(T=9, H=2, P=3, N=4, G=1, seed=11, rows=1, lengths=None):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((rows, T, H, P))
    la = -rng.uniform(0.05, 0.8, size=(rows, T, H))
    B = rng.standard_normal((rows, T, G, N))
    C = rng.standard_normal((rows, T, G, N))
    dY = rng.standard_normal((rows, T, H, P))
    S = rows if lengths is None else len(lengths)
    dfin = rng.standard_normal((S, H, P, N))
    init = rng.standard_normal((S, H, P, N))
    cu = None if lengths is None else np.concatenate([[0], np.cumsum(lengths)])
    return X, la, B, C, dY, dfin, init, cu


def _loss(X, la, B, C, dY, dfin, init, cu):
    Y, fin = oracle.forward(X, la, B, C, cu_seqlens=cu, init=init)
    return float(np.sum(dY * Y) + np.sum(dfin * fin))


def _fd_errors(g, case):
    """Central differences of the loss along one random direction per input, against <grad, v>."""
    X, la, B, C, dY, dfin, init, cu = case
    rng = np.random.default_rng(5)
    args = dict(X=X, la=la, B=B, C=C, init=init)
    grads = dict(X=g["dX"], la=g["dlog_a"], B=g["dB"], C=g["dC"], init=g["dinit"])
    out = {}
    eps = 1e-6
    for k in args:
        v = rng.standard_normal(args[k].shape)
        ap, am = dict(args), dict(args)
        ap[k] = args[k] + eps * v
        am[k] = args[k] - eps * v
        fd = (_loss(ap["X"], ap["la"], ap["B"], ap["C"], dY, dfin, ap["init"], cu) -
              _loss(am["X"], am["la"], am["B"], am["C"], dY, dfin, am["init"], cu)) / (2 * eps)
        an = float(np.sum(grads[k] * v))
        out[k] = abs(fd - an) / max(abs(fd), 1e-12)
    return out


@pytest.mark.parametrize("G,H", [(1, 2), (2, 4), (3, 3)])
def test_backward_matches_finite_differences(G, H):
    case = _bwd_case(H=H, G=G, seed=20 + G)
    X, la, B, C, dY, dfin, init, cu = case
    g = oracle.backward(X, la, B, C, dY, dfinal=dfin, init=init)
    for k, e in _fd_errors(g, case).items():
        assert e < 1e-7, (k, e)


def test_backward_packed_finite_differences_and_separate_runs():
    lengths = [3, 1, 6, 2]
    case = _bwd_case(T=sum(lengths), H=2, G=1, seed=31, lengths=lengths)
    X, la, B, C, dY, dfin, init, cu = case
    g = oracle.backward(X, la, B, C, dY, dfinal=dfin, cu_seqlens=cu, init=init)
    for k, e in _fd_errors(g, case).items():
        assert e < 1e-7, (k, e)
    for s in range(len(lengths)):
        b, e = int(cu[s]), int(cu[s + 1])
        gs = oracle.backward(X[:, b:e], la[:, b:e], B[:, b:e], C[:, b:e], dY[:, b:e], dfinal=dfin[s:s + 1],
                             init=init[s:s + 1])
        for k in ("dX", "dlog_a", "dB", "dC"):
            np.testing.assert_allclose(g[k][:, b:e], gs[k], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(g["dinit"][s], gs["dinit"][0], rtol=1e-13, atol=1e-13)


def test_backward_scalar_closed_form():
    # N = P = 1, B = C = 1, a = 1/2: y_t = sum_{j<=t} 2^-(t-j) x_j, so with dY = 1 and no
    # final-state gradient dx_j = sum_{t=j}^{T-1} 2^-(t-j) = 2 (1 - 2^-(T-j)).
    T = 6
    X = np.arange(1.0, T + 1).reshape(1, T, 1, 1)
    la = np.full((1, T, 1), math.log(0.5))
    one = np.ones((1, T, 1, 1))
    g = oracle.backward(X, la, one, one, np.ones_like(X))
    want = [2 * (1 - 2.0 ** -(T - j)) for j in range(T)]
    np.testing.assert_allclose(g["dX"][0, :, 0, 0], want, rtol=1e-14)
    np.testing.assert_allclose(g["dB"][0, :, 0, 0], np.array(want) * X[0, :, 0, 0], rtol=1e-14)


def test_backward_log_decay_identity():
    # d/dcs_k of <dY, M X> is dY_k . y_k - x_k . dx_k (the two exponents of every
    # L_ij = exp(cs_i - cs_j)), plus <dfinal, h_last> at the last token, and
    # log a_t enters every cs_k with k >= t: d log a = reverse cumsum of that.
    case = _bwd_case(T=12, H=3, G=1, seed=41)
    X, la, B, C, dY, dfin, init, cu = case
    g = oracle.backward(X, la, B, C, dY, dfinal=dfin, init=init)
    Y, fin = oracle.forward(X, la, B, C, init=init)
    gk = np.sum(dY * Y, axis=-1) - np.sum(X * g["dX"], axis=-1)
    gk[:, -1] += np.sum(dfin * fin, axis=(-2, -1))
    want = np.flip(np.cumsum(np.flip(gk, axis=1), axis=1), axis=1)
    np.testing.assert_allclose(g["dlog_a"], want, rtol=1e-11, atol=1e-11)


def _bwd_pins(mutant):
    failed = []
    case = _bwd_case(T=8, H=2, G=1, seed=51)
    X, la, B, C, dY, dfin, init, cu = case
    g = oracle.backward(X, la, B, C, dY, dfinal=dfin, init=init, mutant=mutant)
    errs = _fd_errors(g, case)
    failed += [k for k, e in errs.items() if e > 1e-7]
    return failed


@pytest.mark.parametrize("name", sorted(oracle.BACKWARD_MUTANTS))
def test_backward_mutants_are_caught(name):
    assert _bwd_pins(0) == []
    assert _bwd_pins(oracle.BACKWARD_MUTANTS[name]), f"mutant {name} passed every pin"


# ---------------------------------------------------------------------------
# Backward of the Mamba-2 call: central differences of the pinned
# mamba2_forward along one random direction per input.
# ---------------------------------------------------------------------------
def _m2_case(T=9, H=2, P=3, N=4, G=1, seed=61, lengths=None, skip=True, gate=True, bias=True):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((1, T, H, P))
    dt = rng.uniform(-3.0, 1.0, size=(1, T, H))
    dtb = rng.uniform(-1.0, 0.5, size=H) if bias else None
    A_log = rng.uniform(-1.0, 1.5, size=H)
    D = rng.standard_normal(H) if skip else None
    z = rng.standard_normal((1, T, H, P)) * 2.0 if gate else None
    B = rng.standard_normal((1, T, G, N))
    C = rng.standard_normal((1, T, G, N))
    dY = rng.standard_normal((1, T, H, P))
    S = 1 if lengths is None else len(lengths)
    dfin = rng.standard_normal((S, H, P, N))
    init = rng.standard_normal((S, H, P, N))
    cu = None if lengths is None else np.concatenate([[0], np.cumsum(lengths)])
    return dict(X=X, dt=dt, dt_bias=dtb, A_log=A_log, D=D, z=z, B=B, C=C, init=init), dY, dfin, cu


def _m2_fd_errors(g, case):
    args, dY, dfin, cu = case

    def loss(a):
        Y, fin = oracle.mamba2_forward(a["X"], a["dt"], a["dt_bias"], a["A_log"], a["D"], a["z"], a["B"], a["C"],
                                       cu_seqlens=cu, init=a["init"])
        return float(np.sum(dY * Y) + np.sum(dfin * fin))

    names = dict(X="dX", dt="ddt", dt_bias="ddt_bias", A_log="dA_log", D="dD", z="dz", B="dB", C="dC",
                 init="dinit")
    rng = np.random.default_rng(7)
    out = {}
    eps = 1e-6
    for k, gk in names.items():
        if args[k] is None:
            continue
        v = rng.standard_normal(np.shape(args[k]))
        ap, am = dict(args), dict(args)
        ap[k] = args[k] + eps * v
        am[k] = args[k] - eps * v
        fd = (loss(ap) - loss(am)) / (2 * eps)
        an = float(np.sum(g[gk] * v))
        out[k] = abs(fd - an) / max(abs(fd), 1e-12)
    return out


@pytest.mark.parametrize("skip,gate,bias", [(True, True, True), (False, True, False), (True, False, True),
                                            (False, False, False)])
def test_mamba2_backward_matches_finite_differences(skip, gate, bias):
    case = _m2_case(skip=skip, gate=gate, bias=bias, seed=62 + 2 * skip + gate)
    args, dY, dfin, cu = case
    g = oracle.mamba2_backward(**args, dY=dY, dfinal=dfin, cu_seqlens=cu)
    errs = _m2_fd_errors(g, case)
    assert errs and all(e < 1e-6 for e in errs.values()), errs
    assert (g["dD"] is None) == (not skip) and (g["dz"] is None) == (not gate)


def test_mamba2_backward_packed_grouped():
    case = _m2_case(T=11, H=4, G=2, lengths=[4, 1, 6], seed=70)
    args, dY, dfin, cu = case
    g = oracle.mamba2_backward(**args, dY=dY, dfinal=dfin, cu_seqlens=cu)
    errs = _m2_fd_errors(g, case)
    assert all(e < 1e-6 for e in errs.values()), errs


def test_mamba2_backward_without_gate_and_skip_is_the_chain_rule_of_backward():
    # no gate, no skip, no bias: dX = dx~ dt', and the recurrence gradients are backward()'s
    case = _m2_case(T=7, seed=71, skip=False, gate=False, bias=False)
    args, dY, dfin, cu = case
    g = oracle.mamba2_backward(**args, dY=dY, dfinal=dfin)
    dtp, la = oracle.mamba2_discretize(args["dt"], None, args["A_log"])
    gs = oracle.backward(args["X"] * dtp[..., None], la, args["B"], args["C"], dY, dfinal=dfin, init=args["init"])
    np.testing.assert_allclose(g["dX"], gs["dX"] * dtp[..., None], rtol=1e-13)
    np.testing.assert_allclose(g["dB"], gs["dB"], rtol=1e-13)


@pytest.mark.parametrize("name", sorted(oracle.MAMBA2_BACKWARD_MUTANTS))
def test_mamba2_backward_mutants_are_caught(name):
    case = _m2_case(seed=73)
    args, dY, dfin, cu = case
    ok = oracle.mamba2_backward(**args, dY=dY, dfinal=dfin)
    assert all(e < 1e-6 for e in _m2_fd_errors(ok, case).values())
    bad = oracle.mamba2_backward(**args, dY=dY, dfinal=dfin, mutant=oracle.MAMBA2_BACKWARD_MUTANTS[name])
    assert any(e > 1e-4 for e in _m2_fd_errors(bad, case).values()), f"mutant {name} passed"
