"""GPU: the state chain as one cooperative launch against two launches.

ssd_set_state_chain(1) runs chunk_state and state_passing as one cooperative
launch with a grid-wide barrier between them whenever the grid can be
resident; mode 0 (the default) always runs the two launches. Both run the same block
computation and the same recurrence, so every output must be bitwise equal.
The parity of the outputs themselves against the oracle is covered by the
other GPU tests, which run in the default mode; the module's last test runs a
shape grid against the oracle in mode 1. Every test first asserts, through
ssd_state_chain_cooperative, that mode 1 does run the cooperative kernel for
its shape, so the comparisons are never two-launch against two-launch.
"""
import sys

import pytest
import torch

import ssd_chunked_scan_fwd_amd as ssd
from ssd_chunked_scan_fwd_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ssd.lib()


@pytest.fixture(autouse=True)
def _restore_mode():
    prev = ssd.set_state_chain(0)
    yield
    ssd.set_state_chain(prev)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def both_modes(fn):
    ssd.set_state_chain(1)
    a = fn()
    torch.cuda.synchronize()
    ssd.set_state_chain(0)
    b = fn()
    torch.cuda.synchronize()
    ssd.set_state_chain(0)
    return a, b


def assert_cooperative(X, B, Q, gs, cu=None):
    sh = ssd.make_shape(X, B, cu)
    assert ssd.state_chain_cooperative(sh, Q, gs), "mode 1 would not launch the cooperative kernel here"


def assert_bitwise(a, b, what):
    assert a.shape == b.shape, what
    assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), what


@pytest.mark.parametrize("case", [
    # (batch, T, H, P, N, Q, gs, lengths)
    (1, 16384, 32, 64, 128, 128, 0, None),        # the headline workload (512 workgroups: all resident)
    (2, 3000, 8, 64, 64, 128, 4, None),
    (1, 5000, 6, 32, 128, 128, 2, None),
    (1, 4321, 4, 128, 128, 64, 8, None),
    (1, 0, 4, 64, 128, 128, 2, [1, 200, 1100, 65, 3, 900, 1, 90]),   # packed
], ids=["headline", "b2-N64", "P32", "P128-N128", "packed"])
def test_forward_chain_bitwise(case):
    b, T, H, P, N, Q, gs, lengths = case
    if lengths:
        T = sum(lengths)
    d = synth.make_forward_inputs(b, T, H, P, N, 1, dtype=torch.bfloat16, seed=4100 + T, lengths=lengths)
    X, la, B, C = (d[k].cuda() for k in ("X", "log_a", "B", "C"))
    cu = d["cu_seqlens"].cuda() if d.get("cu_seqlens") is not None else None
    say(f"[chain] forward X{tuple(X.shape)} N={N} gs={gs} packed={cu is not None}")
    assert_cooperative(X, B, Q, gs, cu)
    (Y1, f1), (Y0, f0) = both_modes(lambda: ssd.fwd(X, la, B, C, cu_seqlens=cu, chunk=Q, state_block=gs))
    assert_bitwise(Y1, Y0, "Y")
    assert_bitwise(f1, f0, "final state")


def test_mamba2_chain_bitwise():
    m = synth.make_mamba2_inputs(1, 4096, 8, 64, 128, 1, torch.bfloat16, seed=4200)
    t = {k: v.cuda() for k, v in m.items() if isinstance(v, torch.Tensor)}
    say("[chain] mamba2 call T=4096 H=8")
    assert_cooperative(t["X"], t["B"], 128, 0)
    (Y1, f1), (Y0, f0) = both_modes(lambda: ssd.fwd_mamba2(t["X"], t["dt"], t["A_log"], t["B"], t["C"],
                                                           dt_bias=t["dt_bias"], D=t["D"], z=t["z"], chunk=128))
    assert_bitwise(Y1, Y0, "Y")
    assert_bitwise(f1, f0, "final state")


def test_backward_chain_bitwise():
    b, T, H, P, N = 1, 4096, 8, 64, 128
    d = synth.make_forward_inputs(b, T, H, P, N, 1, dtype=torch.bfloat16, seed=4300)
    ct = synth.make_cotangents(b, T, H, P, N, b, dtype=torch.bfloat16, seed=4301)
    X, la, B, C, dY = (t.cuda() for t in (d["X"], d["log_a"], d["B"], d["C"], ct["dY"]))
    dfin = ct["dfinal"].cuda() * 0.01
    say("[chain] backward T=4096 H=8")
    assert_cooperative(X, B, 128, 8)
    g1, g0 = both_modes(lambda: ssd.bwd(X, la, B, C, dY, chunk=128, state_block=8, dfinal_state=dfin,
                                        want_dinit=True))
    for k in ("dX", "dlog_a", "dB", "dC", "dinit"):
        assert_bitwise(g1[k], g0[k], k)


@pytest.mark.parametrize("case", [(1, 700, 4, 64, 128, 64, 4), (2, 1500, 6, 32, 128, 128, 2)])
def test_chain_against_oracle(case):
    from oracle import oracle
    from parity import assert_close, to_f64
    b, T, H, P, N, Q, gs = case
    d = synth.make_forward_inputs(b, T, H, P, N, 1, dtype=torch.bfloat16, seed=4400 + T)
    X, la, B, C = (d[k].cuda() for k in ("X", "log_a", "B", "C"))
    assert_cooperative(X, B, Q, gs)
    ssd.set_state_chain(1)
    Y, fin = ssd.fwd(X, la, B, C, chunk=Q, state_block=gs)
    torch.cuda.synchronize()
    ssd.set_state_chain(0)
    Yr, fr = oracle.forward(to_f64(d["X"]), to_f64(d["log_a"]), to_f64(d["B"]), to_f64(d["C"]))
    assert_close(to_f64(Y), Yr, "bf16", "chain Y")
    assert_close(to_f64(fin), fr, "bf16", "chain final")
