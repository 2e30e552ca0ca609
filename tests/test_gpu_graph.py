"""GPU: calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The library allocates nothing, never synchronises and issues no memset: each
entry point only enqueues kernels on the caller's stream, so a call captured
in a graph must reproduce the eager call bitwise on every replay. Each test
captures one call (the forward pass, the Mamba-2 call, the backward pass, a run
of decode steps) with its buffers fixed, then replays it three times with eager
work and synchronisations in between (other calls on other buffers, the
outputs overwritten) and checks every replay against the eager result.
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


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def assert_bitwise(a, b, what):
    assert a.shape == b.shape and a.dtype == b.dtype, what
    bits = {torch.bfloat16: torch.int16, torch.float32: torch.int32}[a.dtype]
    assert torch.equal(a.view(bits), b.view(bits)), what


def capture(fn):
    """fn() once on a side stream (warm-up), then captured into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="relaxed"):
        out = fn()
    torch.cuda.synchronize()
    return g, out


def replay_and_check(g, outs, refs, between):
    for i in range(3):
        between(i)
        for o in outs:
            o.fill_(float("nan") if o.dtype.is_floating_point else 0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (o, r) in enumerate(zip(outs, refs)):
            assert_bitwise(o, r, f"replay {i}, output {k}")


# (T, H, N, state block, chunk_scan kernel): the whole-chunk two-head kernel;
# the half-chunk kernel with the head-pair chunk_state (768 units); the wide
# half-chunk kernel at N = 256.
@pytest.mark.parametrize("T,H,N,gs,kind", [(3000, 8, 128, 0, "pair"), (3000, 64, 128, 1, "half_pair"),
                                           (1000, 4, 256, 0, "half_pair_wide")])
def test_forward_graph(T, H, N, gs, kind):
    d = synth.make_forward_inputs(1, T, H, 64, N, 1, dtype=torch.bfloat16, seed=6100)
    X, la, B, C = (d[k].cuda() for k in ("X", "log_a", "B", "C"))
    shape = ssd.make_shape(X, B, None)
    assert ssd.chunk_scan_kernel(shape, 128, gs) == kind
    ws = ssd.Workspace(shape, 128, X.device, gs)
    Y0, f0 = ssd.fwd(X, la, B, C, chunk=128, workspace=ws)
    torch.cuda.synchronize()
    Y0, f0 = Y0.clone(), f0.clone()
    Yg, fg = torch.empty_like(Y0), torch.empty_like(f0)
    g, _ = capture(lambda: ssd.fwd(X, la, B, C, chunk=128, Y=Yg, final_state=fg, workspace=ws))
    e = synth.make_forward_inputs(1, T, H, 64, N, 1, dtype=torch.bfloat16, seed=6101)
    Xe, lae, Be, Ce = (e[k].cuda() for k in ("X", "log_a", "B", "C"))
    say(f"[graph] forward T={T} H={H} N={N} ({kind})")
    replay_and_check(g, [Yg, fg], [Y0, f0], lambda i: ssd.fwd(Xe, lae, Be, Ce, chunk=128, workspace=ws))


def test_mamba2_graph():
    m = synth.make_mamba2_inputs(1, 2000, 8, 64, 128, 1, torch.bfloat16, seed=6200)
    t = {k: v.cuda() for k, v in m.items() if isinstance(v, torch.Tensor)}
    args = dict(dt_bias=t["dt_bias"], D=t["D"], z=t["z"], chunk=128)
    Y0, f0 = ssd.fwd_mamba2(t["X"], t["dt"], t["A_log"], t["B"], t["C"], **args)
    torch.cuda.synchronize()
    Y0, f0 = Y0.clone(), f0.clone()
    Yg, fg = torch.empty_like(Y0), torch.empty_like(f0)
    shape = ssd.make_shape(t["X"], t["B"], None)
    ws = ssd.Workspace(shape, 128, Y0.device)
    g, _ = capture(lambda: ssd.fwd_mamba2(t["X"], t["dt"], t["A_log"], t["B"], t["C"], Y=Yg, final_state=fg,
                                          workspace=ws, **args))
    say("[graph] mamba2 call T=2000 H=8")
    replay_and_check(g, [Yg, fg], [Y0, f0],
                     lambda i: ssd.fwd_mamba2(t["X"], t["dt"] * (i + 2), t["A_log"], t["B"], t["C"], **args))


def test_backward_graph():
    d = synth.make_forward_inputs(1, 2500, 8, 64, 128, 1, dtype=torch.bfloat16, seed=6300)
    ct = synth.make_cotangents(1, 2500, 8, 64, 128, 1, dtype=torch.bfloat16, seed=6301)
    X, la, B, C, dY = (v.cuda() for v in (d["X"], d["log_a"], d["B"], d["C"], ct["dY"]))
    dfin = ct["dfinal"].cuda() * 0.01
    shape = ssd.make_shape(X, B, None)
    wsb = torch.empty(ssd.bwd_workspace_bytes(shape, 128, 0), dtype=torch.uint8, device=X.device)
    r0 = ssd.bwd(X, la, B, C, dY, chunk=128, dfinal_state=dfin, want_dinit=True, workspace=wsb)
    torch.cuda.synchronize()
    keys = ("dX", "dlog_a", "dB", "dC", "dinit")
    refs = [r0[k].clone() for k in keys]
    g, rg = capture(lambda: ssd.bwd(X, la, B, C, dY, chunk=128, dfinal_state=dfin, want_dinit=True, workspace=wsb))
    say("[graph] backward T=2500 H=8")
    replay_and_check(g, [rg[k] for k in keys], refs,
                     lambda i: ssd.bwd(X, la, B, C, dY * (i + 2), chunk=128, dfinal_state=dfin, want_dinit=True))


def test_decode_graph():
    b, H, P, N, steps = 16, 8, 64, 128, 16
    dd = synth.make_decode_inputs(b, steps, H, P, N, 1, torch.bfloat16, seed=6400)
    xs, las, Bs, Cs = (dd[k].cuda() for k in ("x", "log_a", "B", "C"))
    state0 = torch.randn(b, H, P, N, device="cuda")
    ys = torch.empty(steps, b, H, P, dtype=torch.bfloat16, device="cuda")
    state = state0.clone()
    for t in range(steps):
        ssd.step(state, xs[t], las[t], Bs[t], Cs[t], y=ys[t])
    torch.cuda.synchronize()
    refs = [state.clone(), ys.clone()]
    sg = state0.clone()
    yg = torch.empty_like(ys)

    def run():
        for t in range(steps):
            ssd.step(sg, xs[t], las[t], Bs[t], Cs[t], y=yg[t])

    g, _ = capture(run)
    other = torch.zeros_like(state0)

    def between(i):
        ssd.step(other, xs[i], las[i], Bs[i], Cs[i])
        sg.copy_(state0)   # each replay runs the steps from the same state

    say(f"[graph] decode b={b} H={H}: {steps} steps per replay")
    for i in range(3):
        between(i)
        yg.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_bitwise(sg, refs[0], f"replay {i}, state")
        assert_bitwise(yg, refs[1], f"replay {i}, y")
