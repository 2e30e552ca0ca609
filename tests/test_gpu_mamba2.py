"""GPU parity of the Mamba-2 block's SSD call (ssd_fwd_mamba2, ssd_step_mamba2)
against the fp64 oracle (oracle.mamba2_forward / mamba2_step).

The HIP path discretises inside the cumsum stage (dt' = softplus(dt + dt_bias),
log a = dt' * A, A = -exp(A_log)), carries dt' in the key-side weights instead
of scaling x, adds the skip D x on the diagonal of the diagonal key block and
gates the output with silu(z) before its one rounding. The oracle takes the
plain definition: x * dt' into the recurrence, then + D x, then * silu(z).
"""
import sys

import numpy as np
import pytest
import torch

import ssd_chunked_scan_fwd_amd as ssd
from ssd_chunked_scan_fwd_amd import synth
from oracle import oracle
from parity import assert_close, assert_close_gated, dtype_name, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ssd.lib()


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _opt(d, key, use):
    return d[key] if use else None


def gpu_m2(d, Q, gs=0, gate=True, skip=True, bias=True, init=None):
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    Y, fin = ssd.fwd_mamba2(dev["X"], dev["dt"], dev["A_log"], dev["B"], dev["C"],
                            dt_bias=_opt(dev, "dt_bias", bias), D=_opt(dev, "D", skip), z=_opt(dev, "z", gate),
                            cu_seqlens=dev.get("cu_seqlens"), chunk=Q, state_block=gs,
                            initial_state=None if init is None else init.cuda())
    torch.cuda.synchronize()
    return Y, fin


def oracle_m2(d, gate=True, skip=True, bias=True, init=None):
    cu = d.get("cu_seqlens")
    return oracle.mamba2_forward(to_f64(d["X"]), to_f64(d["dt"]), to_f64(d["dt_bias"]) if bias else None,
                                 to_f64(d["A_log"]), to_f64(d["D"]) if skip else None,
                                 to_f64(d["z"]) if gate else None, to_f64(d["B"]), to_f64(d["C"]),
                                 cu_seqlens=None if cu is None else cu.numpy(),
                                 init=None if init is None else init.double().numpy())


def check_y(Y, Yr, d, what, gate=True, **kw):
    """Y against the oracle: the gated bar when the output is gated, else the plain one."""
    dt = dtype_name(d["X"])
    if not gate:
        return assert_close(to_f64(Y), Yr, dt, what)
    Yu, _ = oracle_m2(d, gate=False, **kw)
    return assert_close_gated(to_f64(Y), Yr, Yu, oracle.silu(to_f64(d["z"])), dt, what)


def check_m2(d, Q, what, gs=0, gate=True, **kw):
    say(f"[mamba2] {what}: X{tuple(d['X'].shape)} {d['X'].dtype} N={d['B'].shape[-1]} Q={Q} gs={gs} "
        f"gate={gate} {kw}")
    Y, fin = gpu_m2(d, Q, gs, gate=gate, **kw)
    Yr, fr = oracle_m2(d, gate=gate, **kw)
    ey = check_y(Y, Yr, d, what + " Y", gate=gate, **kw)
    ef = assert_close(to_f64(fin), fr, dtype_name(d["X"]), what + " final")
    say(f"[mamba2] {what}: Y {ey} final {ef}")
    return Y, fin


# Both bf16 chunk_scan kernels (head pairs: even heads per group, P <= 64,
# N <= 128, Q <= 128; single heads otherwise) and the fp32 path.
CASES = [
    # (batch, T, H, P, N, G, dtype, Q)
    (1, 300, 4, 64, 128, 1, torch.bfloat16, 128),   # head pairs, ragged tail
    (2, 200, 3, 64, 64, 1, torch.bfloat16, 64),     # odd heads per group: single-head kernel
    (1, 129, 4, 16, 32, 2, torch.bfloat16, 32),     # P = 16 (8-byte output pieces), two groups
    (1, 333, 2, 128, 128, 1, torch.bfloat16, 128),  # P = 128
    (1, 300, 2, 64, 256, 1, torch.bfloat16, 128),   # N = 256
    (1, 600, 2, 64, 128, 1, torch.bfloat16, 256),   # Q = 256 (two tiles per wave)
    (1, 1, 2, 64, 64, 1, torch.bfloat16, 64),       # a single token
    (1, 77, 3, 16, 16, 1, torch.float32, 16),       # fp32
    (2, 300, 2, 128, 256, 2, torch.float32, 256),   # fp32, large tiles
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}-T{}-H{}-P{}-N{}-G{}-{}-Q{}".format(
    *c[:6], "bf16" if c[6] == torch.bfloat16 else "fp32", c[7]))
def test_mamba2_shapes(case):
    b, T, H, P, N, G, dt, Q = case
    d = synth.make_mamba2_inputs(b, T, H, P, N, G, dtype=dt, seed=2000 + T + N)
    check_m2(d, Q, f"shape {case}")


@pytest.mark.parametrize("gate,skip,bias", [(False, False, False), (True, False, True), (False, True, True),
                                            (True, True, False)])
@pytest.mark.parametrize("dt,H", [(torch.bfloat16, 4), (torch.bfloat16, 3), (torch.float32, 2)])
def test_mamba2_optional_parts(gate, skip, bias, dt, H):
    d = synth.make_mamba2_inputs(1, 260, H, 32 if dt == torch.bfloat16 else 16, 64 if dt == torch.bfloat16 else 16,
                                 1, dtype=dt, seed=2100 + H)
    check_m2(d, 64, f"gate={gate} skip={skip} bias={bias}", gate=gate, skip=skip, bias=bias)


def test_mamba2_headline_size():
    """The headline shape (T = 16384, H = 32, P = 64, N = 128, Q = 128) with Mamba-2 inputs, in full."""
    w = synth.WORKLOADS[synth.HEADLINE]
    d = synth.make_mamba2_inputs(w.batch, w.T, w.H, w.P, w.N, w.G, dtype=w.torch_dtype, seed=w.seed)
    check_m2(d, w.Q, "headline shape")
    check_m2(d, w.Q, "headline shape, one chunk per state block", gs=1)


@pytest.mark.parametrize("gs", [1, 4])
def test_mamba2_packed_with_initial_states(gs):
    d = synth.make_mamba2_inputs(1, 1500, 4, 64, 128, 1, dtype=torch.bfloat16, seed=2200 + gs, varlen=(1, 600))
    S = d["cu_seqlens"].numel() - 1
    p = synth.make_mamba2_inputs(S, 150, 4, 64, 128, 1, dtype=torch.float32, seed=2201)
    _, h0 = oracle.mamba2_forward(to_f64(p["X"]), to_f64(p["dt"]), to_f64(d["dt_bias"]), to_f64(d["A_log"]),
                                  None, None, to_f64(p["B"]), to_f64(p["C"]))
    check_m2(d, 128, f"packed S={S}", gs=gs, init=torch.from_numpy(h0).float())


def test_mamba2_extreme_step_sizes_and_gates():
    """dt' from ~0 (raw -100: no update, no decay; the key exponent is +inf) to
    ~30 (decay below fp32 range within a token), and gates at +-30."""
    d = synth.make_mamba2_inputs(1, 256, 4, 64, 64, 1, dtype=torch.bfloat16, seed=2300)
    rng = np.random.default_rng(2301)
    pick = rng.integers(0, 4, size=d["dt"].shape)
    d["dt"] = torch.from_numpy(np.choose(pick, [d["dt"].numpy(), np.full(d["dt"].shape, -100.0, np.float32),
                                                np.full(d["dt"].shape, 30.0, np.float32),
                                                np.full(d["dt"].shape, -8.0, np.float32)]).astype(np.float32))
    z = d["z"].float().numpy()
    z[..., :4] = 30.0
    z[..., 4:8] = -30.0
    d["z"] = torch.from_numpy(z).to(torch.bfloat16)
    check_m2(d, 64, "extreme dt and z")


def test_mamba2_no_input_path():
    """B = 0: Y = D x silu(z) exactly as the kernels form it (one rounding)."""
    d = synth.make_mamba2_inputs(1, 200, 4, 64, 64, 1, dtype=torch.bfloat16, seed=2400)
    d["B"] = torch.zeros_like(d["B"])
    Y, fin = check_m2(d, 64, "B = 0")
    assert not fin.any()


def test_mamba2_deterministic_and_plain_call_unchanged():
    """Two identical calls agree bitwise; a Mamba-2 call between two plain calls
    leaves the plain call's result unchanged (separate workspace arrays)."""
    d = synth.make_mamba2_inputs(1, 700, 4, 64, 128, 1, dtype=torch.bfloat16, seed=2500)
    p = synth.make_forward_inputs(1, 700, 4, 64, 128, 1, dtype=torch.bfloat16, seed=2501)
    pc = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
    sh = ssd.make_shape(pc["X"], pc["B"])
    ws = ssd.Workspace(sh, 128, pc["X"].device)
    Yp1, _ = ssd.fwd(pc["X"], pc["log_a"], pc["B"], pc["C"], chunk=128, workspace=ws)
    Yp1 = Yp1.clone()
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    Y1, f1 = ssd.fwd_mamba2(dev["X"], dev["dt"], dev["A_log"], dev["B"], dev["C"], dt_bias=dev["dt_bias"],
                            D=dev["D"], z=dev["z"], chunk=128, workspace=ws)
    Y1, f1 = Y1.clone(), f1.clone()
    Y2, f2 = ssd.fwd_mamba2(dev["X"], dev["dt"], dev["A_log"], dev["B"], dev["C"], dt_bias=dev["dt_bias"],
                            D=dev["D"], z=dev["z"], chunk=128, workspace=ws)
    Yp2, _ = ssd.fwd(pc["X"], pc["log_a"], pc["B"], pc["C"], chunk=128, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2) and torch.equal(f1, f2)
    assert torch.equal(Yp1, Yp2)


# ------------------------------------------------------------------ decode step

@pytest.mark.parametrize("dt,N,gate", [(torch.bfloat16, 128, True), (torch.float32, 16, True),
                                       (torch.bfloat16, 64, False)])
def test_mamba2_step_sequence(dt, N, gate):
    b, steps, H, P = 3, 40, 4, 64 if N != 16 else 16
    d = synth.make_mamba2_decode_inputs(b, steps, H, P, N, 2, dtype=dt, seed=2600 + N)
    say(f"[mamba2] step b={b} steps={steps} H={H} P={P} N={N} {dt} gate={gate}")
    dev = {k: v.cuda() for k, v in d.items()}
    state = torch.zeros(b, H, P, N, dtype=torch.float32, device="cuda")
    ys = []
    for t in range(steps):
        ys.append(ssd.step_mamba2(state, dev["x"][t], dev["dt"][t], dev["A_log"], dev["B"][t], dev["C"][t],
                                  dt_bias=dev["dt_bias"], D=dev["D"], z=dev["z"][t] if gate else None))
    torch.cuda.synchronize()
    Yg = torch.stack(ys, 1)
    tr = lambda a: to_f64(a).swapaxes(0, 1)
    Yr, fr = oracle.mamba2_forward(tr(d["x"]), tr(d["dt"]), to_f64(d["dt_bias"]), to_f64(d["A_log"]),
                                   to_f64(d["D"]), tr(d["z"]) if gate else None, tr(d["B"]), tr(d["C"]))
    dts = dtype_name(d["x"])
    if gate:
        Yu, _ = oracle.mamba2_forward(tr(d["x"]), tr(d["dt"]), to_f64(d["dt_bias"]), to_f64(d["A_log"]),
                                      to_f64(d["D"]), None, tr(d["B"]), tr(d["C"]))
        assert_close_gated(to_f64(Yg), Yr, Yu, oracle.silu(tr(d["z"])), dts, "mamba2 step y")
    else:
        assert_close(to_f64(Yg), Yr, dts, "mamba2 step y")
    assert_close(to_f64(state), fr, dts, "mamba2 step state")


def test_mamba2_prefill_then_decode_handoff():
    """ssd_fwd_mamba2 over [0, T1), then ssd_step_mamba2 over [T1, T), equals the oracle over [0, T)."""
    b, T, T1, H, P, N = 2, 300, 229, 4, 64, 128
    d = synth.make_mamba2_inputs(b, T, H, P, N, 1, dtype=torch.bfloat16, seed=2700)
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    cut = lambda k: dev[k][:, :T1].contiguous()
    _, state = ssd.fwd_mamba2(cut("X"), cut("dt"), dev["A_log"], cut("B"), cut("C"), dt_bias=dev["dt_bias"],
                              D=dev["D"], z=cut("z"), chunk=128)
    ys = []
    for t in range(T1, T):
        at = lambda k: dev[k][:, t].contiguous()
        ys.append(ssd.step_mamba2(state, at("X"), at("dt"), dev["A_log"], at("B"), at("C"), dt_bias=dev["dt_bias"],
                                  D=dev["D"], z=at("z")))
    torch.cuda.synchronize()
    Yr, fr = oracle_m2(d)
    Yu, _ = oracle_m2(d, gate=False)
    assert_close_gated(to_f64(torch.stack(ys, 1)), Yr[:, T1:], Yu[:, T1:], oracle.silu(to_f64(d["z"][:, T1:])),
                       "bf16", "mamba2 handoff y")
    assert_close(to_f64(state), fr, "bf16", "mamba2 handoff final")
