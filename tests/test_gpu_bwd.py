"""GPU parity of the backward pass (ssd_bwd) against the fp64 oracle's
reverse mode through the recurrence (oracle.backward).

The HIP path assembles the gradients from forward passes: dX as the same
chunked algorithm over time-reversed sequences with B and C exchanged, dB and
dC with the roles of x, B, C and dY exchanged (summed over the heads of each
group), and d log a chunk by chunk from the pairs of tokens that straddle each
position, using the chunk-entering states of a forward run and the adjoints
of the reversed run.
"""
import sys

import numpy as np
import pytest
import torch

import ssd_chunked_scan_fwd_amd as ssd
from ssd_chunked_scan_fwd_amd import synth
from oracle import oracle
from parity import assert_close, dtype_name, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ssd.lib()


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _init_states(n, H, P, N, seed, T0=120):
    d = synth.make_forward_inputs(n, T0, H, P, N, 1, dtype=torch.float32, seed=seed)
    _, fin = oracle.forward(to_f64(d["X"]), to_f64(d["log_a"]), to_f64(d["B"]), to_f64(d["C"]))
    return torch.from_numpy(fin).float()


def _dfinal_states(n, H, P, N, seed, T1=120):
    """Final-state gradients at the scale a continuation produces: the oracle's
    initial-state gradient of a seeded piece of T1 more tokens (the chunked
    training use, where the next piece hands its gradient back)."""
    d = synth.make_forward_inputs(n, T1, H, P, N, 1, dtype=torch.float32, seed=seed)
    ct = synth.make_cotangents(n, T1, H, P, N, n, dtype=torch.float32, seed=seed + 1)
    g = oracle.backward(to_f64(d["X"]), to_f64(d["log_a"]), to_f64(d["B"]), to_f64(d["C"]), to_f64(ct["dY"]),
                        init=np.zeros((n, H, P, N)))
    return torch.from_numpy(g["dinit"]).float()


def check_bwd(d, Q, what, gs=0, with_final=True, with_init=True, seed=0):
    X, la, B, C = (d[k] for k in ("X", "log_a", "B", "C"))
    cu = d.get("cu_seqlens")
    b, T, H, P = X.shape
    N = B.shape[-1]
    nseq = b if cu is None else cu.numel() - 1
    ct = synth.make_cotangents(b, T, H, P, N, nseq, dtype=X.dtype, seed=seed)
    if with_final:
        ct["dfinal"] = _dfinal_states(nseq, H, P, N, seed + 2)
    init = _init_states(nseq, H, P, N, seed + 1) if with_init else None
    say(f"[bwd] {what}: X{tuple(X.shape)} {X.dtype} N={N} G={B.shape[2]} Q={Q} gs={gs} final={with_final} "
        f"init={with_init}")
    dev = lambda t: None if t is None else t.cuda()
    Xg, lag, Bg, Cg, cug = dev(X), dev(la), dev(B), dev(C), dev(cu)
    g = ssd.bwd(Xg, lag, Bg, Cg, dev(ct["dY"]), cu_seqlens=cug, chunk=Q, state_block=gs, initial_state=dev(init),
                dfinal_state=dev(ct["dfinal"]) if with_final else None, want_dinit=True)
    torch.cuda.synchronize()
    r = oracle.backward(to_f64(X), to_f64(la), to_f64(B), to_f64(C), to_f64(ct["dY"]),
                        dfinal=to_f64(ct["dfinal"]) if with_final else None,
                        cu_seqlens=None if cu is None else cu.numpy(),
                        init=None if init is None else init.double().numpy())
    dt = dtype_name(X)
    errs = {}
    for k, ref in (("dX", r["dX"]), ("dlog_a", r["dlog_a"]), ("dB", r["dB"]), ("dC", r["dC"]),
                   ("dinit", r["dinit"])):
        errs[k] = assert_close(to_f64(g[k]), ref, dt, f"{what} {k}")
    say(f"[bwd] {what}: " + " ".join(f"{k} rel_l2={e['rel_l2']:.2e} max_unit={e['max_unit']:.3f}"
                                     for k, e in errs.items()))
    return g


CASES = [
    # (batch, T, H, P, N, G, dtype, Q)
    (1, 300, 4, 64, 64, 1, torch.bfloat16, 64),     # head pairs in the dX run, ragged tail
    (2, 200, 4, 32, 64, 2, torch.bfloat16, 64),     # two groups
    (1, 257, 3, 64, 128, 1, torch.bfloat16, 128),   # N = 128, odd heads per group
    (1, 129, 2, 128, 32, 1, torch.bfloat16, 32),    # P = 128 (the dB/dC runs have dstate 128)
    (1, 77, 3, 16, 16, 1, torch.float32, 16),       # fp32
    (2, 150, 2, 32, 64, 2, torch.float32, 64),      # fp32, two groups
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}-T{}-H{}-P{}-N{}-G{}-{}-Q{}".format(
    *c[:6], "bf16" if c[6] == torch.bfloat16 else "fp32", c[7]))
def test_bwd_shapes(case):
    b, T, H, P, N, G, dt, Q = case
    d = synth.make_forward_inputs(b, T, H, P, N, G, dtype=dt, seed=3000 + T + N)
    check_bwd(d, Q, f"shape {case}", seed=7)


@pytest.mark.parametrize("with_final,with_init", [(False, False), (True, False), (False, True)])
def test_bwd_optional_states(with_final, with_init):
    d = synth.make_forward_inputs(1, 260, 4, 64, 64, 1, dtype=torch.bfloat16, seed=3100)
    check_bwd(d, 64, "optional states", with_final=with_final, with_init=with_init, seed=8)


@pytest.mark.parametrize("dt,Q,gs", [(torch.bfloat16, 64, 2), (torch.bfloat16, 128, 4), (torch.float32, 32, 1)])
def test_bwd_packed(dt, Q, gs):
    lengths = [1, 200, 64, 65, 3, 129, 1, 90]
    d = synth.make_forward_inputs(1, sum(lengths), 3, 32, 64, 1, dtype=dt, seed=3200, lengths=lengths)
    check_bwd(d, Q, f"packed {lengths}", gs=gs, seed=9)


def test_bwd_head_pair_state_runs():
    """More (state block, head) units than one round of the one-head chunk_state:
    both state runs of the backward take the head-pair form (two heads per
    workgroup), with state blocks of two chunks (chunk_starts expands them)."""
    d = synth.make_forward_inputs(1, 2048, 96, 32, 64, 1, dtype=torch.bfloat16, seed=8801)
    sh = ssd.make_shape(d["X"], d["B"])
    assert ssd.layout(sh, 128, 2).nblocks * 96 > 512
    check_bwd(d, 128, "head-pair state runs", gs=2, seed=8802)


def test_bwd_long_sequence():
    """T = 4096 with the headline head size and state size (8 heads, 4 state blocks of 8 chunks)."""
    d = synth.make_forward_inputs(1, 4096, 8, 64, 128, 1, dtype=torch.bfloat16, seed=3300)
    check_bwd(d, 128, "long sequence", seed=10)


def test_bwd_state_block_invariance():
    d = synth.make_forward_inputs(1, 1100, 4, 64, 128, 1, dtype=torch.bfloat16, seed=3400)
    g1 = check_bwd(d, 128, "gs 1", gs=1, seed=11)
    g8 = check_bwd(d, 128, "gs 8", gs=8, seed=11)
    for k in ("dX", "dB", "dC", "dlog_a"):
        assert_close(to_f64(g8[k]), to_f64(g1[k]), "bf16", f"gs 8 vs gs 1 {k}")


def test_bwd_headline_sampled_heads():
    """The headline workload at full size (T = 16384, H = 32, P = 64, N = 128, Q = 128, default state
    block, as bench.py times it). dX and d log a of two sampled heads depend on those heads alone, so
    the oracle runs on them only; dB and dC sum over heads, so a second GPU call with dY and the
    final-state gradient zero outside the sampled heads gives their share, which the oracle's dB
    and dC on the two heads must match."""
    w = synth.WORKLOADS[synth.HEADLINE]
    d = synth.workload_inputs(w)
    X, la, B, C = (d[k] for k in ("X", "log_a", "B", "C"))
    b, T, H, P = X.shape
    N = B.shape[-1]
    heads = [0, 17]
    ct = synth.make_cotangents(b, T, H, P, N, b, dtype=X.dtype, seed=12)
    dfin = _dfinal_states(b, H, P, N, seed=13)
    say(f"[bwd] headline sampled heads {heads}: X{tuple(X.shape)} Q={w.Q}")
    dev = lambda t: t.cuda()
    Xg, lag, Bg, Cg = dev(X), dev(la), dev(B), dev(C)
    g = ssd.bwd(Xg, lag, Bg, Cg, dev(ct["dY"]), chunk=w.Q, dfinal_state=dev(dfin))
    mask = torch.zeros(H, dtype=torch.bool)
    mask[heads] = True
    dY_s = ct["dY"].clone()
    dY_s[:, :, ~mask] = 0
    dfin_s = dfin.clone()
    dfin_s[:, ~mask] = 0
    g_s = ssd.bwd(Xg, lag, Bg, Cg, dev(dY_s), chunk=w.Q, dfinal_state=dev(dfin_s))
    torch.cuda.synchronize()
    r = oracle.backward(to_f64(X[:, :, heads]), to_f64(la[:, :, heads]), to_f64(B), to_f64(C),
                        to_f64(ct["dY"][:, :, heads]), dfinal=to_f64(dfin[:, heads]))
    assert_close(to_f64(g["dX"][:, :, heads]), r["dX"], "bf16", "headline dX")
    assert_close(to_f64(g["dlog_a"][:, :, heads]), r["dlog_a"], "bf16", "headline dlog_a")
    assert_close(to_f64(g_s["dB"]), r["dB"], "bf16", "headline dB (sampled heads)")
    assert_close(to_f64(g_s["dC"]), r["dC"], "bf16", "headline dC (sampled heads)")
