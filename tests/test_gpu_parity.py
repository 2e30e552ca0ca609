"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every test runs the library on seeded synthetic inputs and compares it element
by element with ``oracle/`` on the same stored (rounded) input values. Sizes
span several chunks and a ragged tail; the named workloads run at full size.
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

LOG2E = 1.4426950408889634


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ssd.lib()  # the HIP library must load: no fallback


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(d):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def gpu_fwd(d, Q, gs=0, **kw):
    dd = to_dev(d)
    Y, fin = ssd.fwd(dd["X"], dd["log_a"], dd["B"], dd["C"], cu_seqlens=dd.get("cu_seqlens"), chunk=Q,
                     state_block=gs, **kw)
    torch.cuda.synchronize()
    return Y, fin


def oracle_fwd(d):
    cu = d.get("cu_seqlens")
    return oracle.forward(to_f64(d["X"]), to_f64(d["log_a"]), to_f64(d["B"]), to_f64(d["C"]),
                          cu_seqlens=None if cu is None else cu.numpy())


def check_fwd(d, Q, what, gs=0):
    say(f"[parity] {what}: X{tuple(d['X'].shape)} {d['X'].dtype} N={d['B'].shape[-1]} Q={Q} state_block={gs}")
    Y, fin = gpu_fwd(d, Q, gs)
    Yr, fr = oracle_fwd(d)
    dt = dtype_name(d["X"])
    ey = assert_close(to_f64(Y), Yr, dt, what + " Y")
    ef = assert_close(to_f64(fin), fr, dt, what + " final")
    say(f"[parity] {what}: Y {ey} final {ef}")
    return Y, fin


# ------------------------------------------------------------------ named workloads

@pytest.mark.parametrize("name", ["tiny-fp32-T256", "b2-T2048-H24-N64", "long-T16384-H32-N128",
                                  "sweep-b8-T4096-N64", "sweep-b8-T4096-N128", "sweep-b8-T4096-N256",
                                  "packed-T32768-H80-N128"])
def test_workload_full_size(name):
    w = synth.WORKLOADS[name]
    d = synth.workload_inputs(w)
    check_fwd(d, w.Q, name)              # the library's default state block
    if w.dtype == "bf16":
        check_fwd(d, w.Q, name + " (one chunk per state block)", gs=1)


# ------------------------------------------------------------------ shapes and edge cases

# The two-head chunk_scan kernel runs when the heads of a group come in pairs,
# P <= 64, N <= 128 and Q <= 128; the single-head kernel covers the rest
# (odd heads per group, P = 128, N = 256, Q = 256). The cases below exercise both.
CASES = [
    # (batch, T, H, P, N, G, dtype, Q)
    (1, 200, 3, 64, 64, 1, torch.bfloat16, 64),     # ragged tail
    (2, 100, 2, 32, 32, 2, torch.bfloat16, 32),     # G = H
    (1, 50, 4, 16, 32, 2, torch.bfloat16, 64),      # T < Q, P = 16, two groups
    (1, 333, 2, 128, 128, 1, torch.bfloat16, 128),  # P = 128
    (1, 300, 2, 64, 256, 1, torch.bfloat16, 128),   # N = 256
    (1, 600, 2, 64, 128, 1, torch.bfloat16, 256),   # Q = 256
    (3, 129, 2, 32, 64, 1, torch.bfloat16, 128),    # one full chunk + 1 token
    (1, 1, 2, 64, 64, 1, torch.bfloat16, 64),       # a single token
    (1, 77, 3, 16, 16, 1, torch.float32, 16),       # fp32, Q = 16
    (2, 500, 2, 128, 256, 2, torch.float32, 256),   # fp32, large tiles
    (1, 300, 4, 32, 64, 4, torch.float32, 64),      # fp32, G = H
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}-T{}-H{}-P{}-N{}-G{}-{}-Q{}".format(
    *c[:6], "bf16" if c[6] == torch.bfloat16 else "fp32", c[7]))
def test_shapes(case):
    b, T, H, P, N, G, dt, Q = case
    d = synth.make_forward_inputs(b, T, H, P, N, G, dtype=dt, seed=1000 + T + N)
    check_fwd(d, Q, f"shape {case}")


@pytest.mark.parametrize("P,N,Q,gs", [(64, 128, 128, 4), (32, 64, 64, 2), (16, 32, 32, 1)])
def test_head_pairs_match_single_heads(P, N, Q, gs):
    """A head pair through the two-head kernel (two heads, one group) against the
    same heads run one at a time (one head per group, which takes the single-head
    kernel): both within the oracle tolerance, and close to each other."""
    d = synth.make_forward_inputs(1, 3 * Q + 17, 2, P, N, 1, dtype=torch.bfloat16, seed=4242 + P + N)
    say(f"[parity] head pairs vs single heads P={P} N={N} Q={Q} gs={gs}")
    Y2, f2 = check_fwd(d, Q, "head pair", gs)
    for h in range(2):
        dh = dict(d)
        dh["X"] = d["X"][:, :, h:h + 1].contiguous()
        dh["log_a"] = d["log_a"][:, :, h:h + 1].contiguous()
        Y1, f1 = check_fwd(dh, Q, f"single head {h}", gs)
        e = assert_close(to_f64(Y2[:, :, h:h + 1]), to_f64(Y1), "bf16", f"pair vs single head {h} Y")
        assert e["rel_l2"] < 5e-3, e
        assert_close(to_f64(f2[:, h:h + 1]), to_f64(f1), "bf16", f"pair vs single head {h} final")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_linear_attention_no_decay(dt):
    d = synth.make_forward_inputs(1, 300, 2, 32, 64, 1, dtype=dt, seed=77)
    d["log_a"].zero_()
    check_fwd(d, 64, "log_a = 0")


def test_strong_decay():
    # dt up to 1, A up to 16: log a down to -16 per token (deep underflow inside chunks)
    d = synth.make_forward_inputs(1, 512, 2, 64, 64, 1, dtype=torch.bfloat16, seed=78, dt_range=(0.1, 1.0))
    check_fwd(d, 128, "strong decay")


@pytest.mark.parametrize("Q", [32, 64, 128, 256])
def test_chunk_size_invariance(Q):
    d = synth.make_forward_inputs(2, 1000, 4, 64, 128, 1, dtype=torch.bfloat16, seed=5)
    check_fwd(d, Q, f"chunk {Q}")


@pytest.mark.parametrize("Q", [16, 32, 64])
def test_chunk_size_invariance_fp32(Q):
    d = synth.make_forward_inputs(1, 400, 2, 16, 16, 1, dtype=torch.float32, seed=6)
    check_fwd(d, Q, f"fp32 chunk {Q}")


# ------------------------------------------------------------------ packed sequences

@pytest.mark.parametrize("dt,Q", [(torch.bfloat16, 64), (torch.bfloat16, 128), (torch.float32, 32)])
def test_packed_ragged_lengths(dt, Q):
    lengths = [1, 200, 64, 65, 3, 129, 1, 300]
    d = synth.make_forward_inputs(1, sum(lengths), 3, 32, 64, 1, dtype=dt, seed=9, lengths=lengths)
    check_fwd(d, Q, f"packed {lengths}")


def test_packed_equals_separate_runs_bitwise():
    lengths = [100, 37, 256, 5]
    d = synth.make_forward_inputs(1, sum(lengths), 2, 64, 64, 1, dtype=torch.bfloat16, seed=10, lengths=lengths)
    Y, fin = gpu_fwd(d, 64)
    cu = d["cu_seqlens"].numpy()
    for s in range(len(lengths)):
        b, e = int(cu[s]), int(cu[s + 1])
        ds = {k: d[k][:, b:e].contiguous() for k in ("X", "log_a", "B", "C")}
        Ys, fs = gpu_fwd(ds, 64)
        assert torch.equal(Y[:, b:e], Ys)
        assert torch.equal(fin[s], fs[0])


def test_many_short_sequences():
    rng = np.random.default_rng(12)
    lengths = list(rng.integers(1, 40, size=120))
    d = synth.make_forward_inputs(1, int(sum(lengths)), 2, 64, 64, 1, dtype=torch.bfloat16, seed=12,
                                  lengths=[int(v) for v in lengths])
    check_fwd(d, 32, "120 short sequences")


# ------------------------------------------------------------------ stage intermediates

def stage_run(d, Q, gs):
    dd = to_dev(d)
    X, la, B, C, cu = dd["X"], dd["log_a"], dd["B"], dd["C"], dd.get("cu_seqlens")
    sh = ssd.make_shape(X, B, cu)
    ws = ssd.Workspace(sh, Q, X.device, gs)
    nseq = X.shape[0] if cu is None else cu.numel() - 1
    fin = torch.empty(nseq, X.shape[2], X.shape[3], B.shape[3], dtype=torch.float32, device=X.device)
    Y = torch.empty_like(X)
    ssd.chunk_cumsum(la, cu, sh, ws)
    ssd.chunk_state(X, B, cu, sh, ws)
    ssd.state_passing(cu, fin, sh, ws)
    ssd.chunk_scan(X, B, C, cu, Y, sh, ws)
    torch.cuda.synchronize()
    return ws, Y, fin


def _slots(units, span, rows, T, cu):
    """Documented slot numbering of chunks (span = Q) or state blocks (span = Gs*Q)."""
    out = []
    if cu is None:
        per_row = -(-T // span) if span else 0
        for (r, b, e) in units:
            out.append(r * per_row + b // span)
    else:
        for (r, b, e) in units:
            s = int(np.searchsorted(cu, b, side="right") - 1)
            out.append(int(cu[s]) // span + s + (b - int(cu[s])) // span)
    return out


@pytest.mark.parametrize("packed", [False, True])
def test_head_pair_chunk_state(packed):
    """Shapes with more than 512 (state block, head) units and heads in pairs take
    the head-pair chunk_state (two heads per workgroup, 64-row passes): its right
    factors against the oracle restarted at every block start, and the stage
    entry point (segment sums from the cumsum stage) bitwise equal to the fused
    form inside ssd_fwd."""
    if packed:
        lengths = [300, 17, 64, 65, 129, 400, 25]
        rows, T, H, P, N, Q, gs = 1, sum(lengths), 64, 32, 64, 64, 2
    else:
        lengths = None
        rows, T, H, P, N, Q, gs = 2, 1100, 32, 64, 128, 128, 1
    d = synth.make_forward_inputs(rows, T, H, P, N, 1, dtype=torch.bfloat16, seed=3301, lengths=lengths)
    say(f"[parity] head-pair chunk_state packed={packed} H={H} P={P} N={N} Q={Q} state_block={gs}")
    ws, Y, fin = stage_run(d, Q, gs)
    assert ws.layout.nblocks * H > 512 and H % 2 == 0
    cu = None if d["cu_seqlens"] is None else d["cu_seqlens"].numpy()
    X, la, B, C = (to_f64(d[k]) for k in ("X", "log_a", "B", "C"))
    blocks = oracle.chunk_segments(rows, T, Q * gs, cu)
    bslots = _slots(blocks, Q * gs, rows, T, cu)
    _, bst_ref, _ = oracle.scan(X, la, B, C, segments=blocks, want_y=False)
    bst = ws.block_states().clone()
    bdec = ws.block_decay().clone()
    assert_close(bst.cpu().numpy()[bslots], bst_ref, "bf16", "head-pair block states")
    dd = to_dev(d)
    ssd.fwd(dd["X"], dd["log_a"], dd["B"], dd["C"], cu_seqlens=dd.get("cu_seqlens"), chunk=Q, state_block=gs,
            workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(ws.block_states()[bslots], bst[bslots])
    assert torch.equal(ws.block_decay()[bslots], bdec[bslots])


@pytest.mark.parametrize("packed,dt,Q,gs", [(False, torch.bfloat16, 64, 1), (True, torch.bfloat16, 64, 1),
                                            (False, torch.bfloat16, 32, 4), (True, torch.bfloat16, 32, 2),
                                            (False, torch.float32, 32, 1), (True, torch.float32, 16, 1)])
def test_stage_intermediates(packed, dt, Q, gs):
    rows = 1 if packed else 2
    lengths = [70, 1, 130, 64, 200] if packed else None
    T = sum(lengths) if packed else 200
    d = synth.make_forward_inputs(rows, T, 3, 32, 64 if dt == torch.bfloat16 else 16, 1, dtype=dt, seed=21,
                                  lengths=lengths)
    say(f"[parity] stage intermediates packed={packed} {dt} Q={Q} state_block={gs}")
    ws, Y, fin = stage_run(d, Q, gs)
    X, la, B, C = (to_f64(d[k]) for k in ("X", "log_a", "B", "C"))
    cu = None if d["cu_seqlens"] is None else d["cu_seqlens"].numpy()
    dts = dtype_name(d["X"])
    chunks = oracle.chunk_segments(rows, T, Q, cu)
    blocks = oracle.chunk_segments(rows, T, Q * gs, cu)
    cslots = _slots(chunks, Q, rows, T, cu)
    bslots = _slots(blocks, Q * gs, rows, T, cu)
    # chunk records and state-block records
    table = ws.table().cpu().numpy()
    for (r, b, e), sl in zip(chunks, cslots):
        assert table[sl, 1] == r * T + b and table[sl, 2] == e - b
    for sl in set(range(table.shape[0])) - set(cslots):
        assert table[sl, 2] == 0
    btable = ws.block_table().cpu().numpy()
    for (r, b, e), bl in zip(blocks, bslots):
        first = cslots[[c[1] for c in chunks if c[0] == r].index(b) + sum(1 for c in chunks if c[0] < r)]
        assert btable[bl, 1] == first and btable[bl, 2] == -(-(e - b) // Q)
    for bl in set(range(btable.shape[0])) - set(bslots):
        assert btable[bl, 2] == 0
    # cumulative log decay, restarted per chunk, log2-scaled
    cs_ref = oracle.chunk_cumsum(la, chunks)
    cs_gpu = ws.cumsum().cpu().numpy()
    for (r, b, e), sl in zip(chunks, cslots):
        ref = cs_ref[r, b:e].T * LOG2E                       # [H, q]
        got = cs_gpu[sl, :, :e - b]
        assert np.max(np.abs(got - ref)) <= 1e-4 + 1e-5 * np.max(np.abs(ref))
        assert np.all(cs_gpu[sl, :, e - b:] == cs_gpu[sl, :, e - b - 1:e - b])  # padding repeats the total
    # block decay = total log2 decay of each block
    bd = ws.block_decay().cpu().numpy()
    for (r, b, e), bl in zip(blocks, bslots):
        ref = la[r, b:e].sum(axis=0) * LOG2E
        assert np.max(np.abs(bd[bl] - ref)) <= 1e-4 + 1e-5 * np.max(np.abs(ref))
    # right factors = oracle restarted at every block start, read at the block end
    _, bst_ref, _ = oracle.scan(X, la, B, C, segments=blocks, want_y=False)
    assert_close(ws.block_states().cpu().numpy()[bslots], bst_ref, dts, "block states")
    # centre factors = oracle state entering each block (zero at sequence starts)
    bounds = set() if cu is None else set(int(v) for v in cu)
    snap = -np.ones(rows * T, np.int32)
    first = []
    for k, (r, b, e) in enumerate(blocks):
        first.append(b == 0 if cu is None else b in bounds)
        if k + 1 < len(blocks) and blocks[k + 1][0] == r and blocks[k + 1][1] == e and e not in bounds:
            snap[r * T + e - 1] = k + 1
    segs = oracle.sequence_segments(rows, T, cu)
    _, _, snaps = oracle.scan(X, la, B, C, segments=segs, want_y=False, snap_slot=snap, nsnaps=len(blocks) + 1)
    st_gpu = ws.start_states().float().cpu().numpy()[bslots]
    for k in range(len(blocks)):
        if first[k]:
            assert np.all(st_gpu[k] == 0)
    idx = [k for k in range(len(blocks)) if not first[k]]
    if idx:
        assert_close(st_gpu[idx], snaps[idx], dts, "start states")
    # outputs, and stage-by-stage equals ssd_fwd_ex bitwise
    Yr, fr = oracle_fwd(d)
    assert_close(to_f64(Y), Yr, dts, "Y")
    assert_close(to_f64(fin), fr, dts, "final")
    Y2, fin2 = gpu_fwd(d, Q, gs)
    assert torch.equal(Y, Y2) and torch.equal(fin, fin2)


def expected_launch_order(counts):
    """The chunk-scan launch order the state-passing stage writes into the block
    records' fourth word: slots ranked by chunk count, most first, ties by slot,
    as (slot + 1) | (nfull << 16) with nfull the number of slots holding the
    largest count."""
    c = np.clip(np.asarray(counts, np.int64), 0, 16)
    order = sorted(range(len(c)), key=lambda m: (-c[m], m))
    nfull = int(np.sum(c == c.max()))
    return np.array([(m + 1) | (nfull << 16) for m in order], np.int64)


@pytest.mark.parametrize("case", ["packed", "ragged rows", "whole blocks"])
def test_block_launch_order(case):
    """Block slots of unequal length are ranked (longest first) for the
    chunk-scan stage; rows made of whole state blocks keep the plain order (the
    word stays 0). Y is the same either way."""
    if case == "packed":
        d = synth.make_forward_inputs(1, 3 * 1024 + 700, 4, 64, 128, 1, dtype=torch.bfloat16, seed=61,
                                      lengths=[1024 + 5, 300, 2048 + 128 + 7, 700 - 440])
    else:
        T = 2 * 1024 + (300 if case == "ragged rows" else 0)
        d = synth.make_forward_inputs(3, T, 4, 64, 128, 1, dtype=torch.bfloat16, seed=62)
    say(f"[parity] block launch order: {case}")
    ws, Y, fin = stage_run(d, 128, 8)
    bt = ws.block_table().cpu().numpy().astype(np.int64)
    if case == "whole blocks":
        assert np.all(bt[:, 3] == 0)
    else:
        assert np.array_equal(bt[:, 3], expected_launch_order(bt[:, 2]))
    Yr, fr = oracle_fwd(d)
    dts = dtype_name(d["X"])
    assert_close(to_f64(Y), Yr, dts, "Y")
    assert_close(to_f64(fin), fr, dts, "final")


@pytest.mark.parametrize("gs", [1, 2, 4, 8, 16])
def test_state_block_invariance(gs):
    d = synth.make_forward_inputs(2, 3000, 4, 64, 128, 1, dtype=torch.bfloat16, seed=44)
    check_fwd(d, 128, f"state block {gs}", gs=gs)


@pytest.mark.parametrize("gs", [2, 8])
def test_state_block_packed(gs):
    lengths = [1, 700, 64, 65, 3, 1290, 1, 300]
    d = synth.make_forward_inputs(1, sum(lengths), 3, 64, 64, 1, dtype=torch.bfloat16, seed=45, lengths=lengths)
    check_fwd(d, 64, f"packed state block {gs}", gs=gs)


@pytest.mark.parametrize("P,N,Q,gs", [(16, 32, 32, 4), (32, 64, 64, 2), (128, 128, 64, 4), (64, 256, 64, 4),
                                      (128, 64, 128, 2), (64, 128, 256, 2)])
def test_state_block_shapes(P, N, Q, gs):
    d = synth.make_forward_inputs(1, 1100, 2, P, N, 1, dtype=torch.bfloat16, seed=46 + P + N)
    check_fwd(d, Q, f"P={P} N={N} Q={Q}", gs=gs)


def test_deterministic():
    d = synth.make_forward_inputs(1, 1024, 4, 64, 128, 1, dtype=torch.bfloat16, seed=31)
    Y1, f1 = gpu_fwd(d, 128)
    Y2, f2 = gpu_fwd(d, 128)
    assert torch.equal(Y1, Y2) and torch.equal(f1, f2)


# ------------------------------------------------------------------ decode step

@pytest.mark.parametrize("dt,N", [(torch.bfloat16, 128), (torch.float32, 16), (torch.bfloat16, 256),
                                  (torch.bfloat16, 32)])
def test_step_sequence(dt, N):
    b, steps, H, P = 3, 40, 4, 64 if N != 16 else 16
    d = synth.make_decode_inputs(b, steps, H, P, N, 2, dtype=dt, seed=50 + N)
    say(f"[parity] step b={b} steps={steps} H={H} P={P} N={N} {dt}")
    state = torch.zeros(b, H, P, N, dtype=torch.float32, device="cuda")
    dd = to_dev(d)
    ys = []
    for t in range(steps):
        ys.append(ssd.step(state, dd["x"][t], dd["log_a"][t], dd["B"][t], dd["C"][t]))
    torch.cuda.synchronize()
    Yg = torch.stack(ys, 1)                          # [b, steps, H, P]
    X = to_f64(d["x"]).transpose(1, 0, 2, 3)
    la = to_f64(d["log_a"]).transpose(1, 0, 2)
    B = to_f64(d["B"]).transpose(1, 0, 2, 3)
    C = to_f64(d["C"]).transpose(1, 0, 2, 3)
    Yr, fr = oracle.forward(X, la, B, C)
    dts = dtype_name(d["x"])
    assert_close(to_f64(Yg), Yr, dts, "step y")
    assert_close(to_f64(state), fr, dts, "step state")


# ------------------------------------------------------------------ initial states

def _init_states(n, H, P, N, seed, T0=200):
    """Initial states at the scale the layer itself produces: the oracle's final
    states after a seeded prefix of T0 tokens (the chunked-prefill use)."""
    d = synth.make_forward_inputs(n, T0, H, P, N, 1, dtype=torch.float32, seed=seed)
    _, fin = oracle.forward(to_f64(d["X"]), to_f64(d["log_a"]), to_f64(d["B"]), to_f64(d["C"]))
    return torch.from_numpy(fin).float()


@pytest.mark.parametrize("dt,Q,gs", [(torch.bfloat16, 64, 2), (torch.bfloat16, 128, 1), (torch.float32, 32, 1)])
def test_initial_state(dt, Q, gs):
    """ssd_fwd_ex from a given initial state per row against the oracle run from it."""
    b, T, H, P, N = 2, 300, 4, 64, 64
    d = synth.make_forward_inputs(b, T, H, P, N, 1, dtype=dt, seed=70 + Q)
    h0 = _init_states(b, H, P, N, 71)
    say(f"[parity] initial state {dt} Q={Q} gs={gs}")
    Y, fin = gpu_fwd(d, Q, gs, initial_state=h0.cuda())
    Yr, fr = oracle.forward(to_f64(d["X"]), to_f64(d["log_a"]), to_f64(d["B"]), to_f64(d["C"]), init=h0.double().numpy())
    assert_close(to_f64(Y), Yr, dtype_name(d["X"]), "initial state Y")
    assert_close(to_f64(fin), fr, dtype_name(d["X"]), "initial state final")


def test_initial_state_packed():
    """Packed sequences, each from its own initial state."""
    d = synth.make_forward_inputs(1, 1500, 4, 64, 128, 1, dtype=torch.bfloat16, seed=72, varlen=(100, 700))
    S = d["cu_seqlens"].numel() - 1
    h0 = _init_states(S, 4, 64, 128, 73)
    say(f"[parity] initial state packed S={S}")
    Y, fin = gpu_fwd(d, 128, 2, initial_state=h0.cuda())
    Yr, fr = oracle.forward(to_f64(d["X"]), to_f64(d["log_a"]), to_f64(d["B"]), to_f64(d["C"]),
                            cu_seqlens=d["cu_seqlens"].numpy(), init=h0.double().numpy())
    assert_close(to_f64(Y), Yr, "bf16", "packed initial state Y")
    assert_close(to_f64(fin), fr, "bf16", "packed initial state final")


def test_prefill_in_pieces():
    """A prompt run in three pieces, each from the previous piece's final state,
    equals the oracle over the whole prompt."""
    b, T, H, P, N = 2, 1000, 4, 64, 128
    cuts = [0, 333, 700, T]
    d = synth.make_forward_inputs(b, T, H, P, N, 1, dtype=torch.bfloat16, seed=74)
    dd = to_dev(d)
    state, ys = None, []
    for a, e in zip(cuts[:-1], cuts[1:]):
        Y, state = ssd.fwd(*(dd[k][:, a:e].contiguous() for k in ("X", "log_a", "B", "C")), chunk=128,
                           initial_state=state)
        ys.append(Y)
    torch.cuda.synchronize()
    Yr, fr = oracle_fwd(d)
    assert_close(to_f64(torch.cat(ys, 1)), Yr, "bf16", "pieces Y")
    assert_close(to_f64(state), fr, "bf16", "pieces final")


def test_prefill_then_decode_handoff():
    """ssd_fwd over [0, T1) then ssd_step over [T1, T) equals the oracle over [0, T)."""
    b, T, T1, H, P, N = 2, 300, 237, 4, 64, 128
    d = synth.make_forward_inputs(b, T, H, P, N, 1, dtype=torch.bfloat16, seed=60)
    dd = to_dev(d)
    _, fin = ssd.fwd(dd["X"][:, :T1].contiguous(), dd["log_a"][:, :T1].contiguous(), dd["B"][:, :T1].contiguous(),
                     dd["C"][:, :T1].contiguous(), chunk=128)
    state = fin.clone()
    ys = []
    for t in range(T1, T):
        ys.append(ssd.step(state, dd["X"][:, t].contiguous(), dd["log_a"][:, t].contiguous(),
                           dd["B"][:, t].contiguous(), dd["C"][:, t].contiguous()))
    torch.cuda.synchronize()
    Yr, fr = oracle_fwd(d)
    assert_close(to_f64(torch.stack(ys, 1)), Yr[:, T1:], "bf16", "handoff y")
    assert_close(to_f64(state), fr, "bf16", "handoff final")


def test_decode_workload_full_size_sampled():
    """All 4096 steps at batch 64, 80 heads; the oracle follows 256 sampled (row, head)
    streams, four heads of every row."""
    w = synth.WORKLOADS["decode-b64-H80-N128"]
    say(f"[parity] decode workload {w}")
    d = synth.workload_inputs(w)
    dd = to_dev(d)
    state = torch.zeros(w.batch, w.H, w.P, w.N, dtype=torch.float32, device="cuda")
    rng = np.random.default_rng(7)
    pairs = [(r, int(h)) for r in range(w.batch) for h in rng.choice(w.H, 4, replace=False)]
    ys = torch.empty(w.steps, len(pairs), w.P, dtype=torch.bfloat16, device="cuda")
    rows = torch.tensor([p[0] for p in pairs], device="cuda")
    heads = torch.tensor([p[1] for p in pairs], device="cuda")
    y = torch.empty(w.batch, w.H, w.P, dtype=torch.bfloat16, device="cuda")
    for t in range(w.steps):
        ssd.step(state, dd["x"][t], dd["log_a"][t], dd["B"][t], dd["C"][t], y=y)
        ys[t] = y[rows, heads]
    torch.cuda.synchronize()
    r = torch.tensor([p[0] for p in pairs])
    h = torch.tensor([p[1] for p in pairs])
    # each sampled stream as its own row of a one-head oracle run (index first, then upcast)
    X = to_f64(d["x"][:, r, h, :]).transpose(1, 0, 2)[:, :, None, :]
    la = to_f64(d["log_a"][:, r, h]).T[:, :, None]
    B = to_f64(d["B"][:, r, 0, :]).transpose(1, 0, 2)[:, :, None, :]
    C = to_f64(d["C"][:, r, 0, :]).transpose(1, 0, 2)[:, :, None, :]
    Yr, fr = oracle.forward(X, la, B, C)
    assert_close(to_f64(ys).transpose(1, 0, 2), Yr[:, :, 0, :], "bf16", "decode y")
    assert_close(to_f64(state[rows, heads]), fr[:, 0], "bf16", "decode state")


def _gpu_errors(got, ref, rows_per_slice=8):
    """For two device tensors with the same first (row) dimension, accumulated in fp64
    over slices of rows to bound device memory: max |d| / rms(ref), ||d|| / ||ref||, and
    the largest |d_i| / (5e-2 rms(ref) + 2^-8 |ref_i|) (the plain bf16 bar plus one
    rounding of the element itself; <= 1 passes)."""
    from parity import BF16_MAXABS_UNIT, BF16_UNIT_ROUNDOFF
    rsq, n = 0.0, 0
    for r0 in range(0, ref.shape[0], rows_per_slice):
        r = ref[r0:r0 + rows_per_slice].double()
        rsq += r.pow(2).sum().item()
        n += r.numel()
    rms = (rsq / n) ** 0.5
    dmax, dsq, worst = 0.0, 0.0, 0.0
    for r0 in range(0, ref.shape[0], rows_per_slice):
        g, r = got[r0:r0 + rows_per_slice].double(), ref[r0:r0 + rows_per_slice].double()
        d = (g - r).abs()
        dmax = max(dmax, d.max().item())
        dsq += d.pow(2).sum().item()
        worst = max(worst, (d / (BF16_MAXABS_UNIT * rms + BF16_UNIT_ROUNDOFF * r.abs())).max().item())
    return dmax / max(rms, 1e-300), dsq ** 0.5 / max(rsq ** 0.5, 1e-300), worst


def test_decode_workload_matches_chunked_forward():
    """Every one of the 5120 (row, head) streams of the decode workload: 4096 decode steps
    from a zero state give the outputs and final state of the chunked forward pass run on
    the same inputs as 64 sequences of 4096 tokens (the recurrence and its chunked form
    are the same map). Each side is rounded to bf16 on its own, so y is held to the bf16
    bar plus one rounding of the element (rel-L2 <= 2e-2, |d_i| <= 5e-2 rms + 2^-8 |y_i|)
    and the fp32 states to the plain bf16 bar; the oracle itself is checked on sampled
    streams above and on the chunked path's workloads."""
    from parity import BF16_MAXABS_UNIT, BF16_RELL2
    w = synth.WORKLOADS["decode-b64-H80-N128"]
    say(f"[parity] decode workload against the chunked forward, all streams")
    d = synth.workload_inputs(w)
    dd = to_dev(d)
    state = torch.zeros(w.batch, w.H, w.P, w.N, dtype=torch.float32, device="cuda")
    ys = torch.empty(w.steps, w.batch, w.H, w.P, dtype=torch.bfloat16, device="cuda")
    for t in range(w.steps):
        ssd.step(state, dd["x"][t], dd["log_a"][t], dd["B"][t], dd["C"][t], y=ys[t])
    X = dd["x"].permute(1, 0, 2, 3).contiguous()
    la = dd["log_a"].permute(1, 0, 2).contiguous()
    B = dd["B"].permute(1, 0, 2, 3).contiguous()
    C = dd["C"].permute(1, 0, 2, 3).contiguous()
    Y, fin = ssd.fwd(X, la, B, C, chunk=128)
    torch.cuda.synchronize()
    my, ly, wy = _gpu_errors(ys.permute(1, 0, 2, 3), Y)
    mf, lf, _ = _gpu_errors(state, fin)
    say(f"[parity] decode vs chunked: y max|d|/rms {my:.3e} rel-L2 {ly:.3e} rounded-bar {wy:.3f}; "
        f"state max|d|/rms {mf:.3e} rel-L2 {lf:.3e}")
    assert wy <= 1 and ly <= BF16_RELL2
    assert mf <= BF16_MAXABS_UNIT and lf <= BF16_RELL2


# ------------------------------------------------------------------ half-chunk kernel

# Shapes that take the half-chunk two-head kernel (four waves, chunks walked in
# halves of 64 tokens, at least 512 (state block, head pair) units): ragged
# tails that end in either half, chunks of 64 and 128, several chunks per
# state block, P = 16 and 32, N = 32 and 64, packed sequences of 1 to 300
# tokens. Each asserts, through ssd_chunk_scan_kernel, that this kernel runs.
HALF_CASES = [
    # (batch, T, H, P, N, G, Q, state_block, varlen)
    (2, 2000, 32, 64, 128, 1, 128, 1, None),      # last chunk 80 tokens: halves of 64 and 16
    (1, 4100, 32, 64, 64, 1, 128, 1, None),       # last chunk 4 tokens
    (2, 2048, 32, 64, 64, 1, 64, 2, None),        # chunks of 64, two per state block
    (4, 1000, 64, 32, 128, 1, 128, 2, None),      # last chunk 104 tokens, two chunks per block
    (2, 700, 64, 16, 32, 2, 64, 1, None),         # P = 16, N = 32, two groups
    (1, 1500, 64, 64, 128, 1, 128, 1, (1, 300)),  # packed: sequences of 1..300 tokens
    (1, 1500, 64, 64, 64, 1, 64, 2, (1, 200)),    # packed, chunks of 64, two chunks per state block
]
# N = 256 takes the eight-wave form of the same kernel whatever the unit count.
HALF_WIDE_CASES = [
    (1, 300, 2, 64, 256, 1, 128, 0, None),        # last chunk 44 tokens
    (2, 700, 4, 32, 256, 2, 64, 2, None),         # P = 32, chunks of 64, two groups
    (1, 1000, 2, 16, 256, 1, 128, 4, None),       # P = 16, last chunk 104 tokens
    (1, 1200, 4, 64, 256, 1, 128, 2, (1, 300)),   # packed
]


@pytest.mark.parametrize("case", [c + ("half_pair",) for c in HALF_CASES] +
                         [c + ("half_pair_wide",) for c in HALF_WIDE_CASES],
                         ids=lambda c: "b{}-T{}-H{}-P{}-N{}-G{}-Q{}-gs{}{}".format(*c[:8], "-packed" if c[8] else ""))
def test_half_chunk_kernel(case):
    b, T, H, P, N, G, Q, gs, varlen, kind = case
    d = synth.make_forward_inputs(b, T, H, P, N, G, dtype=torch.bfloat16, seed=3000 + T + N, varlen=varlen)
    sh = ssd.make_shape(d["X"], d["B"], d.get("cu_seqlens"))
    assert ssd.chunk_scan_kernel(sh, Q, gs) == kind
    check_fwd(d, Q, f"half-chunk {kind} {case}", gs=gs)


def test_wide_kernel_mamba2_and_single_head_fallback():
    """N = 256: the eight-wave half-chunk kernel in the Mamba-2 call (gate, skip,
    dt' weights) from initial states, and odd heads per group still on the
    single-head kernel, both against the oracle."""
    from parity import assert_close_gated
    b, T, H, P, N, Q = 2, 500, 4, 64, 256, 128
    m = synth.make_mamba2_inputs(b, T, H, P, N, 1, dtype=torch.bfloat16, seed=3201)
    sh = ssd.make_shape(m["X"], m["B"])
    assert ssd.chunk_scan_kernel(sh, Q, 0) == "half_pair_wide"
    h0 = _init_states(b, H, P, N, 3202)
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in m.items()}
    say(f"[parity] wide half-chunk Mamba-2 call b={b} T={T} H={H} N={N}")
    Y, fin = ssd.fwd_mamba2(dev["X"], dev["dt"], dev["A_log"], dev["B"], dev["C"], dt_bias=dev["dt_bias"],
                            D=dev["D"], z=dev["z"], chunk=Q, initial_state=h0.cuda())
    torch.cuda.synchronize()
    args = (to_f64(m["X"]), to_f64(m["dt"]), to_f64(m["dt_bias"]), to_f64(m["A_log"]), to_f64(m["D"]))
    init = h0.double().numpy()
    Yr, fr = oracle.mamba2_forward(*args, to_f64(m["z"]), to_f64(m["B"]), to_f64(m["C"]), init=init)
    Yu, _ = oracle.mamba2_forward(*args, None, to_f64(m["B"]), to_f64(m["C"]), init=init)
    assert_close_gated(to_f64(Y), Yr, Yu, oracle.silu(to_f64(m["z"])), "bf16", "wide Mamba-2 Y")
    assert_close(to_f64(fin), fr, "bf16", "wide Mamba-2 final")
    d = synth.make_forward_inputs(1, 300, 3, 64, 256, 1, dtype=torch.bfloat16, seed=3203)
    assert ssd.chunk_scan_kernel(ssd.make_shape(d["X"], d["B"]), 128, 0) == "single"
    check_fwd(d, 128, "N = 256, odd heads per group (single-head kernel)")


def test_half_chunk_kernel_initial_state_and_gate():
    """The half-chunk kernel from given initial states, and in the Mamba-2 call
    (gate, skip, key-side dt' weights), against the oracle."""
    b, T, H, P, N, Q, gs = 4, 1100, 64, 64, 128, 128, 2
    d = synth.make_forward_inputs(b, T, H, P, N, 1, dtype=torch.bfloat16, seed=3101)
    sh = ssd.make_shape(d["X"], d["B"])
    assert ssd.chunk_scan_kernel(sh, Q, gs) == "half_pair"
    h0 = _init_states(b, H, P, N, 3102)
    say(f"[parity] half-chunk initial state b={b} T={T} H={H}")
    Y, fin = gpu_fwd(d, Q, gs, initial_state=h0.cuda())
    Yr, fr = oracle.forward(to_f64(d["X"]), to_f64(d["log_a"]), to_f64(d["B"]), to_f64(d["C"]),
                            init=h0.double().numpy())
    assert_close(to_f64(Y), Yr, "bf16", "half-chunk initial state Y")
    assert_close(to_f64(fin), fr, "bf16", "half-chunk initial state final")
    from parity import assert_close_gated, assert_close_rounded
    m = synth.make_mamba2_inputs(b, T, H, P, N, 1, dtype=torch.bfloat16, seed=3103)
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in m.items()}
    say(f"[parity] half-chunk Mamba-2 call b={b} T={T} H={H}")
    Y, fin = ssd.fwd_mamba2(dev["X"], dev["dt"], dev["A_log"], dev["B"], dev["C"], dt_bias=dev["dt_bias"],
                            D=dev["D"], z=dev["z"], chunk=Q, state_block=gs)
    torch.cuda.synchronize()
    args = (to_f64(m["X"]), to_f64(m["dt"]), to_f64(m["dt_bias"]), to_f64(m["A_log"]), to_f64(m["D"]))
    Yr, fr = oracle.mamba2_forward(*args, to_f64(m["z"]), to_f64(m["B"]), to_f64(m["C"]))
    Yu, _ = oracle.mamba2_forward(*args, None, to_f64(m["B"]), to_f64(m["C"]))
    assert_close_gated(to_f64(Y), Yr, Yu, oracle.silu(to_f64(m["z"])), "bf16", "half-chunk Mamba-2 Y")
    # Across 64 heads the final states are heavy-tailed: in heads with fast
    # decay the state is a few recent terms dt'_j x_j B_j^T, up to 25 rms(ref)
    # here, and each term enters the right factor through one bf16 rounding of
    # x_j w_j. A CPU model of exactly that rounding (one rounding per term,
    # chunks of 128, fp32 elsewhere) gives the GPU's errors to 6 digits
    # (max|d|/rms 0.07028, rel-L2 1.68e-3), so these states take the plain bar
    # plus that rounding of the largest elements, 2^-8 |ref_i|.
    assert_close_rounded(to_f64(fin), fr, "bf16", "half-chunk Mamba-2 final state")
