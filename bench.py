#!/usr/bin/env python3
"""Benchmark of the MI355X chunked SSD forward pass (one GPU).

One step = one ssd_fwd call (chunk_cumsum -> chunk_state -> state_passing ->
chunk_scan) over the long-sequence workload: batch 1, T = 16384 tokens, H = 32
heads, P = 64, N = 128, one B/C group, chunk Q = 128, bf16 inputs with fp32
accumulation; inputs are seeded synthetic and resident in HBM before timing.

Prints ONE JSON line with the headline throughput (tokens/s), the roofline of
the dominant kernel (its algorithmic bytes / its average launch time, timed with
HIP events on the launch stream), per-stage times, the decode-step throughput,
the decode steps replayed from a HIP graph, the Mamba-2 block's call on the
same shape (ssd_fwd_mamba2: raw step sizes, dt_bias, A_log, the D skip and the
silu(z) gate), its backward (ssd_bwd_mamba2) and its decode step, the backward
pass (ssd_bwd) on the same
shape, the forward pass on the other timed workloads (the state-size sweep
b 8, T 4096, N 64/128/256 with its slowdown against N = 64, and the packed
variable-length H = 80 layer), optionally (--with-chain) the state chain as one
cooperative launch, and the fp64 CPU oracle timed on this host as a baseline.

Per-stage times come from each stage's own entry point (the four-launch form
of the stage API); the step itself runs three launches, chunk_state computing
the segment sums itself.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-decode] [--no-mamba2]
                    [--no-bwd] [--no-workloads]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "SSD fwd tokens/s & % of bf16 MFMA peak at T=16K, H=32, P=64, N=128"


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


# Sources each stage's kernel is built from: a counter-based traffic figure is
# reported only while these files are unchanged since the counters were taken.
CSRC = os.path.join(ROOT, "ssd_chunked_scan_fwd_amd", "csrc")
STAGE_SOURCES = {
    "chunk_cumsum": ["ssd_cumsum_passing.hip", "ssd_device.h", "ssd_segsum.h"],
    "state_passing": ["ssd_cumsum_passing.hip", "ssd_device.h"],
    "chunk_state": ["ssd_chunk_state.hip", "ssd_device.h", "ssd_stage.h", "ssd_segsum.h"],
    "chunk_state_fused": ["ssd_chunk_state.hip", "ssd_device.h", "ssd_stage.h", "ssd_segsum.h"],
    "chunk_scan": ["ssd_chunk_scan.hip", "ssd_device.h", "ssd_stage.h"],
    "chunk_scan_gated": ["ssd_chunk_scan.hip", "ssd_device.h", "ssd_stage.h"],
}


def source_digest(stage: str) -> str:
    h = hashlib.sha256()
    for f in STAGE_SOURCES[stage]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(stage: str, workload: str, state_block: int):
    """HBM bytes per launch from the rocprofv3 FETCH_SIZE and WRITE_SIZE passes
    summarised under profiles/ (scaled by the copy-kernel calibration there), or
    None when there is no summary for this kernel, workload and state block or
    the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{stage}_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    fields = dict(re.findall(r"^- (\w+): `([^`]*)`", text, flags=re.M))
    try:
        if fields["source_sha256"] != source_digest(stage) or int(fields["state_block"]) != state_block:
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def stage_bytes(w, nslots: int, nblocks: int, nseq: int) -> dict:
    """Algorithmic HBM bytes of one launch of each stage (each tensor counted once)."""
    esz = 2 if w.dtype == "bf16" else 4
    tok = w.batch * w.T
    X = tok * w.H * w.P * esz
    BC = tok * w.G * w.N * esz
    la = tok * w.H * 4
    cs = nslots * w.H * w.Q * 4
    tables = nslots * 16 + nblocks * 16
    states = nblocks * w.H * w.P * w.N * 4
    starts = nblocks * w.H * w.P * w.N * esz
    final = nseq * w.H * w.P * w.N * 4
    decay = nblocks * w.H * 4
    return {
        "chunk_cumsum": la + cs + tables,
        "chunk_state": X + BC + cs + tables + states + decay,
        "chunk_state_fused": X + BC + la + cs + tables + states + decay,   # writes cs and the tables
        "state_passing": states + decay + starts + final,
        "chunk_scan": X + 2 * BC + cs + tables + starts + X,   # X read, Y written
        # the Mamba-2 call's gated chunk_scan: also z in and the key-side exponents
        "chunk_scan_gated": X + 2 * BC + 2 * cs + tables + starts + X + X,
    }


def useful_flops(w, chunk_lengths) -> float:
    """Useful flops of the forward pass with causal triangles counted exactly.

    Per chunk of q tokens: C B^T lower triangle G*q(q+1)*N, (L o S) X H*q(q+1)*P,
    right and left factors 4*H*q*P*N, centre factor 2*H*P*N.
    """
    f = 0.0
    for q in chunk_lengths:
        f += w.G * q * (q + 1) * w.N + w.H * q * (q + 1) * w.P + 4 * w.H * q * w.P * w.N + 2 * w.H * w.P * w.N
    return f


# The pages' own speed figures, restated: ratios the authors measured on
# hardware and at a precision the pages do not give. Context, not a target.
PAGES_REPORTED = {
    "ssd_vs_mamba1_fused_scan": "2-8x faster than Mamba's fused selective scan at state size 64 "
                                "(paper card TL;DR; paper section 9.3, fig. 10)",
    "ssd_vs_flashattention2": "faster than FlashAttention-2 from sequence length 2K on; about 6x at 16K "
                              "(paper card TL;DR, section 9.3 fig. 10; zh-note speed table)",
    "state_size": "states 8x larger than Mamba's with limited slowdown (zh-note speed table; alex-wiki "
                  "Evidence And Results)",
    "hardware": "unstated",
    "precision": "unstated",
}

# Every forward configuration, in the order of the workload table.
CONFIGS = ["tiny-fp32-T256", "b2-T2048-H24-N64", "long-T16384-H32-N128", "sweep-b8-T4096-N64",
           "sweep-b8-T4096-N128", "sweep-b8-T4096-N256", "packed-T32768-H80-N128"]
FP32_VECTOR_PEAK_TFLOPS = 157.3   # MI355X fp32 vector (the fp32 path runs on FMA, not MFMA)
FLUSH_BYTES = 1 << 30             # written between cold calls: evicts L2 and the 256 MB Infinity Cache


def chunk_lengths_of(w, lengths=None):
    """Chunk lengths of a workload: chunks restart at every sequence start."""
    seqs = list(lengths) if lengths is not None else [w.T] * w.batch
    out = []
    for L in seqs:
        out += [min(w.Q, L - k * w.Q) for k in range(-(-int(L) // w.Q))]
    return out


def compulsory_bytes(w, nseq: int) -> int:
    """X and Y, B and C at the dtype size, log a (fp32) and the final states (fp32)."""
    esz = 2 if w.dtype == "bf16" else 4
    tok = w.batch * w.T
    return tok * w.H * w.P * esz * 2 + tok * w.G * w.N * esz * 2 + tok * w.H * 4 + nseq * w.H * w.P * w.N * 4


def graph_of(torch, fn, n: int = 1):
    """fn() run n times, captured once into a HIP graph (after one eager run on
    a side stream): replays measure GPU time without the host's per-call
    argument checks and launch overhead."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            fn()
    torch.cuda.synchronize()
    return g


def settle_calls(torch, fn, min_calls: int, seconds: float = 0.15):
    """Run fn back to back for at least min_calls calls and `seconds` of wall time."""
    t0, k = time.perf_counter(), 0
    while k < min_calls or time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        k += 8
        torch.cuda.synchronize()


def copy_probe(torch, dev, mib: int) -> None:
    """One elementwise copy (torch.neg, fp32) of `mib` MiB in and out: the known
    bytes that scale the FETCH_SIZE / WRITE_SIZE counters of a profiled run."""
    if mib > 0:
        src = torch.ones(mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()


def timed_calls(torch, stream, fn, n, before=None):
    """Per-call durations (us) of n calls of fn, each between its own HIP events on
    `stream`; `before(i)` runs untimed ahead of call i."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        if before is not None:
            before(i)
        ev[i][0].record(stream)
        fn()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 for a, b in ev]


def median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def oracle_sample(oracle, w, d, budget_s: float):
    """The fp64 oracle on a bounded sample of a workload: the first k heads (k
    doubled until the time budget is used or all heads are in), run back to
    back; tokens/s scaled to all H heads."""
    X, la, B, C = (d[k].double().numpy() for k in ("X", "log_a", "B", "C"))
    cu = d.get("cu_seqlens")
    cu = None if cu is None else cu.numpy()
    nseq = w.batch if cu is None else len(cu) - 1
    cores = len(os.sched_getaffinity(0))
    k, best = 1, None
    while True:
        th = max(1, min(cores, nseq * k))
        runs, t0 = 0, time.perf_counter()
        while True:
            oracle.scan(X[:, :, :k], la[:, :, :k], B, C, segments=oracle.sequence_segments(w.batch, w.T, cu),
                        threads=th)
            runs += 1
            el = time.perf_counter() - t0
            if el >= budget_s / 4 or runs >= 50:
                break
        best = (k, th, runs, el)
        if k >= w.H or el * 2 > budget_s:
            break
        k = min(w.H, 2 * k)
    k, th, runs, el = best
    tok = w.batch * w.T
    return {"tokens_per_s": round(tok * runs / el * k / w.H, 1), "cores": th,
            "sample": f"{k} of {w.H} heads, {runs} run(s) in {el:.2f} s, scaled to {w.H} heads"}


def measure_config(ctx, name, steps, warmup, cpu_budget):
    """Forward pass of one workload: per-call HIP-event times of the call replayed
    from a HIP graph, warm (back to back) and cold (1 GB written before each
    call), the mean of direct calls back to back, rates, roofline fractions, and
    the oracle on a bounded sample of it."""
    torch, ssd, synth, dev, stream, flush = ctx["torch"], ctx["ssd"], ctx["synth"], ctx["dev"], ctx["stream"], \
        ctx["flush"]
    w = synth.WORKLOADS[name]
    d = synth.workload_inputs(w)
    X, la, B, C = (d[k].to(dev) for k in ("X", "log_a", "B", "C"))
    cu = d["cu_seqlens"].to(dev) if d.get("cu_seqlens") is not None else None
    lengths = None if cu is None else [int(v) for v in (d["cu_seqlens"][1:] - d["cu_seqlens"][:-1])]
    nseq = w.batch if cu is None else cu.numel() - 1
    sh = ssd.make_shape(X, B, cu)
    ws = ssd.Workspace(sh, w.Q, dev)
    Y = torch.empty_like(X)
    fin = torch.empty(nseq, w.H, w.P, w.N, dtype=torch.float32, device=dev)

    def step():
        ssd.fwd(X, la, B, C, cu_seqlens=cu, chunk=w.Q, state_block=ws.state_block, Y=Y, final_state=fin,
                workspace=ws)

    # Warm-up by sustained work: the GPU clock settles only after some tens of
    # milliseconds under load (fewer warm-up calls read slower steps).
    settle_calls(torch, step, warmup)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    b2b = a.elapsed_time(b) * 1e3 / steps
    g = graph_of(torch, step)
    settle_calls(torch, g.replay, warmup)
    warm = timed_calls(torch, stream, g.replay, steps)
    cold = timed_calls(torch, stream, g.replay, steps, before=lambda i: flush.fill_(i % 251))
    del g
    tok = w.batch * w.T
    flops = useful_flops(w, chunk_lengths_of(w, lengths))
    comp = compulsory_bytes(w, nseq)
    sb = stage_bytes(w, ws.layout.nslots, ws.layout.nblocks, nseq)
    pipe = sb["chunk_state_fused"] + sb["state_passing"] + sb["chunk_scan"]
    peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_VECTOR_PEAK_TFLOPS
    r = {"dtype": w.dtype, "batch": w.batch, "T": w.T, "H": w.H, "P": w.P, "N": w.N, "G": w.G, "chunk": w.Q,
         "num_seqs": nseq if cu is not None else 0, "state_block": ws.state_block, "steps": steps}
    for tag, us in (("warm", median(warm)), ("cold", median(cold))):
        r[f"{tag}_us_median"] = round(us, 2)
        r[f"{tag}_tokens_per_s"] = round(tok / (us * 1e-6), 1)
        r[f"{tag}_useful_tflops"] = round(flops / (us * 1e-6) / 1e12, 2)
        r[f"{tag}_{'mfma' if w.dtype == 'bf16' else 'fp32_vector'}_frac"] = round(flops / (us * 1e-6) / 1e12 / peak, 5)
        r[f"{tag}_compulsory_hbm_frac"] = round(comp / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
        r[f"{tag}_pipeline_hbm_frac"] = round(pipe / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    r["back_to_back_us_mean"] = round(b2b, 2)
    r["useful_gflop"] = round(flops / 1e9, 4)
    r["compulsory_mb"] = round(comp / 1e6, 2)
    r["pipeline_mb"] = round(pipe / 1e6, 2)
    if cpu_budget > 0:
        from oracle import oracle
        o = oracle_sample(oracle, w, d, cpu_budget)
        r["oracle"] = o
        r["gpu_warm_vs_oracle"] = round(r["warm_tokens_per_s"] / o["tokens_per_s"], 1)
    del X, la, B, C, cu, ws, Y, fin
    return r


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=200, help="untimed steps; the GPU clock settles under load")
    ap.add_argument("--stage-reps", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-mamba2", action="store_true", help="skip the Mamba-2 block-call timing")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward-pass timing")
    ap.add_argument("--with-chain", action="store_true",
                    help="also time the state chain as one cooperative launch (rocprofv3 cannot trace it)")
    ap.add_argument("--bwd-steps", type=int, default=100)
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the per-config forward timing (every workload, warm and cold)")
    ap.add_argument("--wl-steps", type=int, default=50, help="timed calls per config, warm and cold each")
    ap.add_argument("--wl-cpu-seconds", type=float, default=2.0,
                    help="oracle time budget per config (bounded head sample); 0 skips it")
    ap.add_argument("--profile-config", default="", metavar="NAME",
                    help="run only NAME's forward pass (warm-up, then --wl-steps calls) and print a short JSON "
                         "line: the command the per-config rocprofv3 traces are taken with")
    ap.add_argument("--profile-decode", action="store_true",
                    help="run only the decode steps (and --copy-probe): the command of the decode counter passes")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum wall time of the oracle baseline")
    ap.add_argument("--decode-steps", type=int, default=4096)
    ap.add_argument("--state-block", type=int, default=0, help="chunks per state block (0: library default)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="after the run, launch one elementwise copy of MIB MiB (read MIB, write MIB): the "
                         "calibration kernel of the FETCH_SIZE / WRITE_SIZE counter passes")
    ap.add_argument("--no-graph", action="store_true",
                    help="time stages by back-to-back eager launches and skip graph replays (counter passes)")
    ap.add_argument("--print-digest", action="store_true", help="print the source digest of each stage and exit")
    args = ap.parse_args()

    if args.print_digest:
        for st in STAGE_SOURCES:
            print(st, source_digest(st))
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the SSD forward path has no multi-GPU mode "
              "(run with --gpus 1).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import ssd_chunked_scan_fwd_amd as ssd
    from ssd_chunked_scan_fwd_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    ssd.lib()  # fail loudly when the HIP library is missing
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    ctx = {"torch": torch, "ssd": ssd, "synth": synth, "dev": dev, "stream": torch.cuda.current_stream(dev),
           "flush": flush}

    if args.profile_decode:
        wd = synth.WORKLOADS["decode-b64-H80-N128"]
        n = min(args.decode_steps, 64)
        log(f"[bench] profile run: {n} decode steps of {wd.name}")
        dd = synth.make_decode_inputs(wd.batch, n, wd.H, wd.P, wd.N, wd.G, wd.torch_dtype, wd.seed)
        xs, las, Bs, Cs = (dd[k].to(dev) for k in ("x", "log_a", "B", "C"))
        state = torch.zeros(wd.batch, wd.H, wd.P, wd.N, dtype=torch.float32, device=dev)
        y = torch.empty(wd.batch, wd.H, wd.P, dtype=xs.dtype, device=dev)
        for t in range(n):
            ssd.step(state, xs[t], las[t], Bs[t], Cs[t], y=y)
        torch.cuda.synchronize()
        copy_probe(torch, dev, args.copy_probe)
        print(json.dumps({"profile_decode": wd.name, "steps": n}), flush=True)
        return 0

    if args.profile_config:
        log(f"[bench] profile run: forward on {args.profile_config}")
        r = measure_config(ctx, args.profile_config, args.wl_steps, 10, 0.0)
        copy_probe(torch, dev, args.copy_probe)
        print(json.dumps({"profile_config": args.profile_config, "result": r}), flush=True)
        return 0

    w = synth.WORKLOADS[synth.HEADLINE]
    log(f"[bench] workload {w.name}: generating inputs")
    d = synth.workload_inputs(w)
    X, la, B, C = (d[k].to(dev) for k in ("X", "log_a", "B", "C"))
    shape = ssd.make_shape(X, B, None)
    ws = ssd.Workspace(shape, w.Q, dev, args.state_block)
    Y = torch.empty_like(X)
    fin = torch.empty(w.batch, w.H, w.P, w.N, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        ssd.fwd(X, la, B, C, chunk=w.Q, state_block=ws.state_block, Y=Y, final_state=fin, workspace=ws)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3 / args.steps
    ev_ms = e0.elapsed_time(e1) / args.steps
    # the same step replayed from a HIP graph (GPU time without host overhead)
    graph_ms = ev_ms
    if not args.no_graph:
        gstep = graph_of(torch, step, 10)
        for _ in range(5):
            gstep.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(max(1, args.steps // 10)):
            gstep.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        graph_ms = e0.elapsed_time(e1) / (max(1, args.steps // 10) * 10)
        del gstep
    ms_per_step = wall_ms
    tokens = w.batch * w.T
    value = tokens / (ms_per_step * 1e-3)

    # per-stage average launch time: HIP events on the launch stream around
    # graph replays of the stage's own entry point
    log(f"[bench] per-stage timing, {args.stage_reps} launches each")
    stages = [
        ("chunk_cumsum", lambda: ssd.chunk_cumsum(la, None, shape, ws)),
        ("chunk_state", lambda: ssd.chunk_state(X, B, None, shape, ws)),
        ("state_passing", lambda: ssd.state_passing(None, fin, shape, ws)),
        ("chunk_scan", lambda: ssd.chunk_scan(X, B, C, None, Y, shape, ws)),
    ]
    # Each stage's launches captured in a HIP graph (20 per graph) and replayed,
    # so the figure is GPU time rather than the host's per-call overhead.
    acc = {}
    per_graph = 20
    reps = max(1, args.stage_reps // per_graph)
    for name, fn in stages:
        if args.no_graph:
            for _ in range(min(20, args.stage_reps)):
                fn()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(args.stage_reps):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            acc[name] = a.elapsed_time(b) / max(args.stage_reps, 1)
            continue
        g = graph_of(torch, fn, per_graph)
        for _ in range(2):
            g.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        acc[name] = a.elapsed_time(b) / (reps * per_graph)
        del g
    stage_us = {k: v * 1e3 for k, v in acc.items()}
    sbytes = stage_bytes(w, ws.layout.nslots, ws.layout.nblocks, w.batch)
    dominant = max(stage_us, key=stage_us.get)
    # The step runs three launches: chunk_state in its fused form (segment sums
    # computed in the kernel), state_passing, chunk_scan. The fused kernel has no
    # entry point of its own; its time is the step's event time less the other two.
    fused_us = graph_ms * 1e3 - stage_us["state_passing"] - stage_us["chunk_scan"]
    achieved = sbytes[dominant] / (stage_us[dominant] * 1e-6) / 1e9
    chunk_lengths = [min(w.Q, w.T - k * w.Q) for k in range(-(-w.T // w.Q))] * w.batch
    flops = useful_flops(w, chunk_lengths)
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    compulsory = (tokens * w.H * w.P * 2 * 2 + tokens * w.G * w.N * 2 * 2 + tokens * w.H * 4 +
                  w.batch * w.H * w.P * w.N * 4)
    pipeline_bytes = sbytes["chunk_state_fused"] + sbytes["state_passing"] + sbytes["chunk_scan"]   # the step's launches

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded: X~N(0,1), log_a=-dt*A, dt~U(0.001,0.1), A~U(1,16), B,C~N(0,1)/sqrt(N))",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.T, "heads": w.H, "headdim": w.P,
                   "dstate": w.N, "ngroups": w.G, "chunk": w.Q, "state_block": ws.state_block,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(dominant, w.name, ws.state_block),
                     "bytes_per_launch": sbytes[dominant], "avg_launch_us": round(stage_us[dominant], 3)},
        "launches_per_step": ["chunk_state (fused with the segment sums)", "state_passing", "chunk_scan"],
        "stages_us": {k: round(v, 3) for k, v in stage_us.items()},
        "chunk_state_fused_us_derived": round(fused_us, 3),
        "stage_bytes": sbytes,
        "stage_gbs": {k: round(sbytes[k] / (stage_us[k] * 1e-6) / 1e9, 1) for k in stage_us},
        "event_ms_per_step": round(ev_ms, 5),
        "graph_ms_per_step": round(graph_ms, 5),
        "useful_tflops": round(tflops, 2),
        "mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 5),
        "compulsory_bytes": compulsory,
        "compulsory_hbm_frac": round(compulsory / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "pipeline_bytes": pipeline_bytes,
        "pipeline_hbm_frac": round(pipeline_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "pages_reported": PAGES_REPORTED,
    }

    if not args.no_mamba2:
        # The Mamba-2 block's call on the same shape: raw step sizes, dt_bias,
        # A_log, the D skip and the silu(z) gate, all inside the four kernels.
        log(f"[bench] mamba2 block call on {w.name}: {args.steps} steps")
        m = synth.make_mamba2_inputs(w.batch, w.T, w.H, w.P, w.N, w.G, w.torch_dtype, w.seed)
        mX, mdt, mbias, mAl, mD, mz, mB, mC = (m[k].to(dev) for k in ("X", "dt", "dt_bias", "A_log", "D", "z", "B",
                                                                      "C"))

        def mstep():
            ssd.fwd_mamba2(mX, mdt, mAl, mB, mC, dt_bias=mbias, D=mD, z=mz, chunk=w.Q, state_block=ws.state_block,
                           Y=Y, final_state=fin, workspace=ws)

        for _ in range(min(args.warmup, 50)):
            mstep()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        a.record(stream)
        for _ in range(args.steps):
            mstep()
        b.record(stream)
        torch.cuda.synchronize()
        m_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        out["mamba2"] = {"workload": w.name + " (Mamba-2 call: dt, dt_bias, A_log, D, z)", "steps": args.steps,
                         "ms_per_step": round(m_ms, 5), "event_ms_per_step": round(a.elapsed_time(b) / args.steps, 5),
                         "tokens_per_s": round(tokens / (m_ms * 1e-3), 1)}
        if not args.no_bwd:
            # its backward (ssd_bwd_mamba2): every input's gradient from dY
            ctm = synth.make_cotangents(w.batch, w.T, w.H, w.P, w.N, w.batch, w.torch_dtype, w.seed + 2)
            mdY = ctm["dY"].to(dev)
            mws = torch.empty(ssd.bwd_mamba2_workspace_bytes(shape, w.Q, ws.state_block), dtype=torch.uint8,
                              device=dev)

            def mbstep():
                return ssd.bwd_mamba2(mX, mdt, mAl, mB, mC, mdY, dt_bias=mbias, D=mD, z=mz, chunk=w.Q,
                                      state_block=ws.state_block, workspace=mws)

            nb = max(1, min(args.bwd_steps, args.steps))
            for _ in range(min(args.warmup, 10)):
                mbstep()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(nb):
                mbstep()
            torch.cuda.synchronize()
            out["mamba2"]["bwd_ms_per_step"] = round((time.perf_counter() - t0) * 1e3 / nb, 5)
            del mdY, mws
        del mX, mdt, mbias, mAl, mD, mz, mB, mC

    if args.with_chain:
        # The state chain as one cooperative launch (ssd_set_state_chain(1)),
        # against the default two launches: the same step, timed the same way.
        prev = ssd.set_state_chain(1)
        for _ in range(min(args.warmup, 50)):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        c_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        ssd.set_state_chain(prev)
        out["state_chain_cooperative"] = {"ms_per_step": round(c_ms, 5),
                                          "note": "chunk_state and state_passing as one cooperative launch; "
                                                  "not the default (slower on this stack)"}

    if not args.no_bwd:
        # The backward pass (ssd_bwd) on the same shape: dX, d log a, dB, dC
        # and the initial-state gradient from dY and a final-state cotangent.
        nb = max(1, min(args.bwd_steps, args.steps))
        log(f"[bench] backward pass on {w.name}: {nb} steps")
        ct = synth.make_cotangents(w.batch, w.T, w.H, w.P, w.N, w.batch, w.torch_dtype, w.seed + 1)
        dY, dfin = ct["dY"].to(dev), ct["dfinal"].to(dev)
        bws = torch.empty(ssd.bwd_workspace_bytes(shape, w.Q, ws.state_block),
                          dtype=torch.uint8, device=dev)

        def bstep():
            return ssd.bwd(X, la, B, C, dY, chunk=w.Q, state_block=ws.state_block, dfinal_state=dfin,
                           want_dinit=True, workspace=bws)

        for _ in range(min(args.warmup, 20)):
            bstep()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        a.record(stream)
        for _ in range(nb):
            bstep()
        b.record(stream)
        torch.cuda.synchronize()
        b_ms = (time.perf_counter() - t0) * 1e3 / nb
        out["bwd"] = {"workload": w.name + " (backward: dX, dlog_a, dB, dC, dinit)", "steps": nb,
                      "ms_per_step": round(b_ms, 5), "event_ms_per_step": round(a.elapsed_time(b) / nb, 5),
                      "tokens_per_s": round(tokens / (b_ms * 1e-3), 1),
                      "vs_forward": round(b_ms / ms_per_step, 3)}
        del dY, dfin, bws

    if not args.no_decode:
        wd = synth.WORKLOADS["decode-b64-H80-N128"]
        nsteps = min(args.decode_steps, wd.steps)
        log(f"[bench] decode {wd.name}: {nsteps} steps")
        dd = synth.make_decode_inputs(wd.batch, nsteps, wd.H, wd.P, wd.N, wd.G, wd.torch_dtype, wd.seed)
        xs, las, Bs, Cs = (dd[k].to(dev) for k in ("x", "log_a", "B", "C"))
        state = torch.zeros(wd.batch, wd.H, wd.P, wd.N, dtype=torch.float32, device=dev)
        y = torch.empty(wd.batch, wd.H, wd.P, dtype=xs.dtype, device=dev)
        for t in range(min(16, nsteps)):
            ssd.step(state, xs[t], las[t], Bs[t], Cs[t], y=y)
        state.zero_()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for t in range(nsteps):
            ssd.step(state, xs[t], las[t], Bs[t], Cs[t], y=y)
        b.record(stream)
        torch.cuda.synchronize()
        dec_ms = a.elapsed_time(b)
        per_step_bytes = wd.batch * wd.H * wd.P * wd.N * 4 * 2 + wd.batch * wd.H * (wd.P * 2 * 2 + 4) + \
            wd.batch * wd.G * wd.N * 2 * 2
        out["decode"] = {"workload": wd.name, "steps": nsteps, "ms": round(dec_ms, 3),
                         "tokens_per_s": round(wd.batch * nsteps / (dec_ms * 1e-3), 1),
                         "us_per_step": round(dec_ms * 1e3 / nsteps, 3),
                         "gbs_per_step": round(per_step_bytes / (dec_ms * 1e-3 / nsteps) / 1e9, 1)}
        # The same steps from a HIP graph: 64 consecutive steps captured once and
        # replayed back to back (the inputs of steps 0..63 on every replay).
        glen = min(64, nsteps)
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for t in range(glen):
                ssd.step(state, xs[t], las[t], Bs[t], Cs[t], y=y)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, capture_error_mode="relaxed"):
            for t in range(glen):
                ssd.step(state, xs[t], las[t], Bs[t], Cs[t], y=y)
        reps = max(1, nsteps // glen)
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(reps):
            graph.replay()
        b.record(stream)
        torch.cuda.synchronize()
        out["decode"]["graph_us_per_step"] = round(a.elapsed_time(b) * 1e3 / (reps * glen), 3)
        del graph
        # Cold steps: 1 GB written before each, so the 168 MB state comes from
        # HBM and not from the Infinity Cache; a cold step as fast as a warm one
        # means the warm rate is HBM traffic.
        ncold = min(50, nsteps)
        cold = []
        for t in range(ncold):
            flush.fill_(t % 251)
            e0c, e1c = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0c.record(stream)
            ssd.step(state, xs[t], las[t], Bs[t], Cs[t], y=y)
            e1c.record(stream)
            torch.cuda.synchronize()
            cold.append(e0c.elapsed_time(e1c) * 1e3)
        out["decode"]["cold_us_per_step_median"] = round(median(cold), 3)
        out["decode"]["cold_gbs_per_step"] = round(per_step_bytes / (median(cold) * 1e-6) / 1e9, 1)
        # The cold step is the HBM figure: a model's per-layer decode states
        # together exceed the Infinity Cache.
        out["decode"]["cold_hbm_frac"] = round(per_step_bytes / (median(cold) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
        del xs, las, Bs, Cs
        if not args.no_mamba2:
            md = synth.make_mamba2_decode_inputs(wd.batch, nsteps, wd.H, wd.P, wd.N, wd.G, wd.torch_dtype, wd.seed)
            xs, dts, zs, Bs, Cs = (md[k].to(dev) for k in ("x", "dt", "z", "B", "C"))
            bias, Al, Dk = (md[k].to(dev) for k in ("dt_bias", "A_log", "D"))
            state.zero_()
            for t in range(min(16, nsteps)):
                ssd.step_mamba2(state, xs[t], dts[t], Al, Bs[t], Cs[t], dt_bias=bias, D=Dk, z=zs[t], y=y)
            torch.cuda.synchronize()
            a.record(stream)
            for t in range(nsteps):
                ssd.step_mamba2(state, xs[t], dts[t], Al, Bs[t], Cs[t], dt_bias=bias, D=Dk, z=zs[t], y=y)
            b.record(stream)
            torch.cuda.synchronize()
            m_ms = a.elapsed_time(b)
            out["decode"]["mamba2_us_per_step"] = round(m_ms * 1e3 / nsteps, 3)
            del xs, dts, zs, Bs, Cs
        del state

    if not args.no_workloads:
        # Every forward configuration, warm and cold, with its oracle sample.
        res = {}
        for name in CONFIGS:
            log(f"[bench] config {name}: {args.wl_steps} warm + {args.wl_steps} cold calls")
            res[name] = measure_config(ctx, name, args.wl_steps, 10,
                                       0.0 if args.no_cpu_baseline else args.wl_cpu_seconds)
        base = res["sweep-b8-T4096-N64"]["warm_us_median"]
        for name in ("sweep-b8-T4096-N64", "sweep-b8-T4096-N128", "sweep-b8-T4096-N256"):
            res[name]["slowdown_vs_N64"] = round(res[name]["warm_us_median"] / base, 3)
        out["configs"] = res
        hl = res.get(w.name)
        if hl:
            out["cold_ms_per_step"] = round(hl["cold_us_median"] * 1e-3, 5)
            out["cold_tokens_per_s"] = hl["cold_tokens_per_s"]

    if args.copy_probe > 0:
        n = args.copy_probe * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: {args.copy_probe} MiB read + {args.copy_probe} MiB written (torch.neg)")
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    if not args.no_cpu_baseline:
        from oracle import oracle
        cores = len(os.sched_getaffinity(0))
        threads = min(cores, w.batch * w.H)
        log(f"[bench] cpu baseline: fp64 oracle over the whole workload, {threads} threads, repeated for "
            f">= {args.cpu_seconds:.0f} s")
        Xd, lad, Bd, Cd = (d[k].double().numpy() for k in ("X", "log_a", "B", "C"))
        runs, c0 = 0, time.perf_counter()
        while True:
            oracle.scan(Xd, lad, Bd, Cd, threads=threads)
            runs += 1
            if time.perf_counter() - c0 >= args.cpu_seconds:
                break
        secs = time.perf_counter() - c0
        out["cpu_baseline"] = {"value": round(tokens * runs / secs, 1), "unit": "tokens/s", "cores": threads,
                               "kind": "oracle",
                               "sample": f"the whole {w.name} workload ({tokens} tokens x {w.H} heads) run "
                                         f"{runs} times back to back, {secs:.1f} s in all; fp64 token-by-token "
                                         f"recurrence, OpenMP over (row, head) pairs"}

    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
