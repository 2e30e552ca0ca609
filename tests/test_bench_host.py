"""CPU: the host-side arithmetic of bench.py (no GPU).

The roofline figure is algorithmic bytes over launch time, so the byte and flop
counts are checked here against counts made another way: the bytes of each
stage tensor by tensor for the long-sequence workload (T = 16384, H = 32,
P = 64, N = 128, Q = 128, state blocks of 8 chunks), the flop formula against a
direct count of the multiply-adds of the chunked form on small chunks, the
counter-traffic lookup against a summary written here, and the one-GPU rule.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from ssd_chunked_scan_fwd_amd import synth  # noqa: E402


def test_stage_bytes_long_sequence():
    w = synth.WORKLOADS["long-T16384-H32-N128"]
    nslots, nblocks = 16384 // 128, 16384 // (128 * 8)
    sb = bench.stage_bytes(w, nslots, nblocks, 1)
    X = 16384 * 32 * 64 * 2           # bf16 [T, H, P]; Y has the same size
    BC = 16384 * 1 * 128 * 2          # bf16 [T, G, N], each of B and C
    la = 16384 * 32 * 4               # fp32 [T, H]
    cs = nslots * 32 * 128 * 4        # fp32 [slots, H, Q]
    tables = nslots * 16 + nblocks * 16
    states = nblocks * 32 * 64 * 128 * 4
    starts = nblocks * 32 * 64 * 128 * 2
    final = 32 * 64 * 128 * 4
    decay = nblocks * 32 * 4
    assert sb["chunk_scan"] == 2 * X + 2 * BC + cs + tables + starts == 153094400
    assert sb["chunk_state"] == X + BC + cs + tables + states + decay
    assert sb["chunk_state_fused"] == sb["chunk_state"] + la
    assert sb["state_passing"] == states + decay + starts + final
    assert sb["chunk_cumsum"] == la + cs + tables
    assert sb["chunk_scan_gated"] == sb["chunk_scan"] + cs + X   # the key-side exponents and z


def _count_chunk_flops(q, H, G, P, N):
    """Multiply-adds of one chunk of q tokens counted term by term (2 flops each):
    C B^T on the causal triangle per group, (L o S) X on the triangle per head,
    the right and left factors per head, and the centre-factor update per head."""
    tri = sum(i + 1 for i in range(q))          # pairs (i, j) with j <= i
    macs = G * tri * N                           # S_ij = C_i . B_j
    macs += H * tri * P                          # Y_i += (L o S)_ij X_j
    macs += H * q * P * N                        # right factor sum_j x_j B_j^T
    macs += H * q * P * N                        # left factor C_i h^T
    macs += H * P * N                            # centre factor a h + s
    return 2 * macs


@pytest.mark.parametrize("q,H,G,P,N", [(1, 1, 1, 1, 1), (5, 2, 1, 3, 4), (16, 4, 2, 8, 8)])
def test_useful_flops_counts_the_chunked_form(q, H, G, P, N):
    w = synth.Workload("t", "bf16", 1, q, H, P, N, G, q, seed=0)
    assert bench.useful_flops(w, [q]) == _count_chunk_flops(q, H, G, P, N)
    assert bench.useful_flops(w, [q, q, 3]) == 2 * _count_chunk_flops(q, H, G, P, N) + _count_chunk_flops(3, H, G, P, N)


def test_measured_traffic_follows_the_source_digest(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("chunk_scan", "wl", 8) is None          # no summary
    text = ("# summary\n- traffic_bytes_per_launch: `123456`\n- state_block: `8`\n"
            f"- source_sha256: `{bench.source_digest('chunk_scan')}`\n")
    (prof / "chunk_scan_wl_hbm_traffic.md").write_text(text)
    assert bench.measured_traffic("chunk_scan", "wl", 8) == 123456
    assert bench.measured_traffic("chunk_scan", "wl", 4) is None          # other state block
    (prof / "chunk_scan_wl_hbm_traffic.md").write_text(text.replace(bench.source_digest("chunk_scan"), "0" * 64))
    assert bench.measured_traffic("chunk_scan", "wl", 8) is None          # sources changed since


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_config_helpers():
    from ssd_chunked_scan_fwd_amd import synth
    w = synth.WORKLOADS["long-T16384-H32-N128"]
    # compulsory bytes at the headline: X and Y (bf16), B and C (bf16), log a and the final state (fp32)
    assert bench.compulsory_bytes(w, 1) == 145_752_064
    assert bench.chunk_lengths_of(w) == [128] * 128
    p = synth.WORKLOADS["packed-T32768-H80-N128"]
    lens = [700, 1, 129, 31938]
    cl = bench.chunk_lengths_of(p, lens)
    assert sum(cl) == sum(lens) and cl[:8] == [128] * 5 + [60, 1, 128] and max(cl) <= 128
    assert bench.median([3, 1, 2]) == 2 and bench.median([4, 1, 3, 2]) == 2.5
    assert set(bench.CONFIGS) == {k for k, v in synth.WORKLOADS.items() if not v.steps}
    assert bench.PAGES_REPORTED["hardware"] == "unstated"
