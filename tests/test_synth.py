"""Seeded generators: reproducible, in range, and shaped like the named workloads."""
import numpy as np
import torch

from ssd_chunked_scan_fwd_amd import synth


def test_reproducible_and_seed_sensitive():
    a = synth.make_forward_inputs(2, 64, 3, 16, 32, seed=7)
    b = synth.make_forward_inputs(2, 64, 3, 16, 32, seed=7)
    c = synth.make_forward_inputs(2, 64, 3, 16, 32, seed=8)
    for k in ("X", "log_a", "B", "C"):
        assert torch.equal(a[k], b[k])
        assert not torch.equal(a[k], c[k])


def test_value_ranges():
    d = synth.make_forward_inputs(1, 4096, 8, 64, 128, seed=1)
    la = d["log_a"].double().numpy()
    # log_a = -dt * A with dt in [0.001, 0.1], A in [1, 16]
    assert la.max() <= -0.001 and la.min() >= -1.6
    assert d["log_a"].dtype == torch.float32
    assert d["X"].dtype == torch.bfloat16 and d["B"].dtype == torch.bfloat16
    x = d["X"].float().numpy()
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    b = d["B"].float().numpy()
    assert abs(b.std() * np.sqrt(128) - 1) < 0.02


def test_packed_lengths():
    w = synth.WORKLOADS["packed-T32768-H80-N128"]
    rng = np.random.default_rng(w.seed)
    lengths = synth.draw_lengths(rng, w.T, *w.varlen)
    assert sum(lengths) == w.T
    assert all(512 <= n <= 8192 for n in lengths[:-1])
    assert 1 <= lengths[-1] <= 8192
    # the generator draws the lengths first from the same stream
    d = synth.make_forward_inputs(1, 2048, 2, 16, 16, seed=w.seed, varlen=w.varlen, dtype=torch.float32)
    cu = d["cu_seqlens"].numpy()
    assert cu[0] == 0 and cu[-1] == 2048 and np.all(np.diff(cu) > 0)
    assert d["cu_seqlens"].dtype == torch.int32


def test_workload_shapes():
    w = synth.WORKLOADS[synth.HEADLINE]
    assert (w.batch, w.T, w.H, w.P, w.N, w.G, w.Q) == (1, 16384, 32, 64, 128, 1, 128)
    small = synth.WORKLOADS["tiny-fp32-T256"]
    d = synth.workload_inputs(small)
    assert d["X"].shape == (1, 256, 2, 16) and d["X"].dtype == torch.float32
    assert d["B"].shape == (1, 256, 1, 16) and d["log_a"].shape == (1, 256, 2)


def test_decode_inputs_shape():
    d = synth.make_decode_inputs(4, 10, 3, 16, 32, seed=40)
    assert d["x"].shape == (10, 4, 3, 16)
    assert d["log_a"].shape == (10, 4, 3)
    assert d["B"].shape == (10, 4, 1, 32)
