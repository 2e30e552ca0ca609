"""GPU: ssd_fwd_noalloc, the forward pass in the library's static per-GPU
scratch (for callers that cannot allocate), against ssd_fwd with a caller
workspace on the same inputs: two calls in a row, the second with a smaller
input, each equal to ssd_fwd bit for bit (the same kernels, state block and
order of operations) and so within the parity bars of the other tests.
"""
import sys

import pytest
import torch

import ssd_chunked_scan_fwd_amd as ssd
from ssd_chunked_scan_fwd_amd import synth
from parity import assert_close, dtype_name, to_f64

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _one(b, T, H, P, N, Q, dtype, seed, lengths=None):
    if lengths:
        T = sum(lengths)
    d = synth.make_forward_inputs(b, T, H, P, N, 1, dtype=dtype, seed=seed, lengths=lengths)
    X, la, B, C = (d[k].cuda() for k in ("X", "log_a", "B", "C"))
    cu = d["cu_seqlens"].cuda() if d.get("cu_seqlens") is not None else None
    say(f"[noalloc] X{tuple(X.shape)} N={N} Q={Q} {dtype} packed={cu is not None}")
    Yr, fr = ssd.fwd(X, la, B, C, cu_seqlens=cu, chunk=Q)
    nseq = b if cu is None else cu.numel() - 1
    Y = torch.full_like(X, float("nan"))
    fin = torch.full((nseq, H, P, N), float("nan"), dtype=torch.float32, device=X.device)
    ssd.fwd_noalloc(X, la, B, C, Y, fin, cu_seqlens=cu, chunk=Q)
    torch.cuda.synchronize()
    dt = dtype_name(X)
    assert_close(to_f64(Y), to_f64(Yr), dt, "noalloc Y")
    assert_close(to_f64(fin), to_f64(fr), dt, "noalloc final state")
    assert torch.equal(_bits(Y), _bits(Yr)), "Y differs from ssd_fwd's"
    assert torch.equal(_bits(fin), _bits(fr)), "final state differs from ssd_fwd's"


def test_noalloc_twice_second_smaller():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ssd.lib()
    # the headline workload, then a smaller packed call that reuses the same scratch
    _one(1, 16384, 32, 64, 128, 128, torch.bfloat16, seed=2)
    _one(1, 0, 8, 64, 64, 64, torch.bfloat16, seed=7001, lengths=[300, 1, 129, 700, 64, 2000])
