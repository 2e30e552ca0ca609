"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, sizes its workspace, and rejects bad arguments on the host
before any HIP call (each case below fails validation, so nothing is launched).
"""
import ctypes
import os
import re
import subprocess

import pytest

import ssd_chunked_scan_fwd_amd as ssd
from ssd_chunked_scan_fwd_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")

OK, INVALID, UNSUPPORTED, WS_SMALL = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(ssd_[a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_declares_binding_exports():
    assert declared_functions() == sorted(binding.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = ssd.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", binding.library_path()], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\sT\s(ssd_[a-z_0-9]+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported


def test_abi_version_and_status_strings():
    L = ssd.lib()
    assert L.ssd_abi_version() == 6
    for code, name in binding.STATUS.items():
        assert L.ssd_status_string(code).decode() == name


def shape(**kw):
    base = dict(batch=1, seqlen=16384, nheads=32, ngroups=1, headdim=64, dstate=128, num_seqs=0, dtype=1)
    base.update(kw)
    return binding.Shape(*[base[k] for k in ("batch", "seqlen", "nheads", "ngroups", "headdim", "dstate",
                                              "num_seqs", "dtype")])


def ws_bytes(sh, chunk, gs=1):
    n = ctypes.c_size_t(0)
    st = ssd.lib().ssd_fwd_workspace_bytes(ctypes.byref(sh), chunk, gs, ctypes.byref(n))
    return st, n.value


def _align(v):
    return (v + 255) // 256 * 256


def test_workspace_size_matches_layout():
    sh = shape()
    st, n = ws_bytes(sh, 128, 1)
    assert st == OK
    slots = 16384 // 128
    PN = 64 * 128
    expect = _align(slots * 16) * 2 + _align(slots * 32 * 128 * 4) * 2 + _align(slots * 32 * 4) + \
        _align(slots * 32 * PN * 4) + _align(slots * 32 * PN * 2)
    assert n == expect
    L = ssd.layout(sh, 128, 1)
    assert L.slots_per_row == slots and L.nslots == slots and L.nblocks == slots and L.total_bytes == n
    # the key-side exponent (Mamba-2 calls) follows cumsum, same size
    assert L.key_cumsum_offset - L.cumsum_offset == _align(slots * 32 * 128 * 4)
    assert L.block_decay_offset - L.key_cumsum_offset == _align(slots * 32 * 128 * 4)
    # state blocks of 4 chunks: a quarter of the block arrays
    L4 = ssd.layout(sh, 128, 4)
    assert L4.nslots == slots and L4.nblocks == slots // 4
    assert L4.total_bytes == _align(slots * 16) + _align(slots // 4 * 16) + _align(slots * 32 * 128 * 4) * 2 + \
        _align(slots // 4 * 32 * 4) + _align(slots // 4 * 32 * PN * 4) + _align(slots // 4 * 32 * PN * 2)
    # packed rows: floor(T/Q) + S chunk slots, floor(T/(Gs*Q)) + S block slots
    sp = shape(seqlen=32768, nheads=80, num_seqs=7)
    Lp = ssd.layout(sp, 128, 8)
    assert Lp.slots_per_row == 32768 // 128 + 7 and Lp.blocks_per_row == 32768 // 1024 + 7
    # ragged T: ceil(T/Q) chunk slots and ceil(slots/Gs) block slots per row
    Lr = ssd.layout(shape(batch=3, seqlen=1000), 64, 4)
    assert Lr.slots_per_row == 16 and Lr.nslots == 48 and Lr.blocks_per_row == 4 and Lr.nblocks == 12
    # fp32 start states are 4 bytes
    L32 = ssd.layout(shape(dtype=0, seqlen=256, nheads=2, headdim=16, dstate=16), 32, 1)
    assert L32.total_bytes - L32.start_states_offset == _align(8 * 2 * 16 * 16 * 4)


def test_default_state_block():
    L = ssd.lib()
    assert L.ssd_default_state_block(ctypes.byref(shape(dtype=0, seqlen=4096)), 64) == 1
    gs = L.ssd_default_state_block(ctypes.byref(shape()), 128)
    assert gs in (1, 2, 4, 8, 16)
    assert ssd.layout(shape(), 128, 0).nblocks == 128 // gs
    # small problems keep one chunk per state block
    assert L.ssd_default_state_block(ctypes.byref(shape(seqlen=256, nheads=2)), 128) == 1
    # the measured choices: b 2, T 2048, H 24, N 64, chunk 64 -> 4; the headline -> 8;
    # the N = 256 sweep (64 KB states) -> 16; the packed H = 80 layer -> 8
    d = lambda sh, q: L.ssd_default_state_block(ctypes.byref(sh), q)
    assert d(shape(batch=2, seqlen=2048, nheads=24, dstate=64), 64) == 4
    assert d(shape(), 128) == 8
    assert d(shape(batch=8, seqlen=4096, dstate=256), 128) == 16
    assert d(shape(batch=8, seqlen=4096, dstate=128), 128) == 8
    assert d(shape(seqlen=32768, nheads=80, num_seqs=5), 128) == 8


@pytest.mark.parametrize("kw,gs,code", [(dict(), 3, UNSUPPORTED), (dict(), 32, UNSUPPORTED),
                                         (dict(dtype=0, dstate=64), 2, UNSUPPORTED), (dict(), 16, OK)])
def test_state_block_rules(kw, gs, code):
    st, _ = ws_bytes(shape(**kw), 128, gs)
    assert st == code


@pytest.mark.parametrize("kw,chunk,code", [
    (dict(seqlen=0), 128, INVALID),
    (dict(batch=0), 128, INVALID),
    (dict(nheads=6, ngroups=4), 128, INVALID),
    (dict(headdim=0), 128, INVALID),
    (dict(), 0, INVALID),
    (dict(num_seqs=3), 128, INVALID),           # num_seqs without cu_seqlens (checked in ssd_fwd below)
    (dict(headdim=48), 128, UNSUPPORTED),
    (dict(headdim=256), 128, UNSUPPORTED),
    (dict(dstate=512), 128, UNSUPPORTED),
    (dict(dstate=16), 128, UNSUPPORTED),        # bf16 needs dstate >= 32
    (dict(), 16, UNSUPPORTED),                  # bf16 needs chunk >= 32
    (dict(), 96, UNSUPPORTED),
    (dict(), 512, UNSUPPORTED),
    (dict(dtype=7), 128, UNSUPPORTED),
    (dict(headdim=128, dstate=256), 256, UNSUPPORTED),  # tiles exceed the 160 KiB LDS
    (dict(batch=70000, seqlen=16, nheads=1), 32, UNSUPPORTED),
    (dict(seqlen=1 << 20, nheads=64, headdim=64), 128, UNSUPPORTED),  # more than 2^31 elements
])
def test_fwd_rejects_bad_shapes(kw, chunk, code):
    sh = shape(**kw)
    L = ssd.lib()
    st = L.ssd_fwd(FAKE, FAKE, FAKE, FAKE, None, chunk, FAKE, FAKE, ctypes.byref(sh), FAKE, 1 << 40, None)
    assert st == code
    st = L.ssd_fwd_ex(FAKE, FAKE, FAKE, FAKE, None, None, chunk, 1, FAKE, FAKE, ctypes.byref(sh), FAKE, 1 << 40, None)
    assert st == code


def test_fwd_rejects_null_pointers_and_small_workspace():
    L = ssd.lib()
    sh = shape()
    _, need = ws_bytes(sh, 128, 0)
    args = [FAKE, FAKE, FAKE, FAKE, None, 128, FAKE, FAKE, ctypes.byref(sh), FAKE, need, None]
    for i in (0, 1, 2, 3, 6, 9):  # X, log_a, B, C, Y, workspace
        a = list(args)
        a[i] = None
        assert L.ssd_fwd(*a) == INVALID, i
    a = list(args)
    a[10] = need - 1
    assert L.ssd_fwd(*a) == WS_SMALL
    a = list(args)
    a[8] = None
    assert L.ssd_fwd(*a) == INVALID


def test_packed_argument_rules():
    L = ssd.lib()
    sh = shape(batch=2, num_seqs=3)
    assert L.ssd_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, 128, FAKE, None, ctypes.byref(sh), FAKE, 1 << 40, None) == INVALID
    sh = shape(num_seqs=0)
    assert L.ssd_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, 128, FAKE, None, ctypes.byref(sh), FAKE, 1 << 40, None) == INVALID
    sh = shape(seqlen=4, num_seqs=5)
    assert L.ssd_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, 32, FAKE, None, ctypes.byref(sh), FAKE, 1 << 40, None) == INVALID


def test_stage_entry_points_validate():
    L = ssd.lib()
    sh = shape()
    _, need = ws_bytes(sh, 128, 2)
    assert L.ssd_chunk_cumsum(None, None, 128, 2, ctypes.byref(sh), FAKE, need, None) == INVALID
    assert L.ssd_chunk_state(None, FAKE, None, 128, 2, ctypes.byref(sh), FAKE, need, None) == INVALID
    assert L.ssd_chunk_state(FAKE, FAKE, None, 128, 2, ctypes.byref(sh), FAKE, need - 256, None) == WS_SMALL
    assert L.ssd_chunk_state(FAKE, FAKE, None, 128, 1, ctypes.byref(sh), FAKE, need, None) == WS_SMALL
    assert L.ssd_state_passing(None, None, 128, 2, None, ctypes.byref(sh), None, need, None) == INVALID
    assert L.ssd_chunk_scan(FAKE, FAKE, None, None, 128, 2, FAKE, ctypes.byref(sh), FAKE, need, None) == INVALID
    assert L.ssd_chunk_scan(FAKE, FAKE, FAKE, None, 128, 2, None, ctypes.byref(sh), FAKE, need, None) == INVALID
    assert L.ssd_chunk_scan(FAKE, FAKE, FAKE, None, 128, 5, FAKE, ctypes.byref(sh), FAKE, need, None) == UNSUPPORTED


def test_step_validates():
    L = ssd.lib()
    sh = shape(batch=64, nheads=80)
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(sh), None]
    for i in range(6):
        a = list(args)
        a[i] = None
        assert L.ssd_step(*a) == INVALID
    bad = shape(batch=64, nheads=80, dstate=24)
    assert L.ssd_step(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(bad), None) == UNSUPPORTED
    bad = shape(batch=64, nheads=80, ngroups=3)
    assert L.ssd_step(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(bad), None) == INVALID


def test_binding_refuses_host_tensors():
    import torch
    X = torch.zeros(1, 64, 2, 16)
    with pytest.raises(ValueError):
        ssd.fwd(X, torch.zeros(1, 64, 2), torch.zeros(1, 64, 1, 16), torch.zeros(1, 64, 1, 16), chunk=32)


def test_mamba2_entry_points_validate():
    L = ssd.lib()
    sh = shape()
    _, need = ws_bytes(sh, 128, 0)
    # X, dt, dt_bias, A_log, D, z, B, C, cu, init, chunk, gs, Y, final, shape, ws, bytes, stream
    args = [FAKE, FAKE, None, FAKE, None, None, FAKE, FAKE, None, None, 128, 0, FAKE, None, ctypes.byref(sh), FAKE,
            need, None]
    for i in (0, 1, 3, 6, 7, 12, 15):  # X, dt, A_log, B, C, Y, workspace are required
        a = list(args)
        a[i] = None
        assert L.ssd_fwd_mamba2(*a) == INVALID, i
    a = list(args)
    a[16] = need - 1
    assert L.ssd_fwd_mamba2(*a) == WS_SMALL
    a = list(args)
    a[10] = 48
    assert L.ssd_fwd_mamba2(*a) == UNSUPPORTED
    st = shape(batch=64, nheads=80)
    # state, x, dt, dt_bias, A_log, D, z, B, C, y, shape, stream
    sargs = [FAKE, FAKE, FAKE, None, FAKE, None, None, FAKE, FAKE, FAKE, ctypes.byref(st), None]
    for i in (0, 1, 2, 4, 7, 8, 9):
        a = list(sargs)
        a[i] = None
        assert L.ssd_step_mamba2(*a) == INVALID, i
    bad = shape(batch=64, nheads=80, headdim=48)
    a = list(sargs)
    a[10] = ctypes.byref(bad)
    assert L.ssd_step_mamba2(*a) == UNSUPPORTED


def test_mamba2_binding_checks_parameters():
    import torch
    X = torch.zeros(1, 64, 2, 16)
    with pytest.raises(ValueError):
        ssd.fwd_mamba2(X, torch.zeros(1, 64, 2), torch.zeros(2), torch.zeros(1, 64, 1, 16), torch.zeros(1, 64, 1, 16),
                       chunk=32)


def test_alignment_rules():
    L = ssd.lib()
    sh = shape()
    _, need = ws_bytes(sh, 128, 0)
    odd = ctypes.c_void_p(0x1008)   # 8-byte aligned only
    # workspace must be 256-byte aligned
    assert L.ssd_fwd_ex(FAKE, FAKE, FAKE, FAKE, None, None, 128, 0, FAKE, None, ctypes.byref(sh), odd, need,
                        None) == INVALID
    # states move in 16-byte pieces
    assert L.ssd_fwd_ex(FAKE, FAKE, FAKE, FAKE, None, odd, 128, 0, FAKE, None, ctypes.byref(sh), FAKE, need,
                        None) == INVALID
    assert L.ssd_fwd_ex(FAKE, FAKE, FAKE, FAKE, None, None, 128, 0, FAKE, odd, ctypes.byref(sh), FAKE, need,
                        None) == INVALID


def test_bwd_validates():
    L = ssd.lib()
    sh = shape(seqlen=4096, nheads=8)
    n = ctypes.c_size_t(0)
    assert L.ssd_bwd_workspace_bytes(ctypes.byref(sh), 128, 0, ctypes.byref(n)) == OK and n.value > 0
    # X, log_a, B, C, cu, init, dY, dfinal, chunk, gs, dX, dlog_a, dB, dC, dinit, shape, ws, bytes, stream
    args = [FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None, 128, 0, FAKE, FAKE, FAKE, FAKE, None, ctypes.byref(sh),
            FAKE, n.value, None]
    for i in (0, 1, 2, 3, 6, 10, 11, 12, 13, 15, 16):
        a = list(args)
        a[i] = None
        assert L.ssd_bwd(*a) == INVALID, i
    a = list(args)
    a[17] = n.value - 1
    assert L.ssd_bwd(*a) == WS_SMALL
    # dstate 256 has no exchanged-role run (headdim 256), and bf16 headdim 16 none either (dstate 16)
    for bad in (shape(seqlen=512, nheads=8, dstate=256), shape(seqlen=512, nheads=8, headdim=16)):
        assert L.ssd_bwd_workspace_bytes(ctypes.byref(bad), 128, 0, ctypes.byref(n)) == UNSUPPORTED


def test_state_chain_mode_switch():
    # process-wide switch; nothing is launched
    prev = ssd.set_state_chain(0)
    assert prev in (0, 1)
    assert ssd.set_state_chain(1) == 0
    assert ssd.set_state_chain(prev) == 1


def test_bwd_mamba2_validates():
    L = ssd.lib()
    sh = shape(seqlen=4096, nheads=8)
    n = ctypes.c_size_t(0)
    assert L.ssd_bwd_mamba2_workspace_bytes(ctypes.byref(sh), 128, 0, ctypes.byref(n)) == OK and n.value > 0
    # X dt dt_bias A_log D z B C cu init dY dfinal | chunk gs | dX ddt ddt_bias dA_log dD dz dB dC dinit | shape ws n stream
    args = [FAKE, FAKE, None, FAKE, None, None, FAKE, FAKE, None, None, FAKE, None, 128, 0,
            FAKE, FAKE, None, FAKE, None, None, FAKE, FAKE, None, ctypes.byref(sh), FAKE, n.value, None]
    for i in (0, 1, 3, 6, 7, 10, 14, 15, 17, 20, 21, 23, 24):
        a = list(args)
        a[i] = None
        assert L.ssd_bwd_mamba2(*a) == INVALID, i
    for i, j in ((4, 18), (5, 19)):   # D needs dD and z needs dz, and the other way round
        a = list(args)
        a[i] = FAKE
        assert L.ssd_bwd_mamba2(*a) == INVALID, i
        a = list(args)
        a[j] = FAKE
        assert L.ssd_bwd_mamba2(*a) == INVALID, j
    a = list(args)
    a[25] = n.value - 1
    assert L.ssd_bwd_mamba2(*a) == WS_SMALL
    odd = shape(seqlen=512, nheads=8, headdim=18)
    assert L.ssd_bwd_mamba2_workspace_bytes(ctypes.byref(odd), 64, 0, ctypes.byref(n)) != OK


def test_step_rejects_unaligned_state():
    L = ssd.lib()
    sh = shape(batch=64, nheads=80)
    odd = ctypes.c_void_p(0x1008)   # 8-byte aligned only
    assert L.ssd_step(odd, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(sh), None) == INVALID
    assert L.ssd_step_mamba2(odd, FAKE, FAKE, None, FAKE, None, None, FAKE, FAKE, FAKE, ctypes.byref(sh),
                             None) == INVALID


# ---- the binding's own checks: every tensor against the shape it implies ----
# Host tensors are used throughout: structure (shape, dtype, contiguity) is
# checked before the device, so each case below must be refused for the
# mismatch itself, and the well-formed call only for living on the host.

def _fwd_args(b=1, T=64, H=4, P=16, G=2, N=32, dt=None):
    import torch
    dt = dt or torch.bfloat16
    return dict(X=torch.zeros(b, T, H, P, dtype=dt), log_a=torch.zeros(b, T, H), B=torch.zeros(b, T, G, N, dtype=dt),
                C=torch.zeros(b, T, G, N, dtype=dt))


def _refused(fn, what, **kw):
    with pytest.raises(ValueError) as e:
        fn(**kw)
    msg = str(e.value)
    assert what in msg and "device tensor" not in msg, msg


def _fwd_cases():
    import torch
    bf = torch.bfloat16
    return {
        "B rows": (dict(B=torch.zeros(1, 63, 2, 32, dtype=bf)), "B"),
        "C shape": (dict(C=torch.zeros(1, 64, 2, 16, dtype=bf)), "C"),
        "C groups": (dict(C=torch.zeros(1, 64, 1, 32, dtype=bf)), "C"),
        "C dtype": (dict(C=torch.zeros(1, 64, 2, 32)), "C"),
        "log_a shape": (dict(log_a=torch.zeros(1, 64, 2)), "log_a"),
        "log_a dtype": (dict(log_a=torch.zeros(1, 64, 4, dtype=bf)), "log_a"),
        "log_a heads": (dict(log_a=torch.zeros(1, 64, 4, 1)), "log_a"),
        "groups": (dict(B=torch.zeros(1, 64, 3, 32, dtype=bf), C=torch.zeros(1, 64, 3, 32, dtype=bf)), "ngroups"),
        "X strided": (dict(X=torch.zeros(1, 64, 4, 32, dtype=bf)[..., ::2]), "X"),
        "Y shape": (dict(Y=torch.zeros(1, 64, 4, 8, dtype=bf)), "Y"),
        "Y dtype": (dict(Y=torch.zeros(1, 64, 4, 16)), "Y"),
        "final shape": (dict(final_state=torch.zeros(1, 4, 32, 16)), "final_state"),
        "final dtype": (dict(final_state=torch.zeros(1, 4, 16, 32, dtype=bf)), "final_state"),
        "initial shape": (dict(initial_state=torch.zeros(2, 4, 16, 32)), "initial_state"),
        "cu dtype": (dict(cu_seqlens=torch.tensor([0, 64], dtype=torch.int64)), "cu_seqlens"),
        "cu strided": (dict(cu_seqlens=torch.tensor([0, 9, 32, 50, 64], dtype=torch.int32)[::2]), "cu_seqlens"),
    }


@pytest.mark.parametrize("case", sorted(_fwd_cases()))
def test_binding_fwd_refuses_mismatched_tensors(case):
    kw, what = _fwd_cases()[case]
    args = _fwd_args()
    args.update(kw)
    _refused(ssd.fwd, what, chunk=32, **args)


def test_binding_fwd_refuses_batch_with_cu_seqlens():
    import torch
    args = _fwd_args(b=2)
    _refused(ssd.fwd, "batch 1", chunk=32, cu_seqlens=torch.tensor([0, 64], dtype=torch.int32), **args)


def test_binding_fwd_well_formed_host_call_is_refused_for_the_device_only():
    with pytest.raises(ValueError, match="device tensor"):
        ssd.fwd(chunk=32, **_fwd_args())


def test_binding_workspace_must_match_the_call():
    import torch
    a = _fwd_args()
    other = ssd.make_shape(torch.zeros(1, 128, 4, 16, dtype=torch.bfloat16), a["B"])
    ws = ssd.Workspace(other, 32, "cpu", 1)
    _refused(ssd.fwd, "workspace", chunk=32, workspace=ws, **a)
    sh = ssd.make_shape(a["X"], a["B"])
    ws = ssd.Workspace(sh, 32, "cpu", 1)
    _refused(ssd.fwd, "workspace", chunk=64, workspace=ws, **a)


def test_binding_stage_wrappers_check_tensors():
    import torch
    a = _fwd_args()
    sh = ssd.make_shape(a["X"], a["B"])
    ws = ssd.Workspace(sh, 32, "cpu", 1)
    _refused(lambda: ssd.chunk_cumsum(torch.zeros(1, 64, 2), None, sh, ws), "log_a")
    _refused(lambda: ssd.chunk_state(a["X"], torch.zeros(1, 64, 2, 16, dtype=torch.bfloat16), None, sh, ws), "B")
    _refused(lambda: ssd.chunk_scan(a["X"], a["B"], a["C"], None, torch.zeros(1, 64, 4, 16), sh, ws), "Y")
    _refused(lambda: ssd.state_passing(None, torch.zeros(1, 4, 32, 16), sh, ws), "final_state")
    _refused(lambda: ssd.chunk_cumsum(a["log_a"], torch.tensor([0, 64], dtype=torch.int32), sh, ws), "cu_seqlens")
    other = ssd.make_shape(torch.zeros(1, 64, 4, 16, dtype=torch.bfloat16), torch.zeros(1, 64, 1, 32))
    _refused(lambda: ssd.chunk_cumsum(a["log_a"], None, other, ws), "workspace")


def _step_args(b=3, H=4, P=16, G=2, N=32):
    import torch
    bf = torch.bfloat16
    return dict(state=torch.zeros(b, H, P, N), x=torch.zeros(b, H, P, dtype=bf), log_a=torch.zeros(b, H),
                B=torch.zeros(b, G, N, dtype=bf), C=torch.zeros(b, G, N, dtype=bf))


@pytest.mark.parametrize("kw,what", [
    (dict(state=("zeros", (3, 4, 32, 16))), "state"),
    (dict(state=("zeros_bf", (3, 4, 16, 32))), "state"),
    (dict(log_a=("zeros", (3, 2))), "log_a"),
    (dict(B=("zeros_bf", (2, 2, 32))), "B"),
    (dict(C=("zeros_bf", (3, 1, 32))), "C"),
    (dict(C=("zeros", (3, 2, 32))), "C"),
    (dict(y=("zeros_bf", (3, 4, 8))), "y"),
], ids=["state-shape", "state-dtype", "log_a", "B-rows", "C-groups", "C-dtype", "y"])
def test_binding_step_refuses_mismatched_tensors(kw, what):
    import torch
    make = dict(zeros=lambda s: torch.zeros(*s), zeros_bf=lambda s: torch.zeros(*s, dtype=torch.bfloat16))
    args = _step_args()
    for k, (f, s) in kw.items():
        args[k] = make[f](s)
    _refused(ssd.step, what, **args)


def test_binding_step_mamba2_and_bwd_check_tensors():
    import torch
    a = _step_args()
    H = 4
    _refused(ssd.step_mamba2, "dt", state=a["state"], x=a["x"], dt=torch.zeros(3, 2), A_log=torch.zeros(H),
             B=a["B"], C=a["C"])
    _refused(ssd.step_mamba2, "z", state=a["state"], x=a["x"], dt=torch.zeros(3, H), A_log=torch.zeros(H),
             B=a["B"], C=a["C"], z=torch.zeros(3, H, 16))
    f = _fwd_args()
    _refused(ssd.bwd, "dY", dY=torch.zeros(1, 64, 4, 8, dtype=torch.bfloat16), chunk=32, **f)
    _refused(ssd.bwd, "dfinal_state", dY=torch.zeros_like(f["X"]), dfinal_state=torch.zeros(1, 4, 32, 16), chunk=32,
             **f)
    m = dict(X=f["X"], B=f["B"], C=f["C"], dt=torch.zeros(1, 64, H), A_log=torch.zeros(H))
    _refused(ssd.fwd_mamba2, "A_log", **dict(m, A_log=torch.zeros(H + 1)), chunk=32)
    _refused(ssd.fwd_mamba2, "D", **m, D=torch.zeros(H, dtype=torch.bfloat16), chunk=32)
    _refused(ssd.bwd_mamba2, "dY", **m, dY=torch.zeros(1, 64, 4, 16), chunk=32)


def test_state_chain_cooperative_query_validates():
    L = ssd.lib()
    r = ctypes.c_int32(7)
    assert L.ssd_state_chain_cooperative(ctypes.byref(shape()), 128, 0, None) == INVALID
    assert L.ssd_state_chain_cooperative(None, 128, 0, ctypes.byref(r)) == INVALID
    assert L.ssd_state_chain_cooperative(ctypes.byref(shape(headdim=48)), 128, 0, ctypes.byref(r)) == UNSUPPORTED
    assert L.ssd_state_chain_cooperative(ctypes.byref(shape()), 128, 3, ctypes.byref(r)) == UNSUPPORTED
    assert r.value == 7   # untouched on error


def test_fwd_noalloc_validates_and_bounds_its_scratch():
    """ssd_fwd_noalloc checks its arguments like ssd_fwd, and refuses a call whose
    workspace would exceed the static scratch, all before any HIP call."""
    L = ssd.lib()
    sh = shape()
    _, need = ws_bytes(sh, 128, 0)
    assert need <= binding.NOALLOC_SCRATCH_BYTES   # the headline shape fits
    args = [FAKE, FAKE, FAKE, FAKE, None, 128, FAKE, FAKE, ctypes.byref(sh), None]
    for i in (0, 1, 2, 3, 6, 8):   # X, log_a, B, C, Y, shape
        a = list(args)
        a[i] = None
        assert L.ssd_fwd_noalloc(*a) == INVALID, i
    a = list(args)
    a[5] = 96
    assert L.ssd_fwd_noalloc(*a) == UNSUPPORTED
    odd = ctypes.c_void_p(0x1008)
    a = list(args)
    a[7] = odd   # final_state moves in 16-byte pieces
    assert L.ssd_fwd_noalloc(*a) == INVALID
    big = shape(seqlen=32768, nheads=80, num_seqs=7)   # the packed H = 80 layer: ~175 MB of workspace
    _, need_big = ws_bytes(big, 128, 0)
    assert need_big > binding.NOALLOC_SCRATCH_BYTES
    assert L.ssd_fwd_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, 128, FAKE, None, ctypes.byref(big), None) == WS_SMALL
    hdr = open(HEADER).read()
    assert "#define SSD_NOALLOC_SCRATCH_BYTES (64u << 20)" in hdr and binding.NOALLOC_SCRATCH_BYTES == 64 << 20


def test_chunk_scan_kernel_query():
    """ssd_chunk_scan_kernel names the chunk_scan kernel a call takes, with the
    forward call's own shape checks; host logic only."""
    L = ssd.lib()
    r = ctypes.c_int32(9)
    assert L.ssd_chunk_scan_kernel(ctypes.byref(shape()), 128, 0, None) == INVALID
    assert L.ssd_chunk_scan_kernel(None, 128, 0, ctypes.byref(r)) == INVALID
    assert L.ssd_chunk_scan_kernel(ctypes.byref(shape(headdim=48)), 128, 0, ctypes.byref(r)) == UNSUPPORTED
    assert L.ssd_chunk_scan_kernel(ctypes.byref(shape()), 128, 3, ctypes.byref(r)) == UNSUPPORTED
    assert r.value == 9   # untouched on error
    k = binding.chunk_scan_kernel
    # T = 16384, H = 32 at the default state block of 8 chunks: 256 units, one per CU
    assert k(shape(), 128) == "pair"
    # the same with state blocks of 4 chunks: 512 units, two per CU
    assert k(shape(), 128, 4) == "half_pair"
    # the state-size sweep (b 8, T 4096, H 32): 512 units at the default
    assert k(shape(batch=8, seqlen=4096, dstate=64), 128) == "half_pair"
    assert k(shape(batch=8, seqlen=4096, dstate=128), 128) == "half_pair"
    assert k(shape(batch=8, seqlen=4096, dstate=256), 128) == "half_pair_wide"
    assert k(shape(batch=8, seqlen=4096, dstate=256, nheads=3), 128) == "single"
    assert k(shape(batch=8, seqlen=4096, dstate=256), 32) == "single"
    # packed H = 80 layer
    assert k(shape(seqlen=32768, nheads=80, num_seqs=7), 128) == "half_pair"
    # chunks of 64 need 512 units too; chunks of 32 or 256 never take halves
    assert k(shape(batch=2, seqlen=2048, nheads=24, dstate=64), 64) == "pair"
    assert k(shape(batch=2, seqlen=2048, nheads=32, dstate=64), 64, 1) == "half_pair"
    assert k(shape(batch=2, seqlen=2048, nheads=32, dstate=64), 32, 1) == "pair"
    assert k(shape(batch=8, seqlen=4096), 256) == "single"
    # odd heads per group, P = 128, fp32
    assert k(shape(nheads=3), 128, 1) == "single"
    assert k(shape(batch=8, seqlen=4096, headdim=128, dstate=64), 128) == "single"
    assert k(shape(dtype=0), 128) == "f32"
