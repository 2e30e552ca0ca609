"""CPU run of the `-m "not gpu"` suite against sanitizer builds of the HIP
library's host code and of the oracle (AddressSanitizer + UndefinedBehavior
Sanitizer; clang's ASan runtime preloaded into python, leak checks off since
the interpreter itself is not instrumented).

    python tests/sanitize_cpu.py [extra pytest args]

Builds _build/sanitize/libssd_mi355x.so (host code instrumented, device code
as usual) and _build/sanitize/libssd_oracle.so, then runs the suite in a child
process that loads them (SSD_MI355X_LIBRARY, SSD_ORACLE_LIBRARY). Exits with
the suite's status; any sanitizer report aborts the child (UBSan without
recovery, ASan halts on the first error).
"""
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


CANARY = r"""
import ctypes, numpy as np
import ssd_chunked_scan_fwd_amd as ssd
from oracle import oracle
L = oracle._load()
maps = open("/proc/self/maps").read()
ssd.lib()
maps = open("/proc/self/maps").read()
assert "_build/sanitize/libssd_oracle.so" in maps and "_build/sanitize/libssd_mi355x.so" in maps, "not loaded"
print("loaded: sanitized oracle and library", flush=True)
rows, T, H, G, P, N = 1, 8, 1, 1, 2, 2
X = np.zeros((rows, T, H, P)); la = np.zeros((rows, T, H)); B = np.zeros((rows, T, G, N)); C = np.zeros_like(B)
seg = np.array([0, 0, T], np.int32)
Y = np.zeros((rows, T - 1, H, P))              # one token short
fin = np.zeros((1, H, P, N))
dp = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
L.ssd_oracle_scan(rows, T, H, G, P, N, dp(X), dp(la), dp(B), dp(C), 1, seg.ctypes.data_as(ctypes.POINTER(ctypes.c_int)),
                  None, dp(Y), dp(fin), None, None, 1, 0)
print("overflow not reported", flush=True)
"""


def asan_runtime() -> str:
    libs = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not libs:
        raise RuntimeError("clang's ASan runtime (libclang_rt.asan-x86_64.so) not found under /opt/rocm/llvm")
    return libs[-1]


def main() -> int:
    from ssd_chunked_scan_fwd_amd import build as b
    from oracle import oracle
    lib = b.build(sanitize=True)
    orc = oracle.build_sanitized(os.path.join(b.SANITIZE_DIR, "libssd_oracle.so"))
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan_runtime(), SSD_MI355X_LIBRARY=lib, SSD_ORACLE_LIBRARY=orc,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # Canary: the instrumented libraries are the ones loaded, and a heap
    # overflow in them is reported (the oracle handed an output buffer one
    # token short); the child must die with an AddressSanitizer report.
    r = subprocess.run([sys.executable, "-c", CANARY], env=env, cwd=ROOT, capture_output=True, text=True)
    if r.returncode == 0 or "AddressSanitizer: heap-buffer-overflow" not in r.stderr:
        print(r.stdout[-2000:], r.stderr[-4000:])
        raise RuntimeError("the sanitizer canary was not caught: the checking build is not active")
    print("[sanitize] canary caught: " + r.stdout.strip().splitlines()[-1], flush=True)
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-m", "not gpu", "-p",
           "no:cacheprovider"] + sys.argv[1:]
    print("[sanitize] " + " ".join(cmd), flush=True)
    return subprocess.run(cmd, env=env, cwd=ROOT).returncode


if __name__ == "__main__":
    sys.exit(main())
