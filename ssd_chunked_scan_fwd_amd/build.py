"""Build libssd_mi355x.so (gfx950) in-tree with hipcc.

    python -m ssd_chunked_scan_fwd_amd.build

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled, and linked into one shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libssd_mi355x.so")
SOURCES = ["ssd_api.cpp", "ssd_cumsum_passing.hip", "ssd_chunk_state.hip", "ssd_chunk_scan.hip", "ssd_bwd.hip", "ssd_bwd_chunk.hip", "ssd_bwd_mamba2.hip"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


COMMON = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I" + INCLUDE, "-I" + CSRC]


# Host-side sanitizers for the checking build (build(sanitize=True)): every
# flag applies to the host pass only (-Xarch_host); device code is unchanged.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SANITIZE_DIR = os.path.join(BUILD, "sanitize")
SANITIZE_LIB = os.path.join(SANITIZE_DIR, "libssd_mi355x.so")


def _compile(src: str, sanitize: bool = False) -> str:
    out_dir = SANITIZE_DIR if sanitize else BUILD
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    cmd = [hipcc()] + COMMON + (SANITIZE if sanitize else []) + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 8, sanitize: bool = False) -> str:
    """Build libssd_mi355x.so next to this file; with sanitize, a checking build
    with AddressSanitizer and UndefinedBehaviorSanitizer on the host code, in
    _build/sanitize/ (loaded by the tests through SSD_MI355X_LIBRARY, with the
    clang ASan runtime preloaded)."""
    out_dir = SANITIZE_DIR if sanitize else BUILD
    lib = SANITIZE_LIB if sanitize else LIB
    os.makedirs(out_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), SOURCES))
    tmp = lib + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + \
        (SANITIZE + ["-shared-libasan"] if sanitize else []) + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    args = [a for a in sys.argv[1:] if a != "--sanitize"]
    print(build(int(args[0]) if args else 8, sanitize="--sanitize" in sys.argv[1:]))
