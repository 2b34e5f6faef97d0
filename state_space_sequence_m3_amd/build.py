"""Build libm3scan.so in-tree with hipcc for gfx950.

    python -m state_space_sequence_m3_amd.build        # or build() from Python

Each .hip source is compiled to an object in parallel, then linked into
``state_space_sequence_m3_amd/libm3scan.so``.  Packed-fp32 instruction selection is switched off
(``-packed-fp32-ops``) for every HIP translation unit.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build", "m3scan")
LIB = os.path.join(PKG, "libm3scan.so")
SOURCES = ["api.hip", "bcnorm_rope.hip", "prefill.hip", "decode.hip", "backward.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set ROCM_PATH)")


def compile_flags() -> list:
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link the shared library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    flags = compile_flags()

    def one(src):
        obj = os.path.join(BUILD_DIR, src + ".o")
        cmd = [cc] + flags + ["-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
