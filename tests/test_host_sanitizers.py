"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

api.hip is compiled again with the sanitizers on its host pass only (each -fsanitize flag behind
-Xarch_host, so the GPU code is built as usual), linked with the other objects of the regular
build into a library in a temporary folder, and loaded by a child Python process that has the
sanitizer runtime preloaded.  The child runs tests/test_abi_host.py against that library: the
argument checks of every entry point (null, misaligned, overlapping and undersized buffers, bad
dims, the workspace-size queries, the no-device error path), which is all of the host code that
runs without a GPU.  Any report (heap or stack overflow, use after free, signed overflow, a bad
shift, misaligned access, ...) aborts the child, and the test fails with its output."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "state_space_sequence_m3_amd")
CSRC = os.path.join(PKG, "csrc")
OBJS = os.path.join(ROOT, "_build", "m3scan")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

CHILD = r"""
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
from state_space_sequence_m3_amd import m3scan
m3scan.load({lib!r})
assert m3scan._lib._name == {lib!r}
import pytest
sys.exit(pytest.main([{abi!r}, "-q", "-p", "no:cacheprovider"]))
"""


def _runtime():
    hits = sorted(glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    rt = _runtime()
    if not os.path.exists(hipcc) or rt is None:
        pytest.skip("hipcc or the clang sanitizer runtime is not installed")
    others = [os.path.join(OBJS, s + ".o") for s in ("bcnorm_rope.hip", "prefill.hip", "decode.hip", "backward.hip")]
    if not all(os.path.exists(o) for o in others):
        pytest.skip("the regular build's objects are missing (run the build first)")
    obj = str(tmp_path / "api_san.o")
    lib = str(tmp_path / "libm3scan_san.so")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    cc = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC] + san + ["-c", os.path.join(CSRC, "api.hip"), "-o", obj]
    r = subprocess.run(cc, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    ld = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libasan",
          "-o", lib, obj] + others
    r = subprocess.run(ld, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt
    # Python itself leaks by design at exit; every other report aborts the child
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib,
                        abi=os.path.join(ROOT, "tests", "test_abi_host.py"))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert " passed" in r.stdout, out[-3000:]
