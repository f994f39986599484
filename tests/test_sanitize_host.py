"""The library's host code under AddressSanitizer and UndefinedBehavior-
Sanitizer (CPU only): tests/sanitize/abi_host_check.cpp is linked against the
HIP sources with -fsanitize on the host pass (the device code is built as
usual) and exercises the size queries, the CHMC rank, fp16 rounding, the
timing hooks and every entry point's argument checks. Any sanitizer report or
failed check fails the test.
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "post_weight_quantization_hessian_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "sanitize", "abi_host_check.cpp")
OUT_DIR = os.path.join(ROOT, "_build", "sanitize")
EXE = os.path.join(OUT_DIR, "abi_host_check")


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def _build():
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [DRIVER]
    deps = srcs + glob.glob(os.path.join(CSRC, "*.h")) + [os.path.join(ROOT, "include", "gptq.h")]
    if os.path.exists(EXE) and os.path.getmtime(EXE) >= max(os.path.getmtime(f) for f in deps):
        return
    os.makedirs(OUT_DIR, exist_ok=True)
    cmd = [_hipcc(), "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Wno-unused-result",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", EXE + ".tmp"] + srcs
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    os.replace(EXE + ".tmp", EXE)


@pytest.mark.timeout(900)
def test_host_code_under_address_and_ub_sanitizers():
    if _hipcc() is None:
        pytest.skip("hipcc not found")
    _build()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert "host checks passed" in out
