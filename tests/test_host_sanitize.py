"""The C-ABI validation layer (csrc/moe_api.hip) built for the host alone
with AddressSanitizer and UndefinedBehaviorSanitizer, its kernel launches
replaced by counters (tests/host_sanitize/launch_stubs.cpp), and driven
through every entry point with valid, invalid and extreme arguments
(tests/host_sanitize/validation_driver.cpp).  CPU only: no GPU code is
built (host-only compilation) and nothing is launched."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")
CSRC = os.path.join(ROOT, "combine_router_gate_amd", "csrc")
INC = os.path.join(ROOT, "include")


def _hipcc():
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin",
                           "hipcc"), shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def test_validation_layer_under_asan_ubsan(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "validation_driver")
    # host-only compilation: the sanitizers apply to host code alone
    san = ["-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    cmd = [hipcc, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "--cuda-host-only", "-x", "hip", "-I", INC, "-I", CSRC] + san + [
        os.path.join(CSRC, "moe_api.hip"),
        os.path.join(HERE, "launch_stubs.cpp"),
        os.path.join(HERE, "validation_driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env,
                       timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok:" in r.stdout and "0 failed" in r.stdout, r.stdout
