"""The C-ABI's validation code under AddressSanitizer and UndefinedBehaviorSanitizer.

api.cpp is plain host C++ whose only GPU actions are the launchers of
launch.h.  Here it is compiled with the host compiler and the sanitizers, and
linked against recording stand-ins for those launchers (tests/sanitize/), so
that every entry point can be driven on a machine without a GPU: each rejected
call must return its documented status and launch nothing, each accepted call
must make exactly one launch with the caller's sizes, and a failing launch or
workspace lookup must come back as FA_ERR_HIP.  Integer overflow in the size
arithmetic, out-of-bounds accesses and leaks stop the run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_tiled_attention_18_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_validation_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_checks")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-I", SAN, "-I", "/opt/rocm/include", os.path.join(CSRC, "api.cpp"), os.path.join(SAN, "fake_launch.cpp"),
           os.path.join(SAN, "abi_checks.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "checks passed" in r.stdout and "FAIL" not in r.stdout
