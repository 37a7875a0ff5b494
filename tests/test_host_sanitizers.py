"""The library's host-side code (argument validation, workspace layouts, token
order tables: csrc/validate.cpp and csrc/order.cpp) built with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer and exercised by
tests/host_sanitize/host_checks.cpp: every check must pass with no sanitizer
report.  Needs no GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_attention_fractal_amd", "csrc")
ROCM_INCLUDE = "/opt/rocm/include"


def test_host_code_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("g++ or the ROCm headers are missing")
    exe = str(tmp_path / "host_checks")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-isystem", ROCM_INCLUDE, os.path.join(ROOT, "tests", "host_sanitize", "host_checks.cpp"),
           os.path.join(CSRC, "validate.cpp"), os.path.join(CSRC, "order.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host checks ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
