"""The C ABI's host-side argument validation (csrc/validate.cpp) under
AddressSanitizer and UndefinedBehaviorSanitizer: a host-only build with g++
(no device code) of the validation file and a driver
(tests/sanitize/validate_driver.cpp) that feeds it valid arguments, every
error path, and extreme sizes and strides.  Any out-of-bounds access, signed
overflow or pointer wrap-around aborts the driver."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_attention_gilbert_amd", "csrc")


def test_validation_clean_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    hip_inc = "/opt/rocm/include"
    if not gxx or not os.path.isdir(hip_inc):
        pytest.skip("g++ or the HIP headers are missing")
    exe = tmp_path / "validate_driver"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", hip_inc,
           "-I", CSRC, os.path.join(CSRC, "validate.cpp"), os.path.join(ROOT, "tests", "sanitize", "validate_driver.cpp"),
           "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "sanitizer" in (build.stderr or "").lower() and "cannot find" in build.stderr:
        pytest.skip("sanitizer runtimes are not installed")
    assert build.returncode == 0, build.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, (run.stdout[-1000:], run.stderr[-3000:])
    assert "checks passed" in run.stdout and "runtime error" not in run.stderr, run.stderr[-3000:]
