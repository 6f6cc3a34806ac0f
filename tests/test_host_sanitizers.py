"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
on the CPU (no GPU): sketch generation, explicit FQJL products, the operand
images, qjl_make_sketch's device-image layout, the row map and the argument
checks of every entry point, driven by tests/host_sanitize/driver.cpp with
the HIP runtime and the kernel launchers stood in for."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_quantized_jl_amd", "csrc")
SOURCES = [os.path.join(CSRC, f) for f in ("api.cpp", "sketch_host.cpp", "images_host.cpp")]
DRIVER = os.path.join(ROOT, "tests", "host_sanitize", "driver.cpp")


def _compiler():
    for c in ("/opt/rocm/llvm/bin/clang++", shutil.which("clang++"), shutil.which("g++")):
        if c and os.path.exists(c):
            return c
    return None


def test_host_code_under_asan_and_ubsan(tmp_path):
    cxx = _compiler()
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path / "host_sanitize")
    cmd = [cxx, "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           *SOURCES, DRIVER, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "runtime error" not in r.stderr
    assert "all checks passed" in r.stdout
