"""The C ABI's host code (argument checks, workspace carving, pinned-memory
views, keep budget, size arithmetic) built with AddressSanitizer and
UndefinedBehaviorSanitizer and run on the CPU.

api.cpp and host_sizes.cpp are compiled as plain C++ with g++; the kernel
launchers and the two HIP runtime calls the ABI makes are host-only
stand-ins (tests/abi_host/launch_stubs.cpp) that record what reached them.
The driver (tests/abi_host/abi_host_main.cpp) exits non-zero on a failed
check, and any sanitizer report aborts the run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_sparse_apply_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "abi_host")


def test_abi_host_code_under_asan_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "abi_host")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "host_sizes.cpp"),
           os.path.join(HOST, "launch_stubs.cpp"), os.path.join(HOST, "abi_host_main.cpp"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert "0 failed" in r.stdout and "runtime error" not in r.stderr, r.stderr[-4000:]
