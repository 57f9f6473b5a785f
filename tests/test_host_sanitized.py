"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

tests/host/abi_check.cpp links the library's argument-validation layer (csrc/sv_api.cpp, with
the workspace layouts and launch limits of csrc/sv_internal.h) against stub launchers, drives
every validation path of every entry point up to the ABI's extreme shapes, and checks the
workspace layout, every launch's grid (below 2^32 work-items) and the largest element index the
kernels form.  It is compiled here with g++ (host code only, warnings as errors) and must run
clean: no sanitizer report and no failed check.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rejection_sampling_verify_chain_amd", "csrc")
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs g++ and the ROCm headers")
def test_abi_host_code_is_sanitizer_clean(tmp_path):
    exe = tmp_path / "abi_check"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-Wall", "-Wextra", "-Werror",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-I", ROCM_INCLUDE, os.path.join(CSRC, "sv_api.cpp"),
           os.path.join(ROOT, "tests", "host", "abi_check.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "runtime error" not in r.stderr, r.stderr[-4000:]
    assert "0 failed" in r.stdout, r.stdout
