"""The library's host code (tq_host.cpp, tq_api.cpp) built with the address
and undefined-behaviour sanitizers and run without a GPU: host parameters
for every mode, context construction and teardown, getters, and the
argument validation of the entry points (tests/sanitize/driver.cpp).  The
HIP runtime and the kernel launchers are host stand-ins
(tests/sanitize/stubs.cpp), so only host logic runs; a sanitizer finding or
an unexpected status fails the test."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "oblivious_kv_cache_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "sanitize")
ROCM_INC = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INC), reason="g++ or HIP headers missing")
def test_host_code_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "tq_host_sanitized"
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INC, "-I", os.path.join(ROOT, "include"),
           os.path.join(CSRC, "tq_host.cpp"), os.path.join(CSRC, "tq_api.cpp"),
           os.path.join(HERE, "stubs.cpp"), os.path.join(HERE, "driver.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "0 failures" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
