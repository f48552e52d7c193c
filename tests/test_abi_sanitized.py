"""The C ABI's host code (csrc/api.cpp) built with g++ under the address and
undefined-behaviour sanitizers against stand-in launchers (tests/host_sanitized/stubs.cpp),
and driven through every entry point's checks and marshalling by
tests/host_sanitized/driver.cpp. CPU only: no GPU, no HIP runtime."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitized")
CSRC = os.path.join(ROOT, "attention_forward_03_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_api_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_sanitized")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-static-libasan",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, os.path.join(CSRC, "api.cpp"), os.path.join(HERE, "stubs.cpp"),
           os.path.join(HERE, "driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and "ALL OK" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])
