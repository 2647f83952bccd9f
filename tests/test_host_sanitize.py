"""The C ABI's host layer (fa_api.cpp: argument checks, size rules and
dispatch) built with g++ for the host alone, under AddressSanitizer and
UndefinedBehaviorSanitizer, against stub launchers that record launches
instead of running kernels (tests/host/).  The driver runs every rejection
path (each must launch nothing), checks the arguments accepted calls hand
down, and pushes extreme sizes through the size arithmetic.  No GPU and no
HIP runtime are involved."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_api_host_layer_under_sanitizers(tmp_path):
    exe = str(tmp_path / "api_driver")
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           os.path.join(ROOT, "exact_io_aware_30_amd", "csrc", "fa_api.cpp"),
           os.path.join(HERE, "host", "stub_launchers.cpp"), os.path.join(HERE, "host", "api_driver.cpp"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    print(r.stdout[-2000:], r.stderr[-2000:])
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "ALL OK" in r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
