"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

api.cpp (argument validation, workspace checks, the event-based kernel timer)
is built with g++ beside host stand-ins for the kernel launchers and the HIP
event calls (tests/host_sanitize/stubs.cpp), and the driver
(tests/host_sanitize/driver.cpp) calls every entry point with valid
arguments, each documented error and extreme sizes, from eight host threads
with the timer on.  Any memory error, data race on the timer's containers
visible to ASan, signed overflow or other undefined behaviour aborts the run;
any status that differs from the documented one fails it.  No GPU is used.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host_sanitize")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_host_validation_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "dspark_host_sanitize")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", '-DDSPARK_BUILD_ID="host-sanitize"', "-I/opt/rocm/include",
           os.path.join(ROOT, "draft_verify_schedule_amd", "csrc", "api.cpp"),
           os.path.join(SRC, "stubs.cpp"), os.path.join(SRC, "driver.cpp"),
           "-o", exe, "-pthread"]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    print(run.stdout[-2000:])
    assert run.returncode == 0, (run.stdout[-3000:] + run.stderr[-6000:])
    assert "ok:" in run.stdout
