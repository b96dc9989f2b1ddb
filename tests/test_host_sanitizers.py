"""AddressSanitizer + UndefinedBehaviorSanitizer build of the library's host
code, run on the CPU.

g++ compiles the planner (csrc/bbsa_plan.cpp), the work-map query
(csrc/bbsa_host.cpp, which includes the launch sizing and argument
validation of bbsa_forward and the kernels' item mapping from
csrc/bbsa_schedule.h) and tests/host_sanitize_driver.cpp with
-fsanitize=address,undefined and runs the driver; any sanitizer report, or a
failed check, fails the test.  No HIP runtime call is made.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_long_bbsa_amd", "csrc")


def test_host_code_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "host_sanitize")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__host__=", "-D__device__=", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", "/opt/rocm/include",
           os.path.join(CSRC, "bbsa_plan.cpp"), os.path.join(CSRC, "bbsa_host.cpp"),
           os.path.join(ROOT, "tests", "host_sanitize_driver.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    # verify_asan_link_order=0: the process environment may preload another
    # library ahead of the sanitizer runtime; it is left as it is.
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert run.stdout.strip().endswith("ok")
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr
