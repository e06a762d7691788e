"""The C-ABI layer built with AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only, no GPU needed).

fa_api.cpp is compiled by the host compiler together with stand-ins for the
kernel launchers and for the two HIP runtime calls its FA_DEBUG checks make
(tests/sanitize/hip_stubs.cpp), and a driver (tests/sanitize/api_driver.cpp)
that takes every entry point through its argument checks: each invalid
argument, and valid arguments up to the (stubbed) launch.  The run must end
clean: every expected status, and no sanitizer report.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "exact_attention_70_amd", "csrc")
ROCM_INC = os.environ.get("ROCM_PATH", "/opt/rocm") + "/include"


def test_api_validation_under_asan_ubsan(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None or not os.path.isdir(os.path.join(ROCM_INC, "hip")):
        pytest.skip("needs g++ and the HIP headers")
    exe = str(tmp_path / "api_driver")
    cmd = [cxx, "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INC, "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, os.path.join(CSRC, "fa_api.cpp"), os.path.join(SAN, "hip_stubs.cpp"),
           os.path.join(SAN, "api_driver.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    # verify_asan_link_order=0: the environment may preload a library of its own
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
    assert out.startswith("OK: 0 failed expectations"), out
    # FA_DEBUG on: the table checks copy to the host first; with no device the
    # copy fails and the call reports FA_ERR_HIP, still without a sanitizer report
    env["FA_DEBUG"] = "1"
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = run.stdout + run.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
