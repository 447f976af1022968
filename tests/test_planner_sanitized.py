"""The host side of libhs2 (argument checks, split planner, workspace layout) built with
AddressSanitizer and UndefinedBehaviorSanitizer and driven without a GPU.

tests/sanitize/planner_driver.cpp links csrc/hs2_api.cpp with stub launchers that check
what the planner hands to each kernel (workspace regions inside the reported workspace,
well-formed work lists) and calls every entry point with fuzzed descriptors and every
rejection path. Host code only: no device code is built here.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_mqa_amd", "csrc")


def _clang():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    c = os.path.join(rocm, "llvm", "bin", "clang++")
    return c if os.path.exists(c) else shutil.which("clang++")


def test_host_planner_under_asan_and_ubsan(tmp_path):
    clang = _clang()
    if clang is None:
        pytest.skip("clang++ not available")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = tmp_path / "planner_sanitized"
    cmd = [clang, "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1",
           os.path.join(CSRC, "hs2_api.cpp"), os.path.join(ROOT, "tests", "sanitize", "planner_driver.cpp"),
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "failures: 0" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
