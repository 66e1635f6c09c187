"""The C ABI's argument validation and workspace carving (csrc/api.cpp), built for the CPU with
AddressSanitizer and UndefinedBehaviorSanitizer and driven by tests/native/abi_check.cpp: every entry
point is called with valid and invalid arguments, kernel launchers and HIP calls are stand-ins that
record what they were given (tests/native/abi_stubs.cpp).  Any sanitizer report aborts the run."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = [os.path.join(ROOT, "mixed_precision_moe_amd", "csrc", "api.cpp"),
           os.path.join(ROOT, "tests", "native", "abi_stubs.cpp"),
           os.path.join(ROOT, "tests", "native", "abi_check.cpp")]


def test_abi_validation_under_asan_and_ubsan(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path / "abi_check")
    cmd = [cxx, "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), *SOURCES, "-o", exe]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout
    assert "abi checks passed" in r.stdout
    assert "runtime error" not in r.stdout and "AddressSanitizer" not in r.stdout
