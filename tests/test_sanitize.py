"""Sanitizer builds (CPU): the library's host paths (argument checks,
workspace layout, the decode planner on random and out-of-table CSR lists,
the encode and 8-bit pool layouts) and the fp64 oracle, each compiled with
AddressSanitizer and UndefinedBehaviorSanitizer and run on edge cases; any
report fails the test.  GPU kernels are not involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, cwd):
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=cwd)
    assert r.returncode == 0, f"{' '.join(cmd)} failed:\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the HIP headers")
def test_host_library_under_sanitizers(tmp_path):
    csrc = os.path.join(ROOT, "rank_attention_amd", "csrc")
    exe = str(tmp_path / "host_harness")
    _run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          "-I" + os.path.join(ROOT, "include"), "-I" + csrc, os.path.join(HERE, "host_harness.cpp"),
          os.path.join(csrc, "milo_attn.cpp"), os.path.join(csrc, "milo_encode.cpp"), "-o", exe], tmp_path)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failed expectations" in r.stdout and "ERROR" not in r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", *SAN, os.path.join(HERE, "oracle_driver.c"), "-lm", "-o", exe], tmp_path)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV)
    assert r.returncode == 0, r.stdout + r.stderr
    assert " 0 failures" in r.stdout and "runtime error" not in r.stderr
