"""The host code under the address and undefined-behaviour sanitizers (CPU
only): the float64 oracle (oracle/flce_oracle.c) through a C driver, and the
library's host planners (linear_cross_entropy_amd/csrc/flce_plan.h, plain C++
shared with the GPU library) through a C++ driver that plans the test and
workload shapes, seeded random shapes and extreme or invalid sizes and checks
every accepted plan's invariants. Built with gcc / g++ only; no GPU code is
built with a sanitizer."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
           OMP_NUM_THREADS="4")


def _run(cmd, exe, tmp_path):
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    run = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300, cwd=tmp_path)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr, run.stderr[-4000:]
    return run.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_check")
    out = _run(["gcc", "-std=c11", "-fopenmp", "-fno-fast-math", "-ffp-contract=off", *SAN,
                os.path.join(ROOT, "oracle", "flce_oracle.c"), os.path.join(ROOT, "tests", "sanitize", "oracle_check.c"),
                "-o", exe, "-lm"], exe, tmp_path)
    assert "oracle_check ok" in out


@pytest.mark.skipif(shutil.which("g++") is None, reason="no g++")
def test_host_planners_under_sanitizers(tmp_path):
    exe = str(tmp_path / "plan_check")
    out = _run(["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"),
                "-I", os.path.join(ROOT, "linear_cross_entropy_amd", "csrc"),
                os.path.join(ROOT, "tests", "sanitize", "plan_check.cpp"), "-o", exe], exe, tmp_path)
    assert "plan_check ok" in out
