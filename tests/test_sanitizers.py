"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code (no
GPU): the C oracle (oracle/race_oracle.c, OpenMP) driven on small inputs in
every input type, and libraceattn's host-side shape validation and buffer
layouts (linear_lsh_sketch_amd/csrc/race_host.hpp) over valid, boundary and
invalid shapes. Any sanitizer report aborts the driver (no recovery), so the
test fails on the first one."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1",
           OMP_NUM_THREADS="2")


def _run(cmd_build, exe, tmp_path):
    r = subprocess.run(cmd_build, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    print(r.stdout.strip())
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "ERROR" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", *SAN, "-fopenmp", "-std=c11", os.path.join(HERE, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "race_oracle.c"), "-o", exe, "-lm"], exe, tmp_path)


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_validation_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_driver")
    _run(["g++", *SAN, "-std=c++17", "-I", os.path.join(ROOT, "include"),
          "-I", os.path.join(ROOT, "linear_lsh_sketch_amd", "csrc"), os.path.join(HERE, "host_driver.cpp"),
          "-o", exe], exe, tmp_path)
