"""Address- and undefined-behaviour-sanitizer builds of the host code (CPU).

The oracle (oracle/mc2_oracle.c) and libmc2's host-side validation
(csrc/validate.cpp) are compiled with gcc / g++ and
-fsanitize=address,undefined -fno-sanitize-recover into two small drivers
(tests/sanitize/) that call every entry point on small inputs, valid and
invalid; any out-of-bounds access, overflow or invalid shift fails the run.
The GPU kernels are not built here (the sanitizers are host-only).
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd_build, exe, tmp_path):
    r = subprocess.run(cmd_build, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="2")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    return r.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    out = _run(["gcc", "-std=c11", "-fopenmp", "-ffp-contract=off", *SAN,
                os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), os.path.join(ROOT, "oracle", "mc2_oracle.c"),
                "-o", exe, "-lm"], exe, tmp_path)
    assert "clean" in out


def test_validation_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "validate_driver")
    out = _run(["g++", "-std=c++17", *SAN, f"-I{ROOT}/include", f"-I{ROOT}/comm_matmul_tensor_amd/csrc",
                os.path.join(ROOT, "tests", "sanitize", "validate_driver.cpp"),
                os.path.join(ROOT, "comm_matmul_tensor_amd", "csrc", "validate.cpp"), "-o", exe], exe, tmp_path)
    assert "clean" in out
