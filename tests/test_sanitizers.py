"""AddressSanitizer and UndefinedBehaviorSanitizer runs on the CPU (no GPU).

* The oracle (plain C) built with gcc -fsanitize=address,undefined and driven
  through every entry point by tests/sanitize/oracle_check.c.
* The library's host code -- argument checks, kernel planning, workspace
  sizing, the scratch-limit check -- built with hipcc, the sanitizers applied
  to host code only (-Xarch_host), and driven by tests/sanitize/host_check.cpp
  over a grid of several million shapes and argument combinations; no call
  there reaches a kernel launch.
Any sanitizer report aborts the driver (-fno-sanitize-recover), which fails
the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")


def _run(cmd, cwd, timeout):
    p = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=timeout)
    return p.returncode, p.stdout + p.stderr


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_check")
    rc, out = _run(["gcc", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-std=c11",
                    "-ffp-contract=off", "-Wall", "-Wextra", "-o", exe,
                    os.path.join(HERE, "oracle_check.c"), os.path.join(ROOT, "oracle", "lpgemm_oracle.c"),
                    "-lm"], ROOT, 300)
    assert rc == 0, out
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", OMP_NUM_THREADS="2")
    p = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert p.returncode == 0, p.stdout + p.stderr
    assert "all checks passed" in p.stdout


def test_library_host_paths_under_asan_ubsan(tmp_path):
    hipcc = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")
    if hipcc is None:
        pytest.skip("hipcc not found")
    exe = str(tmp_path / "host_check")
    csrc = os.path.join(ROOT, "precision_integer_gemm_amd", "csrc")
    rc, out = _run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-ffp-contract=off",
                    "-I", os.path.join(ROOT, "include"), "-I", csrc, "-o", exe,
                    os.path.join(HERE, "host_check.cpp"), os.path.join(csrc, "lpgemm_api.hip")],
                   ROOT, 900)
    assert rc == 0, out
    p = subprocess.run([exe], capture_output=True, text=True, timeout=600,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"))
    assert p.returncode == 0, p.stdout + p.stderr
    assert "all checks passed" in p.stdout
