"""The narrow-M kernel's first wait, checked in its compiled code (no GPU).

The kernel issues the first strip's direct-to-LDS copies, then A's loads, and
its first `s_waitcnt vmcnt(n)` leaves n operations in flight: n must not
exceed the number of vector-memory operations issued after the last copy, or
the wait could pass before the strip has landed (the whole-line A instances
wait for everything, n = 0).  The loads are counted in
the source (one per step for packed int4 A, two for int8 A); this test builds
every instance the library uses to assembly and counts them in the code the
compiler actually emitted.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "precision_integer_gemm_amd", "csrc")

INSTANCES = [(var, ks, out, False, False) for var in ("W4A8", "I4I4") for ks in (1, 2, 4)
             for out in ("OUT_I32", "OUT_F32", "OUT_BF16", "OUT_F16")]
INSTANCES += [(var, 4, "OUT_I32", True, False) for var in ("W4A8", "I4I4")]
# int8 A over more than 8 rows: whole-line A loads, whose first wait is vmcnt(0)
INSTANCES += [("W4A8", ks, out, False, True) for ks in (1, 2, 4)
              for out in ("OUT_I32", "OUT_F32", "OUT_BF16", "OUT_F16")]
INSTANCES += [("W4A8", 4, "OUT_I32", True, True)]


def _source():
    lines = ['#include "gemm_skinny.hpp"', "namespace lpgemm {"]
    for var, ks, out, split, whole in INSTANCES:
        lines.append(f"template __global__ void gemm_skinny_kernel<{var}, 16, {ks}, {out}, "
                     f"{'true' if split else 'false'}, {'true' if whole else 'false'}>(const uint8_t *, "
                     "const uint8_t *, Epilogue, int, int, int, int);")
    lines.append("}")
    return "\n".join(lines) + "\n"


def first_wait_margin(body):
    """(copies, operations issued after the last copy, n of the first vmcnt wait)."""
    copies = younger = 0
    for line in body.splitlines():
        t = line.strip()
        if t.startswith("s_waitcnt") and "vmcnt" in t:
            return copies, younger, int(re.search(r"vmcnt\((\d+)\)", t).group(1))
        if t.startswith(("buffer_", "global_", "flat_")):
            if re.search(r"\blds\b", t):
                copies, younger = copies + 1, 0
            else:
                younger += 1
    return copies, younger, None


def test_first_wait_covers_the_first_strip(tmp_path):
    hipcc = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")
    if hipcc is None:
        pytest.skip("hipcc not found")
    src = tmp_path / "skinny_instances.hip"
    src.write_text(_source())
    asm = tmp_path / "skinny_instances.s"
    p = subprocess.run([hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-S",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-ffp-contract=off",
                        "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", str(asm), str(src)],
                       capture_output=True, text=True, timeout=600)
    assert p.returncode == 0, p.stdout + p.stderr
    text = asm.read_text()
    bodies = re.findall(r"^(_ZN6lpgemm18gemm_skinny_kernel\S*):[^\n]*\n(.*?)s_endpgm", text, re.M | re.S)
    assert len(bodies) == len(INSTANCES)
    for name, body in bodies:
        copies, younger, n = first_wait_margin(body)
        ks = int(re.search(r"ILi\dELi16ELi(\d)E", name).group(1))
        assert copies == ks, name
        assert n is not None and younger >= n, (name, copies, younger, n)


def test_margin_counter_on_a_hand_written_body():
    body = """
        buffer_load_dwordx4 v1, s[0:3], 0 offen nt lds
        buffer_load_dwordx4 v1, s[0:3], 0 offen nt lds
        buffer_load_dwordx4 v[2:5], v6, s[4:7], 0 offen
        s_waitcnt vmcnt(1)
    """
    assert first_wait_margin(body) == (2, 1, 1)
    assert first_wait_margin("s_waitcnt lgkmcnt(0)\nbuffer_load_dword v1, v2, s[0:3], 0 offen lds\n") == (1, 0, None)
