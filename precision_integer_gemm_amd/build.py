"""Ahead-of-time build of the HIP library for gfx950 (MI355X).

    python -m precision_integer_gemm_amd.build

compiles csrc/lpgemm_api.hip (which includes every kernel) with hipcc into
precision_integer_gemm_amd/_lpgemm.so, next to this file, and the measurement
probe csrc/ceiling_probe.hip into _ceiling.so (loaded only by bench.py).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "lpgemm_api.hip")
LIB = os.path.join(PKG, "_lpgemm.so")
PROBE_SRC = os.path.join(PKG, "csrc", "ceiling_probe.hip")
PROBE_LIB = os.path.join(PKG, "_ceiling.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library needs ROCm's hipcc")


def command(out: str, src: str = SRC) -> list[str]:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
        # packed fp32 VALU forms are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # the scaled epilogue's roundings are part of its definition: no
        # contraction of a multiply into a fused operation
        "-ffp-contract=off",
        "-Wall", "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
        "-o", out, src,
    ]


def compile_one(src: str, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    proc = subprocess.run(command(tmp, src), capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (proc.stdout + proc.stderr).splitlines() if noise not in l]
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    compile_one(SRC, LIB, verbose)
    compile_one(PROBE_SRC, PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
