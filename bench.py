#!/usr/bin/env python3
"""Benchmark of the low-precision integer GEMM on one MI355X.

One step = one call of every workload (the whole hot path: the block-tiled
MFMA kernel for the square and ragged shapes, the narrow-M kernel for the
decode-like W4A8 shapes):

    i4i4 256^3, i4i4 1024^3, W4A8 4096^3, W4A8 16x28672x8192,
    W4A8 1x28672x8192 (same B values, own copy), i4i4 8192^3,
    i4i4 3000x5120x6144

value = sum of 2*M*N*K over the step / wall time per step, in TOP/s.  Inputs
are seeded synthetic bytes already resident in HBM when timing starts; each
call writes its own int32 C.  An instrumented pass of K steps before the timed
region brackets every launch with HIP events on the stream it runs on; its
per-launch averages give each workload's TOP/s and roofline fraction
(`per_config`) and pick the dominant kernel.  The timed region (K steps, the
wall time behind `value`) brackets only the dominant kernel's launches, whose
average gives `roofline`; `ms_per_step_events_every_launch` is the
instrumented pass's step time.
`per_config_isolated` times each workload alone (back-to-back launches, the
decode-shape B rotated over copies larger than the MALL together), free of the
write-back a previous workload leaves behind; `per_config_cold` times each
workload after a 512 MiB read that evicts its operands from L2 and MALL;
`per_config_scaled_bf16` times the scaled product (per-row and per-column
scales, bf16 output) of each workload alone; `per_config_fp8` times the second
workload, the fp8 GEMM (e4m3 and e5m2 operands) with fp32 output, at 4096^3
and 8192^3; `per_config_blockscaled` the per-K-block scaled product (g = 128
and 32, bf16 output) on three workloads; and `per_config_long_k` W4A8 decode
shapes with K = 28672 on the narrow-M kernel's split-K path (all outside the
step and `value`).  `ceiling` holds what the chip sustains, measured
live by the probe kernels of _ceiling.so (matrix cores only, per format; LDS
reads; the FP6 GEMM's inner loop without global memory), and `roofline`
adds the dominant call's fraction of the sustained ceiling of its format.

The CPU baseline times the oracle (plain C, OpenMP over rows) on the first
rows of every workload, and those rows double as a bit-exact parity check of
the GPU output.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--case NAME] [--no-cpu]
    python bench.py --ceiling      # the sustained-ceiling probes alone
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks (dense): int8 MFMA 5.0 POP/s, fp8 5.0 PFLOP/s, FP6
# 10.1 PFLOP/s, HBM3E 8 TB/s.  A workload is priced at the peak of the matrix-core format its
# kernel computes in: int4 x int4 calls that run on the FP6 path at the FP6
# peak, everything else at the int8 peak.
PEAK_INT8_TOPS = 5000.0
PEAK_FP8_TOPS = 5000.0
PEAK_FP6_TOPS = 10100.0
PEAK_HBM_GBS = 8000.0
# Vector ALU, one non-packed 32-bit operation per lane: the published fp32
# vector peak (157.3 TFLOP/s) counts packed FMAs (2 flops x 2 values per
# lane slot), so one plain operation per lane per cycle is a quarter of it:
# 256 CUs x 64 lanes x 2.4 GHz = 39.3 T lane-operations/s.
PEAK_VALU_TOPS = 157.3 / 4.0
# Per output element and K block, the block-scaled product needs at least
# four binary32 operations: convert the partial, two multiplies, one add.
BLOCK_OPS = 4

# Step order: each W4A8 skinny call reads a B that no call has touched for
# >= 300 MB of other traffic, so it streams from HBM, not the 256 MB MALL.
STEP_ORDER = ["w4a8_skinny_m16", "i4i4_8192", "w4a8_skinny_m1", "w4a8_4096", "i4i4_ragged",
              "i4i4_256", "i4i4_1024"]

KERNEL_SYMBOL = {"tiled": "gemm_pipelined_kernel", "skinny": "gemm_skinny_kernel",
                 "general": "gemm_general_kernel",
                 "fp6": "fp6_convert_pair_kernel + gemm_fp6_kernel"}


def mfma_peak(kernel: str) -> float:
    return PEAK_FP6_TOPS if kernel == "fp6" else PEAK_INT8_TOPS


# Sustained ceilings, measured live by the probe kernels of _ceiling.so
# (csrc/ceiling_probe.hip): one workgroup per compute unit keeps the matrix
# cores (or the LDS) busy for a few milliseconds, long enough for the clock to
# settle at what the chip holds under that load.  A GEMM's `sustained_frac`
# sets its throughput against the ceiling of the matrix-core format it runs on.
PROBES = [("fp6_mfma", 0, 24000), ("int8_mfma", 1, 24000), ("fp8_mfma", 2, 12000),
          ("lds_read", 3, 40000), ("fp6_gemm_inner_loop", 4, 12000)]


# The HBM counterpart: one streaming pass over a buffer of the decode shapes'
# packed weights (N * K / 2 bytes), rotated over three copies like the
# isolated decode timing so that every pass reads HBM rather than the 256 MB
# MALL.  The default run times the best configurations of the sweep below
# (`bench.py --stream-sweep`, kept in profiles/) and reports the fastest:
# direct-to-LDS loads of 1 KB per wave instruction with the non-temporal hint,
# one 1024-thread workgroup per compute unit, two pieces in flight per wave;
# buffer loads, 8 x 256 threads per compute unit, one 16-byte non-temporal
# load in flight; the same with 2 x 256 threads and four in flight.
STREAM_COPIES, STREAM_REPS = 3, 21
STREAM_BEST = [(1, 1, 1024, 2, 2), (0, 8, 256, 1, 2), (0, 2, 256, 4, 2)]  # mode, wg/CU, threads, in flight, policy


def stream_read_ceiling(torch, dev, stream, lib, nbytes: int, cus: int) -> dict:
    import ctypes

    lib.ceiling_probe_stream_sweep.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                                               ctypes.c_void_p]
    lib.ceiling_probe_stream_sweep.restype = ctypes.c_int
    n_out = 8 * cus * 1024
    out = torch.empty(n_out, dtype=torch.int32, device=dev)
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device=dev) for _ in range(STREAM_COPIES)]
    best = None
    for mode, wpc, threads, inflight, pol in STREAM_BEST:
        us = []
        for r in range(STREAM_REPS + STREAM_COPIES):  # the first pass over each copy is a warm-up
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            st = lib.ceiling_probe_stream_sweep(bufs[r % STREAM_COPIES].data_ptr(), nbytes, mode,
                                                wpc * cus, threads, inflight, pol, out.data_ptr(),
                                                n_out, stream.cuda_stream)
            e1.record(stream)
            if st != 0:
                raise RuntimeError(f"stream-read probe: status {st}")
            torch.cuda.synchronize()
            if r >= STREAM_COPIES:
                us.append(e0.elapsed_time(e1) * 1e3)
        med = float(np.median(us))
        rec = {"bytes": nbytes, "median_us": round(med, 3), "min_us": round(float(np.min(us)), 3),
               "gb_s": round(nbytes / (med * 1e-6) / 1e9, 1),
               "config": {"loads": "to_lds" if mode else "buffer", "wg_per_cu": wpc,
                          "threads": threads, "in_flight": inflight, "policy": "nt"}}
        if best is None or med < best["median_us"]:
            best = rec
    del bufs
    return best


# The sweep of single streaming passes over the decode shapes' 117 MB: buffer
# loads (workgroups per compute unit, loads in flight per thread, cache
# policy) and direct-to-LDS loads (workgroups, 1 KB pieces in flight per
# wave, non-temporal or not), each over three rotated copies.
SWEEP_BUF = [(w, 256, f, pol) for w in (2, 4, 8, 16, 32) for f in (1, 2, 4, 8) for pol in (0, 2, 1, 16, 18)]
SWEEP_DMA = [(1, 1024, f, pol) for f in (2, 4, 8) for pol in (0, 2)] + \
            [(2, 512, f, pol) for f in (4, 8) for pol in (0, 2)] + \
            [(4, 256, f, pol) for f in (4, 8, 16) for pol in (0, 2)] + \
            [(8, 256, f, 2) for f in (4, 8)]
# The narrow-M GEMM's own copy pattern without its arithmetic: 64 KB strips
# per workgroup, wave w copying row w as four 1 KB `nt` pieces; in flight 0 =
# one strip per workgroup with a barrier per strip (the GEMM's schedule), else
# that many pieces per wave with no barrier.
SWEEP_STRIP = [(1, 1024, f, 2) for f in (0, 4, 8)]


def stream_sweep(torch, dev, stream, nbytes: int) -> dict:
    import ctypes

    lib = ctypes.CDLL(os.path.join(ROOT, "precision_integer_gemm_amd", "_ceiling.so"))
    lib.ceiling_probe_stream_sweep.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                                               ctypes.c_void_p]
    lib.ceiling_probe_stream_sweep.restype = ctypes.c_int
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device=dev) for _ in range(STREAM_COPIES)]
    n_out = 32 * cus * 1024
    out = torch.empty(n_out, dtype=torch.int32, device=dev)
    rows = []
    for mode, table in ((0, SWEEP_BUF), (1, SWEEP_DMA), (2, SWEEP_STRIP)):
        for wpc, threads, inflight, pol in table:
            us = []
            for r in range(STREAM_REPS + STREAM_COPIES):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                st = lib.ceiling_probe_stream_sweep(bufs[r % STREAM_COPIES].data_ptr(), nbytes, mode,
                                                    wpc * cus, threads, inflight, pol, out.data_ptr(),
                                                    n_out, stream.cuda_stream)
                e1.record(stream)
                if st != 0:
                    raise RuntimeError(f"stream sweep {mode} {wpc} {threads} {inflight} {pol}: {st}")
                torch.cuda.synchronize()
                if r >= STREAM_COPIES:
                    us.append(e0.elapsed_time(e1) * 1e3)
            med = float(np.median(us))
            rows.append({"loads": ("buffer", "to_lds", "strips")[mode], "wg_per_cu": wpc,
                         "threads": threads, "in_flight": inflight,
                         "policy": {0: "-", 1: "sc0", 2: "nt", 16: "sc1", 18: "sc1 nt"}[pol],
                         "median_us": round(med, 2), "min_us": round(float(np.min(us)), 2),
                         "gb_s": round(nbytes / (med * 1e-6) / 1e9, 1)})
            print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
    best = min(rows, key=lambda r: r["median_us"])
    return {"bytes": nbytes, "configs": len(rows), "best": best, "rows": rows}


# C-store patterns (`ceiling_probe_store`): 256 workgroups per 64 MB of int32
# C, each writing one 256 x 256 tile in the tiled GEMMs' MFMA layout (32 bytes
# of 32 rows per instruction), as whole 1 KB rows, or staged through LDS as
# the GEMMs' last tile is; four rotated output buffers.
STORE_SHAPES = [(4096, 4096), (3072, 5120), (8192, 8192)]
STORE_PATTERNS = {0: "mfma_layout", 1: "whole_rows", 2: "lds_staged"}


def store_probe(torch, dev, stream) -> dict:
    import ctypes

    lib = ctypes.CDLL(os.path.join(ROOT, "precision_integer_gemm_amd", "_ceiling.so"))
    lib.ceiling_probe_store.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_void_p]
    lib.ceiling_probe_store.restype = ctypes.c_int
    out = []
    for M, N in STORE_SHAPES:
        bufs = [torch.empty((M, N), dtype=torch.int32, device=dev) for _ in range(4)]
        for p in STORE_PATTERNS:  # each pattern writes {m, n, 0, 0} at (m, n .. n + 3)
            bufs[0].fill_(-1)
            if lib.ceiling_probe_store(p, bufs[0].data_ptr(), M, N, stream.cuda_stream) != 0:
                raise RuntimeError(f"store probe {p} {M}x{N} failed")
            v = bufs[0].view(M, N // 4, 4)
            ok = bool((v[:, :, 0] == torch.arange(M, device=dev).view(M, 1)).all()) and \
                bool((v[:, :, 1] == torch.arange(0, N, 4, device=dev).view(1, N // 4)).all())
            if not ok:
                raise RuntimeError(f"store probe {p} {M}x{N} wrote a wrong element")
        us = {name: [] for name in STORE_PATTERNS.values()}
        n = 0
        for r in range(STREAM_REPS + 3):
            for p, name in STORE_PATTERNS.items():
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                lib.ceiling_probe_store(p, bufs[n % 4].data_ptr(), M, N, stream.cuda_stream)
                e1.record(stream)
                torch.cuda.synchronize()
                n += 1
                if r >= 3:
                    us[name].append(e0.elapsed_time(e1) * 1e3)
        med = {k: round(float(np.median(v)), 2) for k, v in us.items()}
        out.append({"M": M, "N": N, "bytes": M * N * 4, "median_us": med,
                    "tb_s": {k: round(M * N * 4 / (v * 1e-6) / 1e12, 2) for k, v in med.items()}})
        print(json.dumps(out[-1]), file=sys.stderr, flush=True)
        del bufs
    return {"store_patterns": out}


def sustained_ceilings(torch, dev, stream, reps: int = 3, stream_bytes: int = 0) -> dict:
    import ctypes

    path = os.path.join(ROOT, "precision_integer_gemm_amd", "_ceiling.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    lib.ceiling_probe_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                     ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.ceiling_probe_wall_clock_khz.restype = ctypes.c_int
    lib.ceiling_probe_run.restype = ctypes.c_int
    lib.ceiling_probe_work.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.ceiling_probe_work.restype = ctypes.c_double
    lib.ceiling_probe_out_floats.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.ceiling_probe_out_floats.restype = ctypes.c_int64
    blocks = torch.cuda.get_device_properties(dev).multi_processor_count
    n_out = max(lib.ceiling_probe_out_floats(k, blocks) for _, k, _ in PROBES)
    out = torch.empty(n_out, dtype=torch.float32, device=dev)
    clk = torch.zeros(2 * blocks, dtype=torch.int64, device=dev)
    wall_khz = lib.ceiling_probe_wall_clock_khz()
    lib.ceiling_probe_max_clock_khz.restype = ctypes.c_int
    max_khz = lib.ceiling_probe_max_clock_khz()
    res = {"compute_units": blocks, "max_sclk_mhz": round(max_khz / 1000.0, 1) if max_khz > 0 else None}
    for name, kind, iters in PROBES:
        ms, mhz = [], []
        for r in range(reps + 1):  # the first launch is a warm-up
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            st = lib.ceiling_probe_run(kind, blocks, iters, out.data_ptr(), n_out, clk.data_ptr(),
                                       stream.cuda_stream)
            e1.record(stream)
            if st != 0:
                raise RuntimeError(f"ceiling probe {name}: status {st}")
            torch.cuda.synchronize()
            if r:
                ms.append(e0.elapsed_time(e1))
                # shader clock over the loop: shader-clock ticks per constant-rate
                # tick, averaged over the workgroups
                c = clk.cpu().numpy().reshape(blocks, 2).astype(np.float64)
                if wall_khz > 0 and (c[:, 1] > 0).all():
                    mhz.append(float(np.mean(c[:, 0] / c[:, 1])) * wall_khz / 1000.0)
        t = float(np.median(ms)) * 1e-3
        work = lib.ceiling_probe_work(kind, blocks, iters)
        if name == "lds_read":
            res[name] = {"tb_s": round(work / t / 1e12, 2),
                         "gb_s_per_cu": round(work / t / 1e9 / blocks, 1), "ms": round(t * 1e3, 3)}
        else:
            res[name] = {"tops": round(work / t / 1e12, 1), "ms": round(t * 1e3, 3)}
        if mhz:
            res[name]["sclk_mhz"] = round(float(np.median(mhz)), 1)
    if stream_bytes:
        res["hbm_stream_read"] = stream_read_ceiling(torch, dev, stream, lib, stream_bytes, blocks)
    return res


# HBM traffic of the dominant call, from two rocprofv3 --pmc runs (FETCH_SIZE,
# then WRITE_SIZE, KiB per dispatch, summed over the call's dispatches: the
# FP6 re-encoding of both operands and the GEMM), each scaled by what the same counter
# reads for a plain 256 MiB device copy (bench.py --copy-calibration 256):
# FETCH_SIZE reads 131072 KiB for 256 MiB read (x2.0), WRITE_SIZE 262144 KiB
# for 256 MiB written (x1.0).  Valid only for the kernel sources it was taken
# on (their SHA-256 below); any change reports null until re-measured.
TRAFFIC = {
    "i4i4_8192": {"fetch_kib": 328244.3, "fetch_scale": 2.0, "write_kib": 361274.0,
                  "write_scale": 1.0, "sources_sha256": "da139566518226640ac6925e97a82a29bde159baca7c6af30b721540fe476688"},
}
TRAFFIC_SOURCES = ["precision_integer_gemm_amd/csrc/gemm_pipelined.hpp",
                   "precision_integer_gemm_amd/csrc/gemm_fp6.hpp",
                   "precision_integer_gemm_amd/csrc/device_common.hpp",
                   "precision_integer_gemm_amd/csrc/lpgemm_api.hip"]


def sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    t = TRAFFIC.get(workload)
    if t is None or t["sources_sha256"] != sources_sha256():
        return None
    return int(t["fetch_kib"] * 1024 * t["fetch_scale"] + t["write_kib"] * 1024 * t["write_scale"])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--case", action="append", default=None,
                    help="restrict the step to these workloads (profiling)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline and parity rows")
    ap.add_argument("--cpu-macs", type=float, default=6e11,
                    help="multiply-accumulates per workload in the CPU baseline sample")
    ap.add_argument("--isolated-reps", type=int, default=20,
                    help="back-to-back launches per workload for the isolated per-kernel times")
    ap.add_argument("--cold-reps", type=int, default=10,
                    help="launches per workload, each after a 512 MiB read that evicts L2 and MALL")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--ceiling", action="store_true",
                    help="run only the sustained-ceiling probes and print their JSON")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the sustained-ceiling probes")
    ap.add_argument("--stream-sweep", action="store_true",
                    help="only sweep the streaming-read probe over the decode weights' size")
    ap.add_argument("--store-probe", action="store_true",
                    help="only time the C-store pattern probes (MFMA layout, whole rows, staged)")
    ap.add_argument("--trace-summary", metavar="CSV",
                    help="summarise a rocprofv3 kernel_trace.csv per kernel and grid (no GPU use)")
    return ap.parse_args()


def trace_summary(path: str) -> int:
    """Average duration per (kernel, grid) of a rocprofv3 kernel trace, so one
    kernel template used by several workloads is split by launch shape."""
    import csv
    from collections import defaultdict
    groups = defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0]
            grid = int(r.get("Grid_Size", r.get("Grid_Size_X", 0)) or 0)
            wg = int(r.get("Workgroup_Size", r.get("Workgroup_Size_X", 0)) or 0)
            dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            groups[(name, grid, wg)].append(dur)
    print("| kernel | grid (threads) | workgroup | calls | avg ns | min ns | max ns |")
    print("|---|---|---|---|---|---|---|")
    for (name, grid, wg), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        print(f"| {name} | {grid} | {wg} | {len(d)} | {sum(d) / len(d):.0f} | {min(d)} | {max(d)} |")
    return 0


def cpu_model() -> str:
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def roofline_time_s(case, kernel: str = "tiled") -> tuple[float, str]:
    t_mfma = case.ops / (mfma_peak(kernel) * 1e12)
    t_hbm = case.alg_bytes / (PEAK_HBM_GBS * 1e9)
    return (t_mfma, "mfma") if t_mfma >= t_hbm else (t_hbm, "hbm")


def main() -> int:
    args = parse()
    if args.trace_summary:
        return trace_summary(args.trace_summary)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the GEMM shards by N or M with no exchange, and the benchmark runs and reports "
              "a single GPU.", file=sys.stderr)
        return 2

    import torch

    import precision_integer_gemm_amd as L
    from precision_integer_gemm_amd.inputs import CASES, operands

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    L.lib()

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}))
        return 0

    decode = CASES["w4a8_skinny_m16"]
    stream_bytes = decode.N * decode.K // 2  # the decode shapes' packed weights
    if args.ceiling:
        print(json.dumps({"ceiling": sustained_ceilings(torch, dev, torch.cuda.current_stream(),
                                                        stream_bytes=stream_bytes)}))
        return 0
    if args.stream_sweep:
        print(json.dumps({"stream_sweep": stream_sweep(torch, dev, torch.cuda.current_stream(),
                                                       stream_bytes)}))
        return 0
    if args.store_probe:
        print(json.dumps(store_probe(torch, dev, torch.cuda.current_stream())))
        return 0

    names = [n for n in STEP_ORDER if args.case is None or n in args.case]
    work = []
    for name in names:
        c = CASES[name]
        A, B = operands(c)
        a = torch.from_numpy(np.ascontiguousarray(A).view(np.uint8)).to(dev)
        b = torch.from_numpy(B).to(dev)  # each workload owns its B copy
        C = torch.empty((c.M, c.N), dtype=torch.int32, device=dev)
        # the entry point with a caller-owned workspace, allocated here, outside
        # the timed region (the FP6 path's re-encoded operands for 8192^3)
        fn = L.lib().lpgemm_int4_int4_ws if c.variant == "i4i4" else L.lib().lpgemm_w4a8_ws
        variant = L.VARIANT_I4I4 if c.variant == "i4i4" else L.VARIANT_W4A8
        nws = L.lpgemm_workspace_size(variant, c.M, c.N, c.K)
        ws_t = torch.empty(nws + L.WORKSPACE_ALIGN, dtype=torch.uint8, device=dev)
        ws = ws_t.data_ptr() + (-ws_t.data_ptr()) % L.WORKSPACE_ALIGN if nws else None
        plan = L.lpgemm_plan(variant, c.M, c.N, c.K, a.data_ptr(), b.data_ptr(), C.data_ptr(),
                             workspace_bytes=nws)
        work.append(dict(case=c, A=A, B=B, a=a, b=b, C=C, fn=fn, plan=plan, ws=ws, nws=nws,
                         ws_t=ws_t))
        print(f"# {name}: {c.variant} {c.M}x{c.N}x{c.K} plan {plan}", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    handle = stream.cuda_stream

    def call(w, b=None):
        c = w["case"]
        st = w["fn"](w["a"].data_ptr(), (b if b is not None else w["b"]).data_ptr(),
                     w["C"].data_ptr(), c.M, c.N, c.K, w["ws"], w["nws"], handle)
        if st != L.OK:
            raise RuntimeError(f"{c.name}: {L.lpgemm_status_string(st)}")

    for _ in range(args.warmup):
        for w in work:
            call(w)
    torch.cuda.synchronize()
    print(f"# warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    # Instrumented pass (outside the timed region): every launch bracketed by
    # HIP events, for each workload's per-launch time and to pick the
    # dominant kernel.  An event record between every pair of launches costs
    # the step tens of microseconds (the command processor handles each
    # marker between the kernels), so the timed region below brackets only
    # the dominant workload's launches.
    events = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in work] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        for i, w in enumerate(work):
            events[s][i][0].record(stream)
            call(w)
            events[s][i][1].record(stream)
    torch.cuda.synchronize()
    wall_instrumented = time.perf_counter() - t0

    ops_step = sum(w["case"].ops for w in work)
    per_config = {}
    dominant = None
    for i, w in enumerate(work):
        c = w["case"]
        us = np.array([events[s][i][0].elapsed_time(events[s][i][1]) * 1e3
                       for s in range(args.steps)])
        avg = float(us.mean())
        t_roof, bound = roofline_time_s(c, w["plan"]["kernel"])
        rec = {"kernel": w["plan"]["kernel"], "avg_us": round(avg, 3),
               "median_us": round(float(np.median(us)), 3), "min_us": round(float(us.min()), 3),
               "p90_us": round(float(np.percentile(us, 90)), 3),
               "tops": round(c.ops / (avg * 1e-6) / 1e12, 2),
               "gbs": round(c.alg_bytes / (avg * 1e-6) / 1e9, 1),
               "bound": bound, "roofline_frac": round(t_roof / (avg * 1e-6), 4)}
        if bound == "mfma":
            rec["mfma_peak_tops"] = mfma_peak(w["plan"]["kernel"])
            rec["int8_peak_frac"] = round(c.ops / (avg * 1e-6) / 1e12 / PEAK_INT8_TOPS, 4)
        per_config[c.name] = rec
        total = avg * args.steps
        if dominant is None or total > dominant[0]:
            dominant = (total, i)

    # The timed region: exactly K steps, events only around the dominant
    # workload's launches (on the stream they run on).
    dom_i = dominant[1]
    dom_events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        for i, w in enumerate(work):
            if i == dom_i:
                dom_events[s][0].record(stream)
                call(w)
                dom_events[s][1].record(stream)
            else:
                call(w)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"# timed {args.steps} steps in {wall:.3f} s "
          f"(instrumented pass {wall_instrumented:.3f} s)", file=sys.stderr, flush=True)
    dom_us = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in dom_events])
    dc = work[dom_i]["case"]
    drec = dict(per_config[dc.name])
    davg = float(dom_us.mean())
    dom_timed = {"avg_us": round(davg, 3), "median_us": round(float(np.median(dom_us)), 3),
                 "min_us": round(float(dom_us.min()), 3),
                 "p90_us": round(float(np.percentile(dom_us, 90)), 3)}

    # Each workload alone: back-to-back launches, B rotated over enough copies
    # that every launch streams B from HBM (three copies exceed the 256 MB
    # MALL for the decode shape), so no launch pays for another workload's
    # write-back and none reads a cache-warm B.
    isolated = {}
    if args.isolated_reps > 0:
        for w in work:
            c = w["case"]
            copies = [w["b"]] + [w["b"].clone() for _ in range(2 if c.b_bytes > (64 << 20) else 0)]
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.isolated_reps)]
            call(w)
            for j, (e0, e1) in enumerate(evs):
                e0.record(stream)
                call(w, copies[j % len(copies)])
                e1.record(stream)
            torch.cuda.synchronize()
            us = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs])
            med = float(np.median(us))
            t_roof, bound = roofline_time_s(c, w["plan"]["kernel"])
            isolated[c.name] = {"median_us": round(med, 3), "min_us": round(float(us.min()), 3),
                                "p90_us": round(float(np.percentile(us, 90)), 3),
                                "tops": round(c.ops / (med * 1e-6) / 1e12, 2),
                                "gbs": round(c.alg_bytes / (med * 1e-6) / 1e9, 1),
                                "bound": bound, "roofline_frac": round(t_roof / (med * 1e-6), 4)}
            if w["plan"]["kernel"] == "fp6":
                # the same workload forced onto the int8 256-tile kernel, for comparison
                L.lpgemm_set_kernel_override(L.KERNEL_TILED_256)
                try:
                    evs8 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                            for _ in range(args.isolated_reps)]
                    call(w)
                    for e0, e1 in evs8:
                        e0.record(stream)
                        call(w)
                        e1.record(stream)
                    torch.cuda.synchronize()
                finally:
                    L.lpgemm_set_kernel_override(L.KERNEL_AUTO)
                us8 = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs8])
                med8 = float(np.median(us8))
                isolated[c.name]["int8_path"] = {
                    "median_us": round(med8, 3), "tops": round(c.ops / (med8 * 1e-6) / 1e12, 2),
                    "int8_peak_frac": round(c.ops / (med8 * 1e-6) / 1e12 / PEAK_INT8_TOPS, 4)}
            del copies

    # The scaled product (per-row / per-column scales, bf16 output) of every
    # workload alone, timed like `per_config_isolated`: the same GEMM with the
    # scaling epilogue; D is half the bytes of the int32 C.
    scaled = {}
    if args.isolated_reps > 0:
        from precision_integer_gemm_amd.inputs import scale_vector
        for w in work:
            c = w["case"]
            sa = torch.from_numpy(scale_vector(c.seed, 0, c.M)).to(dev)
            sb = torch.from_numpy(scale_vector(c.seed, 1, c.N)).to(dev)
            D = torch.empty((c.M, c.N), dtype=torch.bfloat16, device=dev)
            if c.variant == "i4i4":  # with the workspace (the FP6 path for 8192^3)
                def fn(a_, b_, sa_, sb_, d_, o_, m_, n_, k_, h_, w=w):
                    return L.lib().lpgemm_int4_int4_scaled_ws(a_, b_, sa_, sb_, d_, o_, m_, n_, k_,
                                                              w["ws"], w["nws"], h_)
            else:
                fn = L.lib().lpgemm_w4a8_scaled
            copies = [w["b"]] + [w["b"].clone() for _ in range(2 if c.b_bytes > (64 << 20) else 0)]
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.isolated_reps)]
            for j in range(-1, args.isolated_reps):
                if j >= 0:
                    evs[j][0].record(stream)
                st = fn(w["a"].data_ptr(), copies[max(j, 0) % len(copies)].data_ptr(), sa.data_ptr(),
                        sb.data_ptr(), D.data_ptr(), L.OUT_BF16, c.M, c.N, c.K, handle)
                if j >= 0:
                    evs[j][1].record(stream)
                if st != L.OK:
                    raise RuntimeError(f"{c.name} scaled: {L.lpgemm_status_string(st)}")
            torch.cuda.synchronize()
            us = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs])
            med = float(np.median(us))
            d_bytes = c.a_bytes + c.b_bytes + 2 * c.M * c.N + 4 * (c.M + c.N)
            t_mfma = c.ops / (mfma_peak(w["plan"]["kernel"]) * 1e12)
            t_hbm = d_bytes / (PEAK_HBM_GBS * 1e9)
            scaled[c.name] = {"out": "bf16", "median_us": round(med, 3),
                              "tops": round(c.ops / (med * 1e-6) / 1e12, 2),
                              "gbs": round(d_bytes / (med * 1e-6) / 1e9, 1),
                              "bound": "mfma" if t_mfma >= t_hbm else "hbm",
                              "roofline_frac": round(max(t_mfma, t_hbm) / (med * 1e-6), 4)}
            del copies, D

    # The per-K-block scaled product (bf16 output) on three workloads, g = 128
    # and 32, alone and timed like `per_config_scaled_bf16`.  Its roofline
    # takes the largest of the matrix-core time, the HBM time and the vector
    # ALU time of BLOCK_OPS operations per output element and block.
    blockscaled = {}
    if args.isolated_reps > 0:
        from precision_integer_gemm_amd.inputs import block_scale_table
        by_name = {w["case"].name: w for w in work}
        for name, g in (("w4a8_4096", 128), ("w4a8_4096", 32), ("i4i4_8192", 128),
                        ("w4a8_skinny_m16", 128)):
            if name not in by_name:
                continue
            w = by_name[name]
            c = w["case"]
            nb = -(-c.K // g)
            sfa = torch.from_numpy(block_scale_table(c.seed, 0, c.M, c.K, g)).to(dev)
            sfb = torch.from_numpy(block_scale_table(c.seed, 1, c.N, c.K, g)).to(dev)
            D = torch.empty((c.M, c.N), dtype=torch.bfloat16, device=dev)
            fn = L.lib().lpgemm_int4_int4_blockscaled if c.variant == "i4i4" else L.lib().lpgemm_w4a8_blockscaled
            copies = [w["b"]] + [w["b"].clone() for _ in range(2 if c.b_bytes > (64 << 20) else 0)]
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.isolated_reps)]
            for j in range(-1, args.isolated_reps):
                if j >= 0:
                    evs[j][0].record(stream)
                st = fn(w["a"].data_ptr(), copies[max(j, 0) % len(copies)].data_ptr(), sfa.data_ptr(),
                        sfb.data_ptr(), g, D.data_ptr(), L.OUT_BF16, c.M, c.N, c.K, handle)
                if j >= 0:
                    evs[j][1].record(stream)
                if st != L.OK:
                    raise RuntimeError(f"{c.name} blockscaled: {L.lpgemm_status_string(st)}")
            torch.cuda.synchronize()
            us = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs])
            med = float(np.median(us))
            d_bytes = c.a_bytes + c.b_bytes + 2 * c.M * c.N + 4 * nb * (c.M + c.N)
            t_mfma = c.ops / (PEAK_INT8_TOPS * 1e12)
            t_hbm = d_bytes / (PEAK_HBM_GBS * 1e9)
            t_alu = BLOCK_OPS * c.M * c.N * nb / (PEAK_VALU_TOPS * 1e12)
            t_roof = max(t_mfma, t_hbm, t_alu)
            bound = "mfma" if t_roof == t_mfma else "hbm" if t_roof == t_hbm else "alu"
            blockscaled[f"{name}_g{g}"] = {
                "out": "bf16", "g": g, "median_us": round(med, 3), "min_us": round(float(us.min()), 3),
                "tops": round(c.ops / (med * 1e-6) / 1e12, 2), "gbs": round(d_bytes / (med * 1e-6) / 1e9, 1),
                "roofline_us": {"mfma": round(t_mfma * 1e6, 2), "hbm": round(t_hbm * 1e6, 2),
                                "alu": round(t_alu * 1e6, 2)},
                "bound": bound, "roofline_frac": round(t_roof / (med * 1e-6), 4)}
            del copies, D

    # The second workload, the fp8 GEMM (e4m3 and e5m2 operands) with fp32
    # accumulation and fp32 output, alone (not part of the step or of `value`): priced at the
    # 5.0 PFLOP/s dense fp8 peak.
    fp8 = {}
    if args.isolated_reps > 0:
        from precision_integer_gemm_amd.inputs import fp8_codes
        for fmt, (fm, fn_, fk) in [(f, s) for f in ("e4m3", "e5m2")
                                   for s in ((4096, 4096, 4096), (8192, 8192, 8192))]:
            a8 = torch.from_numpy(fp8_codes(fm + fk, 0, fm, fk, fmt)).to(dev)
            b8 = torch.from_numpy(fp8_codes(fm + fk, 1, fn_, fk, fmt)).to(dev)
            c8 = torch.empty((fm, fn_), dtype=torch.float32, device=dev)
            entry = L.lib().lpgemm_fp8_e4m3 if fmt == "e4m3" else L.lib().lpgemm_fp8_e5m2
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.isolated_reps)]
            for j in range(-1, args.isolated_reps):
                if j >= 0:
                    evs[j][0].record(stream)
                st = entry(a8.data_ptr(), b8.data_ptr(), c8.data_ptr(), L.OUT_F32, fm, fn_, fk, handle)
                if j >= 0:
                    evs[j][1].record(stream)
                if st != L.OK:
                    raise RuntimeError(f"fp8 {fmt} {fm}x{fn_}x{fk}: {L.lpgemm_status_string(st)}")
            torch.cuda.synchronize()
            us = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs])
            med = float(np.median(us))
            tops = 2.0 * fm * fn_ * fk / (med * 1e-6) / 1e12
            fp8[f"fp8_{fmt}_{fm}x{fn_}x{fk}"] = {
                "out": "f32", "median_us": round(med, 3), "min_us": round(float(us.min()), 3),
                "tops": round(tops, 2), "bound": "mfma", "mfma_peak_tops": PEAK_FP8_TOPS,
                "roofline_frac": round(tops / PEAK_FP8_TOPS, 4)}
            del a8, b8, c8

    # W4A8 decode shapes with K beyond one workgroup's 8192 (the split-K path
    # of the narrow-M kernel: K ranges added into C), alone, weights rotated
    # over three copies like the isolated decode calls; against HBM.
    long_k = {}
    if args.isolated_reps > 0:
        from precision_integer_gemm_amd.inputs import custom_operands
        for (lm, ln, lk) in ((16, 8192, 28672), (1, 8192, 28672)):
            A_h, B_h = custom_operands("w4a8", lm, ln, lk, seed=lk + lm)
            la = torch.from_numpy(np.ascontiguousarray(A_h).view(np.uint8)).to(dev)
            lbs = [torch.from_numpy(B_h).to(dev)]
            lbs += [lbs[0].clone() for _ in range(2)]
            lc = torch.empty((lm, ln), dtype=torch.int32, device=dev)
            plan = L.lpgemm_plan(L.VARIANT_W4A8, lm, ln, lk, la.data_ptr(), lbs[0].data_ptr(),
                                 lc.data_ptr())
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.isolated_reps)]
            for j in range(-1, args.isolated_reps):
                if j >= 0:
                    evs[j][0].record(stream)
                st = L.lib().lpgemm_w4a8(la.data_ptr(), lbs[max(j, 0) % 3].data_ptr(), lc.data_ptr(),
                                         lm, ln, lk, handle)
                if j >= 0:
                    evs[j][1].record(stream)
                if st != L.OK:
                    raise RuntimeError(f"w4a8 {lm}x{ln}x{lk}: {L.lpgemm_status_string(st)}")
            torch.cuda.synchronize()
            us = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs])
            med = float(np.median(us))
            alg = ln * lk // 2 + lm * lk + 4 * lm * ln
            long_k[f"w4a8_{lm}x{ln}x{lk}"] = {
                "kernel": plan["kernel"], "k_chunks": plan["k_chunks"],
                "median_us": round(med, 3), "min_us": round(float(us.min()), 3),
                "gbs": round(alg / (med * 1e-6) / 1e9, 1), "bound": "hbm",
                "roofline_frac": round(alg / (PEAK_HBM_GBS * 1e9) / (med * 1e-6), 4)}
            del la, lbs, lc

    # Each workload cold: before every timed launch a 512 MiB buffer is read
    # (not timed), which evicts its operands from the L2s and the 256 MB MALL
    # with clean lines (a write would leave 512 MB of write-back competing
    # with the timed launch).
    cold = {}
    if args.cold_reps > 0:
        flush = torch.ones(128 << 20, dtype=torch.int32, device=dev)  # 512 MiB
        for w in work:
            c = w["case"]
            evs = []
            for j in range(args.cold_reps):
                flush.max()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                call(w)
                e1.record(stream)
                evs.append((e0, e1))
            torch.cuda.synchronize()
            us = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs])
            med = float(np.median(us))
            t_roof, bound = roofline_time_s(c, w["plan"]["kernel"])
            cold[c.name] = {"median_us": round(med, 3), "min_us": round(float(us.min()), 3),
                            "p90_us": round(float(np.percentile(us, 90)), 3),
                            "tops": round(c.ops / (med * 1e-6) / 1e12, 2),
                            "gbs": round(c.alg_bytes / (med * 1e-6) / 1e9, 1),
                            "bound": bound, "roofline_frac": round(t_roof / (med * 1e-6), 4)}
        del flush

    ceiling = (None if args.no_ceiling
               else sustained_ceilings(torch, dev, stream, stream_bytes=stream_bytes))
    if ceiling is not None:
        # The decode records against one streaming pass over their weights.
        sus_gbs = ceiling["hbm_stream_read"]["gb_s"]
        decode_names = [w["case"].name for w in work if w["plan"]["kernel"] == "skinny"]
        decode_names += list(long_k)
        for recs in (per_config, isolated, cold, long_k):
            for name in decode_names:
                if name in recs:
                    recs[name]["stream_read_gbs"] = sus_gbs
                    recs[name]["stream_read_frac"] = round(recs[name]["gbs"] / sus_gbs, 4)

    if drec["bound"] == "mfma":
        achieved = dc.ops / (davg * 1e-6) / 1e12
        peak = mfma_peak(drec["kernel"])
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TOP/s", "frac": round(achieved / peak, 4),
                "int8_peak_frac": round(achieved / PEAK_INT8_TOPS, 4)}
        if ceiling is not None:
            sus = ceiling["fp6_mfma" if drec["kernel"] == "fp6" else "int8_mfma"]["tops"]
            roof["sustained_peak"] = sus
            roof["sustained_frac"] = round(achieved / sus, 4)
    else:
        achieved = dc.alg_bytes / (davg * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roof.update({"traffic": measured_traffic(dc.name), "traffic_unit": "bytes per launch",
                 "kernel": KERNEL_SYMBOL[drec["kernel"]], "workload": dc.name,
                 "avg_us": round(davg, 3), "timed_region": dom_timed})

    result = {
        "metric": "int4/W4A8 GEMM TOPS (2MNK/s) and % of int8 MFMA or HBM roofline, 1 GPU",
        "value": round(ops_step * args.steps / wall / 1e12, 2),
        "unit": "TOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "ms_per_step_events_every_launch": round(wall_instrumented / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8-mfma/int32 and fp6-e3m2-mfma/fp32 (exact; int4 and int8 operands)",
        "data": "synthetic (seeded SplitMix64 bytes: uniform int8, uniform int4 nibbles)",
        "config": {"workload": "lpgemm suite: " + ", ".join(w["case"].name for w in work),
                   "cases": {w["case"].name: [w["case"].variant, w["case"].M, w["case"].N,
                                              w["case"].K] for w in work},
                   "ops_per_step": ops_step, "parallelism": "single GPU"},
        "roofline": roof,
        "per_config": per_config,
        "per_config_isolated": isolated,
        "per_config_cold": cold,
        "per_config_scaled_bf16": scaled,
        "per_config_fp8": fp8,
        "per_config_blockscaled": blockscaled,
        "per_config_long_k": long_k,
        "ceiling": ceiling,
    }
    if ceiling is not None:
        # the shader clock measured under sustained matrix-core load (the
        # probes' own clock counters), and the device's maximum
        result["sclk_mhz"] = {"max": ceiling.get("max_sclk_mhz"),
                              **{f"under_{k}": ceiling[k]["sclk_mhz"] for k in
                                 ("int8_mfma", "fp6_mfma", "fp8_mfma", "fp6_gemm_inner_loop")
                                 if "sclk_mhz" in ceiling.get(k, {})}}

    if not args.no_cpu:
        import oracle

        total_ops, total_t, parity_ok, sample = 0.0, 0.0, True, []
        for w in work:
            c = w["case"]
            rows = int(max(1, min(c.M, args.cpu_macs // (c.N * c.K))))
            a_rows = w["A"][:rows]
            t = time.perf_counter()
            if c.variant == "i4i4":
                ref = oracle.gemm_i4i4(a_rows, w["B"], rows, c.N, c.K)
            else:
                ref = oracle.gemm_w4a8(a_rows, w["B"], rows, c.N, c.K)
            dt = time.perf_counter() - t
            total_ops += 2.0 * rows * c.N * c.K
            total_t += dt
            got = w["C"][:rows].cpu().numpy()
            parity_ok &= bool(np.array_equal(got, ref))
            sample.append(f"{c.name}[:{rows}]")
            print(f"# cpu oracle {c.name} rows {rows}: {dt:.2f} s, parity "
                  f"{np.array_equal(got, ref)}", file=sys.stderr, flush=True)
        # one host thread on the two small workloads, whole
        threads = oracle.num_threads()
        one_thread = {}
        oracle.set_num_threads(1)
        try:
            for w in work:
                c = w["case"]
                if c.name not in ("i4i4_256", "i4i4_1024"):
                    continue
                t = time.perf_counter()
                oracle.gemm_i4i4(w["A"], w["B"], c.M, c.N, c.K)
                dt = time.perf_counter() - t
                one_thread[c.name] = {"s": round(dt, 4), "tops": round(c.ops / dt / 1e12, 6)}
        finally:
            oracle.set_num_threads(threads)
        result["cpu_baseline"] = {
            "value": round(total_ops / total_t / 1e12, 5), "unit": "TOP/s",
            "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "first rows of every workload (" + ", ".join(sample) +
                      f"), {total_t:.1f} s wall on {threads} threads",
            "one_thread": one_thread}
        result["parity_sampled_rows"] = parity_ok

    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
