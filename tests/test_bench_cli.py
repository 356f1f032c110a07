"""bench.py's command line on the CPU: one GPU only, and the trace summary."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=120,
                          env={**os.environ, **(env or {})})


def test_more_than_one_gpu_is_refused():
    p = _bench("--gpus", "2")
    assert p.returncode == 2
    assert "one GPU only" in p.stderr and p.stdout == ""


def test_a_second_rank_is_refused():
    p = _bench(env={"WORLD_SIZE": "2"})
    assert p.returncode == 2
    assert "WORLD_SIZE 2" in p.stderr


def test_trace_summary_groups_kernels_by_name_and_grid(tmp_path):
    csv = tmp_path / "trace.csv"
    rows = ["Kernel_Name,Grid_Size,Workgroup_Size,Start_Timestamp,End_Timestamp",
            "kern_a,1024,256,0,1000", "kern_a,1024,256,5000,8000",
            "kern_a,4096,256,10000,10500", "kern_b,64,64,20000,20100"]
    csv.write_text("\n".join(rows) + "\n")
    p = _bench("--trace-summary", str(csv))
    assert p.returncode == 0, p.stderr
    lines = [l for l in p.stdout.splitlines() if l.startswith("| kern_")]
    assert len(lines) == 3
    cells = {tuple(c.strip() for c in l.split("|")[1:3]): [c.strip() for c in l.split("|")[1:-1]]
             for l in lines}
    assert cells[("kern_a", "1024")][3:] == ["2", "2000", "1000", "3000"]
    assert cells[("kern_a", "4096")][3:] == ["1", "500", "500", "500"]
    assert cells[("kern_b", "64")][3:] == ["1", "100", "100", "100"]
