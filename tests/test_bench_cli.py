"""bench.py's command line, checked without a GPU."""
import os
import subprocess
import sys

from conftest import ROOT


def test_bench_refuses_more_than_one_gpu():
    for n in ("2", "8"):
        p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n], cwd=ROOT,
                           stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=60)
        assert p.returncode == 2
        assert "ONE GPU" in p.stderr and p.stdout == ""


def test_traffic_is_reported_only_for_the_profiled_workload_and_source():
    """The committed counter summary gives each main kernel's HBM bytes for the workload it was
    taken on (GPT-175B block, N = 128, rank 63, contributions at the recommended pitch) and for
    the kernel source it was taken with; any other workload or source reports none."""
    import json
    import bench
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    fresh = t["kernel_src_sha256"] == bench.kernel_src_hash()
    got = bench.load_traffic("gpt175b", 128, 63, "pitched")
    if fresh:
        assert set(got) >= {"grad_reduce", "copyout", "adamw", "flatten"}
        for n in ("grad_reduce", "copyout", "adamw", "flatten"):
            v = t["per_kernel"][n]
            assert got[n] == v["read_bytes"] + v["write_bytes"] > 0
        assert got["copyout"] == t["copyout_hbm_bytes_per_launch"]
    else:
        assert got == {}
    assert bench.load_traffic("gpt175b", 128, 0, "pitched") == {}
    assert bench.load_traffic("gpt175b", 120, 59, "pitched") == {}
    assert bench.load_traffic("gpt175b", 128, 63, "stacked") == {}
    assert bench.load_traffic("t5", 128, 63, "pitched") == {}
