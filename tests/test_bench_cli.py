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


def test_mean_split_and_time_statistics():
    """The mean over N ranks is split into pre * post = N with pre = 2^floor(floor(log2 N) / 2),
    the power of two with pre^2 <= N < 4 pre^2; kernel times report the nearest-rank median and
    p90."""
    import bench
    assert bench.pre_post(1) == (1.0, 1.0)
    assert bench.pre_post(3) == (1.0, 3.0)
    assert bench.pre_post(4) == (2.0, 2.0)
    assert bench.pre_post(8) == (2.0, 4.0)
    assert bench.pre_post(128) == (8.0, 16.0)
    assert bench.pre_post(120) == (8.0, 15.0)
    for n in range(1, 300):
        pre, post = bench.pre_post(n)
        assert pre * post == n and pre == 2.0 ** ((n.bit_length() - 1) // 2)
        assert pre * pre <= n < 4 * pre * pre
    assert bench.time_stats([3.0]) == (3.0, 3.0, 3.0, 3.0)
    assert bench.time_stats([4.0, 1.0, 3.0, 2.0]) == (2.5, 2.5, 1.0, 4.0)
    ms = [float(v) for v in range(10, 0, -1)]
    mean, med, lo, p90 = bench.time_stats(ms)
    assert (mean, med, lo, p90) == (5.5, 5.5, 1.0, 9.0)


def test_committed_counter_traffic_matches_the_algorithmic_bytes():
    """The committed PMC summary (GPT-175B block, N = 128, rank 63) shows every main kernel
    reading and writing its algorithmic bytes to within 0.2%: no wasted re-reads."""
    import json
    import bench
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    S, T = 14_157_024, 1_812_099_072
    alg = {"copyout": (4 * T, 2 * T), "grad_reduce": (2 * 128 * S, 4 * S),
           "adamw": (16 * S, 12 * S), "flatten": (4 * S, 4 * S)}
    for name, (rd, wr) in alg.items():
        k = t["per_kernel"][name]
        assert abs(k["read_bytes"] / rd - 1) < 2e-3, (name, k["read_bytes"], rd)
        assert abs(k["write_bytes"] / wr - 1) < 2e-3, (name, k["write_bytes"], wr)
    assert t["copyout_hbm_bytes_per_launch"] == sum(t["per_kernel"]["copyout"].values())
