"""bench.py keeps its output contract: one JSON line with the required keys, consistent
per-kernel numbers, the roofline object of the dominant kernel and the CPU baseline."""
import json
import os
import subprocess
import sys

import pytest

from conftest import ROOT

pytestmark = pytest.mark.gpu

REQUIRED = ["metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
            "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config", "kernels",
            "roofline", "cpu_baseline"]


def _run(*args, timeout=240):
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=timeout)
    return p


def test_bench_json_line_on_the_tiny_unit():
    p = _run("--workload", "tiny", "--steps", "5", "--warmup", "1", "--next", "--sweep-ranks",
             "--graph", "on")
    assert p.returncode == 0, p.stderr[-2000:]
    lines = [l for l in p.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in REQUIRED:
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 1
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True and d["data"] == "synthetic"
    assert set(d["kernels"]) == {"grad_reduce", "copyout", "adamw", "flatten"}
    step_bytes = sum(k["bytes"] for k in d["kernels"].values())
    assert abs(d["value"] - step_bytes / (d["ms_per_step"] * 1e-3) / 1e9) <= 0.01 * d["value"] + 0.1
    # the tiny unit fits the Infinity Cache: kernels run after a flush, the step is their sum
    assert d["config"]["step_time"].startswith("sum of the kernels")
    assert abs(d["ms_per_step"] - sum(k["ms"] for k in d["kernels"].values())) < 1e-3
    for k in d["kernels"].values():
        assert k["ms_min"] <= k["ms_median"] <= k["ms_p90"]
    pr = d["per_rank"]
    assert pr["ranks"] == [0, 1, 2, 3]
    for k in pr["ranks"]:
        assert set(pr[str(k)]) == {"grad_reduce", "adamw", "flatten"}
    assert set(pr["worst"]) == {"grad_reduce", "adamw", "flatten"}
    gr = d["graph"]
    assert gr["ms_per_step"] > 0 and abs(gr["value"] - step_bytes / (gr["ms_per_step"] * 1e-3) / 1e9) \
        <= 0.01 * gr["value"] + 0.1
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["peak"] == 8000.0 and r["unit"] == "GB/s"
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    import bench
    assert d["kernel_src_sha256"] == bench.kernel_src_hash()
    # the committed counter summary covers the GPT-175B unit only
    assert r["traffic"] is None and all(k["traffic"] is None for k in d["kernels"].values())
    # the headline step runs at the rank whose flatten the sweep measured slowest
    assert d["config"]["rank"] == pr["worst"]["flatten"]["rank"]
    assert "slowest" in d["config"]["rank_choice"]
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["cores"] == bench.host_threads() and c["value"] > 0
    assert c["sample"] and set(c["per_kernel_gbs"]) == {"flatten", "copyout", "grad_reduce", "adamw"}
    one = c["single_core"]
    assert one["cores"] == 1 and one["kind"] == "oracle" and one["value"] > 0
    assert "copyin_bf16_all_ranks" in d["next_rows"]


def test_bench_headline_from_graph_replays_without_flush():
    """Without a flush the step is timed from HIP-graph replays; the eager loop is kept."""
    p = _run("--workload", "tiny", "--steps", "5", "--warmup", "1", "--flush", "off",
             "--no-cpu-baseline")
    assert p.returncode == 0, p.stderr[-2000:]
    d = json.loads([l for l in p.stdout.splitlines() if l.startswith("{")][0])
    assert d["config"]["step_time"] == "wall clock of HIP-graph replays of the step"
    step_bytes = sum(k["bytes"] for k in d["kernels"].values())
    assert abs(d["value"] - step_bytes / (d["ms_per_step"] * 1e-3) / 1e9) <= 0.01 * d["value"] + 0.1
    assert d["eager"]["ms_per_step"] > 0 and "graph" not in d
    # the copy ceiling is on by default
    assert d["copy_ceiling"]["ceiling_GB/s"] > 0
    p = _run("--workload", "tiny", "--steps", "2", "--warmup", "1", "--no-cpu-baseline",
             "--no-next", "--no-sweep-ranks", "--no-copy-probe")
    assert p.returncode == 0, p.stderr[-2000:]
    d = json.loads([l for l in p.stdout.splitlines() if l.startswith("{")][0])
    assert "copy_ceiling" not in d and all("frac_of_copy_ceiling" not in k for k in d["kernels"].values())


def test_bench_defaults_probes_and_opt_outs():
    """The rank sweep is on by default (and --no-sweep-ranks removes it); the copy and floor
    probes report what they measure; every line says how its kernel times were taken."""
    p = _run("--workload", "tiny", "--steps", "2", "--warmup", "1", "--no-cpu-baseline",
             "--no-next", "--copy-probe", "--floor-probe", "--contention-probe")
    assert p.returncode == 0, p.stderr[-2000:]
    d = json.loads([l for l in p.stdout.splitlines() if l.startswith("{")][0])
    assert "per_rank" in d and "timing" in d["per_rank"] and "kernel_timing" in d
    assert "next_rows" not in d
    cp = d["copy_ceiling"]
    runs = {k: v for k, v in cp.items() if isinstance(v, dict)}
    assert set(runs) == {"library_copy", "hipMemcpyDtoD"} and all(v["GB/s"] > 0 for v in runs.values())
    assert cp["ceiling_GB/s"] == max(v["GB/s"] for v in runs.values())
    for k in d["kernels"].values():
        assert abs(k["frac_of_copy_ceiling"] - k["GB/s"] / cp["ceiling_GB/s"]) < 1e-3
    ff = d["flatten_floor"]
    N = d["config"]["N"]
    assert len(ff["order"]) == 5 + len({0, 1, max(0, N // 2 - 1), N - 1})
    assert set(ff["cases"]) == set(ff["order"])
    assert all(c["event_ms_median"] > 0 for c in ff["cases"].values())
    ct = d["contention"]
    for kernel in ("tiles", "sweep"):
        assert all(ct[kernel][key] > 0 for key in ("reduce_alone_ms", "reduce_overlapped_ms",
                                                   "gemm_overlapped_ms", "both_done_wall_ms"))
    fl = d["floor_probe"]
    assert [f["elements"] for f in fl] == [1 << lg for lg in range(20, 28)]
    assert all(f["bytes"] == 8 * f["elements"] and f["event_ms_median"] > 0 for f in fl)
    p = _run("--workload", "tiny", "--steps", "2", "--warmup", "1", "--no-cpu-baseline",
             "--no-next", "--no-sweep-ranks")
    assert p.returncode == 0, p.stderr[-2000:]
    d = json.loads([l for l in p.stdout.splitlines() if l.startswith("{")][0])
    assert "per_rank" not in d


def test_bench_reduce_shapes_probe():
    """The reduction-shape probe reports both kernels for every flat and hybrid shape it runs,
    with the bytes of each reduction."""
    p = _run("--workload", "tiny", "--steps", "1", "--warmup", "1", "--no-cpu-baseline",
             "--no-next", "--no-sweep-ranks", "--reduce-shapes", timeout=300)
    assert p.returncode == 0, p.stderr[-2000:]
    d = json.loads([l for l in p.stdout.splitlines() if l.startswith("{")][0])
    import bench
    rs = d["reduce_shapes"]
    assert [(r["ranks"], r["outputs"]) for r in rs if r["group"] == 0] == bench.REDUCE_SHAPES_FLAT
    assert [(r["ranks"], r["outputs"]) for r in rs if r["group"] == 8] == bench.REDUCE_SHAPES_HYBRID
    for r in rs:
        assert r["bytes"] == (2 * r["ranks"] + (8 if r["accumulate"] else 4)) * r["outputs"]
        assert r["accumulate"] == (r["group"] > 0)
        for k in ("tiles", "sweep"):
            assert r[k]["event_ms_median"] > 0 and r[k]["GB/s"] > 0
