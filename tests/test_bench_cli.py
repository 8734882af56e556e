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
    taken on (GPT-175B block, N = 128, contributions at the recommended pitch) and for the kernel
    source it was taken with -- the flatten's for each swept rank, the other kernels' for any rank
    (they move the same bytes at every rank); any other workload or source reports none."""
    import json
    import bench
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    fresh = t["kernel_src_sha256"] == bench.kernel_src_hash()
    for k in (0, 1, 63, 127):
        got = bench.load_traffic("gpt175b", 128, k, "pitched")
        if not fresh:
            assert got == {}
            continue
        assert set(got) >= {"grad_reduce", "copyout", "adamw", "flatten"}
        for n in ("grad_reduce", "copyout", "adamw"):
            v = t["per_kernel"][n]
            assert got[n] == v["read_bytes"] + v["write_bytes"] > 0
        v = t["flatten_by_rank"][str(k)]
        assert got["flatten"] == v["read_bytes"] + v["write_bytes"] > 0
    if fresh:
        assert got["copyout"] == t["copyout_hbm_bytes_per_launch"]
        assert "flatten" not in bench.load_traffic("gpt175b", 128, 5, "pitched")  # not swept
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
    """The committed PMC summary (GPT-175B block, N = 128) shows every kernel -- the four calls
    (the flatten for each swept rank) and the next rows -- reading and writing its algorithmic
    bytes to within 0.2%: no wasted re-reads.  Three independent copies calibrate the counters
    (the library's, hipMemcpyDtoD's and torch's elementwise kernel) and agree to 1e-4."""
    import json
    import bench
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    S, T = 14_157_024, 1_812_099_072
    alg = {"copyout": (4 * T, 2 * T), "grad_reduce": (2 * 128 * S, 4 * S),
           "adamw": (16 * S, 12 * S)}
    for name, (rd, wr) in alg.items():
        k = t["per_kernel"][name]
        assert (k["algorithmic_read"], k["algorithmic_write"]) == (rd, wr), name
    for name, k in t["per_kernel"].items():
        assert abs(k["read_bytes"] / k["algorithmic_read"] - 1) < 2e-3, name
        if k["algorithmic_write"]:
            assert abs(k["write_bytes"] / k["algorithmic_write"] - 1) < 2e-3, name
    assert set(t["flatten_by_rank"]) == {"0", "1", "63", "127"}
    for k in t["flatten_by_rank"].values():
        assert abs(k["read_bytes"] / (4 * S) - 1) < 2e-3 and abs(k["write_bytes"] / (4 * S) - 1) < 2e-3
    assert t["copyout_hbm_bytes_per_launch"] == t["per_kernel"]["copyout"]["read_bytes"] + \
        t["per_kernel"]["copyout"]["write_bytes"]
    scales = [(c["fetch_scale"], c["write_scale"]) for c in t["calibrations"].values()]
    assert len(scales) == 3
    for f, w in scales:
        assert abs(f / scales[0][0] - 1) < 1e-4 and abs(w / scales[0][1] - 1) < 1e-4


def test_all_cores_baseline_slices_reassemble_the_single_call_results():
    """The all-cores CPU baseline runs the unchanged oracle on disjoint output slices from
    several threads; its claim that the results are those of one call rests on the slicing.
    Here the slices of each part (flatten of a rank, copy-out of the unit, reduction, AdamW),
    cut exactly as the baseline cuts them, are reassembled and compared bit for bit with one
    call over the whole range, for a padded unit and a rank whose shard straddles parameters."""
    import numpy as np

    import bench
    import oracle
    import workloads as W

    unit = W.gpt2_large_block(N=8)
    N, k, threads = 7, 3, 5  # N = 7 pads the flat buffer; 5 threads cut uneven slices
    params = W.host_params(unit, seed=1)
    numels = [int(np.prod(s)) if len(s) else 1 for s in unit.shapes]
    T = sum(numels)
    S = -(-T // N)
    whole = oracle.flat_shard(params, N, k)
    real = min(S, max(0, T - k * S))
    pieces = [oracle.flat_shard(bench._flat_pieces(params, numels, k * S + a, k * S + b), 1, 0)
              for a, b in bench._slices(real, threads)]
    assert np.array_equal(np.concatenate(pieces).view(np.uint32), whole[:real].view(np.uint32))

    gathered = oracle.flat_shard(params, N, -1)
    want = np.concatenate([o.reshape(-1) for o in oracle.flat_copyout(unit.shapes, gathered)])
    got = np.concatenate([o.reshape(-1)
                          for a, b in bench._slices(T, threads)
                          for o in oracle.flat_copyout(
                              [(x.size,) for x in bench._flat_pieces(params, numels, a, b)],
                              gathered[a:b])])
    assert np.array_equal(got, want)

    n_red = 12345
    c = W.host_contribs(N, n_red, step=2)
    want = oracle.grad_reduce([c[r] for r in range(N)], 2.0, 3.0)
    got = np.concatenate([oracle.grad_reduce([c[r, a:b] for r in range(N)], 2.0, 3.0)
                          for a, b in bench._slices(n_red, threads)])
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))

    hp = dict(lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01)
    p0 = W.host_normal(9999, 0.02, seed=3)
    g = W.host_normal(9999, 1e-3, seed=4)
    p1, m1, v1 = p0.copy(), np.zeros_like(p0), np.zeros_like(p0)
    oracle.adamw(p1, g, m1, v1, step=1, **hp)
    p2, m2, v2 = p0.copy(), np.zeros_like(p0), np.zeros_like(p0)
    for a, b in bench._slices(p0.size, threads):
        oracle.adamw(p2[a:b], g[a:b], m2[a:b], v2[a:b], step=1, **hp)
    for x, y in ((p1, p2), (m1, m2), (v1, v2)):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


def test_every_committed_profile_was_taken_on_the_current_kernels():
    """Each rocprofv3 summary under profiles/ names the sha256 of the kernel source it was taken
    on; all of them must name the current one, so that no figure quoted from them is stale."""
    import glob
    import json
    import re
    import bench
    cur = bench.kernel_src_hash()
    files = sorted(glob.glob(os.path.join(ROOT, "profiles", "*")))
    assert files
    for path in files:
        with open(path) as f:
            text = f.read()
        if path.endswith(".json"):
            assert json.loads(text)["kernel_src_sha256"] == cur, path
        else:
            found = re.findall(r"kernels\.hip sha256: `([0-9a-f]{64})`", text)
            assert found and all(h == cur for h in found), path
