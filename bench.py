#!/usr/bin/env python3
"""Benchmark of the per-rank FSDP data path on one MI355X.

One step is one pass of the whole hot path for one rank's share of one FSDP unit:
  grad reduce  (N bf16 gradient contributions -> fp32 shard, pre/post divide)
  copy-out     (gathered fp32 unit -> per-parameter bf16 tensors)
  AdamW        (param/grad/m/v shard, in place)
  flatten      (the unit's fp32 parameters -> this rank's shard)
The four run in that order so that every kernel reads data last touched at least
10 GB of traffic earlier: no input can still sit in the 256 MB Infinity Cache,
and every byte counted comes from HBM.  Inputs are synthetic (seeded normals in
the unit's shapes) and already resident in HBM when the timed region starts.

Default workload: GPT-175B style block unit (d = 12288, 1,812,099,072 fp32
elements), FSDP1 flat sharding over N = 128, at the rank whose flatten a rank
sweep (ranks 0, 1, 63, 127) measured slowest; the 128 contributions sit in one
receive buffer with rows at the library's recommended pitch (S rounded up to
whole 128-byte lines).

Prints one JSON line (metric, value in GB/s over the whole step, per-kernel
GB/s, fraction of the 8 TB/s HBM peak and elements/s, the roofline of the
dominant kernel, and the CPU oracle timed on a bounded sample as a baseline).
The step is timed from replays of a HIP graph that records its launches once
(when no cache flush is needed between kernels, as for the default unit); the
eager loop, one host call and an event pair per call, gives the per-kernel
times and is reported beside it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
METRIC = "achieved HBM GB/s (% of peak) + elements/s per kernel, one FSDP unit"
KERNEL_SRC = os.path.join(ROOT, "sharded_fsdp_flatten_amd", "csrc", "kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gpt175b_block.json")


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gpt175b",
                    choices=["gpt175b", "t5", "gpt2l", "rows", "tiny"])
    ap.add_argument("--rank", type=int, default=None,
                    help="rank k of the headline step (default: the rank whose flatten the rank "
                         "sweep measured slowest; N/2 - 1 with --no-sweep-ranks)")
    ap.add_argument("--ranks", type=int, default=None,
                    help="shard the unit over this many ranks instead of its own N")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--contribs", default="pitched", choices=["pitched", "stacked", "separate"],
                    help="gradient contributions as one receive buffer with rows at the library's "
                         "recommended pitch (S rounded up to whole 128-byte lines; default), as one "
                         "[N, S] buffer with rows S apart, or as N separate allocations")
    ap.add_argument("--next", dest="next", action="store_true", default=True,
                    help="also time the next rows (hybrid + accumulating reduce, bf16 copy-in, "
                         "unscale, cast, bf16 copy-out, local accumulation, sums of squares) in a "
                         "second cold-cache loop (the default)")
    ap.add_argument("--no-next", dest="next", action="store_false",
                    help="time the four calls of the step only")
    ap.add_argument("--flush", default="auto", choices=["auto", "on", "off"],
                    help="read 1 GiB before every timed kernel so that nothing it reads can sit in "
                         "the 256 MB Infinity Cache (auto: on when the copy-out moves < 2 GB, where "
                         "the step order alone does not guarantee it); with flushing, the step time "
                         "is the sum of the kernels' event times")
    ap.add_argument("--sweep-ranks", dest="sweep_ranks", action="store_true", default=True,
                    help="(default) first time flatten, reduce and AdamW for every rank (N <= 8) or "
                         "for ranks 0, 1, N/2-1, N-1, each launch after a 1 GiB read flush "
                         "(`per_rank`); the headline step then runs at the rank whose flatten was "
                         "slowest (reduce and AdamW move the same bytes at every rank)")
    ap.add_argument("--no-sweep-ranks", dest="sweep_ranks", action="store_false",
                    help="skip the rank sweep")
    ap.add_argument("--graph", default="auto", choices=["auto", "on", "off"],
                    help="replay the step from a captured HIP graph (its launches recorded once, "
                         "no host launch overhead per step).  auto: on when no flush is needed, and "
                         "then `value` comes from the graph replays (the eager loop with per-kernel "
                         "events is reported beside it); with a flush the graph is only reported")
    ap.add_argument("--copy-probe", dest="copy_probe", action="store_true", default=True,
                    help="time a plain 4 GiB fp32 copy through the library (N = 1 unit) and "
                         "hipMemcpy device-to-device, as copy ceilings, and give every kernel's "
                         "rate as a fraction of the faster one (default)")
    ap.add_argument("--no-copy-probe", dest="copy_probe", action="store_false",
                    help="skip the copy ceilings")
    ap.add_argument("--floor-probe", action="store_true",
                    help="also split the flatten of one rank shard into what any kernel of its "
                         "shape pays: an empty kernel with the flatten's grid and with one wave, "
                         "a read-only, a write-only and a plain copy kernel over the shard's bytes "
                         "(libfsdpprobe.so), beside the flatten of ranks 0, 1, N/2-1 and N-1; and "
                         "run the library's fp32 copy (flatten of a one-parameter unit, N = 1) at "
                         "8 MB .. 1 GB of traffic.  20 launches each, each after a 1 GiB read, for "
                         "rocprofv3's kernel trace (the event times reported here include event "
                         "overhead)")
    ap.add_argument("--contention-probe", action="store_true",
                    help="also time the reduction on the tile kernel and on the row-major sweep "
                         "alone and while a stream of bf16 GEMMs (a backward pass's compute) runs "
                         "on a second stream of the same priority")
    ap.add_argument("--reduce-shapes", action="store_true",
                    help="also time the reduction on the tile kernel and on the row-major sweep "
                         "over 32, 64 and 128 ranks at 4.2 M to 26.2 M outputs (flat sums) and over "
                         "128 ranks in groups of 8, accumulating, at 3.5 M to 14.2 M outputs: 8 "
                         "launches each after a 1 GiB read, for rocprofv3's kernel trace")
    return ap.parse_args()


def kernel_src_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def load_traffic(workload, N, k, contribs):
    """HBM bytes (read + write) per launch of each kernel, from the committed rocprofv3 counter
    summary, or {} when there is none, it was taken on another workload (unit, N, layout of the
    contributions) or the kernel source changed since it was taken.  The flatten's entry is the
    one of rank k (the summary holds the swept ranks); the other kernels move the same bytes at
    every rank."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return {}
    if t.get("kernel_src_sha256") != kernel_src_hash():
        return {}
    if t.get("bench_args") != {"workload": workload, "N": N, "contribs": contribs}:
        return {}
    out = {n: v["read_bytes"] + v["write_bytes"] for n, v in t.get("per_kernel", {}).items()}
    fl = t.get("flatten_by_rank", {}).get(str(k))
    if fl is not None:
        out["flatten"] = fl["read_bytes"] + fl["write_bytes"]
    return out


def time_stats(ms):
    """Mean, median, min and p90 of a list of kernel times (ms)."""
    srt = sorted(ms)
    n = len(srt)
    med = srt[n // 2] if n % 2 else 0.5 * (srt[n // 2 - 1] + srt[n // 2])
    p90 = srt[min(n - 1, max(0, -(-9 * n // 10) - 1))]
    return sum(ms) / n, med, srt[0], p90


def make_unit(name, ranks=None):
    import workloads as W
    make = {"gpt175b": W.gpt175b_block, "t5": W.t5_11b_block, "gpt2l": W.gpt2_large_block,
            "rows": W.gpt2_large_emb_rows, "tiny": W.tiny_mlp}[name]
    return make() if ranks is None else make(N=ranks)


def pre_post(N):
    """Mean over N ranks split into a pre and a post divide (powers of two when N is)."""
    pre = 1.0
    while pre * pre * 4 <= N:
        pre *= 2.0
    return pre, N / pre


def cpu_baseline(host, unit, N, k, S, valid, pre, post, hp, rows):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    flatten of rank k (whole, it builds the full flat buffer first), copy-out of the whole
    unit, the reduction over the first S/8 outputs of the shard (all N ranks), and AdamW
    on the whole shard.  Single thread."""
    import numpy as np
    import oracle

    t_tot, b_tot, parts = 0.0, 0.0, {}

    t0 = time.perf_counter()
    if rows:
        oracle.rows_shard(host["params"], N, k)
    else:
        oracle.flat_shard(host["params"], N, k)
    dt = time.perf_counter() - t0
    parts["flatten"] = (4 * valid + 4 * S, dt)

    t0 = time.perf_counter()
    if rows:
        oracle.rows_copyout(unit.shapes, N, host["gathered"])
    else:
        oracle.flat_copyout(unit.shapes, host["gathered"])
    dt = time.perf_counter() - t0
    parts["copyout"] = (6 * unit.total, dt)

    n_red = S // 8
    cs = [np.ascontiguousarray(host["contribs"][r, :n_red]) for r in range(N)]
    t0 = time.perf_counter()
    g = oracle.grad_reduce(cs, pre, post)
    dt = time.perf_counter() - t0
    parts["grad_reduce"] = ((2 * N + 4) * n_red, dt)

    p = host["adam_p"].copy()
    gg = host["adam_g"]
    m = np.zeros(S, np.float32)
    v = np.zeros(S, np.float32)
    t0 = time.perf_counter()
    oracle.adamw(p, gg, m, v, step=1, **hp)
    dt = time.perf_counter() - t0
    parts["adamw"] = (28 * S, dt)

    for b, dt in parts.values():
        b_tot += b
        t_tot += dt
    return {
        "value": round(b_tot / t_tot / 1e9, 3),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": ("%s unit, N=%d, rank %d: flatten of the rank (whole), copy-out of the whole "
                   "unit, reduction of the first S/8=%d outputs over all %d ranks, AdamW on the "
                   "whole shard; single-threaded C oracle" % (unit.name, N, k, n_red, N)),
        "cpu_model": host_cpu_model(),
        "host": host_facts(),
        "per_kernel_gbs": {name: round(b / dt / 1e9, 3) for name, (b, dt) in parts.items()},
        "seconds": round(t_tot, 2),
    }


def _slices(n, parts):
    """[a, b) bounds cutting range(n) into `parts` nearly equal pieces (empty ones dropped)."""
    step = -(-n // parts) if n else 0
    return [(a, min(n, a + step)) for a in range(0, n, step)] if n else []


def _flat_pieces(params, numels, lo, hi):
    """1-D pieces of the concatenated parameters covering flat elements [lo, hi)."""
    out, off = [], 0
    for p, n in zip(params, numels):
        a, b = max(lo, off), min(hi, off + n)
        if a < b:
            out.append(p.reshape(-1)[a - off:b - off])
        off += n
    return out


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_facts():
    """The host the baseline ran on: logical CPUs the machine has, those this process may use,
    and its memory."""
    ram_gb = None
    try:
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal:"):
                    ram_gb = round(int(line.split()[1]) * 1024 / 1e9, 1)
                    break
    except (OSError, ValueError, IndexError):
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = None
    return {"nproc": os.cpu_count(), "usable_cpus": usable, "ram_gb": ram_gb}


def cpu_baseline_all_cores(host, unit, N, k, S, valid, pre, post, hp, rows, threads):
    """The same sample as cpu_baseline, with the unchanged single-threaded oracle run on
    disjoint output slices by `threads` host threads at once (its C calls release the GIL;
    every output element is independent, so results are those of one call): the flatten and
    the copy-out of a FLAT unit cut into slices of the flat range (each slice's parameter
    pieces flattened or cast as a unit of their own), the reduction and AdamW cut into slices
    of the shard.  The rows layout's flatten and copy-out take whole parameters per thread."""
    from concurrent.futures import ThreadPoolExecutor
    import numpy as np
    import oracle

    parts = {}
    numels = [int(np.prod(s)) if len(s) else 1 for s in unit.shapes]
    T = sum(numels)
    with ThreadPoolExecutor(max_workers=threads) as pool:
        def run(jobs):
            t0 = time.perf_counter()
            for f in [pool.submit(j) for j in jobs]:
                f.result()
            return time.perf_counter() - t0

        if rows:
            groups = [list(range(i, len(unit.shapes), threads)) for i in range(threads)]
            jobs = [lambda g=g: oracle.rows_shard([host["params"][i] for i in g], N, k)
                    for g in groups if g]
        else:
            jobs = [lambda a=a, b=b: oracle.flat_shard(
                _flat_pieces(host["params"], numels, k * S + a, k * S + b), 1, 0)
                for a, b in _slices(min(S, max(0, T - k * S)), threads)]
        parts["flatten"] = (4 * valid + 4 * S, run(jobs))

        g = host["gathered"]
        if rows:
            # a parameter's rows sit in every rank's segment: one call per parameter group
            jobs = [lambda: oracle.rows_copyout(unit.shapes, N, g)]
        else:
            jobs = [lambda a=a, b=b: oracle.flat_copyout(
                [(x.size,) for x in _flat_pieces(host["params"], numels, a, b)], g[a:b])
                for a, b in _slices(T, threads)]
        parts["copyout"] = (6 * unit.total, run(jobs))

        n_red = S // 8
        c = host["contribs"]
        jobs = [lambda a=a, b=b: oracle.grad_reduce([c[r, a:b] for r in range(N)], pre, post)
                for a, b in _slices(n_red, threads)]
        parts["grad_reduce"] = ((2 * N + 4) * n_red, run(jobs))

        p = host["adam_p"].copy()
        gg = host["adam_g"]
        m = np.zeros(S, np.float32)
        v = np.zeros(S, np.float32)
        jobs = [lambda a=a, b=b: oracle.adamw(p[a:b], gg[a:b], m[a:b], v[a:b], step=1, **hp)
                for a, b in _slices(S, threads)]
        parts["adamw"] = (28 * S, run(jobs))

    b_tot = sum(b for b, _ in parts.values())
    t_tot = sum(t for _, t in parts.values())
    return {
        "value": round(b_tot / t_tot / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": ("the single-core sample (%s unit, N=%d, rank %d), each part cut into disjoint "
                   "output slices run by %d threads at once%s" % (
                       unit.name, N, k, threads,
                       "; the rows layout's copy-out on one thread" if rows else "")),
        "per_kernel_gbs": {name: round(b / dt / 1e9, 3) for name, (b, dt) in parts.items()},
        "seconds": round(t_tot, 2),
        "cpu_model": host_cpu_model(),
        "host": host_facts(),
    }


def host_threads():
    """Host threads for the all-cores baseline: the cores this process may run on, at most 16
    (one GPU's share of its host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def time_next_rows(B, u, unit, args, N, k, S, L, T, pre, post, contrib_rows, grad, outs,
                   gathered, adam_p, stream, flush=None):
    """The next rows, in an order where no kernel reads what one of the last few wrote:
    hybrid reduction (groups of 8 ranks) accumulating into the grad shard; copy-in of
    per-parameter bf16 gradients into the ReduceScatter input (all ranks); unscale of the
    grad shard (sharded gradient scaler); cast of rank k's fp32 shard to bf16; bf16
    copy-out of a gathered bf16 unit; local fp32 accumulation of an unsharded bf16
    gradient; per-parameter sums of squares of the grad shard.  Reuses the step's buffers
    as inputs (values do not matter)."""
    import torch
    dev = grad.device
    rs_input = torch.empty(L, dtype=torch.bfloat16, device=dev)
    shard16 = torch.empty(S, dtype=torch.bfloat16, device=dev)
    group = 8 if N % 8 == 0 and N > 8 else 0
    flag = torch.zeros(1, device=dev)
    sq_ws = torch.empty(max(1, B.fsdp_grad_sqnorm_workspace(u, k)), dtype=torch.float64, device=dev)
    sq_out = torch.empty(len(unit.shapes), dtype=torch.float64, device=dev)
    valid = u.info(k)["valid"]
    rows = {
        "grad_reduce_hybrid_accumulate": (lambda: B.fsdp_grad_reduce_shard_ex(
            u, contrib_rows, pre, post, grad, group=group, accumulate=True), (2 * N + 8) * S, S),
        "copyin_bf16_all_ranks": (lambda: B.fsdp_flatten_shard_bf16(
            u, outs, B.FSDP_ALL_RANKS, rs_input), 2 * T + 2 * L, L),
        # inv_scale 1 keeps the shard's values from one repetition to the next
        "grad_unscale_rank": (lambda: B.fsdp_grad_unscale(u, k, grad, 1.0, flag), 8 * S, S),
        "cast_to_bf16_rank": (lambda: B.fsdp_cast_to_bf16(u, k, adam_p, shard16), 6 * S, S),
        "copyout_bf16": (lambda: B.fsdp_unflatten_copyout_bf16(u, rs_input, outs), 4 * T, T),
        "grad_accumulate_all": (lambda: B.fsdp_grad_accumulate(
            u, B.FSDP_ALL_RANKS, rs_input, gathered, False), 10 * L, L),
        # algorithmic bytes: the shard's real elements (8 bytes per 4096-element tile of
        # partial sums, written and read back, are not counted)
        "grad_sqnorm_rank": (lambda: B.fsdp_grad_sqnorm(u, k, grad, sq_out, sq_ws), 4 * valid, valid),
    }
    order = list(rows)
    for _ in range(max(1, args.warmup)):
        for n in order:
            rows[n][0]()
    torch.cuda.synchronize()
    ev = {n: [] for n in order}
    reps = max(5, args.steps // 5)
    for _ in range(reps):
        for n in order:
            if flush is not None:
                flush()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rows[n][0]()
            e1.record(stream)
            ev[n].append((e0, e1))
    torch.cuda.synchronize()
    out = {}
    for n in order:
        ms = sum(a.elapsed_time(b) for a, b in ev[n]) / reps
        fn, nbytes, elems = rows[n]
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[n] = {"ms": round(ms, 4), "bytes": nbytes, "GB/s": round(gbs, 1),
                  "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                  "elements_per_s": float("%.4g" % (elems / (ms * 1e-3))), "reps": reps}
    out["hybrid_group"] = group
    out["timing"] = ("mean of one HIP event pair around each call, each after the flush when one "
                     "runs; a call's launches are all inside its pair (the sums of squares are two, "
                     "a reduction on the grouped sweep one per run), and the pair adds 2-5 us, "
                     "a large share of a shard-sized call; kernel durations without it are in "
                     "the rocprofv3 summaries")
    del rs_input, shard16, sq_ws, sq_out, flag
    return out


def sweep_ranks(B, u, N, contrib_rows, pre, post, hp, params, grad, shard, adam_p, m, v,
                stream, flush, reps=10):
    """Flatten, reduce and AdamW for each swept rank k, each launch after a 1 GiB read flush.
    Reduce and AdamW move the same bytes for every rank (the shard length is the same);
    flatten reads only rank k's real elements."""
    import torch
    ks = list(range(N)) if N <= 8 else sorted({0, 1, max(0, N // 2 - 1), N - 1})
    out = {"ranks": ks, "reps": reps,
           "timing": "one HIP event pair around each single launch, each after a 1 GiB read; the "
                     "pair adds 2-5 us per launch, a few percent on kernels of 20-60 us (kernel "
                     "durations without it: rocprofv3, profiles/)"}
    worst = {}
    for k in ks:
        info = u.info(k)
        S, valid = info["S"], info["valid"]
        kern = {
            "grad_reduce": (lambda: B.fsdp_grad_reduce_shard(u, contrib_rows, pre, post, grad),
                            (2 * N + 4) * S),
            "adamw": (lambda: B.fsdp_adam_shard(u, adam_p, grad, m, v, step=2, **hp), 28 * S),
            "flatten": (lambda k=k: B.fsdp_flatten_shard(u, params, k, shard), 4 * valid + 4 * S),
        }
        row = {}
        for name, (fn, nbytes) in kern.items():
            fn()
            ev = []
            for _ in range(reps):
                flush()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                ev.append((e0, e1))
            torch.cuda.synchronize()
            _, med, _, p90 = time_stats([a.elapsed_time(b) for a, b in ev])
            gbs = nbytes / (med * 1e-3) / 1e9
            row[name] = {"ms_median": round(med, 4), "ms_p90": round(p90, 4),
                         "GB/s": round(gbs, 1), "bytes": nbytes}
            if name not in worst or gbs < worst[name]["GB/s"]:
                worst[name] = {"rank": k, "GB/s": round(gbs, 1),
                               "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}
        out[str(k)] = row
    out["worst"] = worst
    return out


def _event_median(fn, stream, reps, before=None):
    """Median of `reps` single launches of fn timed with an event pair on `stream` (ms)."""
    import torch
    ev = []
    for _ in range(reps):
        if before is not None:
            before()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    return time_stats([a.elapsed_time(b) for a, b in ev])[1]


def flatten_floor(B, u, N, params, stream, dev, gen, reps=20):
    """What any kernel of the flatten's shape pays, beside the flatten itself, each launch after a
    1 GiB read: an empty kernel with the flatten's grid (one 256-thread workgroup per 1024
    elements of the shard) and with one wave; a read-only kernel over the shard's bytes; a
    write-only one; a plain copy (loads, then device-scope nt stores, no segment table); then the
    flatten of ranks 0, 1, N/2-1 and N-1.  The cases run in this order, `reps` launches each, so
    that rocprofv3's kernel trace can be split by order (the probes are kernels of their own)."""
    import ctypes
    import torch
    from sharded_fsdp_flatten_amd import build as lib_build
    if not os.path.exists(lib_build.PROBE_LIB_PATH):
        raise RuntimeError("libfsdpprobe.so is not built; run __graft_entry__.build()")
    P = ctypes.CDLL(lib_build.PROBE_LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    P.fsdp_probe_empty.argtypes = [i64, i32, vp]
    P.fsdp_probe_read.argtypes = [vp, i64, vp, vp]
    P.fsdp_probe_write.argtypes = [vp, i64, vp]
    P.fsdp_probe_copy.argtypes = [vp, vp, i64, vp]
    S = u.info(0)["S"]
    n = S // 4 * 4
    tiles = -(-S // 1024)
    src = torch.randn(S, device=dev, generator=gen)
    dst = torch.empty(S, device=dev)
    sink = torch.zeros(4, device=dev)
    shard = torch.empty(S, device=dev)
    fb = torch.zeros(1 << 28, device=dev)
    fs = torch.zeros((), device=dev)
    sp = stream.cuda_stream

    def flush():
        torch.sum(fb, dim=0, out=fs)

    def probe(rc):
        if rc != 0:
            raise RuntimeError("probe launch failed (code %d)" % rc)

    ks = sorted({0, 1, max(0, N // 2 - 1), N - 1})
    cases = [
        ("empty kernel, flatten grid (%d x 256)" % tiles, 0, lambda: probe(P.fsdp_probe_empty(tiles, 256, sp))),
        ("empty kernel, one wave", 0, lambda: probe(P.fsdp_probe_empty(1, 64, sp))),
        ("read only (%d fp32)" % n, 4 * n, lambda: probe(P.fsdp_probe_read(src.data_ptr(), n, sink.data_ptr(), sp))),
        ("write only (%d fp32)" % n, 4 * n, lambda: probe(P.fsdp_probe_write(dst.data_ptr(), n, sp))),
        ("copy (%d fp32)" % n, 8 * n, lambda: probe(P.fsdp_probe_copy(src.data_ptr(), dst.data_ptr(), n, sp))),
    ]
    for k in ks:
        valid = u.info(k)["valid"]
        cases.append(("flatten rank %d" % k, 4 * valid + 4 * S,
                      lambda k=k: B.fsdp_flatten_shard(u, params, k, shard)))
    out = {"S": S, "reps": reps, "order": [c[0] for c in cases], "cases": {}}
    for name, nbytes, fn in cases:
        fn()
        med = _event_median(fn, stream, reps, before=flush)
        row = {"event_ms_median": round(med, 5), "bytes": nbytes}
        if nbytes:
            row["GB/s"] = round(nbytes / (med * 1e-3) / 1e9, 1)
        out["cases"][name] = row
        print("flatten floor: %s done" % name, file=sys.stderr, flush=True)
    del src, dst, sink, shard, fb
    return out


REDUCE_SHAPES_FLAT = [(n, s) for n in (32, 64, 128) for s in (4 << 20, 8 << 20, 14157024, 25 << 20)]
REDUCE_SHAPES_HYBRID = [(128, s) for s in (3538944, 7077888, 8 << 20, 14157024)]


def reduce_shapes(B, stream, dev, gen, reps=8):
    """The reduction on the tile kernel and on the sweep (whose shape the library picks by the
    length of its runs) over several rank counts and output lengths: flat sums, and hybrid
    accumulating sums in groups of 8.  Contributions are seeded normals (std 1e-3) in one
    receive buffer at the recommended pitch; every launch follows a 1 GiB read.  Event medians
    (ms) are reported; rocprofv3's kernel trace of the same run gives the kernel durations."""
    import torch
    fb = torch.zeros(1 << 28, device=dev)
    fs = torch.zeros((), device=dev)

    def flush():
        torch.sum(fb, dim=0, out=fs)

    out = []
    for group, shapes in ((0, REDUCE_SHAPES_FLAT), (8, REDUCE_SHAPES_HYBRID)):
        for n, s in shapes:
            u = B.fsdp_unit_create(B.FSDP_FLAT, [(n * s,)], n)
            buf = torch.empty((n, u.recv_pitch), dtype=torch.bfloat16, device=dev)
            c = buf[:, :s]
            c.normal_(0.0, 1e-3, generator=gen)
            rows = [c[r] for r in range(n)]
            grad = torch.zeros(s, device=dev)
            accumulate = group > 0
            need = B.fsdp_grad_reduce_workspace(u, group=group, accumulate=accumulate)
            ws = torch.zeros(need, device=dev) if need else None
            row = {"ranks": n, "outputs": s, "group": group, "accumulate": accumulate,
                   "bytes": (2 * n + (8 if accumulate else 4)) * s}
            for kernel in ("tiles", "sweep"):
                def call():
                    B.fsdp_grad_reduce_shard_ex(u, rows, 2.0, 4.0, grad, group=group,
                                                accumulate=accumulate, kernel=kernel, workspace=ws)
                flush()
                call()  # untimed: the sweep's first call per shape reads the device's occupancy
                ms = _event_median(call, stream, reps, before=flush)
                row[kernel] = {"event_ms_median": round(ms, 4),
                               "GB/s": round(row["bytes"] / (ms * 1e-3) / 1e9, 1)}
            out.append(row)
            print("reduce shapes: N=%d S=%d group=%d done" % (n, s, group), file=sys.stderr,
                  flush=True)
            del buf, c, rows, grad, ws
            torch.cuda.empty_cache()
    del fb
    return out


def contention_probe(B, u, N, contrib_rows, pre, post, grad, stream, dev, reps=10):
    """The reduction on the tile kernel and on the row-major sweep, alone and overlapped with a
    stream of bf16 GEMMs on a second stream of the same priority (the backward compute that the
    ReduceScatter overlaps).  Per case: the reduction's duration (events on its stream), the
    GEMM batch's duration, and the wall time until both are done."""
    import torch
    n = 8192
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    side = torch.cuda.Stream(device=dev)
    gemms = 8

    def gemm_batch():
        with torch.cuda.stream(side):
            for _ in range(gemms):
                torch.matmul(a, b, out=c)

    def reduce(kernel):
        B.fsdp_grad_reduce_shard_ex(u, contrib_rows, pre, post, grad, kernel=kernel)

    for kernel in ("tiles", "sweep"):
        reduce(kernel)
    gemm_batch()
    torch.cuda.synchronize()
    out = {"gemm": "%d bf16 matmuls %dx%dx%d on a second stream" % (gemms, n, n, n), "reps": reps}
    e = {k: torch.cuda.Event(enable_timing=True) for k in ("g0", "g1", "r0", "r1")}
    # the GEMM batch alone
    ts = []
    for _ in range(reps):
        e["g0"].record(side)
        gemm_batch()
        e["g1"].record(side)
        torch.cuda.synchronize()
        ts.append(e["g0"].elapsed_time(e["g1"]))
    out["gemm_alone_ms"] = round(time_stats(ts)[1], 4)
    for kernel in ("tiles", "sweep"):
        alone = _event_median(lambda: reduce(kernel), stream, reps)
        red, gem, wall = [], [], []
        for _ in range(reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            e["g0"].record(side)
            gemm_batch()
            e["g1"].record(side)
            # the reduction starts once the GEMMs hold the device
            stream.wait_event(e["g0"])
            e["r0"].record(stream)
            reduce(kernel)
            e["r1"].record(stream)
            torch.cuda.synchronize()
            wall.append((time.perf_counter() - t0) * 1e3)
            red.append(e["r0"].elapsed_time(e["r1"]))
            gem.append(e["g0"].elapsed_time(e["g1"]))
        out[kernel] = {"reduce_alone_ms": round(alone, 4),
                       "reduce_overlapped_ms": round(time_stats(red)[1], 4),
                       "gemm_overlapped_ms": round(time_stats(gem)[1], 4),
                       "both_done_wall_ms": round(time_stats(wall)[1], 4)}
        print("contention: %s done" % kernel, file=sys.stderr, flush=True)
    del a, b, c
    return out


def main():
    args = parse_args()
    if args.gpus != 1:
        print("bench.py measures one rank's share of one FSDP unit on ONE GPU; --gpus %d is not "
              "supported (the library has no collectives: it measures one rank's share)" % args.gpus, file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import workloads as W
    from sharded_fsdp_flatten_amd import binding as B

    if not os.path.exists(B.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    B.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    unit = make_unit(args.workload, args.ranks)
    N = unit.N
    k = args.rank if args.rank is not None else max(0, N // 2 - 1)
    layout = B.FSDP_FLAT if unit.layout == W.FLAT else B.FSDP_ROWS
    u = B.fsdp_unit_create(layout, unit.shapes, N)
    info = u.info(k)
    S, L, T = info["S"], info["L"], info["T"]
    pre, post = pre_post(N)
    hp = dict(unit.adam)

    # ---- inputs, resident in HBM before the timed region -------------------------
    params = W.device_params(unit, seed=0)
    gen = torch.Generator(device=dev).manual_seed(12345)
    gathered = torch.randn(L, device=dev, generator=gen).mul_(unit.std)
    outs = [torch.empty(s, dtype=torch.bfloat16, device=dev) for s in unit.shapes]
    pitch = u.recv_pitch if args.contribs == "pitched" else S
    contribs = W.device_contribs(N, S, step=1, pitch=pitch)
    if args.contribs == "separate":
        contrib_rows = [contribs[r].clone() for r in range(N)]
    else:
        contrib_rows = [contribs[r] for r in range(N)]
    grad = torch.zeros(S, device=dev)  # written by the reduction, read by AdamW
    shard = torch.empty(S, device=dev)
    adam_p = torch.empty(S, device=dev)
    B.fsdp_flatten_shard(u, params, k, adam_p)
    m = torch.zeros(S, device=dev)
    v = torch.zeros(S, device=dev)
    torch.cuda.synchronize()

    flush_on = args.flush == "on" or (args.flush == "auto" and 6 * T < 2e9)
    # The flush READS 1 GiB: that evicts what the cache held and leaves it clean.  Writing
    # 1 GiB instead would leave it full of dirty lines whose write-back the next kernel
    # would pay for (AdamW measured 53% of peak after such a flush, 82% in the step).
    flush_buf = torch.zeros(1 << 28, device=dev)
    flush_sum = torch.zeros((), device=dev)

    def flush():
        torch.sum(flush_buf, dim=0, out=flush_sum)

    stream = torch.cuda.current_stream()
    # the rank sweep first: the headline step runs at its slowest flatten rank
    per_rank = None
    if args.sweep_ranks:
        per_rank = sweep_ranks(B, u, N, contrib_rows, pre, post, hp, params, grad, shard, adam_p,
                               m, v, stream, flush)
        print("rank sweep done", file=sys.stderr, flush=True)
        if args.rank is None:
            k = per_rank["worst"]["flatten"]["rank"]
    rank_choice = ("given (--rank)" if args.rank is not None
                   else "the rank whose flatten the sweep measured slowest" if per_rank
                   else "N/2 - 1 (no rank sweep)")
    valid = u.info(k)["valid"]

    bytes_k = {
        "grad_reduce": (2 * N + 4) * S,
        "copyout": 6 * T,
        "adamw": 28 * S,
        "flatten": 4 * valid + 4 * S,
    }
    elems_k = {"grad_reduce": S, "copyout": T, "adamw": S, "flatten": S}
    order = ["grad_reduce", "copyout", "adamw", "flatten"]
    step_no = [0]

    def run(name):
        if name == "grad_reduce":
            B.fsdp_grad_reduce_shard(u, contrib_rows, pre, post, grad)
        elif name == "copyout":
            B.fsdp_unflatten_copyout(u, gathered, outs)
        elif name == "adamw":
            step_no[0] += 1
            B.fsdp_adam_shard(u, adam_p, grad, m, v, step=step_no[0], **hp)
        else:
            B.fsdp_flatten_shard(u, params, k, shard)

    def step(events=None):
        for name in order:
            if flush_on:
                flush()
            if events is not None:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                run(name)
                e1.record(stream)
                events[name].append((e0, e1))
            else:
                run(name)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = {n: [] for n in order}
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(events)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    times = {n: [a.elapsed_time(b) for a, b in events[n]] for n in order}
    ms_k = {n: sum(times[n]) / args.steps for n in order}
    # with flushing the fills sit between the kernels, so the step is the kernels' sum
    ms_step = sum(ms_k.values()) if flush_on else wall * 1e3 / args.steps
    step_bytes = sum(bytes_k.values())
    traffic = load_traffic(args.workload, N, k, args.contribs)
    kernels = {}
    for n in order:
        gbs = bytes_k[n] / (ms_k[n] * 1e-3) / 1e9
        _, med, lo, p90 = time_stats(times[n])
        kernels[n] = {"ms": round(ms_k[n], 4), "bytes": bytes_k[n], "GB/s": round(gbs, 1),
                      "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                      "elements_per_s": float("%.4g" % (elems_k[n] / (ms_k[n] * 1e-3))),
                      "ms_median": round(med, 4), "ms_min": round(lo, 4), "ms_p90": round(p90, 4),
                      "traffic": traffic.get(n)}
    kernels["grad_reduce"]["input_elements_per_s"] = float(
        "%.4g" % (N * S / (ms_k["grad_reduce"] * 1e-3)))

    dom = max(order, key=lambda n: ms_k[n])
    achieved = bytes_k[dom] / (ms_k[dom] * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "%s unit (%d params, T=%d fp32 elements), %s sharding over "
                               "N=%d, rank %d" % (unit.name, len(unit.shapes), T,
                                                  "FSDP1 flat" if layout == B.FSDP_FLAT
                                                  else "FSDP2 dim-0 row", N, k),
                   "N": N, "rank": k, "rank_choice": rank_choice, "S": S, "T": T,
                   "pre_divide": pre, "post_divide": post,
                   "contribs": args.contribs if args.contribs == "separate"
                   else "%s (one buffer, row pitch %d elements)" % (args.contribs, pitch),
                   "step_time": ("sum of the kernels' event times, 1 GiB read before each kernel"
                                 if flush_on else "wall clock")},
        "kernels": kernels,
        "kernel_timing": ("HIP events recorded around each call on its stream in the eager loop "
                          "(a reduction on the grouped sweep is one call of two launches); an event "
                          "pair adds 2-5 us, a few percent on the short kernels (flatten, AdamW); "
                          "rocprofv3 kernel durations are in profiles/"),
        "kernel_src_sha256": kernel_src_hash(),
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic.get(dom)},
    }

    use_graph = args.graph == "on" or (args.graph == "auto" and not flush_on)
    if use_graph:
        # capture one step (AdamW keeps the step number it was captured with)
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for name in order:
                run(name)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for name in order:
                run(name)
        for _ in range(max(1, args.warmup)):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        ms_graph = (time.perf_counter() - t0) * 1e3 / args.steps
        graph_res = {"ms_per_step": round(ms_graph, 4),
                     "value": round(step_bytes / (ms_graph * 1e-3) / 1e9, 1)}
        del graph
        if flush_on:
            graph_res["note"] = "wall clock of graph replays; no flush between kernels"
            result["graph"] = graph_res
        else:
            # the headline: whole-step throughput from graph replays; the eager loop (one
            # host call per kernel, with an event pair around each) is kept beside it
            result["eager"] = {"ms_per_step": result["ms_per_step"], "value": result["value"],
                               "step_time": "wall clock, one host call and an event pair per kernel"}
            result["ms_per_step"] = graph_res["ms_per_step"]
            result["value"] = graph_res["value"]
            result["config"]["step_time"] = "wall clock of HIP-graph replays of the step"

    if args.next:
        result["next_rows"] = time_next_rows(B, u, unit, args, N, k, S, L, T, pre, post, contrib_rows,
                                             grad, outs, gathered, adam_p, stream,
                                             flush if flush_on else None)

    if per_rank is not None:
        result["per_rank"] = per_rank
    del flush_buf

    if args.copy_probe:
        n = 1 << 30
        a = torch.randn(n, device=dev, generator=gen)
        b = torch.empty(n, device=dev)
        cu = B.fsdp_unit_create(B.FSDP_FLAT, [(n,)], 1)
        for _ in range(3):
            B.fsdp_flatten_shard(cu, [a], 0, b)
            b.copy_(a)
        torch.cuda.synchronize()
        probe = {}
        for name, fn in (("library_copy", lambda: B.fsdp_flatten_shard(cu, [a], 0, b)),
                         ("hipMemcpyDtoD", lambda: b.copy_(a))):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 10
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            probe[name] = {"bytes": 8 * n, "ms": round(ms, 4),
                           "GB/s": round(8 * n / (ms * 1e-3) / 1e9, 1)}
        ceiling = max(v["GB/s"] for v in probe.values())
        probe["ceiling_GB/s"] = ceiling
        probe["timing"] = "ten back-to-back copies between one HIP event pair, after three untimed"
        result["copy_ceiling"] = probe
        for kd in result["kernels"].values():
            kd["frac_of_copy_ceiling"] = round(kd["GB/s"] / ceiling, 4)
        del a, b

    if args.floor_probe:
        result["flatten_floor"] = flatten_floor(B, u, N, params, stream, dev, gen)
    if args.contention_probe:
        result["contention"] = contention_probe(B, u, N, contrib_rows, pre, post, grad, stream, dev)
    if args.reduce_shapes:
        result["reduce_shapes"] = reduce_shapes(B, stream, dev, gen)
    if args.floor_probe:
        fb = torch.zeros(1 << 28, device=dev)
        fs = torch.zeros((), device=dev)
        a = torch.randn(1 << 27, device=dev, generator=gen)
        b = torch.empty(1 << 27, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        floor = []
        for lg in range(20, 28):
            n = 1 << lg
            cu = B.fsdp_unit_create(B.FSDP_FLAT, [(n,)], 1)
            ts = []
            for _ in range(20):
                torch.sum(fb, dim=0, out=fs)  # evicts the source and destination
                e0.record(stream)
                B.fsdp_flatten_shard(cu, [a[:n]], 0, b[:n])
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            ts.sort()
            floor.append({"elements": n, "bytes": 8 * n, "event_ms_median": round(ts[len(ts) // 2], 4)})
        result["floor_probe"] = floor
        del a, b, fb

    if not args.no_cpu_baseline:
        host = {
            "params": [p.cpu().numpy() for p in params],
            "gathered": gathered.cpu().numpy(),
            "contribs": contribs[:, : S // 8].contiguous().view(torch.int16).cpu().numpy()
                        .view(np.uint16),
            "adam_p": adam_p.cpu().numpy(),
            "adam_g": grad.cpu().numpy(),
        }
        one = cpu_baseline(host, unit, N, k, S, valid, pre, post, hp, rows=layout == B.FSDP_ROWS)
        print("cpu baseline: one core done", file=sys.stderr, flush=True)
        allc = cpu_baseline_all_cores(host, unit, N, k, S, valid, pre, post, hp,
                                      rows=layout == B.FSDP_ROWS, threads=host_threads())
        allc["single_core"] = one
        result["cpu_baseline"] = allc
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
