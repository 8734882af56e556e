"""The gradient reduction's row-major sweep, the path a flat sum takes over at least 32
contributions that are all 4-byte aligned, into a 16-byte-aligned output of at least 12,288
whole 512-element tiles.  Parity with the oracle element by element: the tile the output's
end cuts and the single tiles before the sweep waves, outputs long enough to be split into
several runs, launches chained over more than 128 ranks (sweep after sweep, tile kernel after
sweep), accumulation, the three kinds of pre-divide (none, an exact reciprocal, a true
division) and special values, among them columns that are -0 in every rank (the sweep starts
its sums from -0, which must leave -0 + -0 + ... = -0)."""
import gc

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import assert_f32_tol_then_bits, dev, to_dev, to_host
from sharded_fsdp_flatten_amd import binding as B

pytestmark = pytest.mark.gpu

TILE = 512
MIN_TILES = 12288  # the shortest output (in whole tiles) the sweep takes


@pytest.fixture(autouse=True)
def _free():
    B.load()
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _contribs(N, S, step):
    """Pitched device rows (the library's recommended receive layout) and their host copy."""
    pitch = -(-S // 64) * 64
    c = W.device_contribs(N, S, step=step, pitch=pitch)
    return c, to_host(c)


def _reduce(u, c, pre, post, out=None, accumulate=False):
    S = c.shape[1]
    if out is None:
        out = torch.full((S,), float("nan"), device=dev())
    rows = [c[r] for r in range(c.shape[0])]
    if accumulate:
        need = B.fsdp_grad_reduce_workspace(u, accumulate=True)
        ws = torch.full((need,), float("nan"), device=dev()) if need else None
        B.fsdp_grad_reduce_shard_ex(u, rows, pre, post, out, accumulate=True, workspace=ws)
    else:
        B.fsdp_grad_reduce_shard(u, rows, pre, post, out)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("N,tiles,tail,pre,post", [
    (32, MIN_TILES, 0, 2.0, 16.0),          # exact multiple of 16 tiles: sweep waves only
    (32, MIN_TILES, 517, 4.0, 8.0),         # plus a cut tile (517 = 64 * 8 + 5)
    (48, 13000, 7, 3.0, 16.0),              # 8 single tiles, a cut tile of 7, true division
    (64, 12345, 300, 1.0, 64.0),            # 9 single tiles, no pre-divide
    (33, 12290, 511, -8.0, 4.125),          # negative power-of-two pre, non-power post
    (128, 27650, 224, 8.0, 16.0),           # the GPT-175B shard length at 128 ranks
    (128, 20000, 77, 8.0, 16.0),            # runs of 10,000 tiles: the wide shape
    (32, 24000, 0, 2.0, 16.0),              # runs of 12,000 tiles: the wide shape
])
def test_sweep_reduce(N, tiles, tail, pre, post):
    S = tiles * TILE + tail
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(N * S,)], N)
    assert u.S == S
    c, ch = _contribs(N, S, step=3)
    out = _reduce(u, c, pre, post)
    assert_f32_tol_then_bits(to_host(out), oracle.grad_reduce(list(ch), pre, post),
                             "sweep N=%d S=%d pre=%g post=%g" % (N, S, pre, post))


def test_sweep_split_into_runs():
    """65,029 whole tiles cannot all be resident at once (16 tiles per wave), so the output
    is reduced in several runs, one launch each, the last with the cut tile."""
    N, S = 32, 65029 * TILE + 77
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(N * S,)], N)
    c, ch = _contribs(N, S, step=4)
    out = _reduce(u, c, 2.0, 16.0)
    assert_f32_tol_then_bits(to_host(out), oracle.grad_reduce(list(ch), 2.0, 16.0),
                             "sweep in runs S=%d" % S)


@pytest.mark.parametrize("group,tiles,tail", [
    (0, 150001, 261),   # flat, 16 tiles per wave: five runs at 2,048 resident workgroups
    (8, 70001, 13),     # hybrid groups of 8, accumulating, 8 tiles per wave: five runs
])
def test_sweep_runs_over_several_launches(group, tiles, tail):
    """Five runs (five launches), the last with the cut tile; a hybrid wave's group sums
    start afresh in every run."""
    N, S = 32, tiles * TILE + tail
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(N * S,)], N)
    c, ch = _contribs(N, S, step=9)
    old = W.host_normal(S, 1e-3, seed=23)
    out = to_dev(old)
    B.fsdp_grad_reduce_shard_ex(u, [c[r] for r in range(N)], 2.0, 16.0, out, group=group,
                                accumulate=group > 0, kernel="sweep")
    torch.cuda.synchronize()
    if group:
        want = oracle.grad_reduce_ex(list(ch), 2.0, 16.0, group=group, out=old)
    else:
        want = oracle.grad_reduce(list(ch), 2.0, 16.0)
    assert_f32_tol_then_bits(to_host(out), want, "sweep runs group=%d S=%d" % (group, S))


@pytest.mark.parametrize("N,group,tiles,accumulate", [
    (288, 144, 14336, True),   # groups longer than a launch: partial group sums carried
    (256, 8, 13000, False),    # groups of 8 in two launches of 16 groups each
    (128, 8, 16384, True),     # runs of 8,192 tiles: one rank in flight
])
def test_hybrid_sweep_shapes_and_carries(N, group, tiles, accumulate):
    """Hybrid sums on the grouped sweep: runs of at least 12,288 tiles take the shape with two
    ranks in flight, shorter ones the shape with one; across launches the total and the partial
    group sums travel through the caller's workspace exactly."""
    S = tiles * TILE + 45
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(N * S,)], N)
    c, ch = _contribs(N, S, step=12)
    old = W.host_normal(S, 1e-3, seed=24)
    out = to_dev(old) if accumulate else torch.full((S,), float("nan"), device=dev())
    need = B.fsdp_grad_reduce_workspace(u, group=group, accumulate=accumulate)
    ws = torch.full((need,), float("nan"), device=dev()) if need else None
    B.fsdp_grad_reduce_shard_ex(u, [c[r] for r in range(N)], 4.0, 16.0, out, group=group,
                                accumulate=accumulate, kernel="sweep", workspace=ws)
    torch.cuda.synchronize()
    want = oracle.grad_reduce_ex(list(ch), 4.0, 16.0, group=group,
                                 out=old if accumulate else None)
    assert_f32_tol_then_bits(to_host(out), want, "hybrid sweep N=%d group=%d" % (N, group))


@pytest.mark.parametrize("N,tiles", [(160, MIN_TILES), (130, MIN_TILES), (300, MIN_TILES),
                                     (160, 20000)])
def test_sweep_chained_over_more_than_128_ranks(N, tiles):
    """160 = 128 + 32 (two sweeps), 130 = 128 + 2 (a sweep, then the tile kernel continues
    from the partial sums), 300 = 128 + 128 + 44 (a middle launch neither first nor last);
    12,289 whole tiles take the grouped shape (the flat sum as one group whose running sum
    crosses the launches), 20,000 the wide one."""
    S = tiles * TILE + 1000
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(N * S,)], N)
    c, ch = _contribs(N, S, step=5)
    pre = 8.0 if N != 300 else 3.0
    out = _reduce(u, c, pre, N / pre)
    assert_f32_tol_then_bits(to_host(out), oracle.grad_reduce(list(ch), pre, N / pre),
                             "chained N=%d" % N)


@pytest.mark.parametrize("N,tiles", [(64, MIN_TILES + 5), (64, 20000), (160, MIN_TILES + 5)])
def test_sweep_accumulate(N, tiles):
    """Accumulation on the grouped shape, on the wide one, and over two launches (160 ranks:
    the running sum crosses them in the caller's workspace, the old value stays in the
    output until the last)."""
    S = tiles * TILE + 33
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(N * S,)], N)
    old = W.host_normal(S, 1e-3, seed=21)
    acc = to_dev(old)
    for t, (pre, post) in enumerate([(8.0, 8.0), (3.0, 7.0)]):
        c, ch = _contribs(N, S, step=30 + t)
        _reduce(u, c, pre, post, out=acc, accumulate=True)
        oracle.grad_reduce_ex(list(ch), pre, post, out=old)
        assert_f32_tol_then_bits(to_host(acc), old, "sweep accumulate N=%d S=%d step %d" % (N, S, t))
        del c, ch


@pytest.mark.parametrize("pre,post", [(1.0, 1.0), (4.0, 8.0), (3.0, 5.0)])
def test_sweep_special_values(pre, post):
    N, S = 32, MIN_TILES * TILE + 9
    rng = np.random.Generator(np.random.PCG64(22))
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(N * S,)], N)
    c, ch = _contribs(N, S, step=6)
    ch = ch.copy()
    # scattered specials: +-0, +-inf, quiet NaN, the smallest subnormals, +-max finite
    specials = np.asarray([0x8000, 0x0000, 0x7F80, 0xFF80, 0x7FC0, 0x0001, 0x8001, 0x7F7F,
                           0xFF7F], np.uint16)
    for r in range(N):
        idx = rng.integers(0, S, size=2000)
        ch[r, idx] = rng.choice(specials, size=idx.size)
    # then columns -0 in every rank, in a sweep wave's tiles and in the cut tile
    zero_cols = (0, 4096 * TILE + 3, S - 9)
    for lo in zero_cols:
        ch[:, lo:lo + 9] = 0x8000
    # subnormal in every rank: the pre-divide of a subnormal term
    ch[:, 100:140] = 0x0001
    c.copy_(to_dev(ch))
    out = _reduce(u, c, pre, post)
    got = to_host(out)
    want = oracle.grad_reduce(list(ch), pre, post)
    assert_f32_tol_then_bits(got, want, "sweep specials pre=%g post=%g" % (pre, post))
    for lo in zero_cols:
        assert np.all(got[lo:lo + 9].view(np.uint32) == 0x80000000), "-0 column at %d" % lo


_FRESH_CAPTURE = r"""
import sys
sys.path.insert(0, %(root)r)
import numpy as np, torch
import workloads as W
from sharded_fsdp_flatten_amd import binding as B
N, S = 32, %(S)d
u = B.fsdp_unit_create(B.FSDP_FLAT, [(N * S,)], N)
c = W.device_contribs(N, S, step=7, pitch=-(-S // 64) * 64)
rows = [c[r] for r in range(N)]
out_g = torch.empty(S, device="cuda:0")
out_e = torch.empty(S, device="cuda:0")
torch.cuda.synchronize()
g = torch.cuda.CUDAGraph()
with torch.cuda.graph(g):  # the library's first call in this process is captured
    B.fsdp_grad_reduce_shard(u, rows, 4.0, 8.0, out_g)
B.fsdp_grad_reduce_shard(u, rows, 4.0, 8.0, out_e)
for rep in range(3):
    out_g.fill_(float("nan"))
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out_g.view(torch.int32), out_e.view(torch.int32)), rep
print("fresh-capture OK", flush=True)
"""


def test_sweep_first_call_captured_in_a_fresh_process():
    """The sweep reads the device's occupancy on its first call; that call may be the one a
    caller captures into a HIP graph.  A child process whose first library call is captured,
    replayed three times and compared bit for bit with an eager call.  (Had the runtime refused
    the query during capture, the captured call would have taken the tile kernel: the result
    must be the same bits either way, and the capture must not fail.)"""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    script = _FRESH_CAPTURE % {"root": root, "S": MIN_TILES * TILE + 5}
    p = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True, timeout=150)
    assert p.returncode == 0 and "fresh-capture OK" in p.stdout, p.stdout[-2000:] + p.stderr[-3000:]


def test_sweep_result_does_not_depend_on_residency():
    """The sweep's grid is sized to be resident at once, but no wave waits for another: with a
    long kernel holding CUs on a second stream, the result is bit-identical."""
    N, S = 32, MIN_TILES * TILE + 100
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(N * S,)], N)
    c, ch = _contribs(N, S, step=8)
    alone = _reduce(u, c, 2.0, 16.0)
    side = torch.cuda.Stream()
    big = torch.randn(1 << 28, device=dev())
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(4):
            big.mul_(1.0001).add_(1e-7)  # keeps CUs busy while the reduction runs
    shared = _reduce(u, c, 2.0, 16.0)
    torch.cuda.synchronize()
    assert torch.equal(alone.view(torch.int32), shared.view(torch.int32))
    assert_f32_tol_then_bits(to_host(shared), oracle.grad_reduce(list(ch), 2.0, 16.0),
                             "sweep beside another stream")


_FRESH_THREADS = r"""
import sys, threading
sys.path.insert(0, %(root)r)
import torch
import workloads as W
from sharded_fsdp_flatten_amd import binding as B
S = %(S)d
jobs = [(32, 1), (48, 2), (8, 3), (64, 4)]  # (ranks, step): sweeps and one tile-kernel case
units, rows, outs = [], [], []
for N, step in jobs:
    units.append(B.fsdp_unit_create(B.FSDP_FLAT, [(N * S,)], N))
    c = W.device_contribs(N, S, step=step, pitch=-(-S // 64) * 64)
    rows.append([c[r] for r in range(N)])
    outs.append(torch.empty(S, device="cuda:0"))
torch.cuda.synchronize()
errors = []
def work(i):
    try:
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            B.fsdp_grad_reduce_shard(units[i], rows[i], 2.0, 8.0, outs[i], stream=s)
        s.synchronize()
    except Exception as e:
        errors.append(repr(e))
ts = [threading.Thread(target=work, args=(i,)) for i in range(len(jobs))]
for t in ts: t.start()
for t in ts: t.join()
assert not errors, errors
for i in range(len(jobs)):
    ref = torch.empty(S, device="cuda:0")
    B.fsdp_grad_reduce_shard(units[i], rows[i], 2.0, 8.0, ref)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int32), outs[i].view(torch.int32)), i
print("threads OK", flush=True)
"""


def test_concurrent_first_calls_from_threads_in_a_fresh_process():
    """Four host threads make their first library calls at the same time, each on its own
    stream (three sweeps and one tile-kernel reduction): the per-device occupancy value is
    initialised concurrently, and every result equals a later single-threaded call."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    script = _FRESH_THREADS % {"root": root, "S": MIN_TILES * TILE + 3}
    p = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True, timeout=200)
    assert p.returncode == 0 and "threads OK" in p.stdout, p.stdout[-2000:] + p.stderr[-3000:]
