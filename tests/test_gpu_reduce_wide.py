"""The gradient reduction beyond one launch and on either kernel, against the oracle.

One launch holds 128 ranks.  Longer reductions carry their running sums from launch to
launch: the total through the output, or through the caller's workspace when the output
must keep its old value (accumulation) or when a hybrid group is longer than a launch (its
partial sum).  Cases: accumulation over 129, 256 and 512 ranks; hybrid groups of 129, 150,
200 and 256 ranks (a group split 128 + 1, 128 + 22, 128 + 72, 128 + 128); groups of 8 over
512 ranks.  Each on the tile kernel and on the row-major sweep (forced, so that shards of a
few thousand elements take it), with the workspace filled with NaN so that a read of an
unwritten slot shows.  Also the hybrid sweep on its own (groups of 2 to 64 in 32 to 128
ranks, the three kinds of pre-divide, a cut tile, single tiles) and special values, and the
scalar path (an output not 16-byte aligned) with a workspace.  Results are bit-exact
against the oracle's sequential order (reading: flat sum in rank order; hybrid: each group
in rank order, then the group sums in group order)."""
import gc

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import assert_f32_tol_then_bits, dev, offset_view, to_dev, to_host
from sharded_fsdp_flatten_amd import binding as B

pytestmark = pytest.mark.gpu

TILE = 512


@pytest.fixture(autouse=True)
def _free():
    B.load()
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _pitched(c):
    """Host contributions [N, S] as one device receive buffer with rows on 128-byte lines."""
    N, S = c.shape
    pitch = -(-S // 64) * 64
    buf = torch.zeros((N, pitch), dtype=torch.bfloat16, device=dev())
    buf[:, :S] = to_dev(np.ascontiguousarray(c)).view(N, S)
    return [buf[r, :S] for r in range(N)], buf


def _workspace(u, group, accumulate):
    need = B.fsdp_grad_reduce_workspace(u, group=group, accumulate=accumulate)
    return need, (torch.full((need,), float("nan"), device=dev()) if need else None)


def _run(N, S, group, accumulate, kernel, pre, post, step):
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(N * S,)], N)
    assert u.S == S
    c = W.host_contribs(N, S, step=step)
    rows, keep = _pitched(c)
    old = W.host_normal(S, 1e-3, seed=step)
    out = to_dev(old) if accumulate else torch.full((S,), float("nan"), device=dev())
    need, ws = _workspace(u, group, accumulate)
    B.fsdp_grad_reduce_shard_ex(u, rows, pre, post, out, group=group, accumulate=accumulate,
                                kernel=kernel, workspace=ws)
    torch.cuda.synchronize()
    want = old.copy() if accumulate else None
    ref = oracle.grad_reduce_ex(list(c), pre, post, group=group, out=want)
    return to_host(out), (want if accumulate else ref), need


@pytest.mark.parametrize("kernel", ["tiles", "sweep"])
@pytest.mark.parametrize("N,group,accumulate,need_slots", [
    (129, 0, True, 1),      # flat, 128 + 1 ranks, the old value kept in the output
    (256, 0, True, 1),
    (512, 0, True, 1),
    (512, 0, False, 0),     # flat sum: the output carries it
    (512, 8, True, 1),      # groups of 8, four launches of 16 whole groups
    (256, 128, True, 1),    # a group fills a launch exactly
    (258, 129, True, 2),    # groups split 128 + 1
    (300, 150, False, 1),   # groups split 128 + 22, total in the output
    (400, 200, True, 2),    # groups split 128 + 72
    (512, 256, False, 1),   # the pages' 512 GPUs, sharding factor 256
    (512, 256, True, 2),
])
def test_many_rank_reduction(kernel, N, group, accumulate, need_slots):
    S = 17 * TILE + 5  # 17 whole tiles and a cut tile of 5
    pre = 16.0 if N >= 256 else 8.0
    post = N / pre
    got, want, need = _run(N, S, group, accumulate, kernel, pre, post, step=7)
    assert need == need_slots * (-(-S // 64) * 64)
    assert_f32_tol_then_bits(got, want, "N=%d group=%d acc=%s %s" % (N, group, accumulate, kernel))


@pytest.mark.parametrize("N,group,pre,post,tiles,tail,accumulate", [
    (32, 8, 2.0, 16.0, 16, 0, False),      # two sweep waves of 8 tiles
    (32, 2, 4.0, 8.0, 19, 517, False),     # 3 single tiles, a cut tile
    (64, 16, 3.0, 16.0, 25, 7, True),      # true division, accumulation
    (128, 8, 8.0, 16.0, 40, 224, True),    # the hybrid accumulating reduction's shape
    (128, 64, 1.0, 128.0, 9, 300, False),  # no pre-divide
    (96, 32, -8.0, 12.0, 8, 0, False),     # negative power-of-two pre
])
def test_hybrid_sweep(N, group, pre, post, tiles, tail, accumulate):
    S = tiles * TILE + tail
    results = {}
    for kernel in ("sweep", "tiles"):
        got, want, _ = _run(N, S, group, accumulate, kernel, pre, post, step=11)
        assert_f32_tol_then_bits(got, want, "hybrid %s N=%d group=%d" % (kernel, N, group))
        results[kernel] = got
    assert np.array_equal(results["sweep"].view(np.uint32), results["tiles"].view(np.uint32))


def test_hybrid_sweep_special_values():
    """+-0 (columns that are -0 in every rank), subnormals, +-inf and NaN in the hybrid
    sweep: the group sums start from -0 and must keep -0 + -0 = -0."""
    N, group, S = 64, 8, 12 * TILE + 9
    rng = np.random.Generator(np.random.PCG64(77))
    c = W.host_contribs(N, S, step=4)
    specials = np.array([0x8000, 0x0000, 0x0001, 0x8001, 0x7F80, 0xFF80, 0x7FC0, 0x0080],
                        np.uint16)
    for col in rng.choice(S, 400, replace=False):
        c[:, col] = specials[rng.integers(0, specials.size, N)]
    neg0 = rng.choice(S, 50, replace=False)
    c[:, neg0] = 0x8000
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(N * S,)], N)
    rows, keep = _pitched(c)
    out = torch.full((S,), float("nan"), device=dev())
    B.fsdp_grad_reduce_shard_ex(u, rows, 2.0, 32.0, out, group=group, kernel="sweep")
    torch.cuda.synchronize()
    want = oracle.grad_reduce_ex(list(c), 2.0, 32.0, group=group)
    assert np.all(np.signbit(want[neg0])) and np.all(want[neg0] == 0)
    assert_f32_tol_then_bits(to_host(out), want, "hybrid sweep specials")


def test_workspace_carries_on_the_scalar_path():
    """An output 4 bytes off 16: every output takes the one-element path, and the carried
    sums go through the workspace element by element."""
    N, group, S = 300, 150, 4099
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(N * S,)], N)
    c = W.host_contribs(N, S, step=13)
    rows, keep = _pitched(c)
    old = W.host_normal(S, 1e-3, seed=14)
    out, ob = offset_view(S, torch.float32, 1)
    out.copy_(to_dev(old))
    need, ws = _workspace(u, group, True)
    assert need > 0
    B.fsdp_grad_reduce_shard_ex(u, rows, 16.0, 300 / 16.0, out, group=group, accumulate=True,
                                workspace=ws)
    torch.cuda.synchronize()
    want = old.copy()
    oracle.grad_reduce_ex(list(c), 16.0, 300 / 16.0, group=group, out=want)
    assert_f32_tol_then_bits(to_host(out), want, "scalar path with workspace")


def test_repeated_calls_share_a_workspace():
    """Calls on one stream that share a workspace run in order: micro-batches accumulated over
    512 ranks in groups of 256, one workspace for all of them."""
    N, group, S = 512, 256, 3 * TILE + 1
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(N * S,)], N)
    need, ws = _workspace(u, group, True)
    acc = torch.zeros(S, device=dev())
    h_acc = np.zeros(S, np.float32)
    keep = []
    for t in range(3):
        c = W.host_contribs(N, S, step=20 + t)
        rows, buf = _pitched(c)
        keep.append(buf)
        B.fsdp_grad_reduce_shard_ex(u, rows, 16.0, 32.0, acc, group=group, accumulate=True,
                                    workspace=ws)
        oracle.grad_reduce_ex(list(c), 16.0, 32.0, group=group, out=h_acc)
    torch.cuda.synchronize()
    assert_f32_tol_then_bits(to_host(acc), h_acc, "three micro-batches, shared workspace")
