"""Pins of the oracle's next rows: 16-bit layouts (cast before the gather, FSDP2
copy-in), the hybrid two-level reduction, and gradient accumulation with and
without communication.

What pins them: torch's cat/pad/chunk on int16 tensors and exact widening into
the already pinned fp32 layouts; the special cases that reduce to the flat
reduction (one group of N, N groups of one); exact integer sums and the
hybrid-sharding decomposition ("PyTorch FSDP ..." summary §3.4, the sum over all
ranks equals the sum of the per-group sums); Higham's bound; closed forms that
tell each reading's operation order apart from the alternatives.
"""
import numpy as np
import pytest
import torch

import workloads as W

U = 2.0 ** -24


def _bits16(rng, shape):
    """Random bf16 bit patterns, NaNs excluded (so widening round-trips exactly)."""
    h = rng.integers(0, 1 << 16, size=shape, dtype=np.uint32).astype(np.uint16)
    nan = ((h & 0x7F80) == 0x7F80) & ((h & 0x7F) != 0)
    h[nan] = 0x3F80
    return h


def _widen(h):
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _narrow(x):
    b = np.asarray(x, np.float32).view(np.uint32)
    assert np.all((b & 0xFFFF) == 0)
    return (b >> 16).astype(np.uint16)


def test_u16_flat_layout_matches_widened_fp32_and_torch(orc):
    rng = np.random.Generator(np.random.PCG64(21))
    for trial in range(60):
        shapes = W.random_unit_shapes(rng, max_params=5, max_dim=5)
        params = [_bits16(rng, s) for s in shapes]
        if sum(p.size for p in params) == 0:
            continue
        for N in (1, 2, 3, 5, 8):
            full = orc.flat_shard_u16(params, N, -1)
            wide = orc.flat_shard([_widen(p) for p in params], N, -1)
            assert np.array_equal(full, _narrow(wide))
            flat = torch.cat([torch.from_numpy(p.view(np.int16)).reshape(-1) for p in params])
            L = -(-flat.numel() // N) * N
            F = torch.nn.functional.pad(flat, (0, L - flat.numel()))
            for k, chunk in enumerate(torch.chunk(F, N)):
                assert np.array_equal(orc.flat_shard_u16(params, N, k), chunk.numpy().view(np.uint16))
            outs = orc.flat_copyout_u16(shapes, full)
            for p, o in zip(params, outs):
                assert np.array_equal(o, p)


def test_u16_rows_layout_matches_widened_fp32_and_torch_chunk(orc):
    rng = np.random.Generator(np.random.PCG64(22))
    for trial in range(60):
        shapes = W.random_unit_shapes(rng, max_params=4, max_dim=7)
        params = [_bits16(rng, s) for s in shapes]
        for N in (1, 2, 3, 4, 7):
            full = orc.rows_shard_u16(params, N, -1)
            assert np.array_equal(full, _narrow(orc.rows_shard([_widen(p) for p in params], N, -1)))
            P_r = orc.rows_sizes(shapes, N)
            for k in range(N):
                seg = orc.rows_shard_u16(params, N, k)
                assert np.array_equal(seg, full[k * P_r:(k + 1) * P_r])
                # torch.chunk as the library routine for rank k's rows of parameter 0
                if shapes and len(shapes[0]) >= 1 and shapes[0][0] > 0:
                    t = torch.from_numpy(params[0].view(np.int16))
                    ch = torch.chunk(t, N, dim=0)
                    want = ch[k].reshape(-1).numpy().view(np.uint16) if k < len(ch) else np.zeros(0, np.uint16)
                    assert np.array_equal(seg[:want.size], want)
            outs = orc.rows_copyout_u16(shapes, N, full)
            for p, o in zip(params, outs):
                assert np.array_equal(o, p)


@pytest.mark.parametrize("N", [1, 2, 4, 8, 16, 128])
def test_hybrid_one_group_and_singleton_groups_equal_flat(orc, N):
    c = W.host_contribs(N, 4000, step=3)
    flat = orc.grad_reduce(list(c), 2.0, 3.0)
    for g in (N, 1):
        out = orc.grad_reduce_ex(list(c), 2.0, 3.0, group=g)
        assert np.array_equal(out.view(np.uint32), flat.view(np.uint32)), g


def test_hybrid_integer_sums_exact_for_every_group_size(orc):
    rng = np.random.Generator(np.random.PCG64(9))
    N = 32
    ints = rng.integers(-100, 101, size=(N, 3000)).astype(np.float32)
    cs = [_narrow(row) for row in ints]
    want = ints.astype(np.int64).sum(axis=0).astype(np.float32)
    for g in (1, 2, 4, 8, 16, 32):
        assert np.array_equal(orc.grad_reduce_ex(cs, 1.0, 1.0, group=g), want)


def test_hybrid_order_closed_form(orc):
    """Groups of 2 over [1, 2^-24 | 2^-24, 2^-24]: the first group rounds back to 1.0 (a tie),
    the second is exactly 2^-23, so the two-level sum is 1 + 2^-23; the flat sequential
    sum stays 1.0."""
    cs = [_narrow(np.full(4, v, np.float32)) for v in (1.0, 2.0 ** -24, 2.0 ** -24, 2.0 ** -24)]
    assert np.all(orc.grad_reduce_ex(cs, 1.0, 1.0, group=2) == np.float32(1.0 + 2.0 ** -23))
    assert np.all(orc.grad_reduce_ex(cs, 1.0, 1.0, group=4) == np.float32(1.0))


@pytest.mark.parametrize("g", [2, 4, 8, 16])
def test_hybrid_within_higham_bound(orc, g):
    N = 64
    c = W.host_contribs(N, 10000, step=4)
    out = orc.grad_reduce_ex(list(c), 4.0, 16.0, group=g).astype(np.float64)
    terms = _widen(c).astype(np.float64)
    exact = terms.sum(axis=0) / 64.0
    k = N + 1
    gamma = k * U / (1 - k * U)
    assert np.all(np.abs(out - exact) <= gamma * np.abs(terms).sum(axis=0) / 64.0)


def test_accumulate_adds_fresh_result_after_post_divide(orc):
    """out = old + (sum/post), not (old*post + sum)/post: old = 1, one contribution 2, post 2
    gives 1 + 1 = 2 (the other reading would give 1.5)."""
    old = np.full(8, 1.0, np.float32)
    out = orc.grad_reduce_ex([_narrow(np.full(8, 2.0, np.float32))], 1.0, 2.0, out=old)
    assert out is old and np.all(old == 2.0)


def test_accumulate_integer_micro_batches_exact(orc):
    rng = np.random.Generator(np.random.PCG64(10))
    N, n, steps = 8, 2000, 6
    acc = np.zeros(n, np.float32)
    want = np.zeros(n, np.int64)
    for t in range(steps):
        ints = rng.integers(-50, 51, size=(N, n)).astype(np.float32)
        orc.grad_reduce_ex([_narrow(r) for r in ints], 1.0, 1.0, out=acc)
        want += ints.astype(np.int64).sum(axis=0)
    assert np.array_equal(acc, want.astype(np.float32))


@pytest.mark.parametrize("pre,post", [(2.0, 4.0), (3.0, 5.0)])
def test_accumulate_matches_sequential_fp32_addition(orc, pre, post):
    """old + fresh is one binary32 addition: compare with numpy's float32 add (IEEE) of the
    oracle's own non-accumulating result.  With a post that is not a power of two this also
    tells old + sum/post apart from (old*post + sum)/post, which rounds differently."""
    c = W.host_contribs(8, 5000, step=6)
    old = W.host_normal(5000, 1e-3, seed=3)
    fresh = orc.grad_reduce_ex(list(c), pre, post)
    acc = old.copy()
    orc.grad_reduce_ex(list(c), pre, post, out=acc)
    assert np.array_equal(acc.view(np.uint32), (old + fresh).view(np.uint32))


def test_local_accumulation(orc):
    rng = np.random.Generator(np.random.PCG64(11))
    n = 4096
    acc = np.full(n, 123.0, np.float32)
    ints = [rng.integers(-64, 65, size=n).astype(np.float32) for _ in range(5)]
    orc.grad_accumulate(_narrow(ints[0]), acc, init=True)
    assert np.array_equal(acc, ints[0])                       # init: exact widening
    for x in ints[1:]:
        orc.grad_accumulate(_narrow(x), acc, init=False)
    assert np.array_equal(acc, np.sum(np.stack(ints).astype(np.int64), axis=0).astype(np.float32))
    g = W.host_contribs(1, n, step=9)[0]
    before = acc.copy()
    orc.grad_accumulate(g, acc, init=False)
    assert np.array_equal(acc.view(np.uint32), (before + _widen(g)).view(np.uint32))
