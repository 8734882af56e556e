"""Segment and run tables of every size the library picks.

A launch passes its segments (flatten, copy-out) or runs (sums of squares) by value in a table of
1, 4, 8, 16 or 48 entries; tiles of the segment with the most tiles take a direct path and the
others count the segment starts. Units of 1, 2, 4, 5, 8, 9, 16, 17, 48 and 49 parameters cross
every boundary of that ladder (49 takes two launches), with one multi-tile parameter first, in
the middle or last, so that the other tiles sit after, around or before it. Each case checks
the flatten of every rank and of the gathered layout, the copy-out and the per-parameter sums of
squares against the oracle, bit for bit (integer gradients make every sum of squares exact)."""
import gc

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_bf16_bits, assert_f32_bits, dev, to_dev, to_host
from sharded_fsdp_flatten_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    d = dev()
    B.load()
    yield d
    gc.collect()
    torch.cuda.empty_cache()


COUNTS = [1, 2, 4, 5, 8, 9, 16, 17, 48, 49]
WHERE = {"first": lambda n: 0, "middle": lambda n: n // 2, "last": lambda n: n - 1}


def _shapes(n, where, seed):
    """n one-dimensional parameters of 1..2,499 elements (one to three tiles), one of them
    9,000..12,999 elements (9 to 13 fp32 tiles) at the given place."""
    rng = np.random.Generator(np.random.PCG64(seed))
    shapes = [(int(rng.integers(1, 2500)),) for _ in range(n)]
    shapes[WHERE[where](n)] = (int(rng.integers(9000, 13000)),)
    return shapes


@pytest.mark.parametrize("where", list(WHERE))
@pytest.mark.parametrize("n", COUNTS)
def test_flatten_copyout_and_sqnorm_for_every_table_size(n, where):
    shapes = _shapes(n, where, 1000 * n + len(where))
    rng = np.random.Generator(np.random.PCG64(7 * n + len(where)))
    params = [rng.standard_normal(size=s).astype(np.float32) for s in shapes]
    d_params = [to_dev(p) for p in params]
    for N in (1, 3):
        tag = "n=%d big %s N=%d" % (n, where, N)
        u = B.fsdp_unit_create(B.FSDP_FLAT, shapes, N)
        gathered = torch.full((u.L,), float("nan"), device=dev())
        B.fsdp_flatten_shard(u, d_params, B.FSDP_ALL_RANKS, gathered)
        torch.cuda.synchronize()
        assert_f32_bits(to_host(gathered), oracle.flat_shard(params, N, -1), tag + " gathered")
        for k in range(N):
            shard = torch.full((u.S,), float("nan"), device=dev())
            B.fsdp_flatten_shard(u, d_params, k, shard)
            g = rng.integers(-1024, 1025, u.S).astype(np.float32)
            ws = torch.empty(max(1, B.fsdp_grad_sqnorm_workspace(u, k)), dtype=torch.float64,
                             device=dev())
            sq = torch.full((n,), float("nan"), dtype=torch.float64, device=dev())
            B.fsdp_grad_sqnorm(u, k, to_dev(g), sq, ws)
            torch.cuda.synchronize()
            assert_f32_bits(to_host(shard), oracle.flat_shard(params, N, k), tag + " k=%d" % k)
            assert np.array_equal(to_host(sq), oracle.flat_sqnorm(shapes, N, k, g)), tag + " k=%d" % k
        src = rng.standard_normal(u.L).astype(np.float32)
        outs = [torch.empty(s, dtype=torch.bfloat16, device=dev()) for s in shapes]
        B.fsdp_unflatten_copyout(u, to_dev(src), outs)
        torch.cuda.synchronize()
        for i, (o, w) in enumerate(zip(outs, oracle.flat_copyout(shapes, src))):
            assert_bf16_bits(to_host(o), w, tag + " copy-out param %d" % i)
