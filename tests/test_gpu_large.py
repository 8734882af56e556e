"""Units and shards larger than 2^31 elements: every index and offset in the kernels is
64-bit.  Whole-buffer checks run on the device against torch (layout identities and torch's
own bf16 cast, a library routine); element values are checked against the CPU oracle on
samples (all of the first and last elements, those around 2^31, and random ones)."""
import gc

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_bf16_bits, assert_f32_tol_then_bits, dev, to_host
from sharded_fsdp_flatten_amd import binding as B

pytestmark = pytest.mark.gpu

BIG = 2 ** 31


@pytest.fixture(autouse=True)
def _free():
    B.load()
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _sync():
    torch.cuda.synchronize()


def _same_bits(a, b):
    """Bitwise equality of two same-dtype device tensors (viewed as integers)."""
    it = {torch.float32: torch.int32, torch.bfloat16: torch.int16}[a.dtype]
    return torch.equal(a.view(it), b.view(it))


def _sample_idx(n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    parts = [np.arange(0, 4096), np.arange(n - 4096, n), rng.integers(0, n, 200_000)]
    if n > BIG + 4096:
        parts.append(np.arange(BIG - 4096, BIG + 4096))
    return np.unique(np.concatenate(parts)).astype(np.int64)


def test_flatten_and_copyout_of_a_unit_beyond_2_31_elements():
    """T = 2^31 + 4995 over N = 3: the gathered flat buffer, rank 2's shard and the second
    parameter all sit past 2^31 elements."""
    shapes = [(BIG - 5,), (5000,)]
    N = 3
    u = B.fsdp_unit_create(B.FSDP_FLAT, shapes, N)
    T = BIG - 5 + 5000
    assert (u.S, u.L) == (-(-T // N), N * -(-T // N))
    gen = torch.Generator(device=dev()).manual_seed(1)
    params = [torch.randn(s, device=dev(), generator=gen) for s in shapes]
    gathered = torch.empty(u.L, device=dev())
    B.fsdp_flatten_shard(u, params, B.FSDP_ALL_RANKS, gathered)
    _sync()
    n0 = shapes[0][0]
    assert _same_bits(gathered[:n0], params[0])
    assert _same_bits(gathered[n0:T], params[1])
    assert torch.count_nonzero(gathered[T:].view(torch.int32)).item() == 0
    shard = torch.empty(u.S, device=dev())
    B.fsdp_flatten_shard(u, params, 2, shard)
    _sync()
    assert _same_bits(shard, gathered[2 * u.S:3 * u.S])
    del shard
    outs = [torch.empty(s, dtype=torch.bfloat16, device=dev()) for s in shapes]
    B.fsdp_unflatten_copyout(u, gathered, outs)
    _sync()
    for o, p in zip(outs, params):
        assert _same_bits(o, p.to(torch.bfloat16))
    # and the cast itself against the oracle on samples
    idx = _sample_idx(n0, 2)
    ti = torch.from_numpy(idx).to(dev())
    assert_bf16_bits(to_host(outs[0].view(torch.int16).index_select(0, ti)).view(np.uint16),
                     oracle.bf16(to_host(params[0].index_select(0, ti))), "copy-out samples")


def test_reduce_over_a_shard_beyond_2_31_elements():
    """N = 2 contributions of S = 2^31 + 77 elements, true division by pre and post."""
    S = BIG + 77
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(2 * S,)], 2)
    assert u.S == S
    gen = torch.Generator(device=dev()).manual_seed(3)
    c = [torch.randn(S, device=dev(), generator=gen).mul_(1e-3).to(torch.bfloat16) for _ in range(2)]
    out = torch.empty(S, device=dev())
    B.fsdp_grad_reduce_shard(u, c, 3.0, 5.0, out)
    _sync()
    idx = _sample_idx(S, 4)
    ti = torch.from_numpy(idx).to(dev())
    cs = [to_host(x.view(torch.int16).index_select(0, ti)).view(np.uint16) for x in c]
    assert_f32_tol_then_bits(to_host(out.index_select(0, ti)), oracle.grad_reduce(cs, 3.0, 5.0),
                             "reduce samples")


def test_adamw_on_a_shard_beyond_2_31_elements():
    S = BIG + 77
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(S,)], 1)
    gen = torch.Generator(device=dev()).manual_seed(5)
    p = torch.randn(S, device=dev(), generator=gen).mul_(0.02)
    g = torch.randn(S, device=dev(), generator=gen).mul_(1e-3)
    m = torch.zeros(S, device=dev())
    v = torch.zeros(S, device=dev())
    pb = torch.empty(S, dtype=torch.bfloat16, device=dev())
    idx = _sample_idx(S, 6)
    ti = torch.from_numpy(idx).to(dev())
    hp, hg = to_host(p.index_select(0, ti)), to_host(g.index_select(0, ti))
    hm, hv = np.zeros_like(hp), np.zeros_like(hp)
    hyper = dict(lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01)
    B.fsdp_adam_shard(u, p, g, m, v, step=1, param_bf16=pb, **hyper)
    _sync()
    hpb = oracle.adamw(hp, hg, hm, hv, step=1, want_bf16=True, **hyper)
    assert_f32_tol_then_bits(to_host(p.index_select(0, ti)), hp, "adamw p samples")
    assert_f32_tol_then_bits(to_host(m.index_select(0, ti)), hm, "adamw m samples")
    assert_f32_tol_then_bits(to_host(v.index_select(0, ti)), hv, "adamw v samples")
    assert_bf16_bits(to_host(pb.view(torch.int16).index_select(0, ti)).view(np.uint16), hpb,
                     "adamw bf16 samples")


def test_many_rank_sweep_over_a_shard_beyond_2_31_elements():
    """32 ranks of 2^31 + 1000 outputs (137 GB of contributions): the row-major sweep, split
    into ~130 runs of resident waves, with tile offsets past 2^31 and a cut tile at the end.
    Contributions follow a position-dependent pattern of small integers times 2^-10 (exact in
    bf16; a misread column shows); outputs are checked against the oracle on samples."""
    N, S = 32, BIG + 1000
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(N * S,)], N)
    assert u.S == S
    c = torch.empty((N, S), dtype=torch.bfloat16, device=dev())
    idx = torch.arange(S, dtype=torch.int64, device=dev())
    for r in range(N):
        t = idx.mul(2 * r + 1)
        t.add_(7 * r).remainder_(251).sub_(125)
        c[r].copy_(t.to(torch.float32).mul_(2.0 ** -10))
        del t
    del idx
    torch.cuda.empty_cache()
    out = torch.empty(S, device=dev())
    B.fsdp_grad_reduce_shard(u, [c[r] for r in range(N)], 4.0, 8.0, out)
    _sync()
    sample = _sample_idx(S, 9)
    ti = torch.from_numpy(sample).to(dev())
    cs = [to_host(c[r].view(torch.int16).index_select(0, ti)).view(np.uint16) for r in range(N)]
    assert_f32_tol_then_bits(to_host(out.index_select(0, ti)), oracle.grad_reduce(cs, 4.0, 8.0),
                             "sweep samples beyond 2^31")


@pytest.mark.parametrize("rem", [0, 1, 3, 7, 2047])
def test_xcd_ordered_launches_cover_every_tile_once(rem):
    """Launches of at least 2^18 tiles run in XCD-chunked order (in each group of 8 x 256
    tiles every XCD takes 256 consecutive ones; a partial last group is split evenly, the
    first G % 8 XCDs one tile more).  Here G = 2^18 + rem tiles of 1024 fp32 (rem = 2047: a
    partial group of 2047) with a ragged last tile and a segment boundary inside an XCD's run
    (two parameters, N = 1, so the shard is the concatenation): every element must land once,
    bit for bit, and the fp32 -> bf16 copy-out of the same layout (2048-element tiles, so
    about as many tiles) must match torch's cast."""
    tiles = (1 << 18) + rem
    n = tiles * 1024 - 5
    a_n = 37 * 1024 * 1024 + 11  # the boundary falls mid-tile, inside one XCD's run
    shapes = [(a_n,), (n - a_n,)]
    u = B.fsdp_unit_create(B.FSDP_FLAT, shapes, 1)
    assert u.S == n
    gen = torch.Generator(device=dev()).manual_seed(500 + rem)
    params = [torch.randn(s, device=dev(), generator=gen) for s in shapes]
    shard = torch.full((n,), float("nan"), device=dev())
    B.fsdp_flatten_shard(u, params, 0, shard)
    _sync()
    assert _same_bits(shard, torch.cat(params)), rem
    # copy-out: 2048-element tiles, so twice the size again crosses 2^18 tiles
    big_n = 2 * n
    u2 = B.fsdp_unit_create(B.FSDP_FLAT, [(big_n - a_n,), (a_n,)], 1)
    g = torch.randn(big_n, device=dev(), generator=gen)
    outs = [torch.empty(big_n - a_n, dtype=torch.bfloat16, device=dev()),
            torch.empty(a_n, dtype=torch.bfloat16, device=dev())]
    B.fsdp_unflatten_copyout(u2, g, outs)
    _sync()
    assert _same_bits(torch.cat(outs), g.to(torch.bfloat16)), rem
    idx = _sample_idx(big_n, 600 + rem)
    got = to_host(torch.cat(outs))[idx]
    assert_bf16_bits(got, oracle.bf16(to_host(g)[idx]), "copy-out samples rem=%d" % rem)
