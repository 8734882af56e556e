"""Pins of the oracle's FSDP1 FlatParameter (flatten + pad + equal split, copy-out).

Each test checks the oracle against something other than itself: a worked
example printed on the pages, torch's own cat/pad/chunk/split routines, a
closed-form slice formula, or an invariant the pages state.
"""
import numpy as np
import pytest
import torch

import workloads as W
from conftest import golden_path


def _labelled(shapes):
    """Parameters whose elements are labelled 1..T in flatten order (exact in fp32)."""
    out, nxt = [], 1
    for s in shapes:
        n = int(np.prod(s, dtype=np.int64)) if len(s) else 1
        out.append((np.arange(n, dtype=np.float32) + nxt).reshape(s))
        nxt += n
    return out


def _torch_padded_flat(params, N):
    """torch.cat of the flattened params, right-padded with zeros to a multiple of N."""
    flat = torch.cat([torch.from_numpy(np.ascontiguousarray(p)).reshape(-1) for p in params])
    T = flat.numel()
    L = -(-T // N) * N
    return torch.nn.functional.pad(flat, (0, L - T))


def _read_fig3():
    rows = []
    with open(golden_path("fig3_linear_n16.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, N, shapes, vals = [x.strip() for x in line.split("|")]
            shp = [tuple(int(d) for d in s.split("x")) for s in shapes.split(";")]
            rows.append((name, int(N), shp, [float(v) for v in vals.split()]))
    return rows


@pytest.mark.parametrize("case", _read_fig3(), ids=lambda c: c[0])
def test_fig3_worked_example(orc, case):
    """FSDP paper Fig. 3: one Linear over 16 GPUs, one element per GPU, last rank padded."""
    name, N, shapes, expected = case
    params = _labelled(shapes)
    T, S, L, pad = orc.flat_sizes([p.size for p in params], N)
    assert S == 1
    for k in range(N):
        shard = orc.flat_shard(params, N, k)
        assert shard.shape == (1,)
        assert shard[0] == expected[k], (name, k)


def test_flat_shard_matches_torch_cat_pad_chunk(orc):
    """Brute force over tiny units (T <= 64 after padding rules, N <= 17, every k)
    against torch.cat + pad + chunk as library routines."""
    rng = np.random.Generator(np.random.PCG64(1234))
    n_checked = 0
    for trial in range(150):
        shapes = W.random_unit_shapes(rng, max_params=5, max_dim=4)
        params = [rng.standard_normal(size=s).astype(np.float32) for s in shapes]
        T = sum(p.size for p in params)
        if T == 0 or T > 64:
            continue
        for N in range(1, 18):
            F = _torch_padded_flat(params, N)
            chunks = torch.chunk(F, N)
            assert len(chunks) == N
            full = orc.flat_shard(params, N, -1)
            assert np.array_equal(full.view(np.uint32), F.numpy().view(np.uint32))
            for k in range(N):
                shard = orc.flat_shard(params, N, k)
                assert np.array_equal(shard.view(np.uint32), chunks[k].numpy().view(np.uint32)), \
                    (shapes, N, k)
                n_checked += 1
    assert n_checked > 500


def test_gather_of_shards_is_the_flat_parameter(orc):
    """AllGather of the shards in rank order is the unsharded FlatParameter (FSDP paper §3.4,
    communication layout): concatenating all ranks' shards gives the padded flat buffer."""
    unit = W.tiny_mlp()
    params = W.host_params(unit, seed=0)
    for N in (1, 3, 4, 5, 7, 16, 3152, 3153, 5000):
        full = orc.flat_shard(params, N, -1)
        shards = [orc.flat_shard(params, N, k) for k in range(min(N, 64))] if N <= 64 else None
        if shards is not None:
            assert np.array_equal(np.concatenate(shards), full)
        T, S, L, pad = orc.flat_sizes(unit.numels, N)
        flat = np.concatenate([p.reshape(-1) for p in params])
        assert np.array_equal(full[:T], flat)
        assert np.all(full[T:] == 0) and np.all(np.signbit(full[T:]) == False)  # noqa: E712


@pytest.mark.parametrize("T,N", [(0, 1), (0, 8), (1, 1), (1, 8), (15, 16), (16, 16), (17, 16),
                                 (3152, 3), (3152, 5), (3152, 7), (19677440, 3), (19677440, 6),
                                 (19677440, 7), (1812099072, 120), (1812099072, 128)])
def test_flat_sizes_pad_bound(orc, T, N):
    """Pad on the right so the length divides by the sharding factor; at most F-1 pad
    elements (FSDP paper §3.4, flatten-concat-chunk)."""
    T2, S, L, pad = orc.flat_sizes([T], N)
    assert T2 == T
    assert L == N * S and L >= T
    assert 0 <= pad <= N - 1
    assert L - N < T or T == 0  # minimal: one fewer row of N would not hold the unit


def test_p3_floor_slices_when_divisible(orc):
    """"FSDP Architecture" page: GPU k holds elements floor(kP/N) .. floor((k+1)P/N)-1.
    With N | T this is the equal split with no padding."""
    rng = np.random.Generator(np.random.PCG64(7))
    for T, N in [(3152, 4), (3152, 8), (3152, 16), (4096, 64), (60, 12)]:
        params = [rng.standard_normal(T).astype(np.float32)]
        for k in range(N):
            lo, hi = (k * T) // N, ((k + 1) * T) // N
            assert np.array_equal(orc.flat_shard(params, N, k), params[0][lo:hi])


def test_config_sizes():
    """Unit sizes of the five synthetic units, worked by hand from their shapes."""
    import oracle
    expect = {
        "tiny-mlp": (3152, 788, 0),
        "gpt2-large-block": (19677440, 2459680, 0),
        "t5-11b-block": (201327616, 25165952, 0),
        "gpt-175b-block": (1812099072, 14157024, 0),
    }
    for u in W.all_units():
        if u.name in expect:
            T, S, L, pad = oracle.flat_sizes(u.numels, u.N)
            assert (T, S, pad) == expect[u.name]
    # tiny unit offsets 0/2048/2112/3136: rank 2 straddles W1|b1|W2, rank 3 straddles W2|b2
    u = W.tiny_mlp()
    assert list(np.cumsum([0] + u.numels[:-1])) == [0, 2048, 2112, 3136]


def test_flat_copyout_roundtrip_matches_torch_cast(orc):
    """copy-out(gather(all shards)) == bf16(original params), with torch's CPU cast as
    the library routine, and torch.split with the parameters' sizes as the slicer."""
    rng = np.random.Generator(np.random.PCG64(99))
    for trial in range(60):
        shapes = W.random_unit_shapes(rng, max_params=5, max_dim=5)
        params = [rng.standard_normal(size=s).astype(np.float32) * 3 for s in shapes]
        for N in (1, 2, 3, 8):
            full = orc.flat_shard(params, N, -1)
            outs = orc.flat_copyout(shapes, full)
            pieces = torch.split(torch.from_numpy(full[:sum(p.size for p in params)]),
                                 [p.size for p in params])
            for p, o, piece in zip(params, outs, pieces):
                ref = piece.reshape(p.shape).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
                assert o.shape == p.shape
                assert np.array_equal(o, ref)


def test_cast_before_gather_equals_cast_after(orc):
    """The pages cast before the AllGather; the copy-out casts after it.  Casting is
    elementwise and the gather only moves elements, so the two agree bit for bit."""
    unit = W.tiny_mlp(N=5)
    params = W.host_params(unit, seed=3)
    shards = [orc.flat_shard(params, unit.N, k) for k in range(unit.N)]
    gathered_bf16 = np.concatenate([orc.bf16(s) for s in shards])     # cast, then gather
    outs = orc.flat_copyout(unit.shapes, np.concatenate(shards))      # gather, then cast
    off = 0
    for o in outs:
        assert np.array_equal(o.reshape(-1), gathered_bf16[off:off + o.size])
        off += o.size
