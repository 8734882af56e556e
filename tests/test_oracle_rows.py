"""Pins of the oracle's FSDP2 per-parameter dim-0 sharding.

The pages fix: torch.chunk splits each parameter along dim 0 ("FSDP"
concept page, FSDP1 vs FSDP2), each rank holding complete rows ("FSDP Under The
Hood", section 2).  torch.chunk itself is the library routine checked against.
"""
import numpy as np
import pytest
import torch

import workloads as W


def _rows_of(shape):
    if len(shape) == 0:
        return 1, 1
    r = 1
    for d in shape[1:]:
        r *= d
    return shape[0], r


def _torch_rank_segment(params, N, k):
    """Rank k's segment built from torch.chunk(dim=0): its chunk (or nothing when torch
    makes fewer than N chunks), zero-padded to the chunk size c = ceil(m/N)."""
    pieces = []
    for p in params:
        t = torch.from_numpy(np.ascontiguousarray(p))
        if t.dim() == 0:
            t = t.reshape(1)
        m, r = _rows_of(p.shape)
        c = -(-m // N)
        chunks = torch.chunk(t, N, dim=0) if m > 0 else ()
        mine = chunks[k].reshape(-1) if k < len(chunks) else torch.zeros(0)
        pieces.append(mine)
        pieces.append(torch.zeros(c * r - mine.numel()))
    return torch.cat(pieces) if pieces else torch.zeros(0)


def test_rows_shard_matches_torch_chunk(orc):
    rng = np.random.Generator(np.random.PCG64(2024))
    checked = 0
    for trial in range(120):
        shapes = W.random_unit_shapes(rng, max_params=4, max_dim=7)
        params = [rng.standard_normal(size=s).astype(np.float32) for s in shapes]
        for N in (1, 2, 3, 4, 5, 8, 9):
            P_r = orc.rows_sizes(shapes, N)
            full = orc.rows_shard(params, N, -1)
            assert full.size == N * P_r
            for k in range(N):
                seg = orc.rows_shard(params, N, k)
                ref = _torch_rank_segment(params, N, k).numpy()
                assert seg.size == P_r == ref.size
                assert np.array_equal(seg.view(np.uint32), ref.view(np.uint32)), (shapes, N, k)
                assert np.array_equal(full[k * P_r:(k + 1) * P_r], seg)
                checked += 1
    assert checked > 1000


@pytest.mark.parametrize("m,N,rows", [(5, 4, [2, 2, 1, 0]), (6, 4, [2, 2, 2, 0]),
                                      (3, 8, [1, 1, 1, 0, 0, 0, 0, 0]), (8, 8, [1] * 8),
                                      (0, 4, [0, 0, 0, 0]), (50257, 8, [6283] * 7 + [6276])])
def test_rows_per_rank_row_counts(orc, m, N, rows):
    """torch.chunk can make fewer chunks than ranks; trailing ranks then hold no rows.
    Row counts are read off the oracle's segments by labelling every row with its
    index + 1 (zero marks a pad row)."""
    r = 2
    p = (np.repeat(np.arange(m, dtype=np.float32) + 1, r)).reshape(m, r)
    got = []
    for k in range(N):
        seg = orc.rows_shard([p], N, k).reshape(-1, r) if m else np.zeros((0, r))
        got.append(int(np.count_nonzero(seg[:, 0])))
        # complete rows only: every non-pad row is a whole row of the parameter
        for row in seg:
            if row[0] != 0:
                assert np.all(row == row[0])
    assert got == rows
    ref = [c.shape[0] for c in torch.chunk(torch.zeros(m, r), N, dim=0)] if m else []
    assert got[:len(ref)] == ref


def test_rows_rebuild_and_copyout(orc):
    """Concatenating every rank's valid rows rebuilds each parameter; the copy-out casts
    it with torch's RNE bf16 cast as the library routine."""
    rng = np.random.Generator(np.random.PCG64(5))
    for trial in range(60):
        shapes = W.random_unit_shapes(rng, max_params=4, max_dim=6)
        params = [rng.standard_normal(size=s).astype(np.float32) for s in shapes]
        for N in (1, 2, 4, 7):
            full = orc.rows_shard(params, N, -1)
            outs = orc.rows_copyout(shapes, N, full)
            for p, o in zip(params, outs):
                ref = torch.from_numpy(p).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
                assert o.shape == p.shape
                assert np.array_equal(o, ref)


def test_rows_segment_length_same_for_every_rank(orc):
    """AllGather wants equal inputs (FSDP paper §3.4, Fig. 2a): every rank's segment has
    the same length P_r, including ranks that hold no rows at all."""
    params = [np.ones((5, 3), np.float32), np.ones((3,), np.float32), np.ones((), np.float32)]
    N = 4
    P_r = orc.rows_sizes([p.shape for p in params], N)
    assert P_r == 2 * 3 + 1 + 1
    for k in range(N):
        assert orc.rows_shard(params, N, k).size == P_r


def test_rows_config_sizes(orc):
    """FSDP2 unit (embedding [50257,1280] + one GPT-2 Large block, N = 8), worked by hand:
    embedding chunk 6283 rows (rank 7: 6276 + 7 pad rows = 8960 pad elements); every
    block parameter splits evenly, 2,459,680 elements per rank; P_r = 10,501,920."""
    u = W.gpt2_large_emb_rows()
    assert orc.rows_sizes(u.shapes, u.N) == 6283 * 1280 + 19677440 // 8 == 10501920
