"""GPU parity of the next rows against the CPU oracle: casting before the gather,
the bf16 copy-out and copy-in (FSDP2 ReduceScatter input), the hybrid and
accumulating reduction, and local gradient accumulation -- each alone and
chained the way a training step uses them.  Bit-exact throughout (any NaN
matches any NaN; the reductions first within 2 ulp / 1e-6, then bit-exact).
"""
import gc

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import (assert_bf16_bits, assert_f32_bits, assert_f32_tol_then_bits, dev,
                      offset_view, to_dev, to_host)
from sharded_fsdp_flatten_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    d = dev()
    B.load()
    yield d
    gc.collect()
    torch.cuda.empty_cache()


def _sync():
    torch.cuda.synchronize()


def _layout(unit):
    return B.FSDP_FLAT if unit.layout == W.FLAT else B.FSDP_ROWS


def _shard_oracle(unit, params, k):
    return (oracle.flat_shard if unit.layout == W.FLAT else oracle.rows_shard)(params, unit.N, k)


# ---------------------------------------------------------------------------
# cast before the gather (NEXT-1)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "tiny5", "gpt2l", "rows"])
def test_cast_before_gather_equals_cast_after(name):
    unit = {"tiny": lambda: W.tiny_mlp(4), "tiny5": lambda: W.tiny_mlp(5),
            "gpt2l": W.gpt2_large_block, "rows": W.gpt2_large_emb_rows}[name]()
    params = W.host_params(unit, seed=4)
    u = B.fsdp_unit_create(_layout(unit), unit.shapes, unit.N)
    d_params = [to_dev(p) for p in params]
    shards = []
    for k in range(unit.N):
        s32 = torch.empty(u.S, device=dev())
        B.fsdp_flatten_shard(u, d_params, k, s32)
        s16 = torch.empty(u.S, dtype=torch.bfloat16, device=dev())
        B.fsdp_cast_to_bf16(u, k, s32, s16)
        shards.append(s16)
    gathered16 = torch.cat(shards)
    outs = [torch.empty(s, dtype=torch.bfloat16, device=dev()) for s in unit.shapes]
    B.fsdp_unflatten_copyout_bf16(u, gathered16, outs)
    _sync()
    o_shards = [_shard_oracle(unit, params, k) for k in range(unit.N)]
    o_g16 = np.concatenate([oracle.bf16(s) for s in o_shards])
    assert_bf16_bits(to_host(gathered16), o_g16, "%s cast shards" % name)
    if unit.layout == W.FLAT:
        want16 = oracle.flat_copyout_u16(unit.shapes, o_g16)
        want32 = oracle.flat_copyout(unit.shapes, np.concatenate(o_shards))
    else:
        want16 = oracle.rows_copyout_u16(unit.shapes, unit.N, o_g16)
        want32 = oracle.rows_copyout(unit.shapes, unit.N, np.concatenate(o_shards))
    for i, (o, w16, w32) in enumerate(zip(outs, want16, want32)):
        assert_bf16_bits(to_host(o), w16, "%s copy-out %d" % (name, i))
        assert_bf16_bits(w16, w32, "%s cast-before == cast-after %d" % (name, i))


def test_cast_all_ranks_and_special_values():
    x = np.concatenate([np.tile(W.special_f32(), 11), W.random_bits_f32(100003, seed=7)])
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(x.size,)], 3)
    src = torch.from_numpy(np.concatenate([x, np.zeros(u.L - x.size, np.float32)])).to(dev())
    out = torch.empty(u.L, dtype=torch.bfloat16, device=dev())
    B.fsdp_cast_to_bf16(u, B.FSDP_ALL_RANKS, src, out)
    part = torch.empty(u.S, dtype=torch.bfloat16, device=dev())
    B.fsdp_cast_to_bf16(u, 1, src[u.S:2 * u.S], part)
    _sync()
    want = oracle.bf16(to_host(src))
    assert_bf16_bits(to_host(out), want, "cast all")
    assert_bf16_bits(to_host(part), want[u.S:2 * u.S], "cast rank 1")


def test_bf16_copyout_bruteforce_misaligned():
    rng = np.random.Generator(np.random.PCG64(61))
    for trial in range(60):
        shapes = W.random_unit_shapes(rng, max_params=5, max_dim=9)
        layout = B.FSDP_FLAT if trial % 2 == 0 else B.FSDP_ROWS
        N = int(rng.integers(1, 9))
        u = B.fsdp_unit_create(layout, shapes, N)
        g = rng.integers(0, 1 << 16, size=u.L, dtype=np.uint32).astype(np.uint16)
        gv, gb = offset_view(u.L, torch.bfloat16, int(rng.integers(0, 8)))
        gv.copy_(to_dev(g))
        outs, keep = [], []
        for s in shapes:
            n = int(np.prod(s, dtype=np.int64)) if len(s) else 1
            v, base = offset_view(n, torch.bfloat16, int(rng.integers(0, 8)))
            outs.append(v)
            keep.append(base)
        B.fsdp_unflatten_copyout_bf16(u, gv, outs)
        _sync()
        want = (oracle.flat_copyout_u16(shapes, g) if layout == B.FSDP_FLAT
                else oracle.rows_copyout_u16(shapes, N, g))
        for i, (o, w) in enumerate(zip(outs, want)):
            assert np.array_equal(to_host(o), w.reshape(-1)), (trial, i)


# ---------------------------------------------------------------------------
# copy-in: per-parameter bf16 gradients -> ReduceScatter input (NEXT-2)
# ---------------------------------------------------------------------------

def test_copyin_rows_config_every_rank():
    unit = W.gpt2_large_emb_rows(N=8)
    u = B.fsdp_unit_create(B.FSDP_ROWS, unit.shapes, unit.N)
    rng = np.random.Generator(np.random.PCG64(5))
    grads = [rng.integers(0, 1 << 16, size=s, dtype=np.uint32).astype(np.uint16)
             for s in unit.shapes]
    d_grads = [to_dev(g) for g in grads]
    for k in [B.FSDP_ALL_RANKS, 0, 7]:
        out = torch.empty(u.L if k < 0 else u.S, dtype=torch.bfloat16, device=dev())
        B.fsdp_flatten_shard_bf16(u, d_grads, k, out)
        _sync()
        assert np.array_equal(to_host(out), oracle.rows_shard_u16(grads, unit.N, k)), k
        del out


def test_copyin_bruteforce_both_layouts_misaligned():
    rng = np.random.Generator(np.random.PCG64(62))
    for trial in range(60):
        shapes = W.random_unit_shapes(rng, max_params=4, max_dim=9)
        grads = [rng.integers(0, 1 << 16, size=s, dtype=np.uint32).astype(np.uint16) for s in shapes]
        d, keep = [], []
        for g in grads:
            v, base = offset_view(g.size, torch.bfloat16, int(rng.integers(0, 8)))
            v.copy_(to_dev(g.reshape(-1)))
            d.append(v)
            keep.append(base)
        for layout in (B.FSDP_FLAT, B.FSDP_ROWS):
            for N in (1, 2, 3, 5, 8):
                u = B.fsdp_unit_create(layout, shapes, N)
                res = []
                for k in list(range(N)) + [B.FSDP_ALL_RANKS]:
                    out, ob = offset_view(u.L if k < 0 else u.S, torch.bfloat16,
                                          int(rng.integers(0, 8)))
                    out.fill_(float("nan"))
                    B.fsdp_flatten_shard_bf16(u, d, k, out)
                    res.append((k, out, ob))
                _sync()
                f = oracle.flat_shard_u16 if layout == B.FSDP_FLAT else oracle.rows_shard_u16
                for k, out, _ in res:
                    assert np.array_equal(to_host(out), f(grads, N, k)), (trial, layout, N, k)


def test_fsdp2_backward_chain_copyin_then_reduce():
    """N simulated ranks each hold full per-parameter bf16 gradients; each copies them in
    to its ReduceScatter input; rank k reduces slice k of every rank's input."""
    unit = W.gpt2_large_emb_rows(N=8)
    u = B.fsdp_unit_create(B.FSDP_ROWS, unit.shapes, unit.N)
    rs_inputs = []
    host_inputs = []
    for r in range(unit.N):
        grads32 = [W.host_normal(int(np.prod(s)), 1e-3, seed=500 + 31 * r + i).reshape(s)
                   for i, s in enumerate(unit.shapes)]
        grads = [oracle.bf16(g) for g in grads32]
        out = torch.empty(u.L, dtype=torch.bfloat16, device=dev())
        B.fsdp_flatten_shard_bf16(u, [to_dev(g) for g in grads], B.FSDP_ALL_RANKS, out)
        rs_inputs.append(out)
        host_inputs.append(oracle.rows_shard_u16(grads, unit.N, -1))
    k = 5
    contribs = [x[k * u.S:(k + 1) * u.S] for x in rs_inputs]
    grad = torch.empty(u.S, device=dev())
    B.fsdp_grad_reduce_shard(u, contribs, 2.0, 4.0, grad)
    _sync()
    want = oracle.grad_reduce([h[k * u.S:(k + 1) * u.S] for h in host_inputs], 2.0, 4.0)
    assert_f32_tol_then_bits(to_host(grad), want, "fsdp2 backward chain")


# ---------------------------------------------------------------------------
# hybrid and accumulating reduction (NEXT-3 with communication, NEXT-4)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,S,group,pre,post", [
    (8, 100003, 2, 2.0, 4.0), (8, 100003, 4, 2.0, 4.0), (16, 5000, 8, 1.0, 16.0),
    (128, 70001, 8, 8.0, 16.0), (128, 4099, 16, 3.0, 5.0), (256, 2051, 32, 16.0, 16.0),
    (192, 1025, 64, 8.0, 24.0), (12, 33, 3, 1.0, 1.0), (8, 100003, 1, 2.0, 4.0),
    (8, 100003, 8, 2.0, 4.0)])
def test_hybrid_reduce(N, S, group, pre, post):
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(N * S,)], N)
    c = W.host_contribs(N, S, step=2)
    d_c = [to_dev(c[r]) for r in range(N)]
    out = torch.full((S,), float("nan"), device=dev())
    B.fsdp_grad_reduce_shard_ex(u, d_c, pre, post, out, group=group)
    _sync()
    assert_f32_tol_then_bits(to_host(out), oracle.grad_reduce_ex(list(c), pre, post, group=group),
                             "hybrid N=%d group=%d" % (N, group))


@pytest.mark.parametrize("N,group,pre,post", [(8, 0, 2.0, 4.0), (8, 2, 2.0, 4.0),
                                              (128, 0, 8.0, 16.0), (64, 16, 3.0, 1.0)])
def test_accumulating_reduce_over_micro_batches(N, group, pre, post):
    S = 30011
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(N * S,)], N)
    acc = torch.empty(S, device=dev())
    h_acc = np.zeros(S, np.float32)
    for t in range(1, 5):
        c = W.host_contribs(N, S, step=10 + t)
        d_c = [to_dev(c[r]) for r in range(N)]
        if t == 1:
            B.fsdp_grad_reduce_shard_ex(u, d_c, pre, post, acc, group=group)
            h_acc = oracle.grad_reduce_ex(list(c), pre, post, group=group)
        else:
            B.fsdp_grad_reduce_shard_ex(u, d_c, pre, post, acc, group=group, accumulate=True)
            oracle.grad_reduce_ex(list(c), pre, post, group=group, out=h_acc)
        _sync()
        assert_f32_tol_then_bits(to_host(acc), h_acc, "accumulate t=%d" % t)


def test_hybrid_and_accumulate_misaligned_scalar_path():
    rng = np.random.Generator(np.random.PCG64(64))
    N, S = 12, 4097
    c = W.host_contribs(N, S, step=3)
    views, keep = [], []
    for r in range(N):
        v, base = offset_view(S, torch.bfloat16, int(rng.integers(1, 8)))
        v.copy_(to_dev(c[r]))
        views.append(v)
        keep.append(base)
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(N * S,)], N)
    old = W.host_normal(S, 1e-3, seed=8)
    out, ob = offset_view(S, torch.float32, 1)
    out.copy_(to_dev(old))
    B.fsdp_grad_reduce_shard_ex(u, views, 2.0, 6.0, out, group=4, accumulate=True)
    _sync()
    want = old.copy()
    oracle.grad_reduce_ex(list(c), 2.0, 6.0, group=4, out=want)
    assert_f32_tol_then_bits(to_host(out), want, "misaligned hybrid accumulate")


@pytest.mark.parametrize("N,group,accumulate", [(16, 4, True), (12, 3, False), (256, 32, False),
                                                (8, 0, True)])
def test_hybrid_and_accumulate_realigned_contribs(N, group, accumulate):
    """Aligned output, contributions at 2-byte offsets 1..7: the shifted-granule vector
    path under hybrid groups, accumulation and chained launches."""
    rng = np.random.Generator(np.random.PCG64(65 + N))
    S = 6007
    c = W.host_contribs(N, S, step=5)
    views, keep = [], []
    for r in range(N):
        v, base = offset_view(S, torch.bfloat16, int(rng.integers(1, 8)))
        v.copy_(to_dev(c[r]))
        views.append(v)
        keep.append(base)
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(N * S,)], N)
    old = W.host_normal(S, 1e-3, seed=9)
    out = to_dev(old) if accumulate else torch.full((S,), float("nan"), device=dev())
    assert out.data_ptr() % 16 == 0
    B.fsdp_grad_reduce_shard_ex(u, views, 2.0, N / 2.0, out, group=group, accumulate=accumulate)
    _sync()
    want = old.copy() if accumulate else None
    got_want = oracle.grad_reduce_ex(list(c), 2.0, N / 2.0, group=group, out=want)
    assert_f32_tol_then_bits(to_host(out), want if accumulate else got_want,
                             "realigned hybrid N=%d group=%d acc=%d" % (N, group, accumulate))


# ---------------------------------------------------------------------------
# local accumulation without communication (NEXT-3)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,mis", [(1, 0), (7, 0), (2048, 0), (2049, 0), (1000003, 0), (4099, 1),
                                   (4099, 3)])
def test_local_accumulate(n, mis):
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(n,)], 1)
    acc, ab = offset_view(n, torch.float32, mis)
    h_acc = np.zeros(n, np.float32)
    for t in range(4):
        g = W.host_contribs(1, n, step=20 + t)[0]
        gv, gb = offset_view(n, torch.bfloat16, mis)
        gv.copy_(to_dev(g))
        B.fsdp_grad_accumulate(u, 0, gv, acc, t == 0)
        oracle.grad_accumulate(g, h_acc, init=(t == 0))
        _sync()
        assert_f32_tol_then_bits(to_host(acc), h_acc, "accumulate n=%d t=%d" % (n, t))


def test_without_communication_chain():
    """Micro-batches accumulate the unsharded gradient locally in fp32 (all L elements), the
    sum is cast to bf16 once, and the reduction runs only then, on rank k's slices."""
    unit = W.tiny_mlp(N=4)
    u = B.fsdp_unit_create(B.FSDP_FLAT, unit.shapes, unit.N)
    L, S, N = u.L, u.S, unit.N
    send = []
    h_send = []
    for r in range(N):
        acc = torch.empty(L, device=dev())
        h_acc = np.zeros(L, np.float32)
        for t in range(3):
            g = W.host_contribs(1, L, step=100 * r + t)[0]
            B.fsdp_grad_accumulate(u, B.FSDP_ALL_RANKS, to_dev(g), acc, t == 0)
            oracle.grad_accumulate(g, h_acc, init=(t == 0))
        g16 = torch.empty(L, dtype=torch.bfloat16, device=dev())
        B.fsdp_cast_to_bf16(u, B.FSDP_ALL_RANKS, acc, g16)
        send.append(g16)
        h_send.append(oracle.bf16(h_acc))
    k = 2
    out = torch.empty(S, device=dev())
    B.fsdp_grad_reduce_shard(u, [x[k * S:(k + 1) * S] for x in send], 2.0, 2.0, out)
    _sync()
    for r in range(N):
        assert_bf16_bits(to_host(send[r]), h_send[r], "rank %d cast" % r)
    want = oracle.grad_reduce([h[k * S:(k + 1) * S] for h in h_send], 2.0, 2.0)
    assert_f32_tol_then_bits(to_host(out), want, "no-communication chain")
