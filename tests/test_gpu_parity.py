"""GPU parity: every kernel of the library (through its C ABI) against the CPU oracle,
element by element, on seeded inputs.

Bar: flatten, row sharding, copy-out and the bf16 cast are bit-exact (any NaN
matches any NaN); the reduction and AdamW are within 2 fp32 ulp or 1e-6 relative
and, since both sides follow the same operation order, also bit-exact.

Covered: the five synthetic units at full size (GPT-175B block included, in the
launch configuration the benchmark times), padded and misaligned variants, the
FSDP paper's Fig. 3 unit, brute force over tiny random units, ragged tails,
chunked launches (more segments / contributions than one launch holds), special
float values, and empty shards.
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


# ---------------------------------------------------------------------------
# bf16 cast (through the copy-out kernel, N = 1)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kind", ["special", "random_bits", "normal"])
def test_cast_matches_oracle(kind):
    if kind == "special":
        x = np.tile(W.special_f32(), 37)
    elif kind == "random_bits":
        x = W.random_bits_f32((1 << 22) + 13, seed=5)
    else:
        x = W.host_normal((1 << 22) + 5, 1.0, seed=6) * np.float32(1e3)
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(x.size,)], 1)
    out = torch.empty(x.size, dtype=torch.bfloat16, device=dev())
    B.fsdp_unflatten_copyout(u, to_dev(x), [out])
    _sync()
    assert_bf16_bits(to_host(out), oracle.bf16(x), kind)


# ---------------------------------------------------------------------------
# FSDP1 flatten + shard
# ---------------------------------------------------------------------------

def _flat_cases():
    cases = []
    for N in (1, 3, 4, 5, 7, 16):
        cases.append(("tiny", N))
    for N in (8, 3, 6, 7):
        cases.append(("gpt2l", N))
    return cases


def _unit_by_name(name, N):
    return {"tiny": W.tiny_mlp, "gpt2l": W.gpt2_large_block, "t5": W.t5_11b_block,
            "rows": W.gpt2_large_emb_rows}[name](N)


@pytest.mark.parametrize("name,N", _flat_cases())
def test_flat_flatten_every_rank(name, N):
    unit = _unit_by_name(name, N)
    params = W.host_params(unit, seed=0)
    u = B.fsdp_unit_create(B.FSDP_FLAT, unit.shapes, N)
    d_params = [to_dev(p) for p in params]
    ks = list(range(N)) + [B.FSDP_ALL_RANKS]
    outs = {}
    for k in ks:
        n = u.L if k == B.FSDP_ALL_RANKS else u.S
        outs[k] = torch.full((n,), float("nan"), dtype=torch.float32, device=dev())
        B.fsdp_flatten_shard(u, d_params, k, outs[k])
    _sync()
    for k in ks:
        assert_f32_bits(to_host(outs[k]), oracle.flat_shard(params, N, k), "%s N=%d k=%d" % (name, N, k))


def test_flat_parameter_order_moves_only_the_straddles():
    """Reading c of the unit order: the caller's list order.  The GPT-2-L block in module
    registration order (ln1, attention, ln2, MLP) instead of the config order: every rank's
    shard and the gathered layout against the oracle bit for bit, the same sizes, the same
    multiset of flat values, and every parameter's bf16 copy-out identical in both orders."""
    unit = W.gpt2_large_block(N=8)
    reg = [0, 1, 4, 5, 6, 7, 2, 3, 8, 9, 10, 11]  # ln1.w/b, qkv, proj, ln2.w/b, fc, fc2
    assert [unit.names[i] for i in reg][:6] == ["ln1.w", "ln1.b", "attn.qkv.w", "attn.qkv.b",
                                                "attn.proj.w", "attn.proj.b"]
    params = W.host_params(unit, seed=0)
    for N in (8, 7):
        orders = {}
        for name, idx in (("config", list(range(12))), ("registration", reg)):
            shapes = [unit.shapes[i] for i in idx]
            ps = [params[i] for i in idx]
            u = B.fsdp_unit_create(B.FSDP_FLAT, shapes, N)
            d_ps = [to_dev(q) for q in ps]
            gathered = torch.full((u.L,), float("nan"), device=dev())
            B.fsdp_flatten_shard(u, d_ps, B.FSDP_ALL_RANKS, gathered)
            shard = torch.empty(u.S, device=dev())
            for k in range(N):
                B.fsdp_flatten_shard(u, d_ps, k, shard)
                _sync()
                assert_f32_bits(to_host(shard), oracle.flat_shard(ps, N, k),
                                "%s order N=%d k=%d" % (name, N, k))
            outs = [torch.empty(sh, dtype=torch.bfloat16, device=dev()) for sh in shapes]
            B.fsdp_unflatten_copyout(u, gathered, outs)
            _sync()
            g = to_host(gathered)
            assert_f32_bits(g, oracle.flat_shard(ps, N, -1), "%s order N=%d gathered" % (name, N))
            by_param = {idx[j]: to_host(outs[j]) for j in range(12)}
            orders[name] = (u.S, u.L, np.sort(g.view(np.uint32)), by_param)
        a, b = orders["config"], orders["registration"]
        assert a[0] == b[0] and a[1] == b[1]
        assert np.array_equal(a[2], b[2])
        for i in range(12):
            assert np.array_equal(a[3][i], b[3][i]), unit.names[i]


def test_flat_flatten_fig3_units():
    for shapes in ([(3, 4), (3,)], [(4, 3), (4,)]):
        params = [np.arange(np.prod(s), dtype=np.float32).reshape(s) + 1 for s in shapes]
        u = B.fsdp_unit_create(B.FSDP_FLAT, shapes, 16)
        d_params = [to_dev(p) for p in params]
        for k in range(16):
            out = torch.full((1,), float("nan"), device=dev())
            B.fsdp_flatten_shard(u, d_params, k, out)
            _sync()
            assert_f32_bits(to_host(out), oracle.flat_shard(params, 16, k), "fig3 k=%d" % k)


def test_flat_flatten_bruteforce_tiny_units():
    """Random tiny units (0-d and zero-size parameters included), N up to 17, every rank,
    parameters placed at arbitrary 4-byte offsets so that the realigning path runs."""
    rng = np.random.Generator(np.random.PCG64(77))
    for trial in range(60):
        shapes = W.random_unit_shapes(rng, max_params=5, max_dim=7)
        params = [rng.standard_normal(size=s).astype(np.float32) for s in shapes]
        offs = [int(rng.integers(0, 4)) for _ in shapes]
        d_params, keep = [], []
        for p, o in zip(params, offs):
            v, base = offset_view(p.size, torch.float32, o)
            v.copy_(torch.from_numpy(p.reshape(-1)))
            d_params.append(v)
            keep.append(base)
        for N in (1, 2, 3, 4, 5, 8, 13, 17):
            u = B.fsdp_unit_create(B.FSDP_FLAT, shapes, N)
            res = []
            for k in list(range(N)) + [B.FSDP_ALL_RANKS]:
                n = u.L if k == B.FSDP_ALL_RANKS else u.S
                so = int(rng.integers(0, 4))
                out, ob = offset_view(n, torch.float32, so)
                out.fill_(float("nan"))
                B.fsdp_flatten_shard(u, d_params, k, out)
                res.append((k, out, ob))
            _sync()
            for k, out, _ in res:
                assert_f32_bits(to_host(out), oracle.flat_shard(params, N, k),
                                "trial %d %s N=%d k=%d" % (trial, shapes, N, k))


def test_flat_flatten_many_params_chunked_launches():
    """More segments than one launch's argument block holds (61 parameters)."""
    rng = np.random.Generator(np.random.PCG64(3))
    shapes = [(int(rng.integers(1, 300)),) for _ in range(61)]
    params = [rng.standard_normal(size=s).astype(np.float32) for s in shapes]
    for N in (1, 2):
        u = B.fsdp_unit_create(B.FSDP_FLAT, shapes, N)
        d_params = [to_dev(p) for p in params]
        out = torch.full((u.L,), float("nan"), device=dev())
        B.fsdp_flatten_shard(u, d_params, B.FSDP_ALL_RANKS, out)
        _sync()
        assert_f32_bits(to_host(out), oracle.flat_shard(params, N, -1), "61 params N=%d" % N)


# ---------------------------------------------------------------------------
# FSDP1 copy-out
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,N", [("tiny", 4), ("tiny", 3), ("tiny", 7), ("gpt2l", 8),
                                    ("gpt2l", 7)])
def test_flat_copyout(name, N):
    unit = _unit_by_name(name, N)
    u = B.fsdp_unit_create(B.FSDP_FLAT, unit.shapes, N)
    gathered = W.host_normal(u.L, 0.02, seed=11)
    outs = [torch.empty(s, dtype=torch.bfloat16, device=dev()) for s in unit.shapes]
    B.fsdp_unflatten_copyout(u, to_dev(gathered), outs)
    _sync()
    want = oracle.flat_copyout(unit.shapes, gathered)
    for i, (o, w) in enumerate(zip(outs, want)):
        assert_bf16_bits(to_host(o), w, "%s N=%d param %d" % (name, N, i))


def test_flat_copyout_misaligned_outputs_and_bruteforce():
    rng = np.random.Generator(np.random.PCG64(12))
    for trial in range(80):
        shapes = W.random_unit_shapes(rng, max_params=5, max_dim=9)
        N = int(rng.integers(1, 9))
        u = B.fsdp_unit_create(B.FSDP_FLAT, shapes, N)
        go = int(rng.integers(0, 4))
        g_host = (rng.standard_normal(u.L) * 3).astype(np.float32)
        gv, gb = offset_view(u.L, torch.float32, go)
        gv.copy_(torch.from_numpy(g_host))
        outs, keep = [], []
        for s in shapes:
            n = int(np.prod(s, dtype=np.int64)) if len(s) else 1
            v, base = offset_view(n, torch.bfloat16, int(rng.integers(0, 8)))
            outs.append(v)
            keep.append(base)
        B.fsdp_unflatten_copyout(u, gv, outs)
        _sync()
        want = oracle.flat_copyout(shapes, g_host)
        for i, (o, w) in enumerate(zip(outs, want)):
            assert_bf16_bits(to_host(o), w.reshape(-1), "trial %d param %d" % (trial, i))


def test_flat_roundtrip_flatten_then_copyout_is_cast_of_params():
    unit = W.gpt2_large_block(N=8)
    params = W.host_params(unit, seed=2)
    u = B.fsdp_unit_create(B.FSDP_FLAT, unit.shapes, unit.N)
    d_params = [to_dev(p) for p in params]
    gathered = torch.empty(u.L, device=dev())
    B.fsdp_flatten_shard(u, d_params, B.FSDP_ALL_RANKS, gathered)
    outs = [torch.empty(s, dtype=torch.bfloat16, device=dev()) for s in unit.shapes]
    B.fsdp_unflatten_copyout(u, gathered, outs)
    _sync()
    for p, o in zip(params, outs):
        assert_bf16_bits(to_host(o), oracle.bf16(p), "round trip")


# ---------------------------------------------------------------------------
# FSDP2 row sharding and copy-out
# ---------------------------------------------------------------------------

def test_rows_config_every_rank_and_copyout():
    unit = W.gpt2_large_emb_rows(N=8)
    params = W.host_params(unit, seed=0)
    u = B.fsdp_unit_create(B.FSDP_ROWS, unit.shapes, unit.N)
    assert u.S == 10_501_920
    d_params = [to_dev(p) for p in params]
    for k in list(range(unit.N)) + [B.FSDP_ALL_RANKS]:
        n = u.L if k == B.FSDP_ALL_RANKS else u.S
        out = torch.full((n,), float("nan"), device=dev())
        B.fsdp_flatten_shard(u, d_params, k, out)
        _sync()
        assert_f32_bits(to_host(out), oracle.rows_shard(params, unit.N, k), "rows k=%d" % k)
        del out
    gathered = W.host_normal(u.L, 0.02, seed=21)
    outs = [torch.empty(s, dtype=torch.bfloat16, device=dev()) for s in unit.shapes]
    B.fsdp_unflatten_copyout(u, to_dev(gathered), outs)
    _sync()
    want = oracle.rows_copyout(unit.shapes, unit.N, gathered)
    for i, (o, w) in enumerate(zip(outs, want)):
        assert_bf16_bits(to_host(o), w, "rows copy-out param %d" % i)


def test_rows_bruteforce_tiny_units():
    rng = np.random.Generator(np.random.PCG64(41))
    for trial in range(60):
        shapes = W.random_unit_shapes(rng, max_params=4, max_dim=9)
        params = [rng.standard_normal(size=s).astype(np.float32) for s in shapes]
        d_params, keep = [], []
        for p in params:
            v, base = offset_view(p.size, torch.float32, int(rng.integers(0, 4)))
            v.copy_(torch.from_numpy(p.reshape(-1)))
            d_params.append(v)
            keep.append(base)
        for N in (1, 2, 3, 4, 7, 9):
            u = B.fsdp_unit_create(B.FSDP_ROWS, shapes, N)
            res = []
            for k in list(range(N)) + [B.FSDP_ALL_RANKS]:
                n = u.L if k == B.FSDP_ALL_RANKS else u.S
                out, ob = offset_view(n, torch.float32, int(rng.integers(0, 4)))
                out.fill_(float("nan"))
                B.fsdp_flatten_shard(u, d_params, k, out)
                res.append((k, out, ob))
            g_host = (rng.standard_normal(u.L)).astype(np.float32)
            outs = [torch.empty(s, dtype=torch.bfloat16, device=dev()) for s in shapes]
            B.fsdp_unflatten_copyout(u, to_dev(g_host), outs)
            _sync()
            for k, out, _ in res:
                assert_f32_bits(to_host(out), oracle.rows_shard(params, N, k),
                                "trial %d %s N=%d k=%d" % (trial, shapes, N, k))
            for i, (o, w) in enumerate(zip(outs, oracle.rows_copyout(shapes, N, g_host))):
                assert_bf16_bits(to_host(o), w, "trial %d copy-out %d" % (trial, i))


def test_rows_many_ranks_chunked_segments():
    """N = 64 with ragged chunks: the all-ranks shard has more segments than one launch."""
    shapes = [(5, 3), (130, 7), (3,), (), (64, 2), (1, 9)] * 6
    rng = np.random.Generator(np.random.PCG64(8))
    params = [rng.standard_normal(size=s).astype(np.float32) for s in shapes]
    N = 64
    u = B.fsdp_unit_create(B.FSDP_ROWS, shapes, N)
    out = torch.full((u.L,), float("nan"), device=dev())
    B.fsdp_flatten_shard(u, [to_dev(p) for p in params], B.FSDP_ALL_RANKS, out)
    g_host = rng.standard_normal(u.L).astype(np.float32)
    outs = [torch.empty(s, dtype=torch.bfloat16, device=dev()) for s in shapes]
    B.fsdp_unflatten_copyout(u, to_dev(g_host), outs)
    _sync()
    assert_f32_bits(to_host(out), oracle.rows_shard(params, N, -1), "rows N=64 all")
    for i, (o, w) in enumerate(zip(outs, oracle.rows_copyout(shapes, N, g_host))):
        assert_bf16_bits(to_host(o), w, "rows N=64 copy-out %d" % i)


# ---------------------------------------------------------------------------
# gradient reduction
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,S,pre,post", [
    (4, 788, 2.0, 2.0), (8, 2459680, 2.0, 4.0), (8, 10501920, 2.0, 4.0), (6, 1001, 2.0, 3.0),
    (3, 37, 3.0, 1.0), (5, 12345, 1.0, 1.0), (1, 100, 1.0, 1.0), (7, 5, 0.5, 3.0),
    (200, 3001, 8.0, 25.0), (129, 2048, 1.0, 129.0), (16, 2049, -4.0, 4.0), (2, 1, 1.0, 1.0)])
def test_grad_reduce(N, S, pre, post):
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(N * S,)], N)
    assert u.S == S
    c = W.host_contribs(N, S, step=1)
    d_c = [to_dev(c[r]) for r in range(N)]
    out = torch.full((S,), float("nan"), device=dev())
    B.fsdp_grad_reduce_shard(u, d_c, pre, post, out)
    _sync()
    assert_f32_tol_then_bits(to_host(out), oracle.grad_reduce(list(c), pre, post),
                             "N=%d S=%d pre=%g post=%g" % (N, S, pre, post))


def test_grad_reduce_misaligned_and_special_values():
    rng = np.random.Generator(np.random.PCG64(4))
    N, S = 9, 5003
    c = W.host_contribs(N, S, step=2)
    specials = np.asarray([0x8000, 0x0000, 0x7F80, 0xFF80, 0x7FC0, 0x0001, 0x8001, 0x7F7F, 0xFF7F],
                          np.uint16)
    for r in range(N):
        idx = rng.integers(0, S, size=40)
        c[r, idx] = rng.choice(specials, size=40)
    c[:, :16] = 0x8000  # all -0 columns stay -0
    views, keep = [], []
    for r in range(N):
        v, base = offset_view(S, torch.bfloat16, int(rng.integers(0, 8)))
        v.copy_(to_dev(c[r]))
        views.append(v)
        keep.append(base)
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(N * S,)], N)
    for pre, post in [(1.0, 1.0), (2.0, 4.5), (3.0, 3.0)]:
        out, ob = offset_view(S, torch.float32, int(rng.integers(0, 4)))
        B.fsdp_grad_reduce_shard(u, views, pre, post, out)
        _sync()
        assert_f32_tol_then_bits(to_host(out), oracle.grad_reduce(list(c), pre, post),
                                 "misaligned pre=%g post=%g" % (pre, post))


@pytest.mark.parametrize("N,S,pre,post,seed", [
    (9, 5003, 2.0, 4.5, 11), (128, 4101, 8.0, 16.0, 12), (130, 2051, 1.0, 130.0, 13),
    (3, 517, 3.0, 1.0, 14), (16, 100003, 4.0, 4.0, 15), (8, 7, 2.0, 4.0, 16)])
def test_grad_reduce_realigned_contribs(N, S, pre, post, seed):
    """Output 16-byte aligned, each contribution at a 2-byte offset of its own (rank 0
    misaligned, the others drawn from 0..7): the vector path reads the two aligned
    granules around a lane's 8 elements and shifts them into place."""
    rng = np.random.Generator(np.random.PCG64(seed))
    c = W.host_contribs(N, S, step=seed)
    offs = rng.integers(0, 8, size=N)
    offs[0] = 5
    views, keep = [], []
    for r in range(N):
        v, base = offset_view(S, torch.bfloat16, int(offs[r]))
        v.copy_(to_dev(c[r]))
        views.append(v)
        keep.append(base)
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(N * S,)], N)
    out = torch.full((S,), float("nan"), device=dev())
    assert out.data_ptr() % 16 == 0
    B.fsdp_grad_reduce_shard(u, views, pre, post, out)
    _sync()
    assert_f32_tol_then_bits(to_host(out), oracle.grad_reduce(list(c), pre, post),
                             "realigned N=%d S=%d" % (N, S))


@pytest.mark.parametrize("N,S", [(120, 3001), (16, 8197), (7, 1030), (129, 1027), (130, 2050)])
def test_grad_reduce_stacked_rows_off_16_bytes(N, S):
    """Rows of one [N, S] receive buffer with S % 8 != 0 start at every 2-byte offset."""
    c = W.host_contribs(N, S, step=21)
    buf = to_dev(c)
    rows = [buf[r] for r in range(N)]
    assert len({r.data_ptr() % 16 for r in rows}) > 1
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(N * S,)], N)
    out = torch.full((S,), float("nan"), device=dev())
    B.fsdp_grad_reduce_shard(u, rows, 4.0, N / 4.0, out)
    _sync()
    assert_f32_tol_then_bits(to_host(out), oracle.grad_reduce(list(c), 4.0, N / 4.0),
                             "stacked N=%d S=%d" % (N, S))


# ---------------------------------------------------------------------------
# AdamW
# ---------------------------------------------------------------------------

def _adam_run(S, steps, hp, *, misalign=0, bf16=True, seed=0):
    rng = np.random.Generator(np.random.PCG64(seed))
    p = (rng.standard_normal(S) * 0.02).astype(np.float32)
    hp_, hm, hv = p.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32)
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(S,)], 1)
    keep = []

    def buf(a, dtype=torch.float32):
        v, base = offset_view(S, dtype, misalign)
        if a is not None:
            v.copy_(to_dev(a))
        keep.append(base)
        return v

    dp, dm, dv = buf(p), buf(np.zeros(S, np.float32)), buf(np.zeros(S, np.float32))
    dpb = buf(None, torch.bfloat16) if bf16 else None
    for t in range(1, steps + 1):
        g = W.host_normal(S, 1e-3, seed=1000 * t)
        dg = buf(g)
        B.fsdp_adam_shard(u, dp, dg, dm, dv, step=t, param_bf16=dpb, **hp)
        hpb = oracle.adamw(hp_, g, hm, hv, step=t, want_bf16=bf16, **hp)
        _sync()
        what = "S=%d t=%d mis=%d" % (S, t, misalign)
        assert_f32_tol_then_bits(to_host(dp), hp_, "param " + what)
        assert_f32_tol_then_bits(to_host(dm), hm, "exp_avg " + what)
        assert_f32_tol_then_bits(to_host(dv), hv, "exp_avg_sq " + what)
        if bf16:
            assert_bf16_bits(to_host(dpb), hpb, "param_bf16 " + what)


def test_adamw_tiny_config_ten_steps():
    unit = W.tiny_mlp()
    _adam_run(788, 10, dict(unit.adam))


@pytest.mark.parametrize("S", [1, 7, 8, 9, 2047, 2048, 2049, 100003])
def test_adamw_ragged_lengths(S):
    _adam_run(S, 3, dict(lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01), seed=S)


@pytest.mark.parametrize("mis", [1, 2, 3])
def test_adamw_misaligned(mis):
    _adam_run(10007, 2, dict(lr=3e-4, betas=(0.9, 0.95), eps=1e-6, weight_decay=0.1),
              misalign=mis, seed=mis)


@pytest.mark.parametrize("hp", [dict(lr=1e-3, betas=(0.0, 0.999), eps=1e-8, weight_decay=0.0),
                                dict(lr=1e-2, betas=(0.9, 0.0), eps=1e-30, weight_decay=0.5),
                                dict(lr=-1e-3, betas=(0.5, 0.5), eps=0.0, weight_decay=0.01)])
def test_adamw_hyperparameter_corners(hp):
    _adam_run(4099, 3, hp, bf16=False, seed=9)


def test_adamw_resume_bitwise():
    """10 steps equal 5 steps, a host save/restore of (p, m, v), and 5 more steps."""
    S = 50001
    hp = dict(lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01)
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(S,)], 1)
    p0 = W.host_normal(S, 0.02, seed=1)
    grads = [to_dev(W.host_normal(S, 1e-3, seed=t)) for t in range(1, 11)]

    def fresh():
        return to_dev(p0), torch.zeros(S, device=dev()), torch.zeros(S, device=dev())

    a = fresh()
    for t in range(1, 11):
        B.fsdp_adam_shard(u, a[0], grads[t - 1], a[1], a[2], step=t, **hp)
    b = fresh()
    for t in range(1, 6):
        B.fsdp_adam_shard(u, b[0], grads[t - 1], b[1], b[2], step=t, **hp)
    saved = [to_host(x).copy() for x in b]
    b = [to_dev(x) for x in saved]
    for t in range(6, 11):
        B.fsdp_adam_shard(u, b[0], grads[t - 1], b[1], b[2], step=t, **hp)
    _sync()
    for x, y in zip(a, b):
        assert_f32_bits(to_host(x), to_host(y), "resume")


# ---------------------------------------------------------------------------
# full-size units, in the launch configuration the benchmark times
# ---------------------------------------------------------------------------

def test_t5_block_full_size():
    unit = W.t5_11b_block(N=8)
    u = B.fsdp_unit_create(B.FSDP_FLAT, unit.shapes, unit.N)
    d_params = W.device_params(unit, seed=0)
    params = [to_host(p) for p in d_params]
    for k in (0, 7):
        out = torch.empty(u.S, device=dev())
        B.fsdp_flatten_shard(u, d_params, k, out)
        _sync()
        assert_f32_bits(to_host(out), oracle.flat_shard(params, unit.N, k), "t5 flatten k=%d" % k)
        del out
    del d_params
    gathered = torch.randn(u.L, device=dev(), generator=torch.Generator(device=dev()).manual_seed(5))
    outs = [torch.empty(s, dtype=torch.bfloat16, device=dev()) for s in unit.shapes]
    B.fsdp_unflatten_copyout(u, gathered, outs)
    _sync()
    want = oracle.flat_copyout(unit.shapes, to_host(gathered))
    for i, (o, w) in enumerate(zip(outs, want)):
        assert_bf16_bits(to_host(o), w, "t5 copy-out %d" % i)


def test_t5_block_full_size_reduce_and_adamw():
    """T5-11B block shard (S = 25,165,952), N = 8: the reduction of 8 bf16 contributions and
    two AdamW steps, every element against the oracle."""
    unit = W.t5_11b_block(N=8)
    u = B.fsdp_unit_create(B.FSDP_FLAT, unit.shapes, unit.N)
    S = u.S
    c = W.device_contribs(unit.N, S, step=1)
    grad = torch.empty(S, device=dev())
    B.fsdp_grad_reduce_shard(u, [c[r] for r in range(unit.N)], 2.0, 4.0, grad)
    _sync()
    g_host = oracle.grad_reduce(list(to_host(c)), 2.0, 4.0)
    assert_f32_tol_then_bits(to_host(grad), g_host, "t5 reduce")
    del c
    hp = unit.adam
    gen = torch.Generator(device=dev()).manual_seed(3)
    p = torch.randn(S, device=dev(), generator=gen).mul_(unit.std)
    m, v = torch.zeros(S, device=dev()), torch.zeros(S, device=dev())
    hp_, hm, hv = to_host(p).copy(), np.zeros(S, np.float32), np.zeros(S, np.float32)
    for t in (1, 2):
        B.fsdp_adam_shard(u, p, grad, m, v, step=t, **hp)
        oracle.adamw(hp_, g_host, hm, hv, step=t, **hp)
        _sync()
        assert_f32_tol_then_bits(to_host(p), hp_, "t5 adam p t=%d" % t)
        assert_f32_tol_then_bits(to_host(m), hm, "t5 adam m t=%d" % t)
        assert_f32_tol_then_bits(to_host(v), hv, "t5 adam v t=%d" % t)


@pytest.fixture(scope="module")
def big175():
    unit = W.gpt175b_block(N=128)
    u = B.fsdp_unit_create(B.FSDP_FLAT, unit.shapes, unit.N)
    assert (u.S, u.L) == (14_157_024, 1_812_099_072)
    yield unit, u
    gc.collect()
    torch.cuda.empty_cache()


def test_gpt175b_flatten_sampled_ranks(big175):
    unit, u = big175
    d_params = W.device_params(unit, seed=0)
    params = [to_host(p) for p in d_params]
    for k in (0, 1, 63, 127):
        out = torch.empty(u.S, device=dev())
        B.fsdp_flatten_shard(u, d_params, k, out)
        _sync()
        assert_f32_bits(to_host(out), oracle.flat_shard(params, unit.N, k), "175b flatten k=%d" % k)
    del d_params, params


def test_gpt175b_copyout_full(big175):
    unit, u = big175
    gen = torch.Generator(device=dev()).manual_seed(7)
    gathered = torch.randn(u.L, device=dev(), generator=gen).mul_(unit.std)
    outs = [torch.empty(s, dtype=torch.bfloat16, device=dev()) for s in unit.shapes]
    B.fsdp_unflatten_copyout(u, gathered, outs)
    _sync()
    g_host = to_host(gathered)
    del gathered
    want = oracle.flat_copyout(unit.shapes, g_host)
    del g_host
    for i, (o, w) in enumerate(zip(outs, want)):
        assert_bf16_bits(to_host(o), w, "175b copy-out %d" % i)


def test_gpt175b_grad_reduce_full(big175):
    """The benchmarked configuration: 128 contributions in one receive buffer whose rows sit
    at the recommended pitch (S rounded up to whole 128-byte lines)."""
    unit, u = big175
    assert u.recv_pitch == 14_157_056
    c = W.device_contribs(unit.N, u.S, step=1, pitch=u.recv_pitch)
    assert all(c[r].data_ptr() % 128 == c[0].data_ptr() % 128 for r in range(unit.N))
    out = torch.empty(u.S, device=dev())
    B.fsdp_grad_reduce_shard(u, [c[r] for r in range(unit.N)], 8.0, 16.0, out)
    _sync()
    c_host = to_host(c)
    del c
    assert_f32_tol_then_bits(to_host(out), oracle.grad_reduce(list(c_host), 8.0, 16.0),
                             "175b reduce")


def test_gpt175b_adamw_two_steps(big175):
    unit, u = big175
    hp = unit.adam
    S = u.S
    gen = torch.Generator(device=dev()).manual_seed(9)
    p = torch.randn(S, device=dev(), generator=gen).mul_(unit.std)
    m, v = torch.zeros(S, device=dev()), torch.zeros(S, device=dev())
    pb = torch.empty(S, dtype=torch.bfloat16, device=dev())
    hp_, hm, hv = to_host(p).copy(), np.zeros(S, np.float32), np.zeros(S, np.float32)
    for t in (1, 2):
        g = torch.randn(S, device=dev(), generator=gen).mul_(1e-3)
        B.fsdp_adam_shard(u, p, g, m, v, step=t, param_bf16=pb, **hp)
        hpb = oracle.adamw(hp_, to_host(g), hm, hv, step=t, want_bf16=True, **hp)
        _sync()
        assert_f32_tol_then_bits(to_host(p), hp_, "175b adam p t=%d" % t)
        assert_f32_tol_then_bits(to_host(m), hm, "175b adam m t=%d" % t)
        assert_f32_tol_then_bits(to_host(v), hv, "175b adam v t=%d" % t)
        assert_bf16_bits(to_host(pb), hpb, "175b adam bf16 t=%d" % t)


def test_gpt175b_padded_n120_flatten(big175):
    """N = 120: S = 15,100,826 (S % 4 = 2), so rank starts are not 16-byte aligned and
    48 pad elements sit at the end of the last rank."""
    unit, _ = big175
    u = B.fsdp_unit_create(B.FSDP_FLAT, unit.shapes, 120)
    assert u.S % 4 == 2 and u.L - 1_812_099_072 == 48
    d_params = W.device_params(unit, seed=0)
    params = [to_host(p) for p in d_params]
    for k in (1, 119):
        out = torch.empty(u.S, device=dev())
        B.fsdp_flatten_shard(u, d_params, k, out)
        _sync()
        assert_f32_bits(to_host(out), oracle.flat_shard(params, 120, k), "175b N=120 k=%d" % k)


def test_gpt175b_n120_grad_reduce_full(big175):
    """N = 120 on the GPT-175B block: S = 15,100,826, so the rows of the [120, S] receive
    buffer start 0, 4, 8 or 12 bytes past a 16-byte boundary."""
    unit, _ = big175
    u = B.fsdp_unit_create(B.FSDP_FLAT, unit.shapes, 120)
    assert u.S == 15_100_826
    c = W.device_contribs(120, u.S, step=4)
    assert {c[r].data_ptr() % 16 for r in range(120)} == {0, 4, 8, 12}
    out = torch.empty(u.S, device=dev())
    B.fsdp_grad_reduce_shard(u, [c[r] for r in range(120)], 8.0, 15.0, out)
    _sync()
    c_host = to_host(c)
    del c
    assert_f32_tol_then_bits(to_host(out), oracle.grad_reduce(list(c_host), 8.0, 15.0),
                             "175b N=120 reduce")


@pytest.mark.parametrize("layout,name,N", [(B.FSDP_FLAT, "gpt2l", 8), (B.FSDP_FLAT, "tiny", 3),
                                           (B.FSDP_ROWS, "rows", 8)])
def test_multi_rank_without_a_cluster(layout, name, N):
    """N is only a layout parameter: looping k = 0..N-1 on one GPU, the shards concatenate to
    the all-ranks layout (what an AllGather of them returns), and rank k's reduction of the N
    simulated ranks' slices [kS, (k+1)S) of their full gradients is slice k of the reduction of
    the full gradients (what a ReduceScatter returns)."""
    unit = _unit_by_name(name, N)
    params = W.host_params(unit, seed=0)
    u = B.fsdp_unit_create(layout, unit.shapes, N)
    d_params = [to_dev(p) for p in params]
    shards = []
    for k in range(N):
        out = torch.full((u.S,), float("nan"), device=dev())
        B.fsdp_flatten_shard(u, d_params, k, out)
        shards.append(out)
    whole = torch.full((u.L,), float("nan"), device=dev())
    B.fsdp_flatten_shard(u, d_params, B.FSDP_ALL_RANKS, whole)
    _sync()
    assert torch.equal(torch.cat(shards).view(torch.int32), whole.view(torch.int32))
    # ReduceScatter: N simulated ranks, each with a full-length bf16 gradient
    full = W.host_contribs(N, u.L, step=7)
    d_full = [to_dev(full[r]) for r in range(N)]
    red = []
    for k in range(N):
        grad = torch.full((u.S,), float("nan"), device=dev())
        B.fsdp_grad_reduce_shard(u, [d_full[r][k * u.S:(k + 1) * u.S] for r in range(N)],
                                 2.0, N / 2.0, grad)
        red.append(grad)
    _sync()
    assert_f32_bits(to_host(torch.cat(red)), oracle.grad_reduce(list(full), 2.0, N / 2.0),
                    "%s reduce-scatter over N=%d" % (name, N))
