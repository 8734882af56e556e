"""GPU parity of the sharded optimizer statistics (the per-rank half of the sharded
gradient scaler, and per-parameter sums of squares of a gradient shard) against the
oracle, through the C ABI."""
import gc

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import assert_f32_bits, dev, offset_view, to_dev, to_host
from sharded_fsdp_flatten_amd import binding as B

pytestmark = pytest.mark.gpu

U = 2.0 ** -53


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    d = dev()
    B.load()
    yield d
    gc.collect()
    torch.cuda.empty_cache()


def _sync():
    torch.cuda.synchronize()


def _grads(n, seed, scale=1e-3 * 65536.0):
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.standard_normal(n) * scale).astype(np.float32)


# ---------------------------------------------------------------------------
# unscale
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,inv,mis", [(1, 0.5, 0), (4096 * 3 + 17, 2.0 ** -16, 0),
                                       (1000003, 1.0 / 3.0, 0), (5003, 7.5e-5, 1),
                                       (4099, 2.0 ** -8, 3), (16384, 1.0, 0), (4096, 1e-30, 2)])
def test_unscale(n, inv, mis):
    host = _grads(n, seed=n)
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(n,)], 1)
    g, base = offset_view(n, torch.float32, mis)
    g.copy_(to_dev(host))
    flag = torch.zeros(1, device=dev())
    inv32 = float(np.float32(inv))
    B.fsdp_grad_unscale(u, 0, g, inv32, flag)
    _sync()
    want = host.copy()
    wflag = np.zeros(1, np.float32)
    oracle.grad_unscale(want, inv32, wflag)
    assert_f32_bits(to_host(g), want, "unscale n=%d inv=%g mis=%d" % (n, inv, mis))
    assert to_host(flag)[0] == wflag[0] == 0.0


@pytest.mark.parametrize("mis", [0, 1])
def test_unscale_flags_non_finite_inputs_and_shares_the_flag(mis):
    n = 3 * 4096 * 4 + 5
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(n,)], 1)
    flag = torch.zeros(1, device=dev())
    rng = np.random.Generator(np.random.PCG64(7 + mis))
    # a clean shard leaves the flag alone
    g, base = offset_view(n, torch.float32, mis)
    g.copy_(to_dev(_grads(n, 1)))
    B.fsdp_grad_unscale(u, 0, g, 0.25, flag)
    _sync()
    assert to_host(flag)[0] == 0.0
    for special in (np.inf, -np.inf, np.nan):
        host = _grads(n, 2)
        host[int(rng.integers(0, n))] = special
        g.copy_(to_dev(host))
        f = torch.zeros(1, device=dev())
        B.fsdp_grad_unscale(u, 0, g, 0.25, f)
        _sync()
        want = host.copy()
        wflag = np.zeros(1, np.float32)
        oracle.grad_unscale(want, 0.25, wflag)
        assert to_host(f)[0] == wflag[0] == 1.0
        assert_f32_bits(to_host(g), want, "unscale with %r" % special)
    # one flag over several shards: set by the second, kept through the third
    for i, host in enumerate([_grads(n, 3), _grads(n, 4), _grads(n, 5)]):
        if i == 1:
            host[n - 1] = np.inf  # in the ragged tail
        g.copy_(to_dev(host))
        B.fsdp_grad_unscale(u, 0, g, 0.5, flag)
        _sync()
        assert to_host(flag)[0] == (0.0 if i == 0 else 1.0)


@pytest.mark.parametrize("n,mis", [(4096 * 5 + 3, 0), (777, 1)])
def test_scale_without_flag_is_the_same_multiply(n, mis):
    """found_inf NULL: the clip-coefficient multiply; non-finite values pass through."""
    host = _grads(n, 9)
    host[3] = np.inf
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(n,)], 1)
    g, base = offset_view(n, torch.float32, mis)
    g.copy_(to_dev(host))
    coef = float(np.float32(0.123456))
    B.fsdp_grad_unscale(u, 0, g, coef, None)
    _sync()
    want = host.copy()
    oracle.grad_unscale(want, coef, np.zeros(1, np.float32))
    assert_f32_bits(to_host(g), want, "scale only n=%d" % n)


def test_unscale_whole_t5_layout_and_one_rank():
    unit = W.t5_11b_block(N=8)
    u = B.fsdp_unit_create(B.FSDP_FLAT, unit.shapes, 8)
    gen = torch.Generator(device=dev()).manual_seed(11)
    g = torch.randn(u.L, device=dev(), generator=gen)
    host = to_host(g)
    flag = torch.zeros(1, device=dev())
    B.fsdp_grad_unscale(u, B.FSDP_ALL_RANKS, g, 2.0 ** -12, flag)
    _sync()
    want = host.copy()
    wflag = np.zeros(1, np.float32)
    oracle.grad_unscale(want, 2.0 ** -12, wflag)
    assert_f32_bits(to_host(g), want, "T5 unscale, all ranks")
    shard = g[3 * u.S:4 * u.S]
    h3 = to_host(shard)
    B.fsdp_grad_unscale(u, 3, shard, 1.0 / 3.0, flag)
    _sync()
    oracle.grad_unscale(h3, float(np.float32(1.0 / 3.0)), wflag)
    assert_f32_bits(to_host(shard), h3, "T5 unscale, rank 3")
    assert to_host(flag)[0] == wflag[0] == 0.0


# ---------------------------------------------------------------------------
# per-parameter sums of squares
# ---------------------------------------------------------------------------

def _sqnorm_gpu(u, k, shard_dev):
    ws = torch.empty(max(1, B.fsdp_grad_sqnorm_workspace(u, k)), dtype=torch.float64, device=dev())
    out = torch.full((len(u.shapes),), float("nan"), dtype=torch.float64, device=dev())
    B.fsdp_grad_sqnorm(u, k, shard_dev, out, ws)
    _sync()
    return to_host(out)


def _oracle_sq(u, layout, k, shard_host):
    if layout == B.FSDP_FLAT:
        return oracle.flat_sqnorm(u.shapes, u.N, k, shard_host)
    return oracle.rows_sqnorm(u.shapes, u.N, k, shard_host)


def _many_shapes():
    rng = np.random.Generator(np.random.PCG64(61))
    shapes = []
    for i in range(61):
        kind = i % 4
        if kind == 0:
            shapes.append((int(rng.integers(1, 9000)),))
        elif kind == 1:
            shapes.append((int(rng.integers(1, 40)), int(rng.integers(1, 300))))
        elif kind == 2:
            shapes.append(())
        else:
            shapes.append((int(rng.integers(0, 3)), 5))
    return shapes


UNITS = {
    "tiny": (B.FSDP_FLAT, W.tiny_mlp().shapes, 4),
    "tiny_pad": (B.FSDP_FLAT, W.tiny_mlp().shapes, 7),
    "gpt2l": (B.FSDP_FLAT, W.gpt2_large_block().shapes, 8),
    "rows": (B.FSDP_ROWS, W.gpt2_large_emb_rows().shapes, 8),
    "many": (B.FSDP_FLAT, _many_shapes(), 3),
    "many_rows": (B.FSDP_ROWS, _many_shapes(), 5),
}


@pytest.mark.parametrize("name", list(UNITS))
def test_sqnorm_integer_grads_bit_exact_every_rank(name):
    """Integer-valued gradients: every square and every partial sum is an integer below
    2^53, so any summation order gives the exact result: GPU == oracle bit for bit, for
    every rank; padding and FSDP2 zero rows are poisoned and must not count."""
    layout, shapes, N = UNITS[name]
    u = B.fsdp_unit_create(layout, shapes, N)
    rng = np.random.Generator(np.random.PCG64(len(name) * 31 + N))
    for k in range(N):
        host = rng.integers(-1024, 1025, u.S).astype(np.float32)
        if layout == B.FSDP_FLAT:
            host[u.info(k)["valid"]:] = 1e30  # padding sits at the end of the shard
        else:
            q = 0
            for s in shapes:
                m, r = oracle.rows_of(s)
                c = -(-m // N)
                rows = min(m, (k + 1) * c) - min(m, k * c)
                host[q + rows * r:q + c * r] = 1e30
                q += c * r
        got = _sqnorm_gpu(u, k, to_dev(host))
        want = _oracle_sq(u, layout, k, host)
        assert np.array_equal(got, want), (name, k)


@pytest.mark.parametrize("name", ["gpt2l", "rows", "many"])
def test_sqnorm_real_grads_within_the_summation_bound_and_deterministic(name):
    """Real-valued gradients: both sides sum exact binary64 squares, each within (n-1)u of
    the exact sum, so they differ by at most 2(n-1)u times the sum; two calls agree bitwise."""
    layout, shapes, N = UNITS[name]
    u = B.fsdp_unit_create(layout, shapes, N)
    k = N // 2
    host = _grads(u.S, 40 + N, scale=1e-3)
    host[np.random.Generator(np.random.PCG64(3)).integers(0, u.S, 50)] *= 1e5
    d = to_dev(host)
    got = _sqnorm_gpu(u, k, d)
    again = _sqnorm_gpu(u, k, d)
    assert np.array_equal(got.view(np.uint64), again.view(np.uint64))
    want = _oracle_sq(u, layout, k, host)
    runs = _run_lengths(u, layout, k)
    for i, n in enumerate(runs):
        assert abs(got[i] - want[i]) <= 2 * max(n - 1, 0) * U * want[i] * 1.0001, (name, i)


def _run_lengths(u, layout, k):
    out, off = [], 0
    if layout == B.FSDP_FLAT:
        for s in u.shapes:
            n = oracle.numel(s)
            lo, hi = max(off, k * u.S), min(off + n, (k + 1) * u.S)
            out.append(max(0, hi - lo))
            off += n
        return out
    for s in u.shapes:
        m, r = oracle.rows_of(s)
        c = -(-m // u.N)
        out.append((min(m, (k + 1) * c) - min(m, k * c)) * r)
    return out


def test_sqnorm_gpt175b_rank_shard_full_size():
    """The GPT-175B block shard of rank 63 (S = 14,157,024, 5 parameters in it): integer
    gradients bit-exact; real gradients within the bound."""
    unit = W.gpt175b_block(N=128)
    u = B.fsdp_unit_create(B.FSDP_FLAT, unit.shapes, 128)
    for k in (0, 63, 127):
        gen = torch.Generator(device=dev()).manual_seed(100 + k)
        d = torch.randint(-1024, 1025, (u.S,), device=dev(), generator=gen).to(torch.float32)
        host = to_host(d)
        assert np.array_equal(_sqnorm_gpu(u, k, d), oracle.flat_sqnorm(u.shapes, 128, k, host)), k
    d = torch.randn(u.S, device=dev(), generator=torch.Generator(device=dev()).manual_seed(5)) * 1e-3
    host = to_host(d)
    got = _sqnorm_gpu(u, 63, d)
    want = oracle.flat_sqnorm(u.shapes, 128, 63, host)
    for i, n in enumerate(_run_lengths(u, B.FSDP_FLAT, 63)):
        assert abs(got[i] - want[i]) <= 2 * max(n - 1, 0) * U * want[i] * 1.0001, i
