"""Pins of the oracle's sharded optimizer statistics: the per-rank half of the sharded
gradient scaler (unscale + overflow flag) and per-parameter sums of squares of a gradient
shard (FSDP paper summary §3.4 "Native Mixed Precision and the Sharded Gradient Scaler";
§6 "Limitations", statistics of original parameters under flat shards)."""
import math

import numpy as np
import pytest

import oracle
import workloads as W

U = 2.0 ** -53  # unit roundoff of binary64


def _rand_f32(rng, n, lo=-30, hi=30):
    """Finite float32 values with exponents spread over [lo, hi] (both signs, some zeros)."""
    m = rng.uniform(1.0, 2.0, n)
    e = rng.integers(lo, hi, n)
    x = (np.ldexp(m, e) * rng.choice([-1.0, 1.0], n)).astype(np.float32)
    x[rng.integers(0, n, max(1, n // 50))] = 0.0
    return x


# ---------------------------------------------------------------------------
# unscale
# ---------------------------------------------------------------------------

def test_unscale_is_one_rounded_binary32_multiply():
    """The product of two binary32 values is exact in binary64; rounding it once to
    binary32 is the correctly rounded binary32 product."""
    rng = np.random.Generator(np.random.PCG64(1))
    g = np.concatenate([_rand_f32(rng, 20000), _rand_f32(rng, 2000, -149, -120),
                        _rand_f32(rng, 2000, 100, 127)])
    for inv in (2.0 ** -16, 1.0 / 65536.0, 1.0 / 3.0, 7.5e-5, 3.0, 1e-30):
        inv32 = float(np.float32(inv))
        with np.errstate(over="ignore"):  # products beyond binary32 round to +-inf
            want = (g.astype(np.float64) * inv32).astype(np.float32)
        got = g.copy()
        flag = np.zeros(1, np.float32)
        oracle.grad_unscale(got, inv32, flag)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), inv
        assert flag[0] == 0.0


def test_unscale_by_one_is_the_identity():
    rng = np.random.Generator(np.random.PCG64(2))
    g = np.concatenate([_rand_f32(rng, 5000, -149, 127), np.float32([-0.0, 0.0])])
    got = g.copy()
    oracle.grad_unscale(got, 1.0, np.zeros(1, np.float32))
    assert np.array_equal(got.view(np.uint32), g.view(np.uint32))


def test_unscale_flags_exactly_the_non_finite_inputs_and_never_clears():
    rng = np.random.Generator(np.random.PCG64(3))
    for special in (np.inf, -np.inf, np.nan):
        g = _rand_f32(rng, 1000)
        g[rng.integers(0, 1000)] = special
        flag = np.zeros(1, np.float32)
        out = g.copy()
        oracle.grad_unscale(out, 0.25, flag)
        assert flag[0] == 1.0
        assert np.array_equal(np.isfinite(out), np.isfinite(g))
        # a later clean shard leaves the shared flag set
        oracle.grad_unscale(_rand_f32(rng, 100), 0.25, flag)
        assert flag[0] == 1.0
    # finite inputs whose product overflows are not flagged: the check is on the input
    flag = np.zeros(1, np.float32)
    big = np.float32([3e38, -3e38])
    oracle.grad_unscale(big, 4.0, flag)
    assert flag[0] == 0.0 and np.all(np.isinf(big))


# ---------------------------------------------------------------------------
# per-parameter sums of squares
# ---------------------------------------------------------------------------

def _int_params(rng, shapes, lim=1024):
    return [rng.integers(-lim, lim + 1, size=s if len(s) else ()).astype(np.float32)
            for s in shapes]


def _exact_sq(x):
    return sum(int(v) * int(v) for v in np.asarray(x, np.float32).reshape(-1))


@pytest.mark.parametrize("N", [1, 3, 4, 7, 16])
def test_flat_sqnorm_integer_grads_sum_to_each_parameters_norm(N):
    """Integer gradients: every square and partial sum is exact in binary64, so the
    per-rank values must equal integer sums over the rank's part of each parameter, and
    their sum over ranks each parameter's squared norm, whatever the shard boundaries."""
    rng = np.random.Generator(np.random.PCG64(10 + N))
    shapes = [(5, 3), (7,), (), (0, 4), (2, 2, 3), (1,)]
    params = _int_params(rng, shapes)
    T, S, L, pad = oracle.flat_sizes([oracle.numel(s) for s in shapes], N)
    flat = np.concatenate([p.reshape(-1) for p in params] + [np.zeros(pad, np.float32)])
    total = np.zeros(len(shapes))
    offs = np.cumsum([0] + [oracle.numel(s) for s in shapes])
    for k in range(N):
        shard = flat[k * S:(k + 1) * S].copy()
        if k == N - 1 and pad:
            shard[S - pad:] = 1e30  # padding is nobody's: garbage there changes nothing
        got = oracle.flat_sqnorm(shapes, N, k, shard)
        for i in range(len(shapes)):
            lo, hi = max(offs[i], k * S), min(offs[i + 1], (k + 1) * S)
            want = _exact_sq(flat[lo:hi]) if hi > lo else 0
            assert got[i] == want, (k, i)
        total += got
    assert [int(t) for t in total] == [_exact_sq(p) for p in params]


@pytest.mark.parametrize("N", [1, 2, 4, 8, 9])
def test_rows_sqnorm_integer_grads_and_layout_independence(N):
    """FSDP2 segments: only the rows a rank holds count (zero rows and garbage in them
    change nothing), and over all ranks each parameter's total equals the FLAT layout's."""
    rng = np.random.Generator(np.random.PCG64(20 + N))
    shapes = [(5, 3), (7,), (), (3, 2, 2), (2,)]
    params = _int_params(rng, shapes)
    P_r = oracle.rows_sizes(shapes, N)
    gathered = oracle.rows_shard(params, N, -1)
    total = np.zeros(len(shapes))
    q = 0
    starts = []
    for s in shapes:
        m, r = oracle.rows_of(s)
        starts.append((q, m, r))
        q += -(-m // N) * r
    for k in range(N):
        seg = gathered[k * P_r:(k + 1) * P_r].copy()
        for (q0, m, r) in starts:  # poison the pad rows
            c = -(-m // N)
            rows = min(m, (k + 1) * c) - min(m, k * c)
            seg[q0 + rows * r:q0 + c * r] = 1e30
        got = oracle.rows_sqnorm(shapes, N, k, seg)
        total += got
    assert [int(t) for t in total] == [_exact_sq(p) for p in params]
    flat_total = np.zeros(len(shapes))
    T, S, L, pad = oracle.flat_sizes([oracle.numel(s) for s in shapes], N)
    flat = oracle.flat_shard(params, N, -1)
    for k in range(N):
        flat_total += oracle.flat_sqnorm(shapes, N, k, flat[k * S:(k + 1) * S])
    assert np.array_equal(total, flat_total)


def test_flat_sqnorm_within_the_recursive_summation_bound():
    """Real-valued gradients: each square is exact in binary64, so the sequential sum of
    n non-negative terms is within (n-1)u of the correctly rounded math.fsum."""
    rng = np.random.Generator(np.random.PCG64(30))
    unit = W.gpt2_large_block(N=8)
    shapes = unit.shapes
    T, S, L, pad = oracle.flat_sizes([oracle.numel(s) for s in shapes], 8)
    k = 3
    shard = (rng.standard_normal(S) * 1e-3).astype(np.float32)
    shard[rng.integers(0, S, 100)] *= 1e6  # a few large entries
    got = oracle.flat_sqnorm(shapes, 8, k, shard)
    offs = np.cumsum([0] + [oracle.numel(s) for s in shapes])
    for i in range(len(shapes)):
        lo, hi = max(offs[i], k * S) - k * S, min(offs[i + 1], (k + 1) * S) - k * S
        if hi <= lo:
            assert got[i] == 0.0
            continue
        x = shard[lo:hi].astype(np.float64)
        exact = math.fsum((x * x).tolist())
        n = hi - lo
        assert abs(got[i] - exact) <= (n - 1) * U * exact * 1.0001, i


def test_sqnorm_of_the_fig3_unit():
    """Linear(4->3) over 16 ranks (15 elements, pad 1): the weight's 12 elements sit on
    ranks 0-11, the bias on ranks 12-14, and rank 15 holds only padding."""
    shapes = [(3, 4), (3,)]
    vals = np.arange(1, 16, dtype=np.float32)
    flat = np.concatenate([vals, np.float32([5.0])])  # the pad element is not counted
    for k in range(16):
        got = oracle.flat_sqnorm(shapes, 16, k, flat[k:k + 1])
        want = [float(vals[k] ** 2) if k < 12 else 0.0,
                float(vals[k] ** 2) if 12 <= k < 15 else 0.0]
        assert list(got) == want, k
