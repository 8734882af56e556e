"""Pins of the oracle's gradient reduction: fp32 sum of N bf16 contributions with
pre/post divide, sequential over ranks.

What pins it: the F = 1 special case (plain data parallel: nothing to reduce),
exact sums of equal or integer-valued contributions, the hybrid-sharding sum
decomposition (FSDP paper §3.4, the sum over all ranks equals the sum over
sharding groups of the in-group sums), Higham's bound for recursive summation
against a float64 sum, and closed forms that tell a sequential order apart from
any other.
"""
import numpy as np
import pytest

import workloads as W

U = 2.0 ** -24  # unit roundoff of binary32


def _bf16_of(x):
    """bf16 bit patterns of values that are exact in bf16 (upper half of fp32)."""
    bits = np.asarray(x, np.float32).view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0)
    return (bits >> 16).astype(np.uint16)


def _f32(h):
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


def test_single_rank_is_identity(orc):
    """N = 1 (full replication in the FSDP paper's terms): the result is the one
    contribution, widened to fp32 exactly."""
    c = W.host_contribs(1, 10000, step=1)
    out = orc.grad_reduce([c[0]], 1.0, 1.0)
    assert np.array_equal(out.view(np.uint32), _f32(c[0]).view(np.uint32))


@pytest.mark.parametrize("N", [2, 4, 8, 16, 128])
def test_mean_of_equal_contributions_is_exact(orc, N):
    """N equal contributions x with pre*post = N (powers of two): the mean is x exactly."""
    pre = 2.0 ** (int(np.log2(N)) // 2)
    post = N / pre
    x = W.host_contribs(1, 5000, step=3)[0]
    out = orc.grad_reduce([x] * N, pre, post)
    assert np.array_equal(out.view(np.uint32), _f32(x).view(np.uint32))


def test_integer_contributions_sum_exactly_and_decompose(orc):
    """Integer-valued terms sum exactly in fp32; so the total of the W ranks' terms equals the sum
    over W/F sharding groups of the in-group sums (hybrid sharding decomposition)."""
    rng = np.random.Generator(np.random.PCG64(8))
    Wn, F, n = 32, 8, 4096
    ints = rng.integers(-128, 129, size=(Wn, n)).astype(np.float32)
    cs = [_bf16_of(row) for row in ints]
    total = orc.grad_reduce(cs, 1.0, 1.0)
    assert np.array_equal(total, ints.astype(np.int64).sum(axis=0).astype(np.float32))
    groups = [orc.grad_reduce(cs[g * F:(g + 1) * F], 1.0, 1.0) for g in range(Wn // F)]
    assert np.array_equal(np.sum(np.stack(groups).astype(np.float64), axis=0).astype(np.float32),
                          total)


@pytest.mark.parametrize("N,pre,post", [(4, 2, 2), (8, 2, 4), (128, 8, 16), (6, 2, 3),
                                        (5, 1, 1), (3, 3, 1), (7, 0.5, 3)])
def test_within_higham_bound_of_exact_sum(orc, N, pre, post):
    """|out - exact| <= gamma_{N+1} * sum|x_r| / |pre*post|  (N-1 additions, N pre
    divisions, one post division, each rounded once)."""
    c = W.host_contribs(N, 20000, step=2)
    out = orc.grad_reduce(list(c), pre, post).astype(np.float64)
    terms = _f32(c).astype(np.float64)
    exact = terms.sum(axis=0) / (pre * post)
    k = N + 1
    gamma = k * U / (1 - k * U)
    bound = gamma * np.abs(terms).sum(axis=0) / abs(pre * post)
    assert np.all(np.abs(out - exact) <= bound)


def test_sequential_order_closed_form(orc):
    """1.0 followed by N-1 copies of 2^-24: adding 2^-24 to 1.0 is an exact tie that
    rounds back to 1.0, so the sequential sum from rank 0 is exactly 1.0; any order that
    adds the small terms together first gives more."""
    for N in (2, 3, 4, 16, 128):
        cs = [_bf16_of(np.full(8, 1.0))] + [_bf16_of(np.full(8, 2.0 ** -24))] * (N - 1)
        out = orc.grad_reduce(cs, 1.0, 1.0)
        assert np.all(out == 1.0)
        # rank order matters: the small terms first, then 1.0, gives a larger result
        rev = orc.grad_reduce(cs[::-1], 1.0, 1.0)
        if N >= 3:
            assert np.all(rev > 1.0)


def test_negative_zero_survives(orc):
    """The sum starts from rank 0's term, not from +0, so all -0 terms give -0."""
    z = np.full(16, 0x8000, np.uint16)
    out = orc.grad_reduce([z] * 5, 1.0, 1.0)
    assert np.all(out.view(np.uint32) == 0x80000000)


def test_pre_divide_is_true_division(orc):
    """N = 1, pre = 3: each result is x/3 correctly rounded to binary32 (the float64
    quotient of a bf16 value by 3 is never close enough to a binary32 midpoint for the
    second rounding to matter)."""
    c = W.host_contribs(1, 50000, step=4)[0]
    out = orc.grad_reduce([c], 3.0, 1.0)
    want = (_f32(c).astype(np.float64) / 3.0).astype(np.float32)
    assert np.array_equal(out.view(np.uint32), want.view(np.uint32))


def test_pre_divides_each_term_before_the_sum(orc):
    """pre applies to every contribution before it is added (a pre-divide factor), post to
    the sum.  For N = 2 every step is evaluated exactly in float64 and rounded once to
    binary32: fl(x0/3) and fl(x1/3) (quotients never near a binary32 midpoint, see above),
    then their sum (exact in float64 for these magnitudes) rounded once, then / 5."""
    c = W.host_contribs(2, 50000, step=5)
    out = orc.grad_reduce(list(c), 3.0, 5.0)
    x0, x1 = (_f32(r).astype(np.float64) for r in c)
    t0 = (x0 / 3.0).astype(np.float32).astype(np.float64)
    t1 = (x1 / 3.0).astype(np.float32).astype(np.float64)
    s = (t0 + t1).astype(np.float32).astype(np.float64)
    want = (s / 5.0).astype(np.float32)
    assert np.array_equal(out.view(np.uint32), want.view(np.uint32))
    # dividing the sum instead of each term is a different function on these inputs
    alt = ((x0 + x1).astype(np.float32).astype(np.float64) / 15.0).astype(np.float32)
    assert not np.array_equal(out, alt)
