"""Pins of the oracle's fp32 -> bf16 cast (round to nearest, ties to even).

Checked against: a hand-worked table of boundary cases (tests/golden), torch's
CPU cast as a library routine, and a brute-force nearest-value search that uses
neither.
"""
import numpy as np
import torch

import workloads as W
from conftest import golden_path


def _torch_bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _is_nan_bf16(h):
    h = np.asarray(h, np.uint16)
    return ((h & 0x7F80) == 0x7F80) & ((h & 0x007F) != 0)


def test_golden_boundary_cases(orc):
    n = 0
    with open(golden_path("bf16_rne_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            src, exp = line.split()[:2]
            x = np.asarray([int(src, 16)], np.uint32).view(np.float32)
            got = orc.bf16(x)[0]
            if exp == "NaN":
                assert _is_nan_bf16(got), src
            else:
                assert got == int(exp, 16), (src, hex(got), exp)
            n += 1
    assert n >= 25


def test_random_bit_patterns_match_torch(orc):
    x = W.random_bits_f32(1 << 20, seed=11)
    got = orc.bf16(x)
    ref = _torch_bf16_bits(x)
    nan_in = np.isnan(x)
    assert np.array_equal(got[~nan_in], ref[~nan_in])
    assert np.all(_is_nan_bf16(got[nan_in]))


def test_nearest_by_brute_force(orc):
    """The result is a nearest bf16 neighbour, and on a tie the one with an even last bit.
    Computed from the two bf16 values that bracket x, in float64, with no rounding rule."""
    rng = np.random.Generator(np.random.PCG64(3))
    bits = rng.integers(0, 0x7F7FFFFF, size=200000, dtype=np.uint64).astype(np.uint32)
    bits[:1000] = (bits[:1000] & 0xFFFF0000) | 0x8000          # force many exact ties
    sign = rng.integers(0, 2, size=bits.size, dtype=np.uint32) << 31
    x = (bits | sign).view(np.float32)
    got = orc.bf16(x)
    lo = (x.view(np.uint32) >> 16).astype(np.uint32)           # truncation toward zero
    hi = lo + 1

    def as_f64(h):
        # IEEE-754 rounds as if the exponent range were unbounded: the step past the
        # largest finite bf16 is worth 2^128 (and the result of choosing it is infinity).
        v = (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        top = (h & 0x7FFF) == 0x7F80
        return np.where(top, np.where(h & 0x8000, -2.0 ** 128, 2.0 ** 128), v)
    xd = x.astype(np.float64)
    dlo = np.abs(xd - as_f64(lo))
    dhi = np.abs(xd - as_f64(hi))
    want = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    assert np.array_equal(got, want.astype(np.uint16))


def test_exact_values_round_trip(orc):
    """Every non-NaN bf16 value converted to fp32 casts back to itself."""
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ok = ~_is_nan_bf16(h)
    x = (h.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(orc.bf16(x)[ok], h[ok])


def test_monotone(orc):
    x = np.sort(np.random.default_rng(1).standard_normal(100000).astype(np.float32) * 1e3)
    f = (orc.bf16(x).astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.diff(f) >= 0)
