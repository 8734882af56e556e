"""Helpers shared by the GPU parity tests (host <-> device marshalling, comparisons)."""
import numpy as np
import torch

U32 = np.uint32


def dev():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU parity tests need a ROCm GPU (torch.cuda.is_available() is False)")
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, d=None):
    d = d or dev()
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(d).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(d)


def to_host(t) -> np.ndarray:
    if t.dtype in (torch.bfloat16, torch.int16):
        return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def bf16_nan(h):
    h = np.asarray(h, np.uint16)
    return ((h & 0x7F80) == 0x7F80) & ((h & 0x007F) != 0)


def assert_f32_bits(got, want, what=""):
    got = np.asarray(got, np.float32).reshape(-1)
    want = np.asarray(want, np.float32).reshape(-1)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    g, w = got.view(U32), want.view(U32)
    bad = np.nonzero(g != w)[0]
    if bad.size:
        i = bad[0]
        raise AssertionError("%s: %d of %d fp32 elements differ; first at %d: got %08x want %08x"
                             % (what, bad.size, g.size, i, g[i], w[i]))


def assert_bf16_bits(got, want, what=""):
    """Bit-exact bf16, except that any NaN matches any NaN (payload not fixed)."""
    got = np.asarray(got, np.uint16).reshape(-1)
    want = np.asarray(want, np.uint16).reshape(-1)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    nan_w = bf16_nan(want)
    assert np.array_equal(bf16_nan(got), nan_w), "%s: NaN positions differ" % what
    bad = np.nonzero((got != want) & ~nan_w)[0]
    if bad.size:
        i = bad[0]
        raise AssertionError("%s: %d of %d bf16 elements differ; first at %d: got %04x want %04x"
                             % (what, bad.size, got.size, i, got[i], want[i]))


def assert_f32_tol_then_bits(got, want, what=""):
    """The stated tolerance (2 fp32 ulp or 1e-6 relative, NaN where the oracle has NaN),
    then bit-exactness, which the pinned operation order makes possible."""
    g = np.asarray(got, np.float32).reshape(-1)
    w = np.asarray(want, np.float32).reshape(-1)
    assert g.shape == w.shape
    nan_w = np.isnan(w)
    assert np.array_equal(np.isnan(g), nan_w), "%s: NaN positions differ" % what
    fin = ~nan_w
    gd, wd = g[fin].astype(np.float64), w[fin].astype(np.float64)
    inf = np.isinf(wd)
    assert np.array_equal(gd[inf], wd[inf]), "%s: infinities differ" % what
    gd, wd = gd[~inf], wd[~inf]
    err = np.abs(gd - wd)
    ulp = np.spacing(np.abs(w[fin][~inf])).astype(np.float64)
    ok = (err <= 2 * ulp) | (err <= 1e-6 * np.abs(wd))
    assert np.all(ok), "%s: %d elements beyond 2 ulp / 1e-6 relative (max err %g)" % (
        what, int(np.count_nonzero(~ok)), float(err.max()))
    gb, wb = g.view(U32)[fin], w.view(U32)[fin]
    n_bad = int(np.count_nonzero(gb != wb))
    assert n_bad == 0, "%s: within tolerance but %d elements not bit-exact" % (what, n_bad)


def offset_view(t_like_numel: int, dtype, offset: int, d=None):
    """A contiguous tensor of `t_like_numel` elements starting `offset` elements into a
    larger allocation (to exercise unaligned pointers)."""
    d = d or dev()
    base = torch.zeros(t_like_numel + offset + 8, dtype=dtype, device=d)
    return base[offset:offset + t_like_numel], base
