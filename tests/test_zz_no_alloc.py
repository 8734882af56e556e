"""fsdp_grad_sqnorm_noalloc, the per-parameter sums of squares for callers that cannot
allocate device memory: its partial sums live in the library's own per-GPU scratch.  Through
the C ABI, two calls in a row -- the second on a smaller shard, so it reuses the start of the
scratch the first left behind -- each compared with fsdp_grad_sqnorm (the same kernels with a
caller's workspace: bit for bit) and with the oracle (bit for bit on integer gradients, whose
every partial sum is exact; within the summation bound on real ones).  Also a third call on a
unit of many parameters, and a shard that needs more partial sums than the scratch holds
(refused before any launch)."""
import ctypes
import gc

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import dev, to_dev, to_host
from sharded_fsdp_flatten_amd import binding as B

pytestmark = pytest.mark.gpu

U = 2.0 ** -53


@pytest.fixture(autouse=True)
def _free():
    B.load()
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _noalloc(u, k, grad):
    """The new entry point, called through the C ABI with ctypes (no Python wrapper)."""
    out = torch.full((len(u.shapes),), float("nan"), dtype=torch.float64, device=dev())
    lib = B.load()
    st = lib.fsdp_grad_sqnorm_noalloc(u.handle, k, ctypes.c_void_p(grad.data_ptr()),
                                      ctypes.c_void_p(out.data_ptr()),
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, B.fsdp_last_error()
    torch.cuda.synchronize()
    return to_host(out)


def _with_workspace(u, k, grad):
    ws = torch.empty(max(1, B.fsdp_grad_sqnorm_workspace(u, k)), dtype=torch.float64, device=dev())
    out = torch.full((len(u.shapes),), float("nan"), dtype=torch.float64, device=dev())
    B.fsdp_grad_sqnorm(u, k, grad, out, ws)
    torch.cuda.synchronize()
    return to_host(out)


def _runs(u, k):
    out, off = [], 0
    for s in u.shapes:
        n = oracle.numel(s)
        lo, hi = max(off, k * u.S), min(off + n, (k + 1) * u.S)
        out.append(max(0, hi - lo))
        off += n
    return out


@pytest.mark.parametrize("integer", [True, False])
def test_noalloc_sqnorm_two_calls_second_smaller(integer):
    cases = [(W.t5_11b_block(), 3), (W.gpt2_large_block(), 5)]  # 25.2 M then 2.5 M elements
    for unit, k in cases:
        u = B.fsdp_unit_create(B.FSDP_FLAT, unit.shapes, unit.N)
        gen = torch.Generator(device=dev()).manual_seed(200 + k)
        if integer:
            g = torch.randint(-1024, 1025, (u.S,), device=dev(), generator=gen).to(torch.float32)
        else:
            g = torch.randn(u.S, device=dev(), generator=gen).mul_(1e-3)
        got = _noalloc(u, k, g)
        ref = _with_workspace(u, k, g)
        assert np.array_equal(got.view(np.uint64), ref.view(np.uint64)), (unit.name, k)
        want = oracle.flat_sqnorm(u.shapes, u.N, k, to_host(g))
        if integer:
            assert np.array_equal(got, want), (unit.name, k)
        else:
            for i, n in enumerate(_runs(u, k)):
                assert abs(got[i] - want[i]) <= 2 * max(n - 1, 0) * U * want[i] * 1.0001, (unit.name, i)


def test_noalloc_sqnorm_many_parameters_and_rows():
    """61 parameters over 3 ranks (more runs than one launch's table: two launch pairs) and an
    FSDP2 unit, integer gradients: bit for bit against the oracle and the workspace version."""
    rng = np.random.Generator(np.random.PCG64(61))
    shapes = [(int(rng.integers(1, 9000)),) if i % 2 else (int(rng.integers(1, 40)), 300)
              for i in range(61)]
    for layout, shp, N, k in [(B.FSDP_FLAT, shapes, 3, 1), (B.FSDP_ROWS, W.gpt2_large_emb_rows().shapes, 8, 7)]:
        u = B.fsdp_unit_create(layout, shp, N)
        host = rng.integers(-1024, 1025, u.S).astype(np.float32)
        d = to_dev(host)
        got = _noalloc(u, k, d)
        assert np.array_equal(got.view(np.uint64), _with_workspace(u, k, d).view(np.uint64))
        if layout == B.FSDP_FLAT:
            host[u.info(k)["valid"]:] = 0.0  # padding is never counted
            want = oracle.flat_sqnorm(u.shapes, N, k, host)
        else:
            want = oracle.rows_sqnorm(u.shapes, N, k, host)
        assert np.array_equal(got, want)


def test_noalloc_sqnorm_refuses_more_than_its_scratch():
    """2^30 + 4096 elements need 262,145 partial sums, one more than the scratch holds: the
    call is refused before any launch, and the workspace version still takes it."""
    n = (1 << 30) + 4096
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(n,)], 1)
    assert B.fsdp_grad_sqnorm_workspace(u, 0) == (1 << 18) + 1
    lib = B.load()
    fake = ctypes.c_void_p(0x7F0000000000)  # never dereferenced: the call fails validation
    assert lib.fsdp_grad_sqnorm_noalloc(u.handle, 0, fake, fake, None) == 2
    assert "262144" in B.fsdp_last_error()
