"""GPU parity of the next rows at the GPT-175B block size (N = 128, rank 63), in the
configuration bench.py times them: the hybrid (groups of 8) accumulating reduction from a
receive buffer at the recommended pitch, the bf16 copy-in of all ranks and the bf16
copy-out of the whole unit, the cast of the rank shard, the local fp32 accumulation of the
whole unsharded gradient, and the unscale of the rank shard.  Every output is compared
with the CPU oracle element by element (reductions: tolerance, then bits; the rest: bits)."""
import gc

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import (assert_bf16_bits, assert_f32_bits, assert_f32_tol_then_bits, dev,
                      offset_view, to_host)
from sharded_fsdp_flatten_amd import binding as B

pytestmark = pytest.mark.gpu

K = 63


@pytest.fixture(scope="module")
def unit175():
    B.load()
    unit = W.gpt175b_block(N=128)
    u = B.fsdp_unit_create(B.FSDP_FLAT, unit.shapes, unit.N)
    assert (u.S, u.L, u.info(K)["T"]) == (14_157_024, 1_812_099_072, 1_812_099_072)
    yield unit, u
    gc.collect()
    torch.cuda.empty_cache()


def _sync():
    torch.cuda.synchronize()


def _bf16_params(unit, seed):
    gen = torch.Generator(device=dev()).manual_seed(seed)
    return [torch.randn(s, device=dev(), generator=gen).mul_(unit.std).to(torch.bfloat16)
            for s in unit.shapes]


def test_gpt175b_hybrid_accumulating_reduce_full(unit175):
    unit, u = unit175
    c = W.device_contribs(unit.N, u.S, step=1, pitch=u.recv_pitch)
    gen = torch.Generator(device=dev()).manual_seed(11)
    grad = torch.randn(u.S, device=dev(), generator=gen).mul_(1e-3)
    old = to_host(grad).copy()
    B.fsdp_grad_reduce_shard_ex(u, [c[r] for r in range(unit.N)], 8.0, 16.0, grad, group=8,
                                accumulate=True)
    _sync()
    c_host = to_host(c)
    del c
    oracle.grad_reduce_ex(list(c_host), 8.0, 16.0, group=8, out=old)
    del c_host
    assert_f32_tol_then_bits(to_host(grad), old, "175b hybrid accumulating reduce")


def test_gpt175b_bf16_copyin_all_ranks_and_copyout(unit175):
    unit, u = unit175
    params = _bf16_params(unit, 12)
    rs_input = torch.empty(u.L, dtype=torch.bfloat16, device=dev())
    B.fsdp_flatten_shard_bf16(u, params, B.FSDP_ALL_RANKS, rs_input)
    _sync()
    host = [to_host(p) for p in params]
    want = oracle.flat_shard_u16(host, unit.N, -1)
    assert_bf16_bits(to_host(rs_input), want, "175b bf16 copy-in, all ranks")
    del want
    outs = [torch.empty(s, dtype=torch.bfloat16, device=dev()) for s in unit.shapes]
    B.fsdp_unflatten_copyout_bf16(u, rs_input, outs)
    _sync()
    want = oracle.flat_copyout_u16(unit.shapes, to_host(rs_input))
    for i, (o, w, h) in enumerate(zip(outs, want, host)):
        got = to_host(o)
        assert_bf16_bits(got, w, "175b bf16 copy-out %d" % i)
        assert_bf16_bits(got, h, "175b bf16 round trip %d" % i)
    del params, rs_input, outs, host, want


def test_gpt175b_cast_rank_shard(unit175):
    unit, u = unit175
    gen = torch.Generator(device=dev()).manual_seed(13)
    src = torch.randn(u.S, device=dev(), generator=gen).mul_(unit.std)
    dst = torch.empty(u.S, dtype=torch.bfloat16, device=dev())
    B.fsdp_cast_to_bf16(u, K, src, dst)
    _sync()
    assert_bf16_bits(to_host(dst), oracle.bf16(to_host(src)), "175b cast, rank 63")


def test_gpt175b_local_accumulation_all(unit175):
    unit, u = unit175
    grad = torch.cat([p.reshape(-1) for p in _bf16_params(unit, 14)])
    assert grad.numel() == u.L
    gen = torch.Generator(device=dev()).manual_seed(15)
    acc = torch.randn(u.L, device=dev(), generator=gen).mul_(1e-3)
    want = to_host(acc).copy()
    B.fsdp_grad_accumulate(u, B.FSDP_ALL_RANKS, grad, acc, False)
    _sync()
    oracle.grad_accumulate(to_host(grad), want, init=False)
    assert_f32_bits(to_host(acc), want, "175b local accumulation, all L")
    del grad, acc, want


@pytest.mark.parametrize("init,mis_acc,mis_grad", [(True, 0, 0), (False, 0, 2), (False, 1, 1),
                                                   (True, 3, 2)])
def test_long_local_accumulation_variants(init, mis_acc, mis_grad):
    """The accumulation over more than 2^18 blocks (XCD-ordered): from a zero start (init),
    and with accumulator and gradient at element offsets (the one-element path: an
    accumulator not 16-byte aligned; the vector path needs a 16-byte-aligned accumulator and a
    4-byte-aligned gradient), 600 M elements, element by element against the oracle."""
    n = 600_000_000 + 77
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(n,)], 1)
    gen = torch.Generator(device=dev()).manual_seed(17)
    gv, gb = offset_view(n, torch.bfloat16, mis_grad)
    gv.copy_(torch.randn(n, device=dev(), generator=gen).mul_(1e-3).to(torch.bfloat16))
    acc, ab = offset_view(n, torch.float32, mis_acc)
    acc.copy_(torch.randn(n, device=dev(), generator=gen).mul_(1e-3))
    want = to_host(acc).copy()
    B.fsdp_grad_accumulate(u, 0, gv, acc, init)
    _sync()
    oracle.grad_accumulate(to_host(gv), want, init=init)
    assert_f32_bits(to_host(acc), want, "accumulation init=%s offsets %d/%d" % (init, mis_acc, mis_grad))
    del gv, gb, acc, ab, want


def test_gpt175b_unscale_rank_shard(unit175):
    unit, u = unit175
    gen = torch.Generator(device=dev()).manual_seed(16)
    g = torch.randn(u.S, device=dev(), generator=gen).mul_(65536.0 * 1e-3)
    g[u.S // 3] = float("inf")
    host = to_host(g).copy()
    flag = torch.zeros(1, device=dev())
    B.fsdp_grad_unscale(u, K, g, 2.0 ** -16, flag)
    _sync()
    hflag = np.zeros(1, np.float32)
    oracle.grad_unscale(host, 2.0 ** -16, hflag)
    assert_f32_bits(to_host(g), host, "175b unscale, rank 63")
    assert to_host(flag)[0] == hflag[0] == 1.0
