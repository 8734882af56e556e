"""AdamW on non-finite values, and the sharded gradient scaler's skip of the step.

The pages' mixed-precision training scales the loss, and a step whose gradients overflow
is skipped on every rank (FSDP paper summary section 3.4, "Native Mixed Precision and the
Sharded Gradient Scaler").  AdamW itself must treat +-inf and NaN in g, m, v and p exactly
as the oracle's binary32 operations do (any NaN matches any NaN; every other element bit for
bit, the bf16 copy included), on the vector path and on the one-element path.  Then the
chain: unscale the reduced gradient shard, read the flag, and take or skip the step."""
import gc

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import assert_bf16_bits, assert_f32_tol_then_bits, dev, offset_view, to_dev, to_host
from sharded_fsdp_flatten_amd import binding as B

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01)
SPECIALS = np.array([np.inf, -np.inf, np.nan, 0.0, -0.0, 1e-45, -3e38, 3.4e38], np.float32)


@pytest.fixture(autouse=True)
def _free():
    B.load()
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _plant(a, rng, count):
    idx = rng.choice(a.size, count, replace=False)
    a[idx] = SPECIALS[rng.integers(0, SPECIALS.size, count)]
    return a


@pytest.mark.parametrize("S,misalign", [(4099, 0), (4099, 1), (2048 * 3, 0)])
def test_adamw_nonfinite_inputs(S, misalign):
    rng = np.random.Generator(np.random.PCG64(S + misalign))
    p = _plant((rng.standard_normal(S) * 0.02).astype(np.float32), rng, 60)
    g = _plant(W.host_normal(S, 1e-3, seed=5), rng, 60)
    m = _plant((rng.standard_normal(S) * 1e-4).astype(np.float32), rng, 60)
    v = np.abs(_plant((rng.standard_normal(S) * 1e-7).astype(np.float32), rng, 60))
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(S,)], 1)
    keep = []

    def buf(a, dtype=torch.float32):
        t, base = offset_view(S, dtype, misalign)
        if a is not None:
            t.copy_(to_dev(a))
        keep.append(base)
        return t

    dp, dg, dm, dv = buf(p), buf(g), buf(m), buf(v)
    dpb = buf(None, torch.bfloat16)
    hp_, hm, hv = p.copy(), m.copy(), v.copy()
    for t in (1, 2):
        B.fsdp_adam_shard(u, dp, dg, dm, dv, step=t, param_bf16=dpb, **HP)
        hpb = oracle.adamw(hp_, g, hm, hv, step=t, want_bf16=True, **HP)
        torch.cuda.synchronize()
        what = "S=%d mis=%d t=%d" % (S, misalign, t)
        assert np.isnan(hp_).any() and np.isinf(hm).any()  # the specials reached the state
        assert_f32_tol_then_bits(to_host(dp), hp_, "param " + what)
        assert_f32_tol_then_bits(to_host(dm), hm, "exp_avg " + what)
        assert_f32_tol_then_bits(to_host(dv), hv, "exp_avg_sq " + what)
        assert_bf16_bits(to_host(dpb), hpb, "param_bf16 " + what)


@pytest.mark.parametrize("overflow", [False, True])
def test_unscale_flag_skips_the_step(overflow):
    """Rank 5 of 8 on a GPT-2-L-sized shard: reduce, unscale by 1/1024 into a zeroed flag, and
    take the AdamW step only when the flag stayed 0.  With an overflow planted in one
    contribution (bf16 +inf) the flag is 1 and parameters and moments stay bit for bit."""
    N, S = 8, 100003
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(N * S,)], N)
    c = W.host_contribs(N, S, std=1.0, step=3)
    if overflow:
        c[6, 4321] = 0x7F80
    d_c = [to_dev(c[r]) for r in range(N)]
    grad = torch.empty(S, device=dev())
    B.fsdp_grad_reduce_shard(u, d_c, 2.0, 4.0, grad)
    flag = torch.zeros(1, device=dev())
    B.fsdp_grad_unscale(u, 5, grad, 1.0 / 1024, flag)
    p0 = (np.random.Generator(np.random.PCG64(9)).standard_normal(S) * 0.02).astype(np.float32)
    m0 = W.host_normal(S, 1e-5, seed=10)
    v0 = np.abs(W.host_normal(S, 1e-9, seed=11))
    dp, dm, dv = to_dev(p0), to_dev(m0), to_dev(v0)
    found = float(flag.item())  # synchronizes
    if found == 0.0:
        B.fsdp_adam_shard(u, dp, grad, dm, dv, step=4, **HP)
    torch.cuda.synchronize()

    h_grad = oracle.grad_reduce(list(c), 2.0, 4.0)
    h_flag = np.zeros(1, np.float32)
    oracle.grad_unscale(h_grad, 1.0 / 1024, h_flag)
    assert found == float(h_flag[0]) == (1.0 if overflow else 0.0)
    hp_, hm, hv = p0.copy(), m0.copy(), v0.copy()
    if not overflow:
        oracle.adamw(hp_, h_grad, hm, hv, step=4, **HP)
    assert_f32_tol_then_bits(to_host(grad), h_grad, "unscaled grad")
    assert_f32_tol_then_bits(to_host(dp), hp_, "param")
    assert_f32_tol_then_bits(to_host(dm), hm, "exp_avg")
    assert_f32_tol_then_bits(to_host(dv), hv, "exp_avg_sq")
