"""Pins of the oracle's AdamW step on a shard.

What pins it: closed forms of the first step (the update is lr*g/(|g|+eps),
which tends to lr*sign(g)), the constant-gradient invariant (bias-corrected
moments equal g and g^2), torch.optim.AdamW as a library routine at a stated
tolerance, the pages' claim that the step is local to each aligned shard
("FSDP Architecture": parameter, gradient and both moments are held for the
same positions), and padding that must stay zero.
"""
import numpy as np
import pytest
import torch

import workloads as W


def _ulp(x):
    return np.spacing(np.abs(np.asarray(x, np.float32))).astype(np.float64)


def _state(n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    return p, g, np.zeros(n, np.float32), np.zeros(n, np.float32)


def test_first_step_tends_to_lr_sign_g(orc):
    """wd = 0, eps -> 0: p1 = p0 - lr*sign(g)."""
    lr = 1e-3
    p, g, m, v = _state(100000, 1)
    p0 = p.copy()
    orc.adamw(p, g, m, v, lr=lr, betas=(0.9, 0.999), eps=1e-30, weight_decay=0.0, step=1)
    want = p0.astype(np.float64) - lr * np.sign(g)
    err = np.abs(p - want)
    # the update lr*sign(g) passes five rounded operations (1-b1, m, den, m/den,
    # step_size*...), each within u relative; the final subtraction adds half an ulp
    assert np.all(err <= 0.5 * _ulp(want) + 3 * _ulp(lr))


def test_first_step_closed_form_with_decay_and_eps(orc):
    """Any wd and eps: m1 = (1-b1) g and v1 = (1-b2) g^2, so after bias correction
    p1 = p0*(1 - lr*wd) - lr * g / (|g| + eps).  Gradients near eps pin where eps sits
    (outside the square root)."""
    lr, wd, eps = 1e-3, 0.01, 1e-8
    rng = np.random.Generator(np.random.PCG64(2))
    n = 50000
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-8).astype(np.float32)     # |g| ~ eps
    m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
    p0 = p.copy()
    orc.adamw(p, g, m, v, lr=lr, betas=(0.9, 0.999), eps=eps, weight_decay=wd, step=1)
    gd = g.astype(np.float64)
    want = p0.astype(np.float64) * (1 - lr * wd) - lr * gd / (np.abs(gd) + eps)
    assert np.all(np.abs(p - want) <= 1.5 * _ulp(want) + 4 * _ulp(lr))
    assert np.all(np.abs(m - 0.1 * gd) <= 2 * _ulp(m) + 1e-45)
    assert np.all(np.abs(v - 0.001 * gd * gd) <= 2 * _ulp(v) + 1e-45)


def test_constant_gradient_moves_p_linearly(orc):
    """With the same g every step, m_hat_t = g and v_hat_t = g^2 exactly in real
    arithmetic, so each step moves p by lr*g/(|g|+eps) (wd = 0)."""
    lr, eps, t_max = 1e-3, 1e-8, 20
    p, g, m, v = _state(20000, 3)
    p0 = p.astype(np.float64).copy()
    for t in range(1, t_max + 1):
        orc.adamw(p, g, m, v, lr=lr, betas=(0.9, 0.999), eps=eps, weight_decay=0.0, step=t)
    gd = g.astype(np.float64)
    want = p0 - t_max * lr * gd / (np.abs(gd) + eps)
    assert np.max(np.abs(p - want)) <= 1e-6 * t_max * lr + t_max * 2 * np.max(_ulp(p))


def test_matches_torch_adamw_within_tolerance(orc):
    """torch.optim.AdamW (a library routine with its own operation order) on the tiny
    unit for 10 steps: |dp| <= 1e-4*lr*t, |dm| <= 1e-5*max|g|, |dv| <= 1e-5*max g^2."""
    unit = W.tiny_mlp()
    hp = unit.adam
    params = W.host_params(unit, seed=0)
    flat = np.concatenate([p.reshape(-1) for p in params])
    n = flat.size
    p = flat.copy()
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    tp = torch.nn.Parameter(torch.from_numpy(flat.copy()))
    opt = torch.optim.AdamW([tp], lr=hp["lr"], betas=hp["betas"], eps=hp["eps"],
                            weight_decay=hp["weight_decay"], foreach=False)
    gmax = 0.0
    for t in range(1, 11):
        g = W.host_normal(n, 1e-3, seed=1000 * t)
        gmax = max(gmax, float(np.abs(g).max()))
        orc.adamw(p, g, m, v, lr=hp["lr"], betas=hp["betas"], eps=hp["eps"],
                  weight_decay=hp["weight_decay"], step=t)
        tp.grad = torch.from_numpy(g.copy())
        opt.step()
        st = opt.state[tp]
        assert np.max(np.abs(p - tp.detach().numpy())) <= 1e-4 * hp["lr"] * t
        assert np.max(np.abs(m - st["exp_avg"].numpy())) <= 1e-5 * gmax
        assert np.max(np.abs(v - st["exp_avg_sq"].numpy())) <= 1e-5 * gmax ** 2


def test_shard_then_adam_equals_adam_then_shard(orc):
    """The step on each rank's shard alone gives, position by position, the same bits as
    the step on the whole flat buffer (no per-parameter or global statistic enters)."""
    unit = W.tiny_mlp(N=5)
    params = W.host_params(unit, seed=1)
    F = orc.flat_shard(params, unit.N, -1)
    L = F.size
    g = W.host_normal(L, 1e-3, seed=77)
    pf, mf, vf = F.copy(), np.zeros(L, np.float32), np.zeros(L, np.float32)
    for t in (1, 2, 3):
        orc.adamw(pf, g, mf, vf, lr=1e-3, weight_decay=0.01, step=t)
    S = L // unit.N
    for k in range(unit.N):
        sl = slice(k * S, (k + 1) * S)
        ps = orc.flat_shard(params, unit.N, k)
        ms, vs = np.zeros(S, np.float32), np.zeros(S, np.float32)
        gs = np.ascontiguousarray(g[sl])
        for t in (1, 2, 3):
            orc.adamw(ps, gs, ms, vs, lr=1e-3, weight_decay=0.01, step=t)
        assert np.array_equal(ps.view(np.uint32), pf[sl].view(np.uint32))
        assert np.array_equal(ms.view(np.uint32), mf[sl].view(np.uint32))
        assert np.array_equal(vs.view(np.uint32), vf[sl].view(np.uint32))


def test_padding_stays_zero(orc):
    """Pad elements (value +0, gradient 0) stay +0 through any number of steps."""
    n = 64
    p, g, m, v = (np.zeros(n, np.float32) for _ in range(4))
    for t in range(1, 11):
        orc.adamw(p, g, m, v, lr=1e-3, weight_decay=0.01, step=t)
    for a in (p, m, v):
        assert np.all(a.view(np.uint32) == 0)


def test_resume_is_bitwise(orc):
    """10 steps equal 5 steps, a save/restore of (p, m, v, t), and 5 more steps."""
    p, g0, m, v = _state(4096, 9)
    a = [x.copy() for x in (p, m, v)]
    for t in range(1, 11):
        g = W.host_normal(4096, 1e-3, seed=t)
        orc.adamw(a[0], g, a[1], a[2], lr=1e-3, weight_decay=0.01, step=t)
    b = [x.copy() for x in (p, m, v)]
    for t in range(1, 6):
        g = W.host_normal(4096, 1e-3, seed=t)
        orc.adamw(b[0], g, b[1], b[2], lr=1e-3, weight_decay=0.01, step=t)
    saved = [x.tobytes() for x in b]
    b = [np.frombuffer(s, np.float32).copy() for s in saved]
    for t in range(6, 11):
        g = W.host_normal(4096, 1e-3, seed=t)
        orc.adamw(b[0], g, b[1], b[2], lr=1e-3, weight_decay=0.01, step=t)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


def test_bf16_copy_of_new_params(orc):
    p, g, m, v = _state(10000, 4)
    pb = orc.adamw(p, g, m, v, lr=1e-3, weight_decay=0.01, step=1, want_bf16=True)
    ref = torch.from_numpy(p).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(pb, ref)
