"""Every entry point can be captured in a HIP graph: the calls only launch kernels on the
caller's stream (no allocation, no memset, no synchronisation).  A whole step is captured
once and replayed several times, with the program's own eager work and synchronisations
between the replays; every replay is compared bit for bit with the same sequence run
eagerly on a second set of buffers."""
import gc

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import dev, to_host
from sharded_fsdp_flatten_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free():
    B.load()
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _state(u, unit, seed):
    """All buffers of one step, filled deterministically."""
    d = dev()
    gen = torch.Generator(device=d).manual_seed(seed)
    st = {
        "params": [torch.randn(s, device=d, generator=gen).mul_(0.02) for s in unit.shapes],
        "gathered": torch.randn(u.L, device=d, generator=gen).mul_(0.02),
        "outs": [torch.empty(s, dtype=torch.bfloat16, device=d) for s in unit.shapes],
        "contribs": W.device_contribs(u.N, u.S, step=seed, pitch=u.recv_pitch),
        "grad": torch.empty(u.S, device=d),
        "p": torch.randn(u.S, device=d, generator=gen).mul_(0.02),
        "m": torch.zeros(u.S, device=d),
        "v": torch.zeros(u.S, device=d),
        "pb": torch.empty(u.S, dtype=torch.bfloat16, device=d),
        "shard": torch.empty(u.S, device=d),
        "flag": torch.zeros(1, device=d),
        "ws": torch.empty(max(1, B.fsdp_grad_sqnorm_workspace(u, 3)), dtype=torch.float64, device=d),
        "sq": torch.empty(len(unit.shapes), dtype=torch.float64, device=d),
    }
    return st


def _step(u, unit, st):
    hp = unit.adam
    rows = [st["contribs"][r] for r in range(u.N)]
    B.fsdp_grad_reduce_shard(u, rows, 2.0, 4.0, st["grad"])
    B.fsdp_grad_unscale(u, 3, st["grad"], 0.5, st["flag"])
    B.fsdp_grad_sqnorm(u, 3, st["grad"], st["sq"], st["ws"])
    B.fsdp_unflatten_copyout(u, st["gathered"], st["outs"])
    B.fsdp_adam_shard(u, st["p"], st["grad"], st["m"], st["v"], step=1, param_bf16=st["pb"], **hp)
    B.fsdp_flatten_shard(u, st["params"], 3, st["shard"])


def _snapshot(st):
    out = {}
    for k in ("grad", "p", "m", "v", "pb", "shard", "flag", "sq"):
        out[k] = to_host(st[k]).copy()
    out["outs"] = [to_host(o).copy() for o in st["outs"]]
    return out


def _same(a, b, what):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape and a.dtype == b.dtype, what
    assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), what


@pytest.mark.parametrize("name", ["gpt2l", "rows"])
def test_step_replays_from_a_captured_graph(name):
    unit = {"gpt2l": W.gpt2_large_block(N=8), "rows": W.gpt2_large_emb_rows(N=8)}[name]
    layout = B.FSDP_FLAT if unit.layout == W.FLAT else B.FSDP_ROWS
    u = B.fsdp_unit_create(layout, unit.shapes, unit.N)
    eager = _state(u, unit, seed=1)
    graph = _state(u, unit, seed=1)
    # warm up on a side stream (what capture expects), then capture one step
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(u, unit, _state(u, unit, seed=2))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(u, unit, graph)
    torch.cuda.synchronize()
    for rep in range(3):
        g.replay()
        _step(u, unit, eager)
        torch.cuda.synchronize()
        a, b = _snapshot(graph), _snapshot(eager)
        for k in a:
            if k == "outs":
                for i, (x, y) in enumerate(zip(a[k], b[k])):
                    _same(x, y, "%s replay %d outs[%d]" % (name, rep, i))
            else:
                _same(a[k], b[k], "%s replay %d %s" % (name, rep, k))
        # the program's own eager work between replays
        junk = torch.randn(1 << 20, device=dev()).mul_(2.0).sum()
        junk.item()
