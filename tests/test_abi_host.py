"""Host-side checks of the C-ABI library: it loads, exports what the header declares,
plans units exactly as the oracle lays them out, keeps the pages' memory ledger,
and rejects every invalid argument before making any HIP call (so all of this
runs without a GPU)."""
import ctypes
import os
import re

import numpy as np
import pytest

import workloads as W
from conftest import ROOT, golden_path

HEADER = os.path.join(ROOT, "include", "fsdp_flatten.h")


@pytest.fixture(scope="module")
def B():
    from sharded_fsdp_flatten_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from sharded_fsdp_flatten_amd import build
        build.build()
    binding.load()
    return binding


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"FSDP_API\s+[\w\s\*]+?\b(fsdp_\w+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = _declared()
    for n in ("fsdp_flatten_shard", "fsdp_unflatten_copyout", "fsdp_grad_reduce_shard",
              "fsdp_adam_shard"):
        assert n in names


def test_library_exports_every_declared_symbol(B):
    lib = B.load()
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing
    assert sorted(_declared()) == sorted(B.ABI_FUNCTIONS)


def test_abi_version_matches_header(B):
    v = int(re.search(r"#define FSDP_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert B.fsdp_abi_version() == v == B.ABI_VERSION


def _labelled(shapes):
    out = []
    for s in shapes:
        n = int(np.prod(s, dtype=np.int64)) if len(s) else 1
        out.append(np.ones(n, np.float32).reshape(s))
    return out


@pytest.mark.parametrize("layout", [W.FLAT, W.ROWS])
def test_planner_sizes_match_oracle(B, orc, layout):
    """T, S, L, pad, per-rank valid counts and offsets agree with the oracle's own
    layout (valid counts read off the oracle by counting the non-zero elements of a
    shard of all-ones parameters)."""
    rng = np.random.Generator(np.random.PCG64(31))
    for trial in range(80):
        shapes = W.random_unit_shapes(rng, max_params=5, max_dim=6)
        params = _labelled(shapes)
        for N in (1, 2, 3, 5, 8):
            u = B.fsdp_unit_create(layout, shapes, N)
            info = u.info()
            T = sum(p.size for p in params)
            if layout == W.FLAT:
                T2, S, L, pad = orc.flat_sizes([p.size for p in params], N)
                assert (info["T"], info["S"], info["L"], info["pad"]) == (T2, S, L, pad)
                off = 0
                for i, p in enumerate(params):
                    assert u.offset(i) == off
                    off += p.size
            else:
                P_r = orc.rows_sizes(shapes, N)
                assert (info["T"], info["S"], info["L"]) == (T, P_r, N * P_r)
                assert info["pad"] == N * P_r - T
            for k in range(N):
                shard = (orc.flat_shard(params, N, k) if layout == W.FLAT
                         else orc.rows_shard(params, N, k))
                ik = u.info(k)
                assert ik["valid"] == int(np.count_nonzero(shard)), (shapes, N, k)
                assert ik["bytes_per_rank"] == 16 * ik["S"]


def _ledger():
    vals = {}
    with open(golden_path("memory_ledger.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                key, val, unit, dec = [x.strip() for x in line.split("|")]
                vals[key] = (float(val), unit, int(dec))
    return vals


def _gpt2_large_units():
    """GPT-2 Large as the page's script wraps it: one unit per transformer block plus
    the root unit with the embeddings and the final LayerNorm."""
    _, block = W.gpt_block(1280)
    root = [(50257, 1280), (1024, 1280), (1280,), (1280,)]
    return [block] * 36 + [root]


def test_memory_ledger_matches_pages(B):
    """"FSDP Architecture" per-GPU ledger 4P/N + 4P/N + 8P/N with its 13B example, and the
    GPT-2 Large figures of "FSDP Under The Hood" section 5 (Psi = 0.774B)."""
    L = _ledger()
    GB, GiB = 1e9, 2.0 ** 30

    def same(key, x):
        val, unit, dec = L[key]
        scale = {"GB": GB, "GiB": GiB, "G": 1e9}[unit]
        assert round(x / scale, dec) == val, (key, x / scale)

    u13 = B.fsdp_unit_create(B.FSDP_FLAT, [(13_000_000_000,)], 8)
    same("p3_13b_per_gpu_n8", u13.info(0)["bytes_per_rank"])
    same("p3_13b_total", B.fsdp_unit_create(B.FSDP_FLAT, [(13_000_000_000,)], 1).info(0)["bytes_per_rank"])

    units = _gpt2_large_units()
    psi = sum(B.fsdp_unit_create(B.FSDP_ROWS, shapes, 1).info()["T"] for shapes in units)
    assert psi == 774_030_080
    same("p2_psi", psi)
    same("p2_ddp_16psi", sum(B.fsdp_unit_create(B.FSDP_FLAT, s, 1).info(0)["bytes_per_rank"]
                             for s in units))
    fsdp2 = sum(12 * B.fsdp_unit_create(B.FSDP_ROWS, s, 8).info(0)["S"] for s in units)
    same("p2_fsdp2_12psi_over_8", fsdp2)
    same("p2_bf16_model", 2 * psi)
    same("p2_bf16_model_gb", 2 * psi)
    same("p2_fp32_grads", 4 * psi)


# ---------------------------------------------------------------------------
# validation: every error is reported before any HIP call
# ---------------------------------------------------------------------------

FAKE = 0x7F0000000000  # 256-byte aligned address that is never dereferenced


def _status(exc):
    return exc.value.status_name


def test_create_errors(B):
    with pytest.raises(B.FsdpError) as e:
        B.fsdp_unit_create(3, [(4,)], 2)
    assert _status(e) == "FSDP_E_RANGE"
    with pytest.raises(B.FsdpError) as e:
        B.fsdp_unit_create(B.FSDP_FLAT, [(4,)], 0)
    assert _status(e) == "FSDP_E_RANGE"
    with pytest.raises(B.FsdpError) as e:
        B.fsdp_unit_create(B.FSDP_FLAT, [(4, -1)], 2)
    assert _status(e) == "FSDP_E_RANGE"
    with pytest.raises(B.FsdpError) as e:
        B.fsdp_unit_create(B.FSDP_FLAT, [(1,) * 9], 2)
    assert _status(e) == "FSDP_E_RANGE"
    with pytest.raises(B.FsdpError) as e:
        B.fsdp_unit_create(B.FSDP_FLAT, [(2 ** 40, 2 ** 40)], 2)
    assert _status(e) == "FSDP_E_OVERFLOW"
    with pytest.raises(B.FsdpError) as e:
        B.fsdp_unit_create(B.FSDP_FLAT, [(2 ** 62,), (2 ** 62,)], 2)
    assert _status(e) == "FSDP_E_OVERFLOW"
    with pytest.raises(B.FsdpError) as e:
        B.fsdp_unit_create(B.FSDP_ROWS, [(2 ** 62, 3)], 2)
    assert _status(e) == "FSDP_E_OVERFLOW"
    assert "overflow" in B.fsdp_last_error()
    lib = B.load()
    assert lib.fsdp_unit_create(1, 0, None, None, 1, None) == 1  # null out
    import ctypes
    out = ctypes.c_void_p()
    assert lib.fsdp_unit_create(1, 2, None, None, 1, ctypes.byref(out)) == 1  # null tables
    # only scalars: sum(ndims) = 0, so dims may be NULL; a NULL dims with dimensions may not
    nd0 = (ctypes.c_int32 * 2)(0, 0)
    assert lib.fsdp_unit_create(1, 2, nd0, None, 3, ctypes.byref(out)) == 0
    lib.fsdp_unit_destroy(out)
    nd1 = (ctypes.c_int32 * 2)(0, 1)
    assert lib.fsdp_unit_create(1, 2, nd1, None, 3, ctypes.byref(out)) == 1


def test_info_and_offset_errors(B):
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(4,), (3,)], 2)
    for k in (2, -2, 100):
        with pytest.raises(B.FsdpError) as e:
            u.info(k)
        assert _status(e) == "FSDP_E_RANGE"
    with pytest.raises(B.FsdpError):
        u.offset(2)


def test_recv_pitch(B):
    """S rounded up to whole 128-byte lines (64 bf16), for both layouts; null arguments fail."""
    import ctypes
    cases = [(B.FSDP_FLAT, [(W.gpt175b_block().shapes[0])], 128),
             (B.FSDP_FLAT, W.gpt175b_block().shapes, 128), (B.FSDP_FLAT, W.gpt175b_block().shapes, 120),
             (B.FSDP_FLAT, [(64 * 5,)], 5), (B.FSDP_FLAT, [(65,)], 1), (B.FSDP_FLAT, [(3,)], 4),
             (B.FSDP_ROWS, W.gpt2_large_emb_rows().shapes, 8), (B.FSDP_FLAT, [], 3)]
    for layout, shapes, N in cases:
        u = B.fsdp_unit_create(layout, shapes, N)
        p = u.recv_pitch
        assert p % 64 == 0 and u.S <= p < u.S + 64, (u.S, p)
    assert B.fsdp_unit_create(B.FSDP_FLAT, W.gpt175b_block().shapes, 128).recv_pitch == 14_157_056
    assert B.fsdp_unit_create(B.FSDP_FLAT, [(64 * 5,)], 5).recv_pitch == 64
    assert B.fsdp_unit_create(B.FSDP_FLAT, [], 3).recv_pitch == 0
    lib = B.load()
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(4,)], 2)
    assert lib.fsdp_unit_recv_pitch(u.handle, None) == 1
    assert lib.fsdp_unit_recv_pitch(None, ctypes.byref(ctypes.c_int64())) == 1


def test_flatten_errors(B):
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(4,), (3,)], 2)
    cases = [
        (dict(params=[FAKE, FAKE], k=2, shard=FAKE), "FSDP_E_RANGE"),
        (dict(params=[FAKE, FAKE], k=-2, shard=FAKE), "FSDP_E_RANGE"),
        (dict(params=[FAKE, 0], k=0, shard=FAKE), "FSDP_E_ARG"),
        (dict(params=[FAKE + 2, FAKE], k=0, shard=FAKE), "FSDP_E_ALIGN"),
        (dict(params=[FAKE, FAKE], k=0, shard=0), "FSDP_E_ARG"),
        (dict(params=[FAKE, FAKE], k=0, shard=FAKE + 1), "FSDP_E_ALIGN"),
    ]
    for kw, want in cases:
        with pytest.raises(B.FsdpError) as e:
            B.fsdp_flatten_shard(u, kw["params"], kw["k"], kw["shard"], stream=0)
        assert _status(e) == want, kw
    lib = B.load()
    assert lib.fsdp_flatten_shard(u.handle, None, 0, FAKE, None) == 1  # null table


def test_copyout_errors(B):
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(4,), (3,)], 2)
    with pytest.raises(B.FsdpError) as e:
        B.fsdp_unflatten_copyout(u, 0, [FAKE, FAKE], stream=0)
    assert _status(e) == "FSDP_E_ARG"
    with pytest.raises(B.FsdpError) as e:
        B.fsdp_unflatten_copyout(u, FAKE, [FAKE, FAKE + 1], stream=0)
    assert _status(e) == "FSDP_E_ALIGN"
    with pytest.raises(B.FsdpError) as e:
        B.fsdp_unflatten_copyout(u, FAKE + 2, [FAKE, FAKE], stream=0)
    assert _status(e) == "FSDP_E_ALIGN"


def test_reduce_errors(B):
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(16,)], 4)
    good = [FAKE] * 4
    for pre, post in [(0.0, 1.0), (1.0, 0.0), (float("inf"), 1.0), (1.0, float("nan")),
                      (float("nan"), 1.0), (-0.0, 1.0)]:
        with pytest.raises(B.FsdpError) as e:
            B.fsdp_grad_reduce_shard(u, good, pre, post, FAKE, stream=0)
        assert _status(e) == "FSDP_E_RANGE"
    with pytest.raises(B.FsdpError) as e:
        B.fsdp_grad_reduce_shard(u, [FAKE, 0, FAKE, FAKE], 1.0, 1.0, FAKE, stream=0)
    assert _status(e) == "FSDP_E_ARG"
    with pytest.raises(B.FsdpError) as e:
        B.fsdp_grad_reduce_shard(u, [FAKE, FAKE + 1, FAKE, FAKE], 1.0, 1.0, FAKE, stream=0)
    assert _status(e) == "FSDP_E_ALIGN"
    with pytest.raises(B.FsdpError) as e:
        B.fsdp_grad_reduce_shard(u, good, 1.0, 1.0, FAKE + 2, stream=0)
    assert _status(e) == "FSDP_E_ALIGN"
    with pytest.raises(ValueError):
        B.fsdp_grad_reduce_shard(u, good[:3], 1.0, 1.0, FAKE, stream=0)


def test_adam_errors(B):
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(16,)], 4)
    base = dict(lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01, step=1)
    bad = [dict(step=0), dict(step=-3), dict(betas=(1.0, 0.999)), dict(betas=(0.9, -0.1)),
           dict(betas=(float("nan"), 0.9)), dict(eps=-1.0), dict(eps=float("inf")),
           dict(lr=float("nan")), dict(weight_decay=float("inf"))]
    for b in bad:
        kw = dict(base, **b)
        with pytest.raises(B.FsdpError) as e:
            B.fsdp_adam_shard(u, FAKE, FAKE, FAKE, FAKE, stream=0, **kw)
        assert _status(e) == "FSDP_E_RANGE", b
    with pytest.raises(B.FsdpError) as e:
        B.fsdp_adam_shard(u, 0, FAKE, FAKE, FAKE, stream=0, **base)
    assert _status(e) == "FSDP_E_ARG"
    with pytest.raises(B.FsdpError) as e:
        B.fsdp_adam_shard(u, FAKE, FAKE, FAKE + 2, FAKE, stream=0, **base)
    assert _status(e) == "FSDP_E_ALIGN"
    with pytest.raises(B.FsdpError) as e:
        B.fsdp_adam_shard(u, FAKE, FAKE, FAKE, FAKE, param_bf16=FAKE + 1, stream=0, **base)
    assert _status(e) == "FSDP_E_ALIGN"
    lib = B.load()
    assert lib.fsdp_adam_shard(u.handle, FAKE, FAKE, FAKE, FAKE, None, None, None) == 1


def test_empty_unit_calls_are_noops(B):
    """A unit with no elements: every call validates and returns OK without launching."""
    for layout in (B.FSDP_FLAT, B.FSDP_ROWS):
        for shapes in ([], [(0,)], [(0, 5), (3, 0)]):
            u = B.fsdp_unit_create(layout, shapes, 4)
            assert u.info()["T"] == 0
            B.fsdp_flatten_shard(u, [0] * len(shapes), 0, 0, stream=0)
            B.fsdp_flatten_shard(u, [0] * len(shapes), B.FSDP_ALL_RANKS, 0, stream=0)
            B.fsdp_unflatten_copyout(u, 0, [0] * len(shapes), stream=0)
            B.fsdp_grad_reduce_shard(u, [0] * 4, 1.0, 1.0, 0, stream=0)
            B.fsdp_adam_shard(u, 0, 0, 0, 0, lr=1e-3, stream=0)
            assert B.fsdp_last_error() == ""


def test_last_error_is_per_call(B):
    with pytest.raises(B.FsdpError):
        B.fsdp_unit_create(B.FSDP_FLAT, [(4,)], 0)
    assert B.fsdp_last_error() != ""
    B.fsdp_unit_create(B.FSDP_FLAT, [(4,)], 1)
    assert B.fsdp_last_error() == ""
    assert B.fsdp_status_string(3) == "FSDP_E_ALIGN"
    assert B.fsdp_status_string(99) == "FSDP_E_UNKNOWN"


# ---------------------------------------------------------------------------
# next rows: cast before gather, bf16 copy-out / copy-in, hybrid and accumulating
# reduction, local accumulation
# ---------------------------------------------------------------------------

def test_reduce_ex_errors(B):
    lib = B.load()
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(64,)], 8)
    good = [FAKE] * 8
    for group in (3, 5, 7, 9, -1):
        with pytest.raises(B.FsdpError) as e:
            B.fsdp_grad_reduce_shard_ex(u, good, 1.0, 1.0, FAKE, group=group, stream=0)
        assert _status(e) == "FSDP_E_RANGE", group
    for pre, post in [(0.0, 1.0), (1.0, float("inf"))]:
        with pytest.raises(B.FsdpError) as e:
            B.fsdp_grad_reduce_shard_ex(u, good, pre, post, FAKE, group=2, stream=0)
        assert _status(e) == "FSDP_E_RANGE"
    assert lib.fsdp_grad_reduce_shard_ex(u.handle, None, None, FAKE, None) == 1  # opts NULL
    with pytest.raises(ValueError):
        B.fsdp_grad_reduce_shard_ex(u, good, 1.0, 1.0, FAKE, kernel="fast", stream=0)
    opts = B.fsdp_reduce_opts(1.0, 1.0, 0, 0, 3, 0, None, 0)  # kernel 3 is not a kernel
    assert lib.fsdp_grad_reduce_shard_ex(u.handle, None, ctypes.byref(opts), FAKE, None) == 2
    # more ranks than one launch holds (128): the sums carried between launches need the
    # caller's workspace when the output must keep its old value or a group spans launches
    big = B.fsdp_unit_create(B.FSDP_FLAT, [(512 * 4,)], 512)  # S = 4: one slot of 64 floats
    for group, acc, need in [(0, False, 0), (0, True, 64), (8, False, 0), (8, True, 64),
                             (128, True, 64), (256, False, 64), (256, True, 128),
                             (512, True, 64)]:
        assert B.fsdp_grad_reduce_workspace(big, group=group, accumulate=acc) == need, (group, acc)
        if need == 0:
            continue
        with pytest.raises(B.FsdpError) as e:  # no workspace
            B.fsdp_grad_reduce_shard_ex(big, [FAKE] * 512, 1.0, 1.0, FAKE, group=group,
                                        accumulate=acc, stream=0)
        assert _status(e) == "FSDP_E_ARG"
        for ws, ws_len, want in [(FAKE + 8, need, "FSDP_E_ALIGN"), (FAKE, need - 1, "FSDP_E_RANGE")]:
            o = B.fsdp_reduce_opts(1.0, 1.0, group, int(acc), 0, 0, ws, ws_len)
            table = (ctypes.c_void_p * 512)(*([FAKE] * 512))
            st = lib.fsdp_grad_reduce_shard_ex(big.handle, ctypes.cast(table, ctypes.c_void_p),
                                               ctypes.byref(o), FAKE, None)
            assert B.STATUS_NAMES[st] == want, (group, acc)
    for group in (3, 1000):
        with pytest.raises(B.FsdpError) as e:
            B.fsdp_grad_reduce_workspace(big, group=group)
        assert _status(e) == "FSDP_E_RANGE"
    # a shard that is not a multiple of 64: slots are S rounded up to 64 floats
    odd = B.fsdp_unit_create(B.FSDP_FLAT, [(300 * 130,)], 300)  # S = 130
    assert B.fsdp_grad_reduce_workspace(odd, group=150, accumulate=True) == 2 * 192
    assert B.fsdp_grad_reduce_workspace(odd, group=150) == 192
    assert B.fsdp_grad_reduce_workspace(odd, group=100, accumulate=True) == 192
    with pytest.raises(B.FsdpError) as e:
        B.fsdp_grad_reduce_shard_ex(u, [FAKE] * 7 + [FAKE + 1], 1.0, 1.0, FAKE, group=4, stream=0)
    assert _status(e) == "FSDP_E_ALIGN"


def test_cast_copyin_accumulate_errors(B):
    u = B.fsdp_unit_create(B.FSDP_ROWS, [(5, 3), (4,)], 4)
    for k in (4, -2):
        with pytest.raises(B.FsdpError) as e:
            B.fsdp_cast_to_bf16(u, k, FAKE, FAKE, stream=0)
        assert _status(e) == "FSDP_E_RANGE"
        with pytest.raises(B.FsdpError) as e:
            B.fsdp_flatten_shard_bf16(u, [FAKE, FAKE], k, FAKE, stream=0)
        assert _status(e) == "FSDP_E_RANGE"
        with pytest.raises(B.FsdpError) as e:
            B.fsdp_grad_accumulate(u, k, FAKE, FAKE, True, stream=0)
        assert _status(e) == "FSDP_E_RANGE"
    cases = [
        (lambda: B.fsdp_cast_to_bf16(u, 0, 0, FAKE, stream=0), "FSDP_E_ARG"),
        (lambda: B.fsdp_cast_to_bf16(u, 0, FAKE + 2, FAKE, stream=0), "FSDP_E_ALIGN"),
        (lambda: B.fsdp_cast_to_bf16(u, B.FSDP_ALL_RANKS, FAKE, FAKE + 1, stream=0), "FSDP_E_ALIGN"),
        (lambda: B.fsdp_unflatten_copyout_bf16(u, 0, [FAKE, FAKE], stream=0), "FSDP_E_ARG"),
        (lambda: B.fsdp_unflatten_copyout_bf16(u, FAKE, [FAKE, FAKE + 1], stream=0), "FSDP_E_ALIGN"),
        (lambda: B.fsdp_unflatten_copyout_bf16(u, FAKE + 1, [FAKE, FAKE], stream=0), "FSDP_E_ALIGN"),
        (lambda: B.fsdp_flatten_shard_bf16(u, [FAKE, 0], 0, FAKE, stream=0), "FSDP_E_ARG"),
        (lambda: B.fsdp_flatten_shard_bf16(u, [FAKE, FAKE], 0, 0, stream=0), "FSDP_E_ARG"),
        (lambda: B.fsdp_flatten_shard_bf16(u, [FAKE + 1, FAKE], 0, FAKE, stream=0), "FSDP_E_ALIGN"),
        (lambda: B.fsdp_grad_accumulate(u, 0, 0, FAKE, False, stream=0), "FSDP_E_ARG"),
        (lambda: B.fsdp_grad_accumulate(u, 0, FAKE, FAKE + 2, False, stream=0), "FSDP_E_ALIGN"),
    ]
    for fn, want in cases:
        with pytest.raises(B.FsdpError) as e:
            fn()
        assert _status(e) == want


def test_next_rows_noops_on_empty_units(B):
    for layout in (B.FSDP_FLAT, B.FSDP_ROWS):
        for shapes in ([], [(0,)], [(0, 5), (3, 0)]):
            u = B.fsdp_unit_create(layout, shapes, 4)
            B.fsdp_cast_to_bf16(u, 0, 0, 0, stream=0)
            B.fsdp_cast_to_bf16(u, B.FSDP_ALL_RANKS, 0, 0, stream=0)
            B.fsdp_unflatten_copyout_bf16(u, 0, [0] * len(shapes), stream=0)
            B.fsdp_flatten_shard_bf16(u, [0] * len(shapes), B.FSDP_ALL_RANKS, 0, stream=0)
            B.fsdp_grad_reduce_shard_ex(u, [0] * 4, 1.0, 1.0, 0, group=2, accumulate=True, stream=0)
            B.fsdp_grad_accumulate(u, B.FSDP_ALL_RANKS, 0, 0, True, stream=0)
            assert B.fsdp_last_error() == ""


def _runs_by_hand(shapes, N, k, layout_flat=True):
    """Each parameter's element count inside rank k's shard, from the layout definitions."""
    import oracle
    if layout_flat:
        numels = [oracle.numel(sh) for sh in shapes]
        T, S, L, pad = oracle.flat_sizes(numels, N)
        out, off = [], 0
        for n in numels:
            lo, hi = max(off, k * S), min(off + n, (k + 1) * S)
            out.append(max(0, hi - lo))
            off += n
        return out
    out = []
    for sh in shapes:
        m, r = oracle.rows_of(sh)
        c = -(-m // N)
        out.append((min(m, (k + 1) * c) - min(m, k * c)) * r)
    return out


def test_sqnorm_workspace_counts_4096_element_tiles_per_parameter(B):
    for layout, shapes, N in [(B.FSDP_FLAT, W.gpt2_large_block().shapes, 8),
                              (B.FSDP_FLAT, W.gpt175b_block().shapes, 128),
                              (B.FSDP_ROWS, W.gpt2_large_emb_rows().shapes, 8),
                              (B.FSDP_FLAT, [(3, 4), (3,)], 16), (B.FSDP_FLAT, [(5000,), (3,)], 2)]:
        u = B.fsdp_unit_create(layout, shapes, N)
        for k in sorted({0, 1, N // 2, N - 1}):
            runs = _runs_by_hand(shapes, N, k, layout == B.FSDP_FLAT)
            assert B.fsdp_grad_sqnorm_workspace(u, k) == sum(-(-n // 4096) for n in runs)


def test_unscale_and_sqnorm_errors(B):
    import ctypes
    lib = B.load()
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(4,), (3,)], 2)
    g, f, o, w = 0x1000, 0x2000, 0x3000, 0x4000  # never dereferenced: validation fails first
    assert lib.fsdp_grad_unscale(None, 0, g, 0.5, f, None) == 1
    assert lib.fsdp_grad_unscale(u.handle, 2, g, 0.5, f, None) == 2
    assert lib.fsdp_grad_unscale(u.handle, 0, None, 0.5, f, None) == 1
    assert lib.fsdp_grad_unscale(u.handle, 0, g, 0.5, f + 2, None) == 3  # flag must be float-aligned
    assert lib.fsdp_grad_unscale(u.handle, 0, g + 2, 0.5, f, None) == 3  # fp32 needs 4-byte alignment
    for bad in (float("inf"), float("nan")):
        assert lib.fsdp_grad_unscale(u.handle, 0, g, bad, f, None) == 1
    n = ctypes.c_int64()
    assert lib.fsdp_grad_sqnorm_workspace(u.handle, -1, ctypes.byref(n)) == 2  # no ALL-ranks form
    assert lib.fsdp_grad_sqnorm_workspace(u.handle, 0, None) == 1
    # rank 1 holds 3 elements of the second parameter (and the pad): one tile
    assert lib.fsdp_grad_sqnorm_workspace(u.handle, 1, ctypes.byref(n)) == 0 and n.value == 1
    assert lib.fsdp_grad_sqnorm(u.handle, 2, g, w, 8, o, None) == 2
    assert lib.fsdp_grad_sqnorm(u.handle, 1, g, w, 0, o, None) == 2  # workspace too small
    assert "needs 1" in B.fsdp_last_error()
    assert lib.fsdp_grad_sqnorm(u.handle, 1, g, w, 1, None, None) == 1
    assert lib.fsdp_grad_sqnorm(u.handle, 1, None, w, 1, o, None) == 1
    assert lib.fsdp_grad_sqnorm(u.handle, 1, g, None, 1, o, None) == 1
    assert lib.fsdp_grad_sqnorm(u.handle, 1, g, w + 4, 1, o, None) == 3  # doubles need 8-byte alignment
    e = B.fsdp_unit_create(B.FSDP_FLAT, [], 3)  # empty unit: nothing to do, nothing launched
    assert lib.fsdp_grad_unscale(e.handle, 0, None, 0.5, None, None) == 0
    assert lib.fsdp_grad_sqnorm_workspace(e.handle, 0, ctypes.byref(n)) == 0 and n.value == 0
    assert lib.fsdp_grad_sqnorm(e.handle, 0, None, None, 0, None, None) == 0
    # the allocation-free variant validates the same way, and refuses shards whose partial
    # sums do not fit its 262,144-double scratch, before any HIP call
    assert lib.fsdp_grad_sqnorm_noalloc(None, 0, g, o, None) == 1
    assert lib.fsdp_grad_sqnorm_noalloc(u.handle, 2, g, o, None) == 2
    assert lib.fsdp_grad_sqnorm_noalloc(u.handle, 1, None, o, None) == 1
    assert lib.fsdp_grad_sqnorm_noalloc(u.handle, 1, g, None, None) == 1
    assert lib.fsdp_grad_sqnorm_noalloc(u.handle, 1, g, o + 4, None) == 3
    assert lib.fsdp_grad_sqnorm_noalloc(e.handle, 0, None, None, None) == 0
    big = B.fsdp_unit_create(B.FSDP_FLAT, [((1 << 18) * 4096 + 1,)], 1)
    assert lib.fsdp_grad_sqnorm_workspace(big.handle, 0, ctypes.byref(n)) == 0
    assert n.value == (1 << 18) + 1
    assert lib.fsdp_grad_sqnorm_noalloc(big.handle, 0, g, o, None) == 2
    assert "holds 262144" in B.fsdp_last_error()


def test_binding_refuses_host_tensors(B):
    """A host tensor's address would reach the kernels and fault the GPU: the binding refuses
    it before the library is called (and refuses non-contiguous tensors and wrong dtypes)."""
    import torch
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(5, 3), (7,)], 2)
    params = [torch.zeros(5, 3), torch.zeros(7)]
    with pytest.raises(ValueError, match="on the GPU"):
        B.fsdp_flatten_shard(u, params, 0, FAKE, stream=0)
    with pytest.raises(ValueError, match="on the GPU"):
        B.fsdp_flatten_shard(u, [FAKE, FAKE], 0, torch.zeros(u.S), stream=0)
    with pytest.raises(ValueError, match="on the GPU"):
        B.fsdp_grad_reduce_shard(u, [torch.zeros(u.S, dtype=torch.bfloat16)] * 2, 1.0, 1.0, FAKE,
                                 stream=0)
    with pytest.raises(TypeError, match="dtype"):
        B.fsdp_adam_shard(u, torch.zeros(u.S, dtype=torch.float64), FAKE, FAKE, FAKE, lr=1e-3,
                          stream=0)


def test_last_error_is_per_thread(B):
    """fsdp_last_error() holds the calling thread's message: 8 threads fail calls with
    different messages at the same time (ctypes releases the GIL around foreign calls) and each
    must read back its own, then a successful call must leave its thread's message empty."""
    import ctypes
    import threading
    lib = B.load()
    errors = []

    def work(tid):
        try:
            u = B.fsdp_unit_create(B.FSDP_FLAT, [(4 + tid,)], 2)
            for it in range(300):
                if (it + tid) % 2:
                    st = lib.fsdp_unit_create(1, 1, None, None, 2, None)  # out NULL
                    want = b"out is NULL"
                else:
                    st = lib.fsdp_unit_param_offset(u.handle, 5 + tid, None)  # offset NULL
                    want = b"must not be NULL"
                msg = lib.fsdp_last_error()
                if st == 0 or want not in msg:
                    errors.append((tid, it, st, msg))
                    return
            sizes = B.fsdp_unit_sizes()
            if lib.fsdp_unit_info(u.handle, -1, ctypes.byref(sizes)) != 0 or lib.fsdp_last_error() != b"":
                errors.append((tid, "ok call left a message"))
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append((tid, repr(e)))

    threads = [threading.Thread(target=work, args=(t,)) for t in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:3]


def test_documented_error_statuses(B):
    """Every per-call 'Errors:' line of include/fsdp_flatten.h, condition by condition, returns
    the status it names (addresses are never dereferenced: validation precedes any HIP call)."""
    import ctypes
    lib = B.load()
    u = B.fsdp_unit_create(B.FSDP_FLAT, [(6, 5), (7,)], 4)
    h = u.handle
    tab2 = (ctypes.c_void_p * 2)(FAKE, FAKE)
    tab2_null = (ctypes.c_void_p * 2)(FAKE, None)
    tab2_odd = (ctypes.c_void_p * 2)(FAKE, FAKE + 1)
    tab2_two = (ctypes.c_void_p * 2)(FAKE, FAKE + 2)
    tab4 = (ctypes.c_void_p * 4)(FAKE, FAKE, FAKE, FAKE)
    tab4_null = (ctypes.c_void_p * 4)(FAKE, FAKE, None, FAKE)
    tab4_odd = (ctypes.c_void_p * 4)(FAKE, FAKE, FAKE + 1, FAKE)
    c = lambda t: ctypes.cast(t, ctypes.c_void_p)  # noqa: E731

    def adam(**kw):
        cfg = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, step=1)
        ptrs = kw.pop("ptrs", (FAKE, FAKE, FAKE, FAKE))
        pb = kw.pop("pb", None)
        cfg.update(kw)
        s = B.fsdp_adamw_cfg(cfg["lr"], cfg["beta1"], cfg["beta2"], cfg["eps"], cfg["weight_decay"],
                             cfg["step"])
        return lib.fsdp_adam_shard(h, *ptrs, ctypes.byref(s), pb, None)

    inf, nan = float("inf"), float("nan")
    cases = [
        # flatten
        (lambda: lib.fsdp_flatten_shard(None, c(tab2), 0, FAKE, None), "FSDP_E_ARG"),
        (lambda: lib.fsdp_flatten_shard(h, None, 0, FAKE, None), "FSDP_E_ARG"),
        (lambda: lib.fsdp_flatten_shard(h, c(tab2_null), 0, FAKE, None), "FSDP_E_ARG"),
        (lambda: lib.fsdp_flatten_shard(h, c(tab2), 0, None, None), "FSDP_E_ARG"),
        (lambda: lib.fsdp_flatten_shard(h, c(tab2), 4, FAKE, None), "FSDP_E_RANGE"),
        (lambda: lib.fsdp_flatten_shard(h, c(tab2), -2, FAKE, None), "FSDP_E_RANGE"),
        (lambda: lib.fsdp_flatten_shard(h, c(tab2_two), 0, FAKE, None), "FSDP_E_ALIGN"),
        (lambda: lib.fsdp_flatten_shard(h, c(tab2), 0, FAKE + 2, None), "FSDP_E_ALIGN"),
        # copy-out
        (lambda: lib.fsdp_unflatten_copyout(None, FAKE, c(tab2), None), "FSDP_E_ARG"),
        (lambda: lib.fsdp_unflatten_copyout(h, None, c(tab2), None), "FSDP_E_ARG"),
        (lambda: lib.fsdp_unflatten_copyout(h, FAKE, None, None), "FSDP_E_ARG"),
        (lambda: lib.fsdp_unflatten_copyout(h, FAKE, c(tab2_null), None), "FSDP_E_ARG"),
        (lambda: lib.fsdp_unflatten_copyout(h, FAKE + 2, c(tab2), None), "FSDP_E_ALIGN"),
        (lambda: lib.fsdp_unflatten_copyout(h, FAKE, c(tab2_odd), None), "FSDP_E_ALIGN"),
        # reduce
        (lambda: lib.fsdp_grad_reduce_shard(None, c(tab4), 1.0, 1.0, FAKE, None), "FSDP_E_ARG"),
        (lambda: lib.fsdp_grad_reduce_shard(h, None, 1.0, 1.0, FAKE, None), "FSDP_E_ARG"),
        (lambda: lib.fsdp_grad_reduce_shard(h, c(tab4_null), 1.0, 1.0, FAKE, None), "FSDP_E_ARG"),
        (lambda: lib.fsdp_grad_reduce_shard(h, c(tab4), 1.0, 1.0, None, None), "FSDP_E_ARG"),
        (lambda: lib.fsdp_grad_reduce_shard(h, c(tab4), 0.0, 1.0, FAKE, None), "FSDP_E_RANGE"),
        (lambda: lib.fsdp_grad_reduce_shard(h, c(tab4), 1.0, inf, FAKE, None), "FSDP_E_RANGE"),
        (lambda: lib.fsdp_grad_reduce_shard(h, c(tab4), nan, 1.0, FAKE, None), "FSDP_E_RANGE"),
        (lambda: lib.fsdp_grad_reduce_shard(h, c(tab4_odd), 1.0, 1.0, FAKE, None), "FSDP_E_ALIGN"),
        (lambda: lib.fsdp_grad_reduce_shard(h, c(tab4), 1.0, 1.0, FAKE + 2, None), "FSDP_E_ALIGN"),
        # AdamW
        (lambda: lib.fsdp_adam_shard(None, FAKE, FAKE, FAKE, FAKE, None, None, None), "FSDP_E_ARG"),
        (lambda: lib.fsdp_adam_shard(h, FAKE, FAKE, FAKE, FAKE, None, None, None), "FSDP_E_ARG"),
        (lambda: adam(ptrs=(FAKE, FAKE, None, FAKE)), "FSDP_E_ARG"),
        (lambda: adam(step=0), "FSDP_E_RANGE"),
        (lambda: adam(beta1=1.0), "FSDP_E_RANGE"),
        (lambda: adam(beta2=-0.1), "FSDP_E_RANGE"),
        (lambda: adam(lr=nan), "FSDP_E_RANGE"),
        (lambda: adam(weight_decay=inf), "FSDP_E_RANGE"),
        (lambda: adam(eps=-1e-8), "FSDP_E_RANGE"),
        (lambda: adam(eps=inf), "FSDP_E_RANGE"),
        (lambda: adam(ptrs=(FAKE, FAKE + 2, FAKE, FAKE)), "FSDP_E_ALIGN"),
        (lambda: adam(pb=FAKE + 1), "FSDP_E_ALIGN"),
        # cast, bf16 copy-out, bf16 flatten, local accumulation
        (lambda: lib.fsdp_cast_to_bf16(None, 0, FAKE, FAKE, None), "FSDP_E_ARG"),
        (lambda: lib.fsdp_cast_to_bf16(h, 0, None, FAKE, None), "FSDP_E_ARG"),
        (lambda: lib.fsdp_cast_to_bf16(h, 4, FAKE, FAKE, None), "FSDP_E_RANGE"),
        (lambda: lib.fsdp_cast_to_bf16(h, 0, FAKE, FAKE + 1, None), "FSDP_E_ALIGN"),
        (lambda: lib.fsdp_unflatten_copyout_bf16(h, FAKE + 1, c(tab2), None), "FSDP_E_ALIGN"),
        (lambda: lib.fsdp_unflatten_copyout_bf16(h, None, c(tab2), None), "FSDP_E_ARG"),
        (lambda: lib.fsdp_flatten_shard_bf16(h, c(tab2_odd), 0, FAKE, None), "FSDP_E_ALIGN"),
        (lambda: lib.fsdp_flatten_shard_bf16(h, c(tab2), 9, FAKE, None), "FSDP_E_RANGE"),
        (lambda: lib.fsdp_grad_accumulate(None, 0, FAKE, FAKE, 1, None), "FSDP_E_ARG"),
        (lambda: lib.fsdp_grad_accumulate(h, 0, FAKE, None, 1, None), "FSDP_E_ARG"),
        (lambda: lib.fsdp_grad_accumulate(h, -3, FAKE, FAKE, 1, None), "FSDP_E_RANGE"),
        (lambda: lib.fsdp_grad_accumulate(h, 0, FAKE + 1, FAKE, 1, None), "FSDP_E_ALIGN"),
        # plan queries
        (lambda: lib.fsdp_unit_info(None, 0, ctypes.byref(B.fsdp_unit_sizes())), "FSDP_E_ARG"),
        (lambda: lib.fsdp_unit_info(h, 0, None), "FSDP_E_ARG"),
        (lambda: lib.fsdp_unit_info(h, 4, ctypes.byref(B.fsdp_unit_sizes())), "FSDP_E_RANGE"),
        (lambda: lib.fsdp_unit_param_offset(None, 0, ctypes.byref(ctypes.c_int64())), "FSDP_E_ARG"),
        (lambda: lib.fsdp_unit_param_offset(h, 0, None), "FSDP_E_ARG"),
        (lambda: lib.fsdp_unit_param_offset(h, 2, ctypes.byref(ctypes.c_int64())), "FSDP_E_RANGE"),
        (lambda: lib.fsdp_unit_param_offset(h, -1, ctypes.byref(ctypes.c_int64())), "FSDP_E_RANGE"),
        (lambda: lib.fsdp_unit_recv_pitch(None, ctypes.byref(ctypes.c_int64())), "FSDP_E_ARG"),
        (lambda: lib.fsdp_unit_recv_pitch(h, None), "FSDP_E_ARG"),
        (lambda: lib.fsdp_unit_destroy(None), "FSDP_OK"),
    ]
    for i, (call, want) in enumerate(cases):
        got = B.STATUS_NAMES.get(call(), "?")
        assert got == want, (i, got, want, lib.fsdp_last_error())
