"""CPU oracle for the per-rank FSDP data path (test infrastructure only).

A thin ctypes wrapper around ``fsdp_oracle.c``.  Only the test suite, the
package smoke check and the CPU-baseline leg of ``bench.py`` may import this
package; the library under ``sharded_fsdp_flatten_amd`` never does, and the two
share no code.  Inputs and outputs are numpy arrays on the host.

The definitions, the pages they follow and the readings taken where the pages
are silent are stated next to each C function.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fsdp_oracle.c")
_BUILT = os.path.join(_HERE, "liboracle.so")
# FSDP_ORACLE_LIB may name another build of fsdp_oracle.c to load instead; the test suite
# loads copies with planted mistakes this way to check that the pins reject them.
_LIB_PATH = os.environ.get("FSDP_ORACLE_LIB") or _BUILT

CFLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = True, src: str = _SRC, out: str = _BUILT) -> str:
    """Compile fsdp_oracle.c (or another copy of it) with gcc into oracle/liboracle.so."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, src, "-o", tmp, "-lm"])
        os.replace(tmp, out)
    return out


_lib = None

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            if _LIB_PATH != _BUILT:
                raise FileNotFoundError("FSDP_ORACLE_LIB names a missing library: " + _LIB_PATH)
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        lib.orc_bf16.argtypes = [ctypes.c_float]
        lib.orc_bf16.restype = ctypes.c_uint16
        lib.orc_bf16_array.argtypes = [_i64, _p, _p]
        lib.orc_bf16_array.restype = None
        lib.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        lib.orc_bf16_to_f32.restype = ctypes.c_float
        lib.orc_flat_sizes.argtypes = [_i32, _p, _i64, _p]
        lib.orc_flat_sizes.restype = None
        lib.orc_flat_shard.argtypes = [_i32, _p, _p, _i64, _i64, _p]
        lib.orc_flat_shard.restype = ctypes.c_int
        lib.orc_flat_copyout.argtypes = [_i32, _p, _p, _p]
        lib.orc_flat_copyout.restype = None
        lib.orc_rows_sizes.argtypes = [_i32, _p, _p, _i64, _p]
        lib.orc_rows_sizes.restype = None
        lib.orc_rows_shard.argtypes = [_i32, _p, _p, _p, _i64, _i64, _p]
        lib.orc_rows_shard.restype = ctypes.c_int
        lib.orc_rows_copyout.argtypes = [_i32, _p, _p, _i64, _p, _p]
        lib.orc_rows_copyout.restype = None
        lib.orc_grad_reduce.argtypes = [_i64, _i64, _p, ctypes.c_float, ctypes.c_float, _p]
        lib.orc_grad_reduce.restype = None
        lib.orc_adamw.argtypes = [_i64, _p, _p, _p, _p, ctypes.c_double, ctypes.c_double,
                                  ctypes.c_double, ctypes.c_double, ctypes.c_double, _i64, _p]
        lib.orc_adamw.restype = None
        lib.orc_flat_shard_u16.argtypes = [_i32, _p, _p, _i64, _i64, _p]
        lib.orc_flat_shard_u16.restype = ctypes.c_int
        lib.orc_flat_copyout_u16.argtypes = [_i32, _p, _p, _p]
        lib.orc_flat_copyout_u16.restype = None
        lib.orc_rows_shard_u16.argtypes = [_i32, _p, _p, _p, _i64, _i64, _p]
        lib.orc_rows_shard_u16.restype = ctypes.c_int
        lib.orc_rows_copyout_u16.argtypes = [_i32, _p, _p, _i64, _p, _p]
        lib.orc_rows_copyout_u16.restype = None
        lib.orc_grad_reduce_ex.argtypes = [_i64, _i64, _p, ctypes.c_float, ctypes.c_float, _i64,
                                           ctypes.c_int, _p]
        lib.orc_grad_reduce_ex.restype = None
        lib.orc_grad_accumulate.argtypes = [_i64, _p, _p, ctypes.c_int]
        lib.orc_grad_accumulate.restype = None
        lib.orc_grad_unscale.argtypes = [_i64, _p, ctypes.c_float, _p]
        lib.orc_grad_unscale.restype = None
        lib.orc_flat_sqnorm.argtypes = [_i32, _p, _i64, _i64, _p, _p]
        lib.orc_flat_sqnorm.restype = None
        lib.orc_rows_sqnorm.argtypes = [_i32, _p, _p, _i64, _i64, _p, _p]
        lib.orc_rows_sqnorm.restype = None
        _lib = lib
    return _lib


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------

def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _i64_array(xs) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(list(xs), dtype=np.int64))


def _ptr_array(arrays) -> np.ndarray:
    return np.asarray([a.ctypes.data for a in arrays], dtype=np.uint64)


def _f32(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def numel(shape: Sequence[int]) -> int:
    n = 1
    for d in shape:
        n *= int(d)
    return n


def rows_of(shape: Sequence[int]) -> tuple[int, int]:
    """(m, r): dim-0 length and row length; a 0-d tensor is one row of one."""
    if len(shape) == 0:
        return 1, 1
    r = 1
    for d in shape[1:]:
        r *= int(d)
    return int(shape[0]), r


# --------------------------------------------------------------------------
# public oracle API
# --------------------------------------------------------------------------

def bf16(x) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    x = _f32(x)
    y = np.empty(x.shape, dtype=np.uint16)
    _load().orc_bf16_array(x.size, _ptr(x), _ptr(y))
    return y


def bf16_scalar(x: float) -> int:
    return int(_load().orc_bf16(ctypes.c_float(x)))


def flat_sizes(numels: Sequence[int], N: int) -> tuple[int, int, int, int]:
    """(T, S, L, pad) of a FlatParameter over N ranks."""
    n = _i64_array(numels)
    out = np.zeros(4, dtype=np.int64)
    _load().orc_flat_sizes(len(n), _ptr(n), N, _ptr(out))
    return tuple(int(v) for v in out)


def flat_shard(params: Sequence[np.ndarray], N: int, k: int) -> np.ndarray:
    """Rank k's FlatParameter shard (k = -1: the whole padded flat buffer)."""
    params = [_f32(p).reshape(-1) for p in params]
    n = _i64_array(p.size for p in params)
    T, S, L, pad = flat_sizes(n, N)
    out = np.empty(L if k < 0 else S, dtype=np.float32)
    ptrs = _ptr_array(params)
    rc = _load().orc_flat_shard(len(params), _ptr(n), _ptr(ptrs), N, k, _ptr(out))
    if rc != 0:
        raise MemoryError("oracle flat_shard: allocation failed")
    return out


def flat_copyout(shapes: Sequence[Sequence[int]], gathered: np.ndarray) -> list[np.ndarray]:
    """Per-parameter bf16 tensors (uint16 bit patterns) from the gathered flat buffer."""
    g = _f32(gathered).reshape(-1)
    n = _i64_array(numel(s) for s in shapes)
    if int(n.sum()) > g.size:
        raise ValueError("gathered buffer shorter than the unit")
    outs = [np.empty(tuple(s), dtype=np.uint16) for s in shapes]
    ptrs = _ptr_array(outs)
    _load().orc_flat_copyout(len(outs), _ptr(n), _ptr(g), _ptr(ptrs))
    return outs


def rows_sizes(shapes: Sequence[Sequence[int]], N: int) -> int:
    """P_r: the per-rank segment length of an FSDP2 unit."""
    mr = [rows_of(s) for s in shapes]
    m = _i64_array(a for a, _ in mr)
    r = _i64_array(b for _, b in mr)
    out = np.zeros(1, dtype=np.int64)
    _load().orc_rows_sizes(len(mr), _ptr(m), _ptr(r), N, _ptr(out))
    return int(out[0])


def rows_shard(params: Sequence[np.ndarray], N: int, k: int) -> np.ndarray:
    """Rank k's FSDP2 segment (k = -1: all N segments, rank-major)."""
    shapes = [p.shape for p in params]
    flat = [_f32(p).reshape(-1) for p in params]
    mr = [rows_of(s) for s in shapes]
    m = _i64_array(a for a, _ in mr)
    r = _i64_array(b for _, b in mr)
    P_r = rows_sizes(shapes, N)
    out = np.empty(N * P_r if k < 0 else P_r, dtype=np.float32)
    ptrs = _ptr_array(flat)
    _load().orc_rows_shard(len(flat), _ptr(m), _ptr(r), _ptr(ptrs), N, k, _ptr(out))
    return out


def rows_copyout(shapes: Sequence[Sequence[int]], N: int, gathered: np.ndarray) -> list[np.ndarray]:
    g = _f32(gathered).reshape(-1)
    P_r = rows_sizes(shapes, N)
    if g.size < N * P_r:
        raise ValueError("gathered buffer shorter than N*P_r")
    mr = [rows_of(s) for s in shapes]
    m = _i64_array(a for a, _ in mr)
    r = _i64_array(b for _, b in mr)
    outs = [np.empty(tuple(s), dtype=np.uint16) for s in shapes]
    ptrs = _ptr_array(outs)
    _load().orc_rows_copyout(len(outs), _ptr(m), _ptr(r), N, _ptr(g), _ptr(ptrs))
    return outs


def grad_reduce(contribs: Sequence[np.ndarray], pre: float = 1.0, post: float = 1.0) -> np.ndarray:
    """fp32 reduction of N bf16 contributions (uint16 arrays of equal length)."""
    cs = [np.ascontiguousarray(c, dtype=np.uint16).reshape(-1) for c in contribs]
    if not cs:
        raise ValueError("need at least one contribution")
    length = cs[0].size
    if any(c.size != length for c in cs):
        raise ValueError("contributions differ in length")
    out = np.empty(length, dtype=np.float32)
    ptrs = _ptr_array(cs)
    _load().orc_grad_reduce(len(cs), length, _ptr(ptrs), pre, post, _ptr(out))
    return out


def adamw(p: np.ndarray, g: np.ndarray, m: np.ndarray, v: np.ndarray, *, lr: float,
          betas=(0.9, 0.999), eps: float = 1e-8, weight_decay: float = 0.0, step: int = 1,
          want_bf16: bool = False):
    """One AdamW step, in place on p, m, v (contiguous float32). Returns bf16(p) or None."""
    for a in (p, g, m, v):
        if a.dtype != np.float32 or not a.flags["C_CONTIGUOUS"]:
            raise ValueError("adamw wants contiguous float32 arrays")
    n = p.size
    if not (g.size == m.size == v.size == n):
        raise ValueError("adamw: size mismatch")
    pb = np.empty(n, dtype=np.uint16) if want_bf16 else None
    _load().orc_adamw(n, _ptr(p), _ptr(g), _ptr(m), _ptr(v), lr, betas[0], betas[1], eps,
                      weight_decay, step, _ptr(pb) if pb is not None else None)
    return pb


# --------------------------------------------------------------------------
# 16-bit layouts, hybrid / accumulating reduction, local accumulation
# --------------------------------------------------------------------------

def _u16(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.uint16)


def flat_shard_u16(params: Sequence[np.ndarray], N: int, k: int) -> np.ndarray:
    """FlatParameter shard of 16-bit (bf16 bit pattern) parameters (k = -1: all ranks)."""
    params = [_u16(p).reshape(-1) for p in params]
    n = _i64_array(p.size for p in params)
    T, S, L, pad = flat_sizes(n, N)
    out = np.empty(L if k < 0 else S, dtype=np.uint16)
    ptrs = _ptr_array(params)
    if _load().orc_flat_shard_u16(len(params), _ptr(n), _ptr(ptrs), N, k, _ptr(out)) != 0:
        raise MemoryError("oracle flat_shard_u16: allocation failed")
    return out


def flat_copyout_u16(shapes: Sequence[Sequence[int]], gathered: np.ndarray) -> list:
    g = _u16(gathered).reshape(-1)
    n = _i64_array(numel(s) for s in shapes)
    if int(n.sum()) > g.size:
        raise ValueError("gathered buffer shorter than the unit")
    outs = [np.empty(tuple(s), dtype=np.uint16) for s in shapes]
    ptrs = _ptr_array(outs)
    _load().orc_flat_copyout_u16(len(outs), _ptr(n), _ptr(g), _ptr(ptrs))
    return outs


def rows_shard_u16(params: Sequence[np.ndarray], N: int, k: int) -> np.ndarray:
    shapes = [p.shape for p in params]
    flat = [_u16(p).reshape(-1) for p in params]
    mr = [rows_of(s) for s in shapes]
    m = _i64_array(a for a, _ in mr)
    r = _i64_array(b for _, b in mr)
    P_r = rows_sizes(shapes, N)
    out = np.empty(N * P_r if k < 0 else P_r, dtype=np.uint16)
    ptrs = _ptr_array(flat)
    _load().orc_rows_shard_u16(len(flat), _ptr(m), _ptr(r), _ptr(ptrs), N, k, _ptr(out))
    return out


def rows_copyout_u16(shapes: Sequence[Sequence[int]], N: int, gathered: np.ndarray) -> list:
    g = _u16(gathered).reshape(-1)
    P_r = rows_sizes(shapes, N)
    if g.size < N * P_r:
        raise ValueError("gathered buffer shorter than N*P_r")
    mr = [rows_of(s) for s in shapes]
    m = _i64_array(a for a, _ in mr)
    r = _i64_array(b for _, b in mr)
    outs = [np.empty(tuple(s), dtype=np.uint16) for s in shapes]
    ptrs = _ptr_array(outs)
    _load().orc_rows_copyout_u16(len(outs), _ptr(m), _ptr(r), N, _ptr(g), _ptr(ptrs))
    return outs


def grad_reduce_ex(contribs: Sequence[np.ndarray], pre: float = 1.0, post: float = 1.0,
                   group: int = 0, out: np.ndarray = None) -> np.ndarray:
    """Reduction in groups of `group` consecutive ranks (0: one group of all N).  With `out`
    given, the fresh result is added to it in place (accumulation) and `out` is returned."""
    cs = [np.ascontiguousarray(c, dtype=np.uint16).reshape(-1) for c in contribs]
    N = len(cs)
    g = N if group == 0 else group
    if N == 0 or N % g != 0:
        raise ValueError("the group size must divide the number of contributions")
    length = cs[0].size
    if any(c.size != length for c in cs):
        raise ValueError("contributions differ in length")
    acc = out is not None
    if acc:
        if out.dtype != np.float32 or out.size != length or not out.flags["C_CONTIGUOUS"]:
            raise ValueError("out must be a contiguous float32 array of the contribution length")
        res = out
    else:
        res = np.empty(length, dtype=np.float32)
    ptrs = _ptr_array(cs)
    _load().orc_grad_reduce_ex(N, length, _ptr(ptrs), pre, post, g, 1 if acc else 0, _ptr(res))
    return res


def grad_accumulate(grad_bf16: np.ndarray, acc: np.ndarray, init: bool) -> np.ndarray:
    """acc = (init ? 0 : acc) + fp32(grad), in place on the float32 accumulator."""
    g = _u16(grad_bf16).reshape(-1)
    if acc.dtype != np.float32 or acc.size != g.size or not acc.flags["C_CONTIGUOUS"]:
        raise ValueError("acc must be a contiguous float32 array of the gradient's length")
    _load().orc_grad_accumulate(g.size, _ptr(g), _ptr(acc), 1 if init else 0)
    return acc


def grad_unscale(grad: np.ndarray, inv_scale: float, found_inf: np.ndarray) -> np.ndarray:
    """grad *= inv_scale in place (binary32); found_inf[0] = 1 if any input is not finite
    (never cleared here)."""
    if grad.dtype != np.float32 or not grad.flags["C_CONTIGUOUS"]:
        raise ValueError("grad must be a contiguous float32 array")
    if found_inf.dtype != np.float32 or found_inf.size != 1:
        raise ValueError("found_inf must be one float32")
    _load().orc_grad_unscale(grad.size, _ptr(grad), ctypes.c_float(inv_scale), _ptr(found_inf))
    return grad


def flat_sqnorm(shapes: Sequence[Sequence[int]], N: int, k: int, shard: np.ndarray) -> np.ndarray:
    """Per-parameter sums of squares (float64) of rank k's FLAT gradient shard."""
    g = _f32(shard).reshape(-1)
    n = _i64_array(numel(s) for s in shapes)
    T, S, L, pad = flat_sizes(n, N)
    if g.size != S or not 0 <= k < N:
        raise ValueError("shard must hold S elements of a rank in [0, N)")
    out = np.zeros(len(shapes), dtype=np.float64)
    _load().orc_flat_sqnorm(len(shapes), _ptr(n), N, k, _ptr(g), _ptr(out))
    return out


def rows_sqnorm(shapes: Sequence[Sequence[int]], N: int, k: int, seg: np.ndarray) -> np.ndarray:
    """Per-parameter sums of squares (float64) of rank k's FSDP2 gradient segment."""
    g = _f32(seg).reshape(-1)
    mr = [rows_of(s) for s in shapes]
    m = _i64_array(a for a, _ in mr)
    r = _i64_array(b for _, b in mr)
    if g.size != rows_sizes(shapes, N) or not 0 <= k < N:
        raise ValueError("seg must hold P_r elements of a rank in [0, N)")
    out = np.zeros(len(shapes), dtype=np.float64)
    _load().orc_rows_sqnorm(len(shapes), _ptr(m), _ptr(r), N, k, _ptr(g), _ptr(out))
    return out
