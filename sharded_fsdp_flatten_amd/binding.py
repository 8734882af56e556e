"""ctypes binding of libfsdpflat.so, with the C ABI's names.

Argument marshalling only: shapes become the ndims/dims arrays, tensors become
device pointers (``data_ptr()``), the stream defaults to torch's current stream.
Every step of the data path runs in the library's HIP kernels; there is no
Python or CPU fallback, and importing the binding fails loudly when the library
has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

FSDP_FLAT = 1
FSDP_ROWS = 2
FSDP_ALL_RANKS = -1
FSDP_MAX_NDIM = 8
ABI_VERSION = 3  # FSDP_ABI_VERSION of include/fsdp_flatten.h this binding marshals for

STATUS_NAMES = {0: "FSDP_OK", 1: "FSDP_E_ARG", 2: "FSDP_E_RANGE", 3: "FSDP_E_ALIGN",
                4: "FSDP_E_OVERFLOW", 5: "FSDP_E_NOMEM", 6: "FSDP_E_HIP",
                7: "FSDP_E_UNSUPPORTED"}

# The in-tree library; FSDP_FLATTEN_LIB may name another build of the same ABI.
LIB_PATH = os.environ.get("FSDP_FLATTEN_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libfsdpflat.so")


class FsdpError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        self.status_name = STATUS_NAMES.get(status, "FSDP_E_UNKNOWN")
        super().__init__("%s: %s" % (self.status_name, message))


class fsdp_unit_sizes(ctypes.Structure):
    _fields_ = [("layout", ctypes.c_int32), ("n_params", ctypes.c_int32),
                ("N", ctypes.c_int64), ("T", ctypes.c_int64), ("S", ctypes.c_int64),
                ("L", ctypes.c_int64), ("pad", ctypes.c_int64), ("valid", ctypes.c_int64),
                ("bytes_per_rank", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {k: getattr(self, k) for k, _ in self._fields_}


class fsdp_adamw_cfg(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double),
                ("step", ctypes.c_int64)]


class fsdp_reduce_opts(ctypes.Structure):
    _fields_ = [("pre_divide", ctypes.c_float), ("post_divide", ctypes.c_float),
                ("group", ctypes.c_int32), ("accumulate", ctypes.c_int32),
                ("kernel", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_len", ctypes.c_int64)]


# fsdp_reduce_kernel
FSDP_REDUCE_AUTO = 0
FSDP_REDUCE_TILES = 1
FSDP_REDUCE_SWEEP = 2
_REDUCE_KERNELS = {"auto": FSDP_REDUCE_AUTO, "tiles": FSDP_REDUCE_TILES, "sweep": FSDP_REDUCE_SWEEP}


_lib = None
_vp = ctypes.c_void_p


def load() -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libfsdpflat.so is not built; run __graft_entry__.build() or "
                           "`python -m sharded_fsdp_flatten_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    st = ctypes.c_int32
    lib.fsdp_abi_version.argtypes = []
    lib.fsdp_abi_version.restype = ctypes.c_int32
    if lib.fsdp_abi_version() != ABI_VERSION:
        raise RuntimeError("%s implements ABI version %d; this binding needs %d (rebuild it)"
                           % (LIB_PATH, lib.fsdp_abi_version(), ABI_VERSION))
    lib.fsdp_last_error.argtypes = []
    lib.fsdp_last_error.restype = ctypes.c_char_p
    lib.fsdp_status_string.argtypes = [ctypes.c_int32]
    lib.fsdp_status_string.restype = ctypes.c_char_p
    lib.fsdp_unit_create.argtypes = [ctypes.c_int32, ctypes.c_int32, _vp, _vp, ctypes.c_int32,
                                     ctypes.POINTER(_vp)]
    lib.fsdp_unit_create.restype = st
    lib.fsdp_unit_destroy.argtypes = [_vp]
    lib.fsdp_unit_destroy.restype = st
    lib.fsdp_unit_info.argtypes = [_vp, ctypes.c_int32, ctypes.POINTER(fsdp_unit_sizes)]
    lib.fsdp_unit_info.restype = st
    lib.fsdp_unit_param_offset.argtypes = [_vp, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64)]
    lib.fsdp_unit_param_offset.restype = st
    lib.fsdp_unit_recv_pitch.argtypes = [_vp, ctypes.POINTER(ctypes.c_int64)]
    lib.fsdp_unit_recv_pitch.restype = st
    lib.fsdp_flatten_shard.argtypes = [_vp, _vp, ctypes.c_int32, _vp, _vp]
    lib.fsdp_flatten_shard.restype = st
    lib.fsdp_unflatten_copyout.argtypes = [_vp, _vp, _vp, _vp]
    lib.fsdp_unflatten_copyout.restype = st
    lib.fsdp_grad_reduce_shard.argtypes = [_vp, _vp, ctypes.c_float, ctypes.c_float, _vp, _vp]
    lib.fsdp_grad_reduce_shard.restype = st
    lib.fsdp_adam_shard.argtypes = [_vp, _vp, _vp, _vp, _vp, ctypes.POINTER(fsdp_adamw_cfg), _vp,
                                    _vp]
    lib.fsdp_adam_shard.restype = st
    lib.fsdp_cast_to_bf16.argtypes = [_vp, ctypes.c_int32, _vp, _vp, _vp]
    lib.fsdp_cast_to_bf16.restype = st
    lib.fsdp_unflatten_copyout_bf16.argtypes = [_vp, _vp, _vp, _vp]
    lib.fsdp_unflatten_copyout_bf16.restype = st
    lib.fsdp_flatten_shard_bf16.argtypes = [_vp, _vp, ctypes.c_int32, _vp, _vp]
    lib.fsdp_flatten_shard_bf16.restype = st
    lib.fsdp_grad_reduce_shard_ex.argtypes = [_vp, _vp, ctypes.POINTER(fsdp_reduce_opts), _vp, _vp]
    lib.fsdp_grad_reduce_shard_ex.restype = st
    lib.fsdp_grad_reduce_workspace.argtypes = [_vp, ctypes.POINTER(fsdp_reduce_opts),
                                               ctypes.POINTER(ctypes.c_int64)]
    lib.fsdp_grad_reduce_workspace.restype = st
    lib.fsdp_grad_accumulate.argtypes = [_vp, ctypes.c_int32, _vp, _vp, ctypes.c_int32, _vp]
    lib.fsdp_grad_accumulate.restype = st
    lib.fsdp_grad_unscale.argtypes = [_vp, ctypes.c_int32, _vp, ctypes.c_float, _vp, _vp]
    lib.fsdp_grad_unscale.restype = st
    lib.fsdp_grad_sqnorm_workspace.argtypes = [_vp, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64)]
    lib.fsdp_grad_sqnorm_workspace.restype = st
    lib.fsdp_grad_sqnorm_noalloc.argtypes = [_vp, ctypes.c_int32, _vp, _vp, _vp]
    lib.fsdp_grad_sqnorm_noalloc.restype = st
    lib.fsdp_grad_sqnorm.argtypes = [_vp, ctypes.c_int32, _vp, _vp, ctypes.c_int64, _vp, _vp]
    lib.fsdp_grad_sqnorm.restype = st
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        raise FsdpError(status, load().fsdp_last_error().decode())


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _is_tensor(x) -> bool:
    return hasattr(x, "data_ptr") and hasattr(x, "dtype")


def _addr(x, want=None) -> int:
    """Device address of a tensor (checked on the GPU, contiguous and of dtype `want`), or an
    int taken as a device address."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    if _is_tensor(x):
        if want is not None and str(x.dtype) not in want:
            raise TypeError("expected a tensor of dtype %s, got %s" % (" or ".join(want), x.dtype))
        if not getattr(x, "is_cuda", False):
            # a host address would reach the kernels and fault the GPU
            raise ValueError("tensors passed to the library must be on the GPU, got one on %s"
                             % x.device)
        if not x.is_contiguous():
            raise ValueError("tensors passed to the library must be contiguous")
        return int(x.data_ptr())
    raise TypeError("expected a tensor, an int address or None, got %r" % type(x))


def _need(t, n: int, name: str, exact: bool = False) -> None:
    """Tensors must hold what the kernels will touch (the C ABI sees only pointers)."""
    if _is_tensor(t):
        have = t.numel()
        if (have != n) if exact else (have < n):
            raise ValueError("%s holds %d elements, the unit needs %s%d"
                             % (name, have, "" if exact else "at least ", n))


def _ptr_table(items, want) -> ctypes.Array:
    arr = (ctypes.c_void_p * max(1, len(items)))()
    for i, t in enumerate(items):
        arr[i] = _addr(t, want) or None
    return arr


_F32 = ("torch.float32",)
_BF16 = ("torch.bfloat16", "torch.int16", "torch.uint16")


def _stream(stream, *tensors) -> int:
    if stream is not None:
        return int(stream) if isinstance(stream, int) else int(stream.cuda_stream)
    for t in tensors:
        if _is_tensor(t) and getattr(t, "is_cuda", False):
            import torch
            return int(torch.cuda.current_stream(t.device).cuda_stream)
    return 0


# ---------------------------------------------------------------------------
# the ABI
# ---------------------------------------------------------------------------

def fsdp_abi_version() -> int:
    return int(load().fsdp_abi_version())


def fsdp_last_error() -> str:
    return load().fsdp_last_error().decode()


def fsdp_status_string(status: int) -> str:
    return load().fsdp_status_string(status).decode()


class Unit:
    """Owner of an ``fsdp_unit*`` plan handle (freed on garbage collection)."""

    def __init__(self, handle: int, layout: int, shapes, N: int):
        self.handle = handle
        self.layout = layout
        self.shapes = [tuple(int(d) for d in s) for s in shapes]
        self.N = N
        self.numels = []
        for s in self.shapes:
            n = 1
            for d in s:
                n *= d
            self.numels.append(n)
        sizes = fsdp_unit_sizes()
        _check(load().fsdp_unit_info(handle, FSDP_ALL_RANKS, ctypes.byref(sizes)))
        self.S = int(sizes.S)
        self.L = int(sizes.L)

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.fsdp_unit_destroy(self.handle)
            self.handle = None

    def info(self, k: int = FSDP_ALL_RANKS) -> dict:
        return fsdp_unit_info(self, k)

    def offset(self, i: int) -> int:
        return fsdp_unit_param_offset(self, i)

    @property
    def recv_pitch(self) -> int:
        """Recommended row pitch (elements) of a stacked [N, pitch] bf16 receive buffer."""
        return fsdp_unit_recv_pitch(self)


def fsdp_unit_create(layout: int, shapes: Sequence[Sequence[int]], N: int) -> Unit:
    lib = load()
    ndims = (ctypes.c_int32 * max(1, len(shapes)))(*[len(s) for s in shapes])
    flat = [int(d) for s in shapes for d in s]
    dims = (ctypes.c_int64 * max(1, len(flat)))(*flat)
    out = ctypes.c_void_p()
    _check(lib.fsdp_unit_create(layout, len(shapes), ctypes.cast(ndims, _vp),
                                ctypes.cast(dims, _vp), N, ctypes.byref(out)))
    return Unit(out.value, layout, shapes, N)


def fsdp_unit_destroy(unit: Unit) -> None:
    if unit.handle:
        _check(load().fsdp_unit_destroy(unit.handle))
        unit.handle = None


def fsdp_unit_info(unit: Unit, k: int = FSDP_ALL_RANKS) -> dict:
    s = fsdp_unit_sizes()
    _check(load().fsdp_unit_info(unit.handle, k, ctypes.byref(s)))
    return s.as_dict()


def fsdp_unit_param_offset(unit: Unit, i: int) -> int:
    off = ctypes.c_int64()
    _check(load().fsdp_unit_param_offset(unit.handle, i, ctypes.byref(off)))
    return int(off.value)


def fsdp_unit_recv_pitch(unit: Unit) -> int:
    pitch = ctypes.c_int64()
    _check(load().fsdp_unit_recv_pitch(unit.handle, ctypes.byref(pitch)))
    return int(pitch.value)


def fsdp_flatten_shard(unit: Unit, params: Sequence, k: int, shard, stream=None) -> None:
    """Write rank k's shard (k = FSDP_ALL_RANKS: every rank, gathered layout)."""
    if len(params) != len(unit.shapes):
        raise ValueError("need %d parameters, got %d" % (len(unit.shapes), len(params)))
    for i, p in enumerate(params):
        _need(p, unit.numels[i], "params[%d]" % i, exact=True)
    _need(shard, unit.L if k == FSDP_ALL_RANKS else unit.S, "shard")
    table = _ptr_table(params, _F32)
    _check(load().fsdp_flatten_shard(unit.handle, ctypes.cast(table, _vp), k,
                                     _addr(shard, _F32) or None, _stream(stream, shard, *params)))


def fsdp_unflatten_copyout(unit: Unit, gathered, outs: Sequence, stream=None) -> None:
    """Copy the gathered fp32 unit out into per-parameter bf16 tensors."""
    if len(outs) != len(unit.shapes):
        raise ValueError("need %d outputs, got %d" % (len(unit.shapes), len(outs)))
    for i, o in enumerate(outs):
        _need(o, unit.numels[i], "outs[%d]" % i, exact=True)
    _need(gathered, unit.L, "gathered")
    table = _ptr_table(outs, _BF16)
    _check(load().fsdp_unflatten_copyout(unit.handle, _addr(gathered, _F32) or None,
                                         ctypes.cast(table, _vp),
                                         _stream(stream, gathered, *outs)))


def fsdp_grad_reduce_shard(unit: Unit, contribs: Sequence, pre_divide: float, post_divide: float,
                           grad_shard, stream=None) -> None:
    """fp32 reduction of N bf16 contributions (each S elements) into grad_shard."""
    if len(contribs) != unit.N:
        raise ValueError("need exactly N = %d contributions, got %d" % (unit.N, len(contribs)))
    for r, c in enumerate(contribs):
        _need(c, unit.S, "contribs[%d]" % r)
    _need(grad_shard, unit.S, "grad_shard")
    table = _ptr_table(contribs, _BF16)
    _check(load().fsdp_grad_reduce_shard(unit.handle, ctypes.cast(table, _vp),
                                         float(pre_divide), float(post_divide),
                                         _addr(grad_shard, _F32) or None,
                                         _stream(stream, grad_shard, *contribs)))


def fsdp_adam_shard(unit: Unit, param, grad, exp_avg, exp_avg_sq, *, lr: float,
                    betas=(0.9, 0.999), eps: float = 1e-8, weight_decay: float = 0.0,
                    step: int = 1, param_bf16=None, stream=None) -> None:
    """One AdamW step on the rank's aligned (param, grad, exp_avg, exp_avg_sq) shard."""
    for name, t in (("param", param), ("grad", grad), ("exp_avg", exp_avg),
                    ("exp_avg_sq", exp_avg_sq), ("param_bf16", param_bf16)):
        _need(t, unit.S, name)
    cfg = fsdp_adamw_cfg(float(lr), float(betas[0]), float(betas[1]), float(eps),
                         float(weight_decay), int(step))
    _check(load().fsdp_adam_shard(unit.handle, _addr(param, _F32) or None,
                                  _addr(grad, _F32) or None, _addr(exp_avg, _F32) or None,
                                  _addr(exp_avg_sq, _F32) or None, ctypes.byref(cfg),
                                  _addr(param_bf16, _BF16) or None,
                                  _stream(stream, param, grad, exp_avg, exp_avg_sq)))


def fsdp_cast_to_bf16(unit: Unit, k: int, src, dst, stream=None) -> None:
    """bf16(src) over rank k's shard (S elements) or, k = FSDP_ALL_RANKS, the L-element layout."""
    n = unit.L if k == FSDP_ALL_RANKS else unit.S
    _need(src, n, "src")
    _need(dst, n, "dst")
    _check(load().fsdp_cast_to_bf16(unit.handle, k, _addr(src, _F32) or None,
                                    _addr(dst, _BF16) or None, _stream(stream, src, dst)))


def fsdp_unflatten_copyout_bf16(unit: Unit, gathered, outs: Sequence, stream=None) -> None:
    """Copy a gathered bf16 unit out into per-parameter bf16 tensors (cast before gather)."""
    if len(outs) != len(unit.shapes):
        raise ValueError("need %d outputs, got %d" % (len(unit.shapes), len(outs)))
    for i, o in enumerate(outs):
        _need(o, unit.numels[i], "outs[%d]" % i, exact=True)
    _need(gathered, unit.L, "gathered")
    table = _ptr_table(outs, _BF16)
    _check(load().fsdp_unflatten_copyout_bf16(unit.handle, _addr(gathered, _BF16) or None,
                                              ctypes.cast(table, _vp),
                                              _stream(stream, gathered, *outs)))


def fsdp_flatten_shard_bf16(unit: Unit, params: Sequence, k: int, shard, stream=None) -> None:
    """fsdp_flatten_shard for bf16 tensors (k = FSDP_ALL_RANKS on gradients: the copy-in)."""
    if len(params) != len(unit.shapes):
        raise ValueError("need %d tensors, got %d" % (len(unit.shapes), len(params)))
    for i, p in enumerate(params):
        _need(p, unit.numels[i], "params[%d]" % i, exact=True)
    _need(shard, unit.L if k == FSDP_ALL_RANKS else unit.S, "shard")
    table = _ptr_table(params, _BF16)
    _check(load().fsdp_flatten_shard_bf16(unit.handle, ctypes.cast(table, _vp), k,
                                          _addr(shard, _BF16) or None,
                                          _stream(stream, shard, *params)))


def _reduce_opts(pre_divide, post_divide, group, accumulate, kernel, workspace=None):
    if kernel not in _REDUCE_KERNELS:
        raise ValueError("kernel must be one of %s" % ", ".join(_REDUCE_KERNELS))
    ws_len = workspace.numel() if _is_tensor(workspace) else 0
    return fsdp_reduce_opts(float(pre_divide), float(post_divide), int(group),
                            1 if accumulate else 0, _REDUCE_KERNELS[kernel], 0,
                            _addr(workspace, _F32) or None, ws_len)


def fsdp_grad_reduce_workspace(unit: Unit, *, group: int = 0, accumulate: bool = False) -> int:
    """fp32 elements of workspace fsdp_grad_reduce_shard_ex needs for these options (0: none)."""
    n = ctypes.c_int64()
    opts = _reduce_opts(1.0, 1.0, group, accumulate, "auto")
    _check(load().fsdp_grad_reduce_workspace(unit.handle, ctypes.byref(opts), ctypes.byref(n)))
    return int(n.value)


def fsdp_grad_reduce_shard_ex(unit: Unit, contribs: Sequence, pre_divide: float,
                              post_divide: float, grad_shard, *, group: int = 0,
                              accumulate: bool = False, kernel: str = "auto", workspace=None,
                              stream=None) -> None:
    """Reduction in hybrid groups of `group` ranks, optionally accumulating into grad_shard;
    `kernel` is "auto", "tiles" or "sweep"; `workspace` is an fp32 tensor of at least
    fsdp_grad_reduce_workspace(...) elements, or None when that is 0."""
    if len(contribs) != unit.N:
        raise ValueError("need exactly N = %d contributions, got %d" % (unit.N, len(contribs)))
    for r, c in enumerate(contribs):
        _need(c, unit.S, "contribs[%d]" % r)
    _need(grad_shard, unit.S, "grad_shard")
    table = _ptr_table(contribs, _BF16)
    opts = _reduce_opts(pre_divide, post_divide, group, accumulate, kernel, workspace)
    _check(load().fsdp_grad_reduce_shard_ex(unit.handle, ctypes.cast(table, _vp),
                                            ctypes.byref(opts), _addr(grad_shard, _F32) or None,
                                            _stream(stream, grad_shard, *contribs)))


def fsdp_grad_accumulate(unit: Unit, k: int, grad, acc, init: bool, stream=None) -> None:
    """acc = (init ? 0 : acc) + fp32(grad) over rank k's shard or (FSDP_ALL_RANKS) all L."""
    n = unit.L if k == FSDP_ALL_RANKS else unit.S
    _need(grad, n, "grad")
    _need(acc, n, "acc")
    _check(load().fsdp_grad_accumulate(unit.handle, k, _addr(grad, _BF16) or None,
                                       _addr(acc, _F32) or None, 1 if init else 0,
                                       _stream(stream, grad, acc)))


_F64 = ("torch.float64",)


def fsdp_grad_unscale(unit: Unit, k: int, grad, inv_scale: float, found_inf, stream=None) -> None:
    """grad *= inv_scale over rank k's shard or (FSDP_ALL_RANKS) all L; found_inf (one
    float, or None to scale only) is set to 1 if any input was not finite, never cleared."""
    n = unit.L if k == FSDP_ALL_RANKS else unit.S
    _need(grad, n, "grad")
    if found_inf is not None:
        _need(found_inf, 1, "found_inf")
    _check(load().fsdp_grad_unscale(unit.handle, k, _addr(grad, _F32) or None, inv_scale,
                                    _addr(found_inf, _F32) or None, _stream(stream, grad)))


def fsdp_grad_sqnorm_workspace(unit: Unit, k: int) -> int:
    """Doubles of workspace fsdp_grad_sqnorm needs for rank k."""
    n = ctypes.c_int64()
    _check(load().fsdp_grad_sqnorm_workspace(unit.handle, k, ctypes.byref(n)))
    return int(n.value)


def fsdp_grad_sqnorm(unit: Unit, k: int, grad, out, workspace, stream=None) -> None:
    """out[i] = sum of squares (float64) of parameter i's elements in rank k's shard."""
    need = fsdp_grad_sqnorm_workspace(unit, k)
    _need(grad, unit.S, "grad")
    _need(out, len(unit.shapes), "out")
    _need(workspace, need, "workspace")
    ws_len = workspace.numel() if _is_tensor(workspace) else need
    _check(load().fsdp_grad_sqnorm(unit.handle, k, _addr(grad, _F32) or None,
                                   _addr(workspace, _F64) or None, ws_len,
                                   _addr(out, _F64) or None, _stream(stream, grad)))


def fsdp_grad_sqnorm_noalloc(unit: Unit, k: int, grad, out, stream=None) -> None:
    """fsdp_grad_sqnorm with the partial sums in the library's own per-GPU scratch (no
    workspace; calls that overlap on one GPU race)."""
    _need(grad, unit.S, "grad")
    _need(out, len(unit.shapes), "out")
    _check(load().fsdp_grad_sqnorm_noalloc(unit.handle, k, _addr(grad, _F32) or None,
                                           _addr(out, _F64) or None, _stream(stream, grad)))


ABI_FUNCTIONS = ["fsdp_abi_version", "fsdp_last_error", "fsdp_status_string", "fsdp_unit_create",
                 "fsdp_unit_destroy", "fsdp_unit_info", "fsdp_unit_param_offset", "fsdp_unit_recv_pitch",
                 "fsdp_flatten_shard", "fsdp_unflatten_copyout", "fsdp_grad_reduce_shard",
                 "fsdp_adam_shard", "fsdp_cast_to_bf16", "fsdp_unflatten_copyout_bf16",
                 "fsdp_flatten_shard_bf16", "fsdp_grad_reduce_shard_ex", "fsdp_grad_reduce_workspace",
                 "fsdp_grad_accumulate",
                 "fsdp_grad_unscale", "fsdp_grad_sqnorm_workspace", "fsdp_grad_sqnorm",
                 "fsdp_grad_sqnorm_noalloc"]
