"""sharded_fsdp_flatten_amd: the per-rank FSDP data path as HIP kernels for MI355X.

The product is the C-ABI library ``libfsdpflat.so`` (declared in
``include/fsdp_flatten.h``); this package builds it (``build.py``) and binds it
with ctypes under the same names (``binding.py``).
"""
from .binding import (  # noqa: F401
    FSDP_ALL_RANKS,
    FSDP_FLAT,
    FSDP_REDUCE_AUTO,
    FSDP_REDUCE_SWEEP,
    FSDP_REDUCE_TILES,
    FSDP_ROWS,
    FsdpError,
    Unit,
    fsdp_abi_version,
    fsdp_adam_shard,
    fsdp_cast_to_bf16,
    fsdp_flatten_shard,
    fsdp_flatten_shard_bf16,
    fsdp_grad_accumulate,
    fsdp_grad_reduce_shard,
    fsdp_grad_reduce_shard_ex,
    fsdp_grad_reduce_workspace,
    fsdp_grad_sqnorm,
    fsdp_grad_sqnorm_noalloc,
    fsdp_grad_sqnorm_workspace,
    fsdp_grad_unscale,
    fsdp_last_error,
    fsdp_status_string,
    fsdp_unflatten_copyout,
    fsdp_unflatten_copyout_bf16,
    fsdp_unit_create,
    fsdp_unit_destroy,
    fsdp_unit_info,
    fsdp_unit_param_offset,
    fsdp_unit_recv_pitch,
    load,
)
