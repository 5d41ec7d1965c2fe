"""MI355X-native tensor-parallel MLP shard (column-parallel linear + local
GeLU/SwiGLU, row-parallel linear to an fp32 partial, on-device partial sum),
the shard's backward pass, the attention of one head shard (QKV
column-parallel by heads, the attention core, the output projection as the
row-parallel linear), and a whole pre-LayerNorm transformer block of p shards
with its two reductions.

This package is a thin ctypes binding over ``libtpmlp.so`` (declared in
``include/tpmlp.h``, with a measurement aid in ``include/tpmlp_calib.h``): it
turns torch tensors into pointers, sizes and leading dimensions, and the
current torch stream into a ``hipStream_t``.  Every step of
the computation runs in the library's HIP kernels; if the library is missing,
every call raises.  torch is used for device memory and streams only.
"""
from __future__ import annotations

from ._binding import (  # noqa: F401
    ACT,
    DTYPE,
    TpError,
    library,
    library_path,
    tp_abi_version,
    tp_attention,
    tp_backward_workspace_bytes,
    tp_block_simulated,
    tp_block_workspace_bytes,
    tp_calib_hbm_read,
    tp_calib_mfma_bf16,
    tp_col_linear,
    tp_col_linear_train,
    tp_mlp_shard,
    tp_mlp_shard_backward,
    tp_mlp_shard_noalloc,
    tp_mlp_simulated,
    tp_partial_sum,
    tp_qkv_linear,
    tp_qkv_workspace_bytes,
    tp_residual_layernorm,
    tp_row_linear,
    tp_shard_bounds,
    tp_workspace_bytes,
    workspace,
)

__all__ = [
    "ACT", "DTYPE", "TpError", "library", "library_path", "tp_abi_version", "tp_attention",
    "tp_backward_workspace_bytes", "tp_block_simulated", "tp_block_workspace_bytes",
    "tp_calib_hbm_read", "tp_calib_mfma_bf16", "tp_col_linear", "tp_col_linear_train",
    "tp_mlp_shard", "tp_mlp_shard_backward", "tp_mlp_shard_noalloc", "tp_mlp_simulated", "tp_partial_sum", "tp_qkv_linear",
    "tp_qkv_workspace_bytes", "tp_residual_layernorm", "tp_row_linear", "tp_shard_bounds", "tp_workspace_bytes",
    "workspace",
]
