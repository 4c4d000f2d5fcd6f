"""Gated linear-attention token mixer for AMD MI355X (gfx950): the
bidirectional mixer and its backward pass, the projection prologue fused
with it, its block-causal form with a carried state, and the gated softmax
anchor attention of the hybrid's other layers.

The compute path is libgla.so (C ABI in include/gla.h, HIP kernels in
csrc/); this package is its thin ctypes binding.
"""
from .gla import (  # noqa: F401
    EXPORTS,
    GatedLinearAttention,
    GlaError,
    RopeTables,
    alloc_workspace,
    alloc_workspace_backward,
    alloc_workspace_blocks,
    alloc_workspace_proj,
    alloc_workspace_softmax,
    gla_backward,
    gla_backward_check,
    gla_backward_saved,
    gla_backward_saved_check,
    gla_backward_saved_ws,
    gla_backward_workspace_bytes,
    gla_backward_ws,
    gla_forward,
    gla_forward_blocks,
    gla_forward_blocks_check,
    gla_forward_blocks_ws,
    gla_forward_check,
    gla_forward_noalloc,
    gla_forward_proj,
    gla_forward_proj_check,
    gla_forward_proj_ws,
    gla_forward_ws,
    gla_output_ws,
    gla_proj_workspace_bytes,
    gla_rope_create,
    gla_rope_destroy,
    gla_rope_fill_host,
    gla_rope_table_floats,
    gla_softmax_forward,
    gla_softmax_forward_check,
    gla_softmax_forward_ws,
    gla_softmax_workspace_bytes,
    gla_state,
    gla_state_ws,
    gla_stream_probe,
    gla_strerror,
    gla_workspace_bytes,
    gla_workspace_bytes_blocks,
    gated_linear_attention,
    load_library,
)
