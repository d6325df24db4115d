"""Paged-KV GQA + RoPE attention for AMD MI355X (gfx950).

The product is the C-ABI library ``libpkv.so`` (HIP kernels, see ``include/pkv.h``);
``_lib`` is its ctypes binding and ``harness`` drives one step over a batch with
PyTorch-owned device buffers.
"""
from . import _lib  # noqa: F401
from ._lib import (  # noqa: F401
    PkvError, pkv_abi_version, pkv_append_rope, pkv_append_rope_tree, pkv_attention_forward,
    pkv_attention_forward_tree, pkv_kernel_timing_enable,
    pkv_kernel_timings, pkv_last_error, pkv_rope_cos_sin, pkv_set_coschedule, pkv_set_decode_workgroups, pkv_workspace_size,
    pkv_workspace_size_for_batch,
)
