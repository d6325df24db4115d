"""ctypes binding of ``libpkv.so`` (argument marshalling only).

Every function keeps the C name from ``include/pkv.h`` and takes device buffers
as integer addresses and streams as integer handles.  Loading fails loudly when
the library has not been built: there is no other implementation to fall back on.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# PKV_LIB_PATH selects another build of the same library (for A/B measurements)
LIB_PATH = os.environ.get("PKV_LIB_PATH") or os.path.join(HERE, "libpkv.so")

PKV_OK = 0
PKV_ERR_INVALID_ARG = -1
PKV_ERR_UNSUPPORTED = -2
PKV_ERR_ORDER = -3
PKV_ERR_CHUNK_ALIGN = -4
PKV_ERR_BUDGET = -5
PKV_ERR_BLOCK_RANGE = -6
PKV_ERR_WORKSPACE = -7
PKV_ERR_HIP = -8

PKV_FP32, PKV_BF16, PKV_FP8_E4M3, PKV_INT8 = 0, 1, 2, 3
PKV_SCRATCH_BYTES = 64 << 20        # the per-GPU scratch array of pkv_attention_forward_noalloc
PKV_REQ_CONTEXT, PKV_REQ_GENERATION = 0, 1
PKV_ROPE_NONE, PKV_ROPE_NEOX, PKV_ROPE_GPTJ = 0, 1, 2
PKV_NORM_NONE, PKV_NORM_RMS, PKV_NORM_LAYER = 0, 1, 2

_i32p = ctypes.POINTER(ctypes.c_int32)


class pkv_attn_desc(ctypes.Structure):
    _fields_ = [
        ("num_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("tokens_per_block", ctypes.c_int32),
        ("io_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("rope_style", ctypes.c_int32),
        ("rotary_dim", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("k_scale_quant_orig", ctypes.c_float),
        ("v_scale_quant_orig", ctypes.c_float),
        ("max_num_tokens", ctypes.c_int32),
    ]


class pkv_batch_desc(ctypes.Structure):
    _fields_ = [
        ("num_requests", ctypes.c_int32),
        ("num_tokens", ctypes.c_int32),
        ("max_context_length", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("host_request_types", ctypes.c_void_p),
        ("host_context_lengths", ctypes.c_void_p),
        ("host_sequence_lengths", ctypes.c_void_p),
        ("context_lengths", ctypes.c_void_p),
        ("sequence_lengths", ctypes.c_void_p),
        ("kv_cache_block_offsets", ctypes.c_void_p),
        ("host_kv_cache_block_offsets", ctypes.c_void_p),
        ("num_pool_blocks", ctypes.c_int64),
    ]


class pkv_qk_norm(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("eps", ctypes.c_float),
        ("q_weight", ctypes.c_void_p),
        ("k_weight", ctypes.c_void_p),
        ("q_bias", ctypes.c_void_p),
        ("k_bias", ctypes.c_void_p),
    ]


class pkv_spec_tree(ctypes.Structure):
    _fields_ = [
        ("host_position_offsets", ctypes.c_void_p),
        ("position_offsets", ctypes.c_void_p),
        ("host_packed_mask", ctypes.c_void_p),
        ("packed_mask", ctypes.c_void_p),
    ]


class PkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"pkv status {status}: {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(the HIP library is the only implementation)")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
        D, Bt = ctypes.POINTER(pkv_attn_desc), ctypes.POINTER(pkv_batch_desc)
        L.pkv_abi_version.restype = i32
        L.pkv_last_error.restype = ctypes.c_char_p
        L.pkv_workspace_size.argtypes = [D, i32, i32]
        L.pkv_workspace_size.restype = sz
        L.pkv_workspace_size_for_batch.argtypes = [D, Bt]
        L.pkv_workspace_size_for_batch.restype = sz
        L.pkv_rope_cos_sin.argtypes = [ctypes.c_double, i32, i32, vp, vp]
        L.pkv_rope_cos_sin.restype = i32
        L.pkv_append_rope.argtypes = [D, Bt, vp, i64, vp, vp, i64, vp, i32, vp, vp, vp]
        L.pkv_append_rope.restype = i32
        L.pkv_append_qknorm_rope.argtypes = [D, Bt, ctypes.POINTER(pkv_qk_norm), vp, i64, vp, vp, i64, vp, i32,
                                             vp, vp, vp]
        L.pkv_append_qknorm_rope.restype = i32
        L.pkv_attention_forward.argtypes = [D, Bt, vp, i64, vp, vp, vp, sz, vp]
        L.pkv_attention_forward_fp8_out.argtypes = [D, Bt, vp, i64, vp, ctypes.c_float, vp, vp, sz, vp]
        L.pkv_attention_forward_fp8_out.restype = i32
        L.pkv_attention_forward.restype = i32
        L.pkv_attention_forward_noalloc.argtypes = [D, Bt, vp, i64, vp, vp, vp]
        L.pkv_attention_forward_noalloc.restype = i32
        Tr = ctypes.POINTER(pkv_spec_tree)
        L.pkv_append_rope_tree.argtypes = [D, Bt, Tr, vp, i64, vp, vp, i64, vp, i32, vp, vp, vp]
        L.pkv_append_rope_tree.restype = i32
        L.pkv_attention_forward_tree.argtypes = [D, Bt, Tr, vp, i64, vp, vp, vp, sz, vp]
        L.pkv_attention_forward_tree.restype = i32
        L.pkv_kernel_timing_enable.argtypes = [i32]
        L.pkv_kernel_timing_enable.restype = i32
        L.pkv_set_decode_workgroups.argtypes = [i32]
        L.pkv_set_decode_workgroups.restype = i32
        L.pkv_set_coschedule.argtypes = [i32]
        L.pkv_set_coschedule.restype = i32
        L.pkv_kernel_timings.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_float), i32]
        L.pkv_kernel_timings.restype = i32
        _lib = L
    return _lib


def check(status: int) -> int:
    if status != PKV_OK:
        raise PkvError(status, pkv_last_error())
    return status


def pkv_abi_version() -> int:
    return lib().pkv_abi_version()


def pkv_last_error() -> str:
    return lib().pkv_last_error().decode()


def pkv_workspace_size(desc, max_num_requests: int, max_seq_len: int) -> int:
    return lib().pkv_workspace_size(ctypes.byref(desc), max_num_requests, max_seq_len)


def pkv_workspace_size_for_batch(desc, batch) -> int:
    return lib().pkv_workspace_size_for_batch(ctypes.byref(desc), ctypes.byref(batch))


def pkv_rope_cos_sin(base: float, rotary_dim: int, max_pos: int, cos_sin: int, stream: int) -> int:
    return lib().pkv_rope_cos_sin(base, rotary_dim, max_pos, cos_sin, stream)


def pkv_append_rope(desc, batch, q, q_row_stride, k, v, kv_row_stride, rope_cos_sin, rope_max_pos,
                    q_out, kv_pool, stream) -> int:
    return lib().pkv_append_rope(ctypes.byref(desc), ctypes.byref(batch), q, q_row_stride, k, v, kv_row_stride,
                                 rope_cos_sin, rope_max_pos, q_out, kv_pool, stream)


def pkv_append_qknorm_rope(desc, batch, norm, q, q_row_stride, k, v, kv_row_stride, rope_cos_sin, rope_max_pos,
                           q_out, kv_pool, stream) -> int:
    return lib().pkv_append_qknorm_rope(ctypes.byref(desc), ctypes.byref(batch),
                                        ctypes.byref(norm) if norm is not None else None, q, q_row_stride, k, v,
                                        kv_row_stride, rope_cos_sin, rope_max_pos, q_out, kv_pool, stream)


def pkv_attention_forward(desc, batch, q, q_row_stride, kv_pool, out, workspace, workspace_bytes, stream) -> int:
    return lib().pkv_attention_forward(ctypes.byref(desc), ctypes.byref(batch), q, q_row_stride, kv_pool, out,
                                       workspace, workspace_bytes, stream)


def pkv_attention_forward_fp8_out(desc, batch, q, q_row_stride, kv_pool, out_scale_quant_orig, out, workspace,
                                  workspace_bytes, stream) -> int:
    return lib().pkv_attention_forward_fp8_out(ctypes.byref(desc), ctypes.byref(batch), q, q_row_stride, kv_pool,
                                               out_scale_quant_orig, out, workspace, workspace_bytes, stream)


def pkv_attention_forward_noalloc(desc, batch, q, q_row_stride, kv_pool, out, stream) -> int:
    return lib().pkv_attention_forward_noalloc(ctypes.byref(desc), ctypes.byref(batch), q, q_row_stride, kv_pool,
                                               out, stream)


def pkv_append_rope_tree(desc, batch, tree, q, q_row_stride, k, v, kv_row_stride, rope_cos_sin, rope_max_pos,
                         q_out, kv_pool, stream) -> int:
    return lib().pkv_append_rope_tree(ctypes.byref(desc), ctypes.byref(batch),
                                      ctypes.byref(tree) if tree is not None else None, q, q_row_stride, k, v,
                                      kv_row_stride, rope_cos_sin, rope_max_pos, q_out, kv_pool, stream)


def pkv_attention_forward_tree(desc, batch, tree, q, q_row_stride, kv_pool, out, workspace, workspace_bytes,
                               stream) -> int:
    return lib().pkv_attention_forward_tree(ctypes.byref(desc), ctypes.byref(batch),
                                            ctypes.byref(tree) if tree is not None else None, q, q_row_stride,
                                            kv_pool, out, workspace, workspace_bytes, stream)



def pkv_set_decode_workgroups(n: int) -> int:
    """Cap the decode split pass's workgroups at n (0: default, < 0: query); returns the old cap."""
    return lib().pkv_set_decode_workgroups(int(n))


def pkv_set_coschedule(on: int) -> int:
    """Mixed batches in one launch (1, default) or context then generation (0); < 0 queries.
    Returns the previous setting."""
    return lib().pkv_set_coschedule(int(on))


def pkv_kernel_timing_enable(on) -> int:
    """0 / False: off; 1 / True: every kernel launch; 2: every phase (append, context
    attention, generation attention as one span)."""
    return lib().pkv_kernel_timing_enable(int(on))


def pkv_kernel_timings(max_entries: int = 4096) -> list[tuple[str, float]]:
    names = (ctypes.c_char_p * max_entries)()
    ms = (ctypes.c_float * max_entries)()
    n = lib().pkv_kernel_timings(names, ms, max_entries)
    if n < 0:
        raise PkvError(n, pkv_last_error())
    return [(names[i].decode(), float(ms[i])) for i in range(min(n, max_entries))]
