"""Device-side driver for one attention step over one in-flight batch.

PyTorch supplies device memory and the stream; every step of the path runs in the
library's HIP kernels through the C ABI.  A batch object only needs the attributes
of ``workloads.Batch`` (shape, lengths, block table, per-request value arrays in
the io representation); nothing here computes any part of the method.

The cache history (tokens cached before the step) is written by the library's own
append entry point with rotation off and no q: the history values count as
already rotated, and the append stores them in the cache format exactly as it
stores new tokens.
"""
from __future__ import annotations

import ctypes
import math

import numpy as np
import torch

from . import _lib as L

DTYPE_CODE = {"fp32": L.PKV_FP32, "bf16": L.PKV_BF16, "fp8_e4m3": L.PKV_FP8_E4M3, "int8": L.PKV_INT8}
TORCH_STORE = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp8_e4m3": torch.uint8, "int8": torch.uint8}
NUMPY_STORE = {"fp32": np.float32, "bf16": np.uint16, "fp8_e4m3": np.uint8, "int8": np.uint8}
# views of the stored bits with a same-width integer type (for downloads and sentinels)
TORCH_BITS = {"fp32": torch.int32, "bf16": torch.int16, "fp8_e4m3": torch.uint8, "int8": torch.uint8}


def make_desc(shape, rope: bool = True, max_num_tokens: int | None = None) -> L.pkv_attn_desc:
    d = L.pkv_attn_desc()
    d.num_heads = shape.num_heads
    d.num_kv_heads = shape.num_kv_heads
    d.head_dim = shape.head_dim
    d.tokens_per_block = shape.tokens_per_block
    d.io_dtype = DTYPE_CODE[shape.io_dtype]
    d.kv_dtype = DTYPE_CODE[shape.kv_dtype]
    style = {"neox": L.PKV_ROPE_NEOX, "gptj": L.PKV_ROPE_GPTJ, "none": L.PKV_ROPE_NONE}[
        getattr(shape, "rope_style", "neox")]
    d.rope_style = style if rope else L.PKV_ROPE_NONE
    d.rotary_dim = shape.rotary_dim
    d.softmax_scale = 0.0
    d.k_scale_quant_orig = shape.k_scale
    d.v_scale_quant_orig = shape.v_scale
    d.max_num_tokens = shape.max_num_tokens if max_num_tokens is None else max_num_tokens
    return d


def io_to_device(arr: np.ndarray, io_dtype: str, device) -> torch.Tensor:
    """[rows, heads, D] io-representation array -> dense [rows, heads*D] device tensor."""
    rows = arr.shape[0]
    flat = np.ascontiguousarray(arr.reshape(rows, -1))
    if io_dtype == "bf16":
        return torch.from_numpy(flat.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(flat).to(device)


def stored_to_host(t: torch.Tensor, fmt: str) -> np.ndarray:
    """Device tensor in format ``fmt`` -> numpy array of its stored representation."""
    bits = t.view(TORCH_BITS[fmt]).cpu().numpy()
    return bits.view(NUMPY_STORE[fmt])


class _Lengths:
    """Host and device copies of a batch's lengths and block table (kept alive)."""

    def __init__(self, types, ctx, seq, table, num_pool_blocks, device):
        self.types = np.ascontiguousarray(types, np.int32)
        self.ctx = np.ascontiguousarray(ctx, np.int32)
        self.seq = np.ascontiguousarray(seq, np.int32)
        self.table = np.ascontiguousarray(table, np.int32)
        self.d_ctx = torch.from_numpy(self.ctx).to(device)
        self.d_seq = torch.from_numpy(self.seq).to(device)
        self.d_table = torch.from_numpy(self.table).to(device)
        b = L.pkv_batch_desc()
        b.num_requests = int(self.types.shape[0])
        b.num_tokens = int(self.ctx.sum())
        ctx_rows = self.ctx[self.types == L.PKV_REQ_CONTEXT]
        b.max_context_length = int(ctx_rows.max()) if ctx_rows.size else 0
        b.max_blocks_per_seq = int(self.table.shape[1])
        b.host_request_types = self.types.ctypes.data
        b.host_context_lengths = self.ctx.ctypes.data
        b.host_sequence_lengths = self.seq.ctypes.data
        b.context_lengths = self.d_ctx.data_ptr()
        b.sequence_lengths = self.d_seq.data_ptr()
        b.kv_cache_block_offsets = self.d_table.data_ptr()
        b.host_kv_cache_block_offsets = self.table.ctypes.data
        b.num_pool_blocks = int(num_pool_blocks)
        self.desc = b


class PagedStep:
    """Buffers and ABI calls for one batch: history fill, append, attention."""

    def __init__(self, batch, device="cuda", sentinel: bool = True, fill_history: bool = True,
                 history_tokens_per_call: int = 65536, rope_table: np.ndarray | None = None):
        """``rope_table``: optional fp64 [max_pos, rotary_dim/2, 2] cos/sin table handed to the
        append instead of the one the library's pkv_rope_cos_sin fills."""
        self.batch = batch
        self.device = torch.device(device)
        sh = batch.shape
        self.shape = sh
        self.desc = make_desc(sh)
        self.lengths = _Lengths(batch.request_types, batch.context_lengths, batch.sequence_lengths,
                                batch.block_table, batch.num_pool_blocks, self.device)
        self.bdesc = self.lengths.desc
        H, Hkv, D, T = sh.num_heads, sh.num_kv_heads, sh.head_dim, sh.tokens_per_block
        N = batch.num_tokens
        self.N = N
        self.q = io_to_device(batch.packed("new_q"), sh.io_dtype, self.device) if N else \
            torch.empty((0, H * D), dtype=TORCH_STORE[sh.io_dtype], device=self.device)
        self.k = io_to_device(batch.packed("new_k"), sh.io_dtype, self.device) if N else \
            torch.empty((0, Hkv * D), dtype=TORCH_STORE[sh.io_dtype], device=self.device)
        self.v = io_to_device(batch.packed("new_v"), sh.io_dtype, self.device) if N else \
            torch.empty((0, Hkv * D), dtype=TORCH_STORE[sh.io_dtype], device=self.device)
        self.q_out = torch.empty((max(N, 1), H * D), dtype=TORCH_STORE[sh.io_dtype], device=self.device)
        self.out_fp8_scale = float(getattr(sh, "out_fp8_scale", 0.0))
        out_dtype = torch.uint8 if self.out_fp8_scale > 0 else TORCH_STORE[sh.io_dtype]
        self.out = torch.empty((max(N, 1), H * D), dtype=out_dtype, device=self.device)
        self.pool = torch.empty((batch.num_pool_blocks, 2, T, Hkv, D), dtype=TORCH_STORE[sh.kv_dtype],
                                device=self.device)
        if sentinel:
            self.pool.view(torch.uint8).fill_(0xFF)
        self.max_pos = max(int(batch.sequence_lengths.max()) if batch.num_requests else 1, 1)
        self.rot = sh.rot_dim
        if rope_table is not None:
            tab = np.ascontiguousarray(rope_table, dtype=np.float64)
            if tab.ndim != 3 or tab.shape[0] < self.max_pos or tab.shape[1:] != (self.rot // 2, 2):
                raise ValueError(f"rope_table of shape {tab.shape} does not cover ({self.max_pos}, {self.rot // 2}, 2)")
            self.max_pos = int(tab.shape[0])
            self.rope = torch.from_numpy(tab).to(self.device)
        else:
            self.rope = torch.empty((self.max_pos, self.rot // 2, 2), dtype=torch.float64, device=self.device)
            L.check(L.pkv_rope_cos_sin(float(sh.rope_theta), self.rot, self.max_pos, self.rope.data_ptr(),
                                       self.stream))
        self.norm = None
        if getattr(sh, "qk_norm", "none") != "none":
            prm = batch.norm_params()
            self.norm_tensors = {n: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(self.device)
                                 for n, a in prm.items()}
            nrm = L.pkv_qk_norm()
            nrm.kind = {"rms": L.PKV_NORM_RMS, "layer": L.PKV_NORM_LAYER}[sh.qk_norm]
            nrm.eps = sh.norm_eps
            nrm.q_weight = self.norm_tensors["q_weight"].data_ptr()
            nrm.k_weight = self.norm_tensors["k_weight"].data_ptr()
            nrm.q_bias = self.norm_tensors["q_bias"].data_ptr()
            nrm.k_bias = self.norm_tensors["k_bias"].data_ptr()
            self.norm = nrm
        self.tree = None
        if getattr(batch, "tree", False):
            if self.norm is not None or self.out_fp8_scale > 0:
                raise ValueError("draft trees go through pkv_append_rope_tree / pkv_attention_forward_tree, "
                                 "which take no qk norm and write no fp8 output")
            off, mask = batch.spec_inputs()
            self.tree_host = (np.ascontiguousarray(off, np.int32), np.ascontiguousarray(mask, np.uint32))
            self.tree_dev = (torch.from_numpy(self.tree_host[0]).to(self.device),
                             torch.from_numpy(self.tree_host[1].view(np.int32)).to(self.device))
            tr = L.pkv_spec_tree()
            tr.host_position_offsets = self.tree_host[0].ctypes.data
            tr.position_offsets = self.tree_dev[0].data_ptr()
            tr.host_packed_mask = self.tree_host[1].ctypes.data
            tr.packed_mask = self.tree_dev[1].data_ptr()
            self.tree = tr
        self.ws_bytes = L.pkv_workspace_size_for_batch(self.desc, self.bdesc)
        self.ws = torch.empty((max(self.ws_bytes, 256),), dtype=torch.uint8, device=self.device)
        if fill_history:
            self.fill_history(history_tokens_per_call)

    @property
    def stream(self) -> int:
        return torch.cuda.current_stream(self.device).cuda_stream

    def fill_history(self, tokens_per_call: int = 65536):
        b, sh = self.batch, self.shape
        past = b.past_lengths
        reqs = [r for r in range(b.num_requests) if past[r] > 0]
        desc = make_desc(sh, rope=False, max_num_tokens=2 ** 31 - 1)
        i = 0
        while i < len(reqs):
            group, tot = [], 0
            while i < len(reqs) and (not group or tot + int(past[reqs[i]]) <= tokens_per_call):
                group.append(reqs[i])
                tot += int(past[reqs[i]])
                i += 1
            lens = _Lengths(np.zeros(len(group), np.int32), past[group], past[group], b.block_table[group],
                            b.num_pool_blocks, self.device)
            k = io_to_device(np.concatenate([b.hist_k(r) for r in group]), sh.io_dtype, self.device)
            v = io_to_device(np.concatenate([b.hist_v(r) for r in group]), sh.io_dtype, self.device)
            L.check(L.pkv_append_rope(desc, lens.desc, None, 0, k.data_ptr(), v.data_ptr(), k.shape[1],
                                      None, 0, None, self.pool.data_ptr(), self.stream))
            torch.cuda.synchronize(self.device)
            del k, v, lens

    def append(self) -> int:
        if self.tree is not None:
            return L.pkv_append_rope_tree(self.desc, self.bdesc, self.tree, self.q.data_ptr(), self.q.shape[1],
                                          self.k.data_ptr(), self.v.data_ptr(), self.k.shape[1],
                                          self.rope.data_ptr(), self.max_pos, self.q_out.data_ptr(),
                                          self.pool.data_ptr(), self.stream)
        if self.norm is not None:
            return L.pkv_append_qknorm_rope(self.desc, self.bdesc, self.norm, self.q.data_ptr(), self.q.shape[1],
                                            self.k.data_ptr(), self.v.data_ptr(), self.k.shape[1],
                                            self.rope.data_ptr(), self.max_pos, self.q_out.data_ptr(),
                                            self.pool.data_ptr(), self.stream)
        return L.pkv_append_rope(self.desc, self.bdesc, self.q.data_ptr(), self.q.shape[1], self.k.data_ptr(),
                                 self.v.data_ptr(), self.k.shape[1], self.rope.data_ptr(), self.max_pos,
                                 self.q_out.data_ptr(), self.pool.data_ptr(), self.stream)

    def forward(self) -> int:
        if self.tree is not None:
            return L.pkv_attention_forward_tree(self.desc, self.bdesc, self.tree, self.q_out.data_ptr(),
                                                self.q_out.shape[1], self.pool.data_ptr(), self.out.data_ptr(),
                                                self.ws.data_ptr(), self.ws_bytes, self.stream)
        if self.out_fp8_scale > 0:
            return L.pkv_attention_forward_fp8_out(self.desc, self.bdesc, self.q_out.data_ptr(), self.q_out.shape[1],
                                                   self.pool.data_ptr(), self.out_fp8_scale, self.out.data_ptr(),
                                                   self.ws.data_ptr(), self.ws_bytes, self.stream)
        return L.pkv_attention_forward(self.desc, self.bdesc, self.q_out.data_ptr(), self.q_out.shape[1],
                                       self.pool.data_ptr(), self.out.data_ptr(), self.ws.data_ptr(),
                                       self.ws_bytes, self.stream)

    def step(self):
        L.check(self.append())
        L.check(self.forward())

    # ---- downloads (stored representations) --------------------------------
    def q_out_host(self) -> np.ndarray:
        sh = self.shape
        return stored_to_host(self.q_out[:self.N], sh.io_dtype).reshape(self.N, sh.num_heads, sh.head_dim)

    def out_host(self) -> np.ndarray:
        sh = self.shape
        fmt = "fp8_e4m3" if self.out_fp8_scale > 0 else sh.io_dtype
        return stored_to_host(self.out[:self.N], fmt).reshape(self.N, sh.num_heads, sh.head_dim)

    def pool_host(self) -> np.ndarray:
        return stored_to_host(self.pool, self.shape.kv_dtype)

    def rope_host(self) -> np.ndarray:
        return self.rope.cpu().numpy()
