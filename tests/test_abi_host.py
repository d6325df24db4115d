"""The C ABI on the host: the library loads, exports every declared symbol, and
rejects every invalid argument before touching the GPU (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

from paged_kv_gqa_rope_amd import _lib as L
from workloads import synth as W

HERE = os.path.dirname(os.path.abspath(__file__))
HEADER = os.path.join(os.path.dirname(HERE), "include", "pkv.h")

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH), reason="libpkv.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(pkv_[a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 8, names
    lib = L.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert L.pkv_abi_version() == 1


class HostBatch:
    """Host arrays + a batch desc whose 'device' pointers are host addresses.
    Validation never dereferences device pointers, so this is safe on the CPU."""

    def __init__(self, types, ctx, seq, table, pool_blocks, with_host_table=True, max_ctx=None):
        self.types = np.asarray(types, np.int32)
        self.ctx = np.asarray(ctx, np.int32)
        self.seq = np.asarray(seq, np.int32)
        self.table = (np.ascontiguousarray(np.asarray(table, np.int32).reshape(len(types), -1)) if len(types)
                      else np.zeros((0, 1), np.int32))
        b = L.pkv_batch_desc()
        b.num_requests = len(types)
        b.num_tokens = int(self.ctx.sum())
        cm = self.ctx[self.types == 0]
        b.max_context_length = int(cm.max()) if cm.size else 0 if max_ctx is None else max_ctx
        if max_ctx is not None:
            b.max_context_length = max_ctx
        b.max_blocks_per_seq = self.table.shape[1]
        for f, arr in (("host_request_types", self.types), ("host_context_lengths", self.ctx),
                       ("host_sequence_lengths", self.seq), ("context_lengths", self.ctx),
                       ("sequence_lengths", self.seq), ("kv_cache_block_offsets", self.table)):
            setattr(b, f, arr.ctypes.data)
        b.host_kv_cache_block_offsets = self.table.ctypes.data if with_host_table else None
        b.num_pool_blocks = pool_blocks
        self.desc = b


def desc_for(shape=W.SHAPES[4], **over):
    from paged_kv_gqa_rope_amd.harness import make_desc
    d = make_desc(shape)
    for k, v in over.items():
        setattr(d, k, v)
    return d


BUF = np.zeros(1 << 16, np.uint8)
P = (BUF.ctypes.data + 255) // 256 * 256          # an aligned host address used as a stand-in


def append(desc, hb, q=P, qs=None, k=P, v=P, kvs=None, rope=P, max_pos=10 ** 6, q_out=P, pool=P):
    qs = desc.num_heads * desc.head_dim if qs is None else qs
    kvs = desc.num_kv_heads * desc.head_dim if kvs is None else kvs
    return L.pkv_append_rope(desc, hb.desc, q, qs, k, v, kvs, rope, max_pos, q_out, pool, None)


def forward(desc, hb, q=P, qs=None, pool=P, out=P, ws=P, ws_bytes=1 << 40):
    qs = desc.num_heads * desc.head_dim if qs is None else qs
    return L.pkv_attention_forward(desc, hb.desc, q, qs, pool, out, ws, ws_bytes, None)


def ok_batch():
    # 1 chunked context request (64 cached + 70 new) then 2 generation requests
    return HostBatch([0, 1, 1], [70, 1, 1], [134, 6, 131], [[0, 1, 2], [3, -1, -1], [4, 5, 6]], 8)


def expect(code, rc):
    assert rc == code, (rc, L.pkv_last_error())
    assert L.pkv_last_error() != ""


def test_context_after_generation_is_an_ordering_error():
    hb = HostBatch([1, 0], [1, 5], [6, 5], [[0], [1]], 4)
    expect(L.PKV_ERR_ORDER, append(desc_for(), hb))
    expect(L.PKV_ERR_ORDER, forward(desc_for(), hb))


def test_ragged_earlier_chunk_is_a_chunk_alignment_error():
    hb = HostBatch([0], [10], [40], [[0]], 4)          # 30 cached tokens, T = 64
    expect(L.PKV_ERR_CHUNK_ALIGN, append(desc_for(), hb))
    expect(L.PKV_ERR_CHUNK_ALIGN, forward(desc_for(), hb))


def test_token_budget():
    hb = HostBatch([0], [9000], [9000], [list(range(141))], 141)
    expect(L.PKV_ERR_BUDGET, append(desc_for(), hb))
    hb2 = HostBatch([0], [100], [100], [[0, 1]], 2)
    expect(L.PKV_ERR_BUDGET, forward(desc_for(max_num_tokens=99), hb2))


def test_block_table_range():
    expect(L.PKV_ERR_BLOCK_RANGE, append(desc_for(), HostBatch([1], [1], [200], [[0, 1, 2]], 8)))   # needs 4 blocks
    expect(L.PKV_ERR_BLOCK_RANGE, append(desc_for(), HostBatch([1], [1], [100], [[0, 9]], 8)))      # id 9 >= 8
    expect(L.PKV_ERR_BLOCK_RANGE, forward(desc_for(), HostBatch([1], [1], [100], [[-1, 0]], 8)))
    # without a host table copy the device-side checks are the only guard: validation passes
    hb = HostBatch([1], [1], [100], [[0, 9]], 8, with_host_table=False)
    assert L.pkv_workspace_size_for_batch(desc_for(), hb.desc) >= 0


def test_invalid_arguments():
    hb = ok_batch()
    expect(L.PKV_ERR_INVALID_ARG, append(desc_for(num_kv_heads=7), hb))             # 64 % 7
    expect(L.PKV_ERR_INVALID_ARG, append(desc_for(), hb, k=None))
    expect(L.PKV_ERR_INVALID_ARG, append(desc_for(), hb, q_out=None))                # q without q_out
    expect(L.PKV_ERR_INVALID_ARG, append(desc_for(), hb, q=P + 2))                    # misaligned
    expect(L.PKV_ERR_INVALID_ARG, append(desc_for(), hb, qs=64 * 128 - 8))            # stride < row
    expect(L.PKV_ERR_INVALID_ARG, append(desc_for(), hb, kvs=8 * 128 + 1))            # row starts misaligned
    expect(L.PKV_ERR_INVALID_ARG, append(desc_for(), hb, rope=None))
    expect(L.PKV_ERR_INVALID_ARG, append(desc_for(), hb, max_pos=133))                # position 133 not covered
    expect(L.PKV_ERR_INVALID_ARG, forward(desc_for(), hb, out=None))
    expect(L.PKV_ERR_INVALID_ARG, forward(desc_for(softmax_scale=float("nan")), hb))
    bad = ok_batch(); bad.desc.num_tokens = 71
    expect(L.PKV_ERR_INVALID_ARG, append(desc_for(), bad))
    bad = ok_batch(); bad.desc.max_context_length = 69
    expect(L.PKV_ERR_INVALID_ARG, forward(desc_for(), bad))
    expect(L.PKV_ERR_INVALID_ARG, append(desc_for(), HostBatch([0], [5], [4], [[0]], 1)))   # S < n
    expect(L.PKV_ERR_INVALID_ARG, append(desc_for(), HostBatch([2], [1], [4], [[0]], 1)))   # type 2
    expect(L.PKV_ERR_INVALID_ARG, append(desc_for(), HostBatch([0], [0], [0], [[0]], 1)))   # empty context
    fp8 = desc_for(W.SHAPES[5], k_scale_quant_orig=0.0)
    expect(L.PKV_ERR_INVALID_ARG, append(fp8, ok_batch()))
    int8 = desc_for(W.SHAPES[5], kv_dtype=L.PKV_INT8, v_scale_quant_orig=float("inf"))
    expect(L.PKV_ERR_INVALID_ARG, forward(int8, ok_batch()))
    expect(L.PKV_ERR_UNSUPPORTED, append(desc_for(kv_dtype=4), ok_batch()))


def test_unsupported_configurations():
    hb = ok_batch()
    expect(L.PKV_ERR_UNSUPPORTED, append(desc_for(head_dim=96), hb))
    expect(L.PKV_ERR_UNSUPPORTED, append(desc_for(tokens_per_block=8), hb))
    expect(L.PKV_ERR_UNSUPPORTED, append(desc_for(tokens_per_block=48), hb))
    expect(L.PKV_ERR_UNSUPPORTED, append(desc_for(io_dtype=L.PKV_FP8_E4M3), hb))
    expect(L.PKV_ERR_UNSUPPORTED, append(desc_for(io_dtype=L.PKV_INT8), hb))
    expect(L.PKV_ERR_UNSUPPORTED, append(desc_for(rope_style=7), hb))
    expect(L.PKV_ERR_UNSUPPORTED, append(desc_for(rotary_dim=40), hb))
    # generation requests carry at most 64 new tokens (a token and its draft tokens)
    expect(L.PKV_ERR_UNSUPPORTED, forward(desc_for(), HostBatch([1], [65], [70], [[0, 1]], 2)))


def test_qk_norm_arguments():
    hb = ok_batch()
    d = desc_for()

    def call(kind=L.PKV_NORM_RMS, eps=1e-6, qw=P, kw=P, qb=None, kb=None, q=P, q_out=P, desc=d):
        n = L.pkv_qk_norm()
        n.kind, n.eps, n.q_weight, n.k_weight, n.q_bias, n.k_bias = kind, eps, qw, kw, qb, kb
        qs, kvs = desc.num_heads * desc.head_dim, desc.num_kv_heads * desc.head_dim
        return L.pkv_append_qknorm_rope(desc, hb.desc, n, q, qs, P, P, kvs, P, 10 ** 6, q_out, P, None)

    expect(L.PKV_ERR_INVALID_ARG, call(kind=3))
    expect(L.PKV_ERR_INVALID_ARG, call(eps=-1.0))
    expect(L.PKV_ERR_INVALID_ARG, call(eps=float("inf")))
    expect(L.PKV_ERR_INVALID_ARG, call(kw=None))
    expect(L.PKV_ERR_INVALID_ARG, call(qw=None))                       # q given without its weights
    expect(L.PKV_ERR_INVALID_ARG, call(qw=P + 4))                      # misaligned
    expect(L.PKV_ERR_INVALID_ARG, call(kind=L.PKV_NORM_LAYER, qb=P + 8))
    # 256 + 32 heads exceed the per-token limit of the norm pre-pass
    expect(L.PKV_ERR_UNSUPPORTED, call(desc=desc_for(num_heads=256, num_kv_heads=32)))
    # the same arguments are rejected by the shared validation first
    expect(L.PKV_ERR_INVALID_ARG, call(q_out=None))


def test_fp8_output_scale():
    hb = ok_batch()
    d = desc_for()
    qs = d.num_heads * d.head_dim
    for s in (0.0, -1.0, float("inf"), float("nan"), 1e-45):     # 1e-45: reciprocal overflows
        expect(L.PKV_ERR_INVALID_ARG,
               L.pkv_attention_forward_fp8_out(d, hb.desc, P, qs, P, s, P, P, 1 << 40, None))
    expect(L.PKV_ERR_INVALID_ARG, L.pkv_attention_forward_fp8_out(d, hb.desc, P, qs, P, 1.0, None, P, 1 << 40, None))


def test_empty_batch_is_a_no_op():
    hb = HostBatch([], [], [], np.zeros((0, 1)), 1)
    assert append(desc_for(), hb, q=None, q_out=None, k=None, v=None, pool=None) == L.PKV_OK
    assert forward(desc_for(), hb, q=None, pool=None, out=None, ws=None, ws_bytes=0) == L.PKV_OK


def test_workspace_bounds_cover_every_batch():
    rng = np.random.default_rng(0)
    for k in (2, 4, 5):
        d = desc_for(W.SHAPES[k])
        for _ in range(30):
            B = int(rng.integers(1, 40))
            seq = rng.integers(65, 40000, B).astype(np.int32)
            gen_n = rng.integers(1, 65, B) if rng.random() < 0.5 else np.ones(B, np.int64)  # with draft tokens
            T = d.tokens_per_block
            width = int((seq.max() + T - 1) // T)
            hb = HostBatch([1] * B, gen_n.tolist(), seq, np.zeros((B, width)), 1, with_host_table=False)
            d.max_num_tokens = 1 << 20
            need = L.pkv_workspace_size_for_batch(d, hb.desc)
            bound = L.pkv_workspace_size(d, B, int(seq.max()))
            assert need <= bound, (k, B, need, bound)
            if need > 0:
                expect(L.PKV_ERR_WORKSPACE, forward(d, hb, ws_bytes=need - 1))
                expect(L.PKV_ERR_WORKSPACE, forward(d, hb, ws=None))


def test_noalloc_rejects_a_batch_beyond_its_scratch_before_any_launch():
    """The scratch entry point checks the batch's need against its array's size on the host."""
    d = L.pkv_attn_desc()
    d.num_heads, d.num_kv_heads, d.head_dim, d.tokens_per_block = 64, 8, 128, 64
    d.io_dtype = d.kv_dtype = L.PKV_BF16
    d.rope_style, d.max_num_tokens = L.PKV_ROPE_NEOX, 1 << 20
    B, S = 2048, 4096
    hb = HostBatch([1] * B, [1] * B, [S] * B, np.arange(B * 64, dtype=np.int32), B * 64)
    need = L.pkv_workspace_size_for_batch(d, hb.desc)
    assert need > L.PKV_SCRATCH_BYTES
    rc = L.pkv_attention_forward_noalloc(d, hb.desc, 16, 128 * 64, 16, 16, None)
    assert rc == L.PKV_ERR_WORKSPACE and "scratch" in L.pkv_last_error()


def test_decode_workgroup_cap_set_and_query():
    assert L.pkv_set_decode_workgroups(-1) == 0          # default
    assert L.pkv_set_decode_workgroups(7) == 0
    assert L.pkv_set_decode_workgroups(-1) == 7
    assert L.pkv_set_decode_workgroups(0) == 7
    assert L.pkv_set_decode_workgroups(-1) == 0


def test_coschedule_switch_set_and_query():
    assert L.pkv_set_coschedule(-1) == 1                 # default: mixed batches in one launch
    assert L.pkv_set_coschedule(0) == 1
    assert L.pkv_set_coschedule(-1) == 0
    assert L.pkv_set_coschedule(5) == 0                  # any nonzero value turns it on
    assert L.pkv_set_coschedule(-1) == 1


def test_timed_launch_wrappers_return(tmp_path):
    """Every launch goes through the timing wrappers (a phase span around per-kernel
    records); with timing off, at either level or without a device they must return:
    run in a child process under a time limit."""
    import subprocess
    import sys
    code = (
        "import ctypes\n"
        "from paged_kv_gqa_rope_amd import _lib as L\n"
        "buf = (ctypes.c_double * (8 * 32 * 2))()\n"
        "rc = L.lib().pkv_rope_cos_sin(1e4, 64, 8, ctypes.addressof(buf), None)\n"
        "assert rc in (L.PKV_OK, L.PKV_ERR_HIP), rc\n"
        "print('returned', rc)\n"
    )
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=120)
    assert res.returncode == 0 and "returned" in res.stdout, res.stderr[-2000:]


def _tree(off, mask_words, dev=True):
    off = np.ascontiguousarray(off, np.int32)
    mask = np.ascontiguousarray(np.asarray(mask_words, np.uint32).reshape(-1, 2))
    t = L.pkv_spec_tree()
    t.host_position_offsets = off.ctypes.data
    t.position_offsets = P if dev else None
    t.host_packed_mask = mask.ctypes.data
    t.packed_mask = P if dev else None
    return t, (off, mask)


def test_draft_tree_inputs_are_validated_on_the_host():
    # one context request (5 tokens), then generation requests with 3 and 2 tokens
    hb = HostBatch([0, 1, 1], [5, 3, 2], [5, 13, 12], [[0], [1], [2]], 4)
    good_off = [0, 0, 0, 0, 0, 0, 1, 1, 0, 1]
    good_mask = [0, 0] * 5 + [1, 0, 3, 0, 5, 0, 1, 0, 3, 0]   # token 2 of request 1 is a sibling of token 1
    bad = [
        ([0] * 5 + [0, 1, 3, 0, 1], good_mask, "position offset"),      # offset 3 >= n = 3
        ([0] * 5 + [0, 1, 1, 0, -1], good_mask, "position offset"),     # negative
        (good_off, [0, 0] * 5 + [1, 0, 1, 0, 5, 0, 1, 0, 3, 0], "own mask bit"),   # token 1 lacks bit 1
        (good_off, [0, 0] * 5 + [1, 0, 3, 0, 13, 0, 1, 0, 3, 0], "past n"),        # bit 3 with n = 3
        (good_off, [0, 0] * 5 + [1, 0, 3, 0, 5, 1, 1, 0, 3, 0], "past n"),         # high word
    ]
    d = desc_for()
    for off, mask, what in bad:
        t, keep = _tree(off, mask)
        rc = L.pkv_append_rope_tree(d, hb.desc, t, P, d.num_heads * d.head_dim, P, P, d.num_kv_heads * d.head_dim,
                                    P, 10 ** 6, P, P, None)
        expect(L.PKV_ERR_INVALID_ARG, rc)
        assert what in L.pkv_last_error(), (what, L.pkv_last_error())
        rc = L.pkv_attention_forward_tree(d, hb.desc, t, P, d.num_heads * d.head_dim, P, P, P, 1 << 40, None)
        expect(L.PKV_ERR_INVALID_ARG, rc)
    t, keep = _tree(good_off, good_mask, dev=False)                      # device copies missing
    expect(L.PKV_ERR_INVALID_ARG, L.pkv_attention_forward_tree(d, hb.desc, t, P, d.num_heads * d.head_dim, P, P, P,
                                                               1 << 40, None))
    expect(L.PKV_ERR_INVALID_ARG, L.pkv_attention_forward_tree(d, hb.desc, None, P, d.num_heads * d.head_dim, P, P,
                                                               P, 1 << 40, None))
