"""GPU parity: the HIP path through the C ABI against the CPU oracle, at sizes the
oracle finishes in seconds (several blocks, ragged tails, every workload shape)."""
import dataclasses

import numpy as np
import pytest
import torch

from batch_util import as_crafted, copy_values, crafted
from oracle import codecs as C
from oracle import rope as OR
from oracle import step as O
from parity_util import assert_bits_equal, bits_of, compare_attention
from workloads import synth as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def H():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from paged_kv_gqa_rope_amd import _lib, harness
    _lib.lib()                       # raises if the library was not built
    return harness


def case(*a):
    print("CASE", *a, flush=True)


def sentinel(fmt):
    return int(np.iinfo(O.BITS[fmt]).max)


def run_step(H, batch, **kw):
    st = H.PagedStep(batch, **kw)
    st.step()
    torch.cuda.synchronize()
    return st


def test_rope_table_matches_oracle(H):
    from paged_kv_gqa_rope_amd import _lib as L
    for base, rot, max_pos in [(1e4, 64, 64), (1e4, 128, 4200), (5e5, 128, 33000), (5e5, 32, 100)]:
        case("rope", base, rot, max_pos)
        t = torch.empty((max_pos, rot // 2, 2), dtype=torch.float64, device="cuda")
        L.check(L.pkv_rope_cos_sin(base, rot, max_pos, t.data_ptr(), torch.cuda.current_stream().cuda_stream))
        g = t.cpu().numpy()
        c, s = OR.neox_tables(base, rot, max_pos)
        # angles reach 3.3e4 rad, where one ulp of theta_j moves the angle by ~4e-12
        assert np.max(np.abs(g[..., 0] - c)) <= 1e-11
        assert np.max(np.abs(g[..., 1] - s)) <= 1e-11
        exact = np.mean((g[..., 0] == c) & (g[..., 1] == s))
        print(f"rope base={base} rot={rot} max_pos={max_pos}: {exact:.4f} of entries bit-identical")


@pytest.mark.parametrize("k", W.SMALL_WORKLOADS)
def test_small_workload_append_is_bit_exact(H, k):
    b = W.small_workload(k)
    case("append", b.label, b.shape.name)
    st = run_step(H, b)
    ref_q = np.concatenate([O.append_request(b, r, O.tables(b))[0] for r in range(b.num_requests)])
    assert_bits_equal(st.q_out_host(), ref_q, "q_out")
    want = O.expected_pool(b, sentinel(b.shape.kv_dtype))
    assert_bits_equal(bits_of(st.pool_host()), want, "pool (history + new tokens + untouched sentinel)")


@pytest.mark.parametrize("k", W.SMALL_WORKLOADS)
def test_small_workload_attention_matches_oracle(H, k):
    b = W.small_workload(k)
    case("attention", b.label, b.shape.name)
    st = run_step(H, b)
    ref = O.run(b)
    stats = compare_attention(st.out_host(), ref["out"], b.shape, b.label)
    print(b.label, stats)


@pytest.mark.parametrize("k,rot", [(1, 0), (1, 32), (3, 0), (3, 64), (4, 64), (5, 128)])
def test_interleaved_rope_append_and_attention(H, k, rot):
    """RoPE on interleaved pairs (2j, 2j+1), whole head or a leading part of it."""
    sh = dataclasses.replace(W.SHAPES[k], rope_style="gptj", rotary_dim=rot)
    b = W.small_workload(k, shape=sh)
    case("gptj rope", b.label, sh.name, "rotary_dim", rot)
    st = run_step(H, b)
    tabs = O.tables(b)
    ref_q = np.concatenate([O.append_request(b, r, tabs)[0] for r in range(b.num_requests)])
    assert_bits_equal(st.q_out_host(), ref_q, "q_out")
    assert_bits_equal(bits_of(st.pool_host()), O.expected_pool(b, sentinel(sh.kv_dtype)), "pool")
    stats = compare_attention(st.out_host(), O.run(b)["out"], sh, b.label)
    print(b.label, "gptj", rot, stats)


QKNORM_CASES = [
    # (workload shape, norm, rope style, rotary_dim, kv dtype)
    (1, "rms", "neox", 0, None),            # fp32 io and cache
    (1, "layer", "gptj", 32, None),         # interleaved pairs on half the head
    (3, "rms", "neox", 0, None),            # bf16, GQA-4
    (3, "layer", "neox", 64, None),         # partial rotary: normalised pass-through dims
    (4, "layer", "gptj", 0, None),          # GQA-8, chunks on cached prefixes, generation rows
    (5, "rms", "neox", 0, None),            # fp8 cache
    (5, "layer", "neox", 0, "int8"),        # int8 cache
]


@pytest.mark.parametrize("case_i", range(len(QKNORM_CASES)))
def test_qk_norm_append_and_attention(H, case_i):
    """Per-head q/k normalisation before RoPE: q_out and the whole pool bit-exact,
    attention within the bars."""
    k, kind, style, rot, kv = QKNORM_CASES[case_i]
    sh = dataclasses.replace(W.SHAPES[k], qk_norm=kind, rope_style=style, rotary_dim=rot, norm_eps=1e-5)
    if kv == "int8":
        sh = dataclasses.replace(sh, kv_dtype=W.INT8, k_scale=2.0 ** -5, v_scale=2.0 ** -5)
    b = W.small_workload(k, shape=sh)
    case("qk norm", b.label, sh.name, kind, style, rot, sh.kv_dtype)
    st = run_step(H, b)
    tabs = O.tables(b)
    ref_q = np.concatenate([O.append_request(b, r, tabs)[0] for r in range(b.num_requests)])
    assert_bits_equal(st.q_out_host(), ref_q, "q_out")
    assert_bits_equal(bits_of(st.pool_host()), O.expected_pool(b, sentinel(sh.kv_dtype)), "pool")
    stats = compare_attention(st.out_host(), O.run(b)["out"], sh, b.label)
    print(b.label, kind, style, rot, stats)


# Mixed batches (context chunks and generation requests) run as one launch that splits the
# CUs between the context schedule and the split pass.  Same decode workgroup count in
# both modes, so the split pass covers the same ranges: outputs must be bitwise equal to
# the serial launches and within the bars against the oracle.
MIXED_CASES = [
    # (shape, kv dtype, decode workgroups, context chunks (n, cached: a multiple of the block),
    #  cached lengths of generation requests, their new tokens (None: one each), draft trees)
    (4, None, 16, [(128, 0), (192, 128), (100, 384)], [20, 77, 140, 333, 500, 9], None, False),   # GQA-8 bf16
    (3, None, 8, [(300, 0), (65, 640)], [1, 64, 65, 900], None, False),                            # GQA-4 bf16
    (2, None, 32, [(70, 0)], [0, 63, 64, 700, 1000], None, False),                                 # MHA bf16
    (5, "fp8", 24, [(200, 128)], [1000, 2500, 3000], None, False),                                 # GQA-4 fp8
    (4, "int8", 8, [(64, 64), (33, 0)], [5, 511, 512], None, False),                               # GQA-8 int8
    (4, None, 16, [(128, 0), (64, 128)], [20, 300, 77, 900], [2, 1, 2, 1], True),                  # GQA-8, draft trees
    (2, None, 16, [(70, 0)], [63, 700, 5], [4, 8, 16], True),                                      # MHA, draft trees
]


@pytest.mark.parametrize("case_i", range(len(MIXED_CASES)))
def test_mixed_launch_matches_serial(H, case_i):
    from paged_kv_gqa_rope_amd import _lib as L
    k, kv, wgs, ctx, past, new, tree = MIXED_CASES[case_i]
    sh = W.SHAPES[k]
    if kv == "fp8":
        sh = dataclasses.replace(sh, kv_dtype=W.FP8_E4M3, k_scale=2.0 ** -6, v_scale=2.0 ** -6)
    elif kv == "int8":
        sh = dataclasses.replace(sh, kv_dtype=W.INT8, k_scale=2.0 ** -5, v_scale=2.0 ** -5)
    b = W.make_batch(sh, ctx=ctx, gen_past=past, gen_new=new, seed=6100 + case_i, pool_blocks_min=4,
                     label=f"mixed-{case_i}", tree=tree)
    case("mixed", b.label, sh.name, sh.kv_dtype, wgs, "tree", tree)
    old_w = L.pkv_set_decode_workgroups(wgs)
    old_c = L.pkv_set_coschedule(1)
    try:
        st = run_step(H, b)
        L.check(L.pkv_kernel_timing_enable(1))
        st.step()
        torch.cuda.synchronize()
        names = {n for n, _ in L.pkv_kernel_timings()}
        L.check(L.pkv_kernel_timing_enable(0))
        # one launch for a bf16 cache; one-byte caches take the generic context kernel,
        # so their batches run as two launches even when asked for one
        assert ("mixed" in names) == (kv is None), names
        mixed = st.out_host()
        L.pkv_set_coschedule(0)
        serial = run_step(H, b).out_host()
    finally:
        L.pkv_set_coschedule(old_c)
        L.pkv_set_decode_workgroups(old_w)
    assert_bits_equal(bits_of(mixed), bits_of(serial), "mixed vs serial output")
    compare_attention(mixed, O.run(b)["out"], sh, b.label)


class _SpanBatch(W.Batch):
    """Queries and new keys with heads whose squares span many binades, where the
    index-order sums round differently from other orders: on even tokens every fourth
    head holds one value 2^24 times smaller than the rest (or a subnormal); on odd tokens
    heads are all zero, hold one nonzero value, or are drawn as usual."""

    def _draw(self, tag, r, rows, heads):
        x = super()._draw(tag, r, rows, heads)
        if tag not in ("q", "k"):
            return x
        f = (x.astype(np.uint32) << 16).view(np.float32).copy()
        for t in range(rows):
            for h in range(heads):
                if t % 2 == 0 and h % 4 == 0:
                    f[t, h, (t + h) % f.shape[2]] *= np.float32(2.0 ** -24)
                elif t % 2 == 0 and h % 4 == 1:
                    f[t, h, 3] = np.float32(2.0 ** -130)          # a bf16 subnormal
                elif t % 2 == 1 and h % 4 == 0:
                    f[t, h, :] = 0
                elif t % 2 == 1 and h % 4 == 1:
                    f[t, h, :] = 0
                    f[t, h, h % f.shape[2]] = np.float32(-3.0)
        return (f.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("kind", ["rms", "layer"])
def test_qk_norm_wide_binade_spans(H, kind):
    """The norm statistics follow the index-order sums bit for bit on heads where the
    order matters (tiny and subnormal values among large ones, zero heads)."""
    sh = dataclasses.replace(W.SHAPES[3], qk_norm=kind, norm_eps=1e-5)
    b0 = W.small_workload(3, shape=sh)
    b = _SpanBatch(**{f.name: getattr(b0, f.name) for f in dataclasses.fields(W.Batch)})
    case("qk norm spans", kind, b.label)
    st = run_step(H, b)
    tabs = O.tables(b)
    ref_q = np.concatenate([O.append_request(b, r, tabs)[0] for r in range(b.num_requests)])
    assert_bits_equal(st.q_out_host(), ref_q, "q_out")
    assert_bits_equal(bits_of(st.pool_host()), O.expected_pool(b, sentinel(sh.kv_dtype)), "pool")


FP8_OUT_CASES = [
    # (workload shape, output scale, no saturation): scales that fit the outputs (decode
    # outputs stay below ~0.2, early prompt rows reach ~4); mostly subnormal codes; a scale
    # that saturates every output above 448 * 2^-14; fp32 io (generic kernel); an fp8 cache
    (2, 2.0 ** -9, True), (3, 2.0 ** -6, True), (3, 2.0 ** -2, True), (4, 2.0 ** -14, False),
    (1, 2.0 ** -5, True), (5, 2.0 ** -10, True),
]


@pytest.mark.parametrize("case_i", range(len(FP8_OUT_CASES)))
def test_fp8_attention_output(H, case_i):
    """Attention output quantised to e4m3 inside the attention kernels."""
    from parity_util import compare_fp8_output
    k, s, fits = FP8_OUT_CASES[case_i]
    sh = dataclasses.replace(W.SHAPES[k], out_fp8_scale=s)
    b = W.small_workload(k, shape=sh)
    case("fp8 out", b.label, sh.name, "scale", s)
    st = run_step(H, b)
    out = O.run(b)["out"]
    stats = compare_fp8_output(st.out_host(), out, sh, b.label, check_values=fits)
    print(b.label, "fp8 out", s, stats)
    if not fits:                                      # large outputs saturate exactly
        big = np.abs(out) > 1.1 * 448 * s
        assert big.mean() > 0.1 and np.array_equal(st.out_host()[big], O.output_codes(b, out)[big])


SPEC_CASES = [
    # (shape, cached lengths, new tokens per generation request, context requests)
    (2, [70, 300, 5], [2, 4, 7], []),                         # MHA: up to 7 x 1 columns
    (5, [1500, 700, 64], [4, 1, 3], []),                      # fp8 cache, G = 4
    (4, [300, 90, 1000, 63], [8, 2, 5, 1], []),               # G = 8: 64 columns, 4 blocks
    (4, [200, 1200], [9, 3], []),                             # 72 columns: generic kernel
    (1, [40, 9], [3, 6], [(20, 16)]),                         # fp32: generic kernel
    (4, [500, 250], [4, 6], [(100, 0), (64, 128)]),           # context chunks, then drafts
]


@pytest.mark.parametrize("case_i", range(len(SPEC_CASES)))
def test_generation_requests_with_draft_tokens(H, case_i):
    """Generation requests with 1 + k new tokens: token i at position p + i sees keys
    0 .. p + i (causal among the drafts)."""
    k, past, new, ctx = SPEC_CASES[case_i]
    sh = dataclasses.replace(W.SHAPES[k], max_num_tokens=1 << 16)
    b = W.make_batch(sh, ctx=ctx, gen_past=past, gen_new=new, seed=3100 + case_i, pool_blocks_min=8,
                     label=f"spec{case_i}")
    case("draft tokens", b.label, sh.name, "new", new, "past", past, "ctx", ctx)
    st = run_step(H, b)
    tabs = O.tables(b)
    ref_q = np.concatenate([O.append_request(b, r, tabs)[0] for r in range(b.num_requests)])
    assert_bits_equal(st.q_out_host(), ref_q, "q_out")
    assert_bits_equal(bits_of(st.pool_host()), O.expected_pool(b, sentinel(sh.kv_dtype)), "pool")
    stats = compare_attention(st.out_host(), O.run(b)["out"], sh, b.label)
    print(b.label, stats)


TREE_CASES = [
    # (shape, cached lengths, new tokens per generation request, context requests, kv override)
    (2, [70, 300, 5], [2, 4, 7], [], None),                   # MHA: one column block, 4 heads per segment
    (5, [1500, 700, 64], [4, 1, 3], [], W.FP8_E4M3),          # fp8 cache (fitted scales), G = 4
    (4, [300, 90, 1000, 63], [8, 2, 5, 1], [], None),         # G = 8: 64 columns, 4 column-block waves per head
    (4, [300, 0, 640, 31], [4, 3, 2, 4], [], None),           # G = 8: 2 column-block waves per head; an empty cache
    (4, [200, 1200], [9, 3], [], None),                       # 72 columns: generic kernel
    (1, [40, 9], [3, 6], [(20, 16)], None),                   # fp32: generic kernel, context rows first
    (4, [500, 250, 33], [4, 6, 2], [(100, 0), (64, 128)], W.INT8),   # context chunks, then tree drafts (int8)
    (4, [4000, 77], [33, 64], [], None),                      # trees as wide as the masks (33 and 64 tokens)
    (2, [100, 2000], [33, 40], [], None),                     # MHA, 33 and 40 tokens: the masks' high word in the split pass
]


@pytest.mark.parametrize("case_i", range(len(TREE_CASES)))
def test_generation_requests_with_draft_trees(H, case_i):
    """Draft tokens as random trees (pkv_append_rope_tree, pkv_attention_forward_tree):
    token i is rotated at p + its depth, stored at cache position p + i, and sees the
    cache and its ancestors; q_out and the pool bit-exact, attention within the bars."""
    k, past, new, ctx, kv = TREE_CASES[case_i]
    sh = dataclasses.replace(W.SHAPES[k], max_num_tokens=1 << 16)
    b = W.make_batch(sh, ctx=ctx, gen_past=past, gen_new=new, seed=3500 + case_i, pool_blocks_min=8,
                     label=f"tree{case_i}", tree=True)
    if kv is not None:
        b = W.fitted(b, kv)
    case("draft trees", b.label, b.shape.name, "new", new, "past", past, "ctx", ctx)
    assert any(b.draft_parents(r)[i] != i - 1 for r in range(b.num_requests) for i in range(1, int(b.context_lengths[r])))
    st = run_step(H, b)
    tabs = O.tables(b)
    ref_q = np.concatenate([O.append_request(b, r, tabs)[0] for r in range(b.num_requests)])
    assert_bits_equal(st.q_out_host(), ref_q, "q_out")
    assert_bits_equal(bits_of(st.pool_host()), O.expected_pool(b, sentinel(b.shape.kv_dtype)), "pool")
    ref = O.run(b)["out"]
    stats = compare_attention(st.out_host(), ref, b.shape, b.label)
    # a tree differs from the chain read of the same inputs wherever a token is not its
    # predecessor's child: the chain's attention must fail the bars somewhere
    chain = O.run(b, tree=False)["out"]
    assert np.max(np.abs(chain - ref)) > 0.05, "the case must tell a tree from a chain"
    print(b.label, stats)


HEAD64_CASES = [
    # (Hkv, G, T, cache, draft tokens per request or None, tree, context chunks, split workgroups)
    (8, 4, 64, W.BF16, None, False, [], 0),             # four KV heads per workgroup
    (32, 1, 16, W.BF16, None, False, [(40, 32)], 0),    # MHA, tiles over two blocks, a context chunk first
    (4, 8, 32, W.FP8_E4M3, 4, False, [], 13),           # two column blocks: two waves share each tile
    (4, 8, 64, W.INT8, 8, True, [], 0),                 # four column blocks, draft trees
    (2, 8, 64, W.BF16, None, False, [], 5),             # one KV head per workgroup, waves share the tiles
    (3, 4, 16, W.FP8_E4M3, 3, False, [], 0),            # one head per segment, several column blocks
    (8, 8, 128, W.BF16, 2, True, [(64, 128)], 0),       # trees after a context chunk
]


@pytest.mark.parametrize("case_i", range(len(HEAD64_CASES)))
def test_head_dim_64_generation(H, case_i):
    """head_dim 64 on the MFMA split pass (every segment layout, bf16 / fp8 / int8
    caches, chains and trees of draft tokens): q_out and the pool bit-exact, attention
    within the bars."""
    from paged_kv_gqa_rope_amd import _lib as L
    Hkv, G, T, kv, draft, tree, ctx, wgs = HEAD64_CASES[case_i]
    sh = W.Shape(f"d64-{case_i}", Hkv * G, Hkv, 64, T, W.BF16, kv, 1e4, max_num_tokens=1 << 16)
    pasts = [0, 1, 31, 32, 63, 100, 511, 700, 1500, 5]
    gen_new = None if draft is None else [1 + (i % draft) for i in range(len(pasts))]
    b = W.make_batch(sh, ctx=ctx, gen_past=pasts, gen_new=gen_new, seed=5400 + case_i, pool_blocks_min=3,
                     label=f"d64-{case_i}", tree=tree)
    if kv in (W.FP8_E4M3, W.INT8):
        b = W.fitted(b)
    case("head_dim 64", b.label, b.shape.kv_dtype, "drafts", draft, "tree", tree, "ctx", ctx, "W", wgs)
    old = L.pkv_set_decode_workgroups(wgs)
    try:
        st = run_step(H, b)
    finally:
        L.pkv_set_decode_workgroups(old)
    tabs = O.tables(b)
    ref_q = np.concatenate([O.append_request(b, r, tabs)[0] for r in range(b.num_requests)])
    assert_bits_equal(st.q_out_host(), ref_q, "q_out")
    assert_bits_equal(bits_of(st.pool_host()), O.expected_pool(b, sentinel(b.shape.kv_dtype)), "pool")
    compare_attention(st.out_host(), O.run(b)["out"], b.shape, b.label)


def test_full_tiny_workload(H):
    b = W.workload(1)
    case("full", b.label)
    st = run_step(H, b)
    ref = O.run(b)
    assert_bits_equal(st.q_out_host(), ref["q_out"], "q_out")
    assert_bits_equal(bits_of(st.pool_host()), O.expected_pool(b, sentinel(b.shape.kv_dtype)), "pool")
    print(compare_attention(st.out_host(), ref["out"], b.shape, b.label))


@pytest.mark.parametrize("k", [2, 4, 5])
def test_outputs_are_bitwise_invariant_to_block_placement_and_reruns(H, k):
    b = W.small_workload(k)
    outs = []
    for seed in (7, 8, 9):
        other = W.make_batch(b.shape, ctx=[(int(n), int(s - n)) for n, s, t in
                                          zip(b.context_lengths, b.sequence_lengths, b.request_types) if t == 0],
                             gen_past=[int(s - 1) for s, t in zip(b.sequence_lengths, b.request_types) if t == 1],
                             seed=seed, pool_blocks_min=b.num_pool_blocks + 5)
        assert not np.array_equal(other.block_table, b.block_table)
        pb = copy_values(b, as_crafted(b, table=other.block_table, pool_blocks=other.num_pool_blocks))
        case("placement", b.label, seed)
        st = run_step(H, pb)
        outs.append(st.out_host().copy())
        assert st.forward() == 0
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(st.out_host()), bits_of(outs[-1])), "rerun differs"
    for o in outs[1:]:
        assert np.array_equal(bits_of(o), bits_of(outs[0])), "block placement changes the output"


@pytest.mark.parametrize("kv", [W.BF16, W.FP8_E4M3, W.INT8])
def test_gqa_equals_mha_with_replicated_kv_heads(H, kv):
    G = 4
    gqa = W.Shape("gqa", 16, 4, 128, 64, W.BF16, kv, 5e5, k_scale=2.0 ** -6, v_scale=2.0 ** -6)
    mha = W.Shape("mha", 16, 16, 128, 64, W.BF16, kv, 5e5, k_scale=2.0 ** -6, v_scale=2.0 ** -6)
    src = W.make_batch(gqa, ctx=[(150, 64)], gen_past=[300, 77, 1000], seed=31)
    a = as_crafted(src)
    copy_values(src, a)
    m = as_crafted(src, shape=mha)
    R = range(src.num_requests)
    rep = lambda x: np.repeat(x, G, axis=1)
    m.set_values([src.new_q(r) for r in R], [rep(src.new_k(r)) for r in R], [rep(src.new_v(r)) for r in R],
                 [rep(src.hist_k(r)) for r in R], [rep(src.hist_v(r)) for r in R])
    case("gqa-vs-mha", kv)
    og = run_step(H, a).out_host()
    om = run_step(H, m).out_host()
    ref = O.run(a)["out"]
    compare_attention(og, ref, gqa, "gqa")
    compare_attention(om, ref, mha, "mha")
    d = np.abs(C.decode(og, W.BF16) - C.decode(om, W.BF16))
    assert d.max() <= 2 ** -7 * np.abs(ref).max() + 1e-6


def test_chunked_prefill_equals_unchunked(H):
    sh = W.SHAPES[3]
    full = W.make_batch(sh, ctx=[(200, 0)], seed=41)
    st_full = run_step(H, full, fill_history=False)
    table = full.block_table
    parts, outs, pool = [(0, 128), (128, 192), (192, 200)], [], None
    for lo, hi in parts:
        c = W.Batch(sh, full.seed, np.array([0], np.int32), np.array([hi - lo], np.int32),
                    np.array([hi], np.int32), table, full.num_pool_blocks)
        cc = as_crafted(c)
        cc.set_values([full.new_q(0)[lo:hi]], [full.new_k(0)[lo:hi]], [full.new_v(0)[lo:hi]],
                      [full.new_k(0)[:0]], [full.new_v(0)[:0]])
        case("chunk", lo, hi)
        st = H.PagedStep(cc, fill_history=False, sentinel=pool is None)
        if pool is not None:
            st.pool = pool                       # earlier chunks' K/V are already in the cache
        st.step()
        torch.cuda.synchronize()
        pool = st.pool
        outs.append(st.out_host().copy())
    got = np.concatenate(outs)
    assert_bits_equal(bits_of(pool.cpu().view(torch.int16).numpy()), bits_of(st_full.pool.cpu().view(torch.int16).numpy()),
                      "chunked cache")
    ref = O.run(full)["out"]
    compare_attention(got, ref, sh, "chunked")
    diff = np.abs(C.decode(got, W.BF16) - C.decode(st_full.out_host(), W.BF16))
    assert diff.max() <= 2 ** -7 * np.abs(ref).max() + 1e-6


def test_zero_keys_average_exactly_the_visible_values(H):
    # K = 0 makes every visible score equal, so each row must average V over
    # positions 0..m: pins causal length, past offset and the block-table gather.
    sh = W.Shape("zk", 8, 2, 128, 64, W.BF16, W.BF16, 1e4)
    def val(t):
        return np.float32((t % 16) / 4.0)
    def fill(tag, r, rows, heads):
        if tag in ("v", "hv"):
            base = 0 if tag == "hv" else int(b_len[r][1])
            x = np.array([val(base + i) for i in range(rows)], np.float32)[:, None, None] * np.ones((1, heads, 128), np.float32)
            return (x.view(np.uint32) >> 16).astype(np.uint16)
        if tag == "q":
            rng = np.random.default_rng(r)
            x = rng.standard_normal((rows, heads, 128)).astype(np.float32)
            return (x.view(np.uint32) >> 16).astype(np.uint16)
        return np.zeros((rows, heads, 128), np.uint16)
    ctx, gen = [(100, 0), (70, 128), (1, 0)], [0, 63, 64, 700]
    b_len = [(n, p) for n, p in ctx] + [(1, p) for p in gen]
    b = crafted(sh, ctx=ctx, gen_past=gen, seed=5, fill=fill)
    case("zero-keys")
    out = C.decode(run_step(H, b).out_host(), W.BF16)
    row = 0
    for (n, p) in b_len:
        for i in range(n):
            m = p + i
            want = np.mean([val(t) for t in range(m + 1)])
            np.testing.assert_allclose(out[row], want, rtol=2 ** -8, atol=0, err_msg=f"row {row} m={m}")
            row += 1


def test_empty_batch_launches_nothing(H):
    from paged_kv_gqa_rope_amd import _lib as L
    sh = W.SHAPES[4]
    b = W.make_batch(sh, seed=1)
    lens = H._Lengths(b.request_types, b.context_lengths, b.sequence_lengths, np.zeros((0, 1), np.int32), 1, "cuda")
    d = H.make_desc(sh)
    s = torch.cuda.current_stream().cuda_stream
    assert L.pkv_append_rope(d, lens.desc, None, 0, None, None, 0, None, 0, None, None, s) == 0
    assert L.pkv_attention_forward(d, lens.desc, None, 0, None, None, None, 0, s) == 0


# ------------------------------------------------------------------ decode kernel edges
@pytest.mark.parametrize("T,G,kv", [(16, 1, W.BF16), (32, 2, W.BF16), (64, 4, W.FP8_E4M3), (128, 8, W.BF16),
                                    (256, 16, W.BF16), (16, 8, W.FP8_E4M3), (64, 3, W.BF16),
                                    (32, 4, W.INT8), (256, 16, W.INT8), (16, 1, W.INT8)])
def test_decode_lengths_blocks_and_groups(H, T, G, kv):
    Hkv = 2
    sh = W.Shape(f"dec-T{T}-G{G}", Hkv * G, Hkv, 128, T, W.BF16, kv, 1e4, k_scale=2.0 ** -6, v_scale=2.0 ** -6)
    # S = p + 1: a lone token, a partial tile, exact tile and chunk edges, a long tail
    pasts = [0, 1, 15, 63, 64, 127, 511, 512, 1000, 2500]
    b = W.make_batch(sh, gen_past=pasts, seed=T * 31 + G, pool_blocks_min=3)
    case("decode", sh.name, kv)
    st = run_step(H, b)
    assert_bits_equal(bits_of(st.pool_host()), O.expected_pool(b, sentinel(kv)), "pool")
    compare_attention(st.out_host(), O.run(b)["out"], sh, sh.name)


# The same length edges with 4 and 8 KV heads (several heads' pieces in every cache row):
# tiles that span two blocks (T = 16), one block, or part of one, for bf16, fp8 and int8
# caches, with single tokens and with draft tokens.
HEAD_GROUP_CASES = [
    # (Hkv, T, G, kv, draft tokens per request or None)
    (4, 16, 1, W.BF16, None),
    (8, 32, 2, W.FP8_E4M3, None),
    (4, 64, 4, W.INT8, None),
    (4, 128, 3, W.BF16, None),
    (4, 16, 8, W.FP8_E4M3, None),
    (8, 256, 2, W.BF16, None),
    (4, 64, 2, W.BF16, 3),
    (8, 16, 1, W.INT8, 5),
    (4, 16, 8, W.BF16, None),        # bf16 with 4-head workgroups (groups of 8+, one column block)
    (8, 64, 16, W.BF16, None),
    (4, 32, 8, W.BF16, 2),           # 16 columns: still one block
    (4, 64, 8, W.BF16, 3),           # two column blocks: one head per workgroup
]


@pytest.mark.parametrize("case_i", range(len(HEAD_GROUP_CASES)))
def test_decode_head_groups(H, case_i):
    Hkv, T, G, kv, draft = HEAD_GROUP_CASES[case_i]
    sh = W.Shape(f"decgrp-{case_i}", Hkv * G, Hkv, 128, T, W.BF16, kv, 1e4, k_scale=2.0 ** -6, v_scale=2.0 ** -6)
    pasts = [0, 1, 15, 63, 64, 127, 511, 512, 1000, 2500]
    gen_new = None if draft is None else [1 + (i % draft) for i in range(len(pasts))]
    b = W.make_batch(sh, gen_past=pasts, seed=4000 + case_i, pool_blocks_min=3, gen_new=gen_new)
    case("decode head groups", sh.name, kv, draft)
    st = run_step(H, b)
    assert_bits_equal(bits_of(st.pool_host()), O.expected_pool(b, sentinel(kv)), "pool")
    compare_attention(st.out_host(), O.run(b)["out"], sh, sh.name)


# The split pass shares the batch's 32-key tiles among W workgroups in equal ranges; a
# range cuts segments into pieces and each wave streams its pieces back to back.  Small
# batches normally give one tile per workgroup, so these cases cap W (process-wide) to
# force long ranges: many pieces per workgroup (W = 1 also lists them in several
# batches), pieces of one tile next to long ones, ranges that start and end inside
# segments, with and without the XCD-contiguous range order (W a multiple of 8 or not).
STREAM_CASES = [
    # (Hkv, T, G, kv, draft tokens per request or None, context chunks)
    (4, 16, 1, W.BF16, None, []),         # one head per workgroup, tiles over two blocks
    (8, 64, 8, W.BF16, None, []),         # four heads per workgroup (bf16, GQA-8)
    (8, 32, 4, W.FP8_E4M3, None, []),
    (4, 64, 2, W.INT8, None, []),
    (4, 32, 8, W.BF16, 4, []),            # draft tokens: up to 3 column blocks, plain loads
    (4, 16, 1, W.BF16, 6, []),            # draft tokens, one column block
    (8, 64, 8, W.BF16, None, [(100, 0), (64, 128)]),   # context requests first
]


@pytest.mark.parametrize("wgs", [1, 3, 8, 13, 24])
@pytest.mark.parametrize("case_i", range(len(STREAM_CASES)))
def test_decode_split_workgroup_counts(H, case_i, wgs):
    from paged_kv_gqa_rope_amd import _lib as L
    Hkv, T, G, kv, draft, ctx = STREAM_CASES[case_i]
    sh = W.Shape(f"stream-{case_i}", Hkv * G, Hkv, 128, T, W.BF16, kv, 1e4, k_scale=2.0 ** -6, v_scale=2.0 ** -6,
                 max_num_tokens=1 << 16)
    pasts = [0, 1, 15, 31, 32, 63, 64, 127, 511, 512, 700, 1000, 2500, 5]
    gen_new = None if draft is None else [1 + (i % draft) for i in range(len(pasts))]
    b = W.make_batch(sh, ctx=ctx, gen_past=pasts, seed=5000 + 10 * case_i + wgs, pool_blocks_min=3, gen_new=gen_new)
    case("decode split workgroups", sh.name, kv, draft, ctx, "W", wgs)
    old = L.pkv_set_decode_workgroups(wgs)
    try:
        st = run_step(H, b)
    finally:
        L.pkv_set_decode_workgroups(old)
    compare_attention(st.out_host(), O.run(b)["out"], sh, sh.name)


@pytest.mark.parametrize("wgs", [116, 120, 122, 124, 126, 128, 132, 140])
def test_combine_piece_counts_around_one_wave(H, wgs):
    """One long request with draft tokens next to two short ones, cut into about 58 to 70
    pieces (W / 2 ranges over 128 tiles): the combine's single-round-trip path up to 64
    pieces, its remainder loads past the first pieces, and the general path above 64."""
    from paged_kv_gqa_rope_amd import _lib as L
    sh = W.Shape("combine-pieces", 32, 8, 128, 64, W.BF16, W.BF16, 1e4, max_num_tokens=1 << 14)
    b = W.make_batch(sh, gen_past=[3996, 2, 40], gen_new=[4, 2, 3], seed=5300 + wgs, pool_blocks_min=3)
    case("combine piece counts", sh.name, "W", wgs)
    old = L.pkv_set_decode_workgroups(wgs)
    try:
        st = run_step(H, b)
    finally:
        L.pkv_set_decode_workgroups(old)
    compare_attention(st.out_host(), O.run(b)["out"], sh, sh.name)


def test_decode_fp8_saturating_values(H):
    # values beyond 448 * scale saturate on write; the oracle reads the same codes
    sh = W.Shape("fp8-sat", 8, 2, 128, 64, W.BF16, W.FP8_E4M3, 1e4, k_scale=2.0 ** -9, v_scale=2.0 ** -9)
    b = W.make_batch(sh, gen_past=[200, 70], seed=3)
    case("fp8-saturation")
    st = run_step(H, b)
    want = O.expected_pool(b, sentinel(W.FP8_E4M3))
    assert np.any((want & 0x7F) == 0x7E), "expected some saturated codes"
    assert_bits_equal(bits_of(st.pool_host()), want, "pool")
    compare_attention(st.out_host(), O.run(b)["out"], sh, "fp8-sat")


def test_decode_int8_saturating_values(H):
    # values beyond 127.5 * scale (or below -128.5 * scale) saturate on write
    sh = W.Shape("int8-sat", 8, 2, 128, 64, W.BF16, W.INT8, 1e4, k_scale=2.0 ** -6, v_scale=2.0 ** -6)
    b = W.make_batch(sh, gen_past=[200, 70], seed=3)
    case("int8-saturation")
    st = run_step(H, b)
    want = O.expected_pool(b, sentinel(W.INT8))
    assert np.any(want == 0x7F) and np.any(want == 0x80), "expected saturated codes of both signs"
    assert_bits_equal(bits_of(st.pool_host()), want, "pool")
    compare_attention(st.out_host(), O.run(b)["out"], sh, "int8-sat")


def _int8_shape(k, scale=2.0 ** -5, **kw):
    return dataclasses.replace(W.SHAPES[k], name=W.SHAPES[k].name + "-int8kv", kv_dtype=W.INT8,
                               k_scale=scale, v_scale=scale, **kw)


INT8_CASES = [
    # (label, batch builder): the int8 cache on every attention path
    ("decode-gqa4", lambda: W.small_workload(5, shape=_int8_shape(5))),
    ("decode-mha", lambda: W.small_workload(2, shape=_int8_shape(2))),
    ("mixed-gqa8", lambda: W.small_workload(4, shape=_int8_shape(4))),
    ("prefill-gqa4", lambda: W.small_workload(3, shape=_int8_shape(3))),
    ("fp32-io", lambda: W.small_workload(1, shape=_int8_shape(1, scale=2.0 ** -4))),
    ("drafts-gqa8", lambda: W.make_batch(_int8_shape(4, max_num_tokens=1 << 16), ctx=[(64, 128)],
                                         gen_past=[300, 1000, 63], gen_new=[4, 8, 2], seed=77, pool_blocks_min=4)),
    ("gptj-half", lambda: W.small_workload(4, shape=_int8_shape(4, rope_style="gptj", rotary_dim=64))),
]


@pytest.mark.parametrize("case_i", range(len(INT8_CASES)))
def test_int8_cache_step(H, case_i):
    """INT8 KV cache ("TensorRT-LLM 1.0 study notes", 6.4): the append quantises with
    1/scale and stores codes bit-exactly as the oracle does; attention dequantises on read."""
    label, make = INT8_CASES[case_i]
    b = make()
    case("int8", label, b.shape.name)
    st = run_step(H, b)
    tabs = O.tables(b)
    ref_q = np.concatenate([O.append_request(b, r, tabs)[0] for r in range(b.num_requests)])
    assert_bits_equal(st.q_out_host(), ref_q, "q_out")
    assert_bits_equal(bits_of(st.pool_host()), O.expected_pool(b, sentinel(W.INT8)), "pool")
    stats = compare_attention(st.out_host(), O.run(b)["out"], b.shape, label)
    print("int8", label, stats)


# ------------------------------------------------------------------ context kernel edges
@pytest.mark.parametrize("T,G", [(64, 1), (16, 2), (32, 4), (128, 8), (256, 4), (64, 16)])
def test_context_chunks_blocks_and_groups(H, T, G):
    Hkv = 2
    sh = W.Shape(f"ctx-T{T}-G{G}", Hkv * G, Hkv, 128, T, W.BF16, W.BF16, 5e5)
    # ragged chunk lengths on block-aligned cached prefixes, a 1-token prompt, and a
    # chunk that starts mid-way through a long prefix; then two generation requests
    ctx = [(1, 0), (31, 0), (100, T * 2), (65, 0), (257, T * 5)]
    b = W.make_batch(sh, ctx=ctx, gen_past=[40, 300], seed=T + G, pool_blocks_min=2)
    case("context", sh.name)
    st = run_step(H, b)
    assert_bits_equal(st.q_out_host(), O.run(b)["q_out"], "q_out")
    compare_attention(st.out_host(), O.run(b)["out"], sh, sh.name)


# The context kernel is persistent: it orders up to 512 requests per launch by their number
# of tiles and deals the (request, KV head, query tile) items to its workgroups in rounds.
# Cases: more requests than one launch takes (two launches, one query tile each), KV heads
# that do not split over the 8 XCD groups, and one chunk far longer than the rest (its
# items span several rounds); blocks of 16 and 32 tokens take the multi-block tile path.
PERSIST_CASES = [
    # (Hkv, G, T, requests, longest random chunk, one long chunk)
    (8, 1, 16, 520, 40, 40),
    (3, 2, 32, 40, 600, 600),
    (8, 2, 16, 24, 200, 1100),
]


@pytest.mark.parametrize("case_i", range(len(PERSIST_CASES)))
def test_context_persistent_schedule(H, case_i):
    Hkv, G, T, R, nmax, nlong = PERSIST_CASES[case_i]
    rng = np.random.default_rng(7000 + case_i)
    ns = rng.integers(1, nmax + 1, size=R)
    ns[R // 2] = nlong
    pasts = T * rng.integers(0, 4, size=R)
    sh = W.Shape(f"persist-{case_i}", Hkv * G, Hkv, 128, T, W.BF16, W.BF16, 5e5, max_num_tokens=int(ns.sum()) + 1)
    b = W.make_batch(sh, ctx=list(zip(ns.tolist(), pasts.tolist())), gen_past=[77], seed=7100 + case_i)
    case("persistent", sh.name, R, int(ns.sum()))
    st = run_step(H, b)
    ref = O.run(b)
    assert_bits_equal(st.q_out_host(), ref["q_out"], "q_out")
    compare_attention(st.out_host(), ref["out"], sh, sh.name)


def test_fp64_to_bf16_store_edge_values(H):
    # fp32 io into a bf16 cache: every stored element is one fp64 -> bf16 rounding.
    # History values hit exact bf16 ties (both parities), fp32 subnormals, values at the
    # bf16 overflow boundary and signed zeros; the oracle's codec decides every bit.
    sh = W.Shape("cvt", 2, 1, 128, 16, W.FP32, W.BF16, 1e4)
    rng = np.random.default_rng(77)
    ties = (np.arange(1, 257, dtype=np.uint32) << 16 | 0x8000).view(np.float32)            # x.5 ulp, both parities
    special = np.array([0.0, -0.0, 1e-39, -1e-39, 3e-45, 1.17549435e-38, 3.3895314e38, 3.3961e38, 3.4e38, -3.4e38,
                        1.0000001, 0.99999994, 65504.0, 2.0 ** -133, 1.5 * 2.0 ** -133], np.float32)
    pool_vals = np.concatenate([ties, -ties, special,
                                rng.standard_normal(4000).astype(np.float32) * np.exp2(rng.integers(-130, 120, 4000)).astype(np.float32)])
    def fill(tag, r, rows, heads):
        if tag in ("hk", "hv"):
            n = rows * heads * 128
            return np.resize(pool_vals if tag == "hk" else pool_vals[::-1], n).reshape(rows, heads, 128).astype(np.float32)
        return rng.standard_normal((rows, heads, 128)).astype(np.float32)
    b = crafted(sh, gen_past=[40, 3], seed=8, fill=fill)
    case("fp64->bf16 store edges")
    st = run_step(H, b)
    assert_bits_equal(bits_of(st.pool_host()), O.expected_pool(b, sentinel(W.BF16)), "bf16 pool")
