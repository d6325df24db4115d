"""Seeded random batches against the oracle (the last 16 with 64-dim heads): head counts,
head size, block size, cache and io formats, context chunks on cached prefixes, generation requests with draft tokens
as chains or trees, and the split-pass workgroup count all drawn per case.  Each case
checks q_out and the whole pool bit for bit and the attention within the bars."""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import step as O
from parity_util import assert_bits_equal, bits_of, compare_attention
from workloads import synth as W

pytestmark = pytest.mark.gpu

HEADS = [(32, 32), (32, 8), (64, 8), (16, 4), (8, 1), (12, 4), (64, 16), (32, 2)]


def random_batch(i: int):
    rng = np.random.default_rng(9000 + i)
    H, Hkv = HEADS[int(rng.integers(len(HEADS)))]
    T = int(16 << rng.integers(0, 5))
    io = W.FP32 if rng.random() < 0.1 else W.BF16
    kv = W.FP32 if io == W.FP32 and rng.random() < 0.5 else [W.BF16, W.FP8_E4M3, W.INT8][int(rng.integers(3))]
    D = 64 if rng.random() < 0.15 else 128
    if i >= 32:                                        # cases 32 on: 64-dim heads on the MFMA split pass
        io, D = W.BF16, 64
        kv = [W.BF16, W.FP8_E4M3, W.INT8][i % 3]
    style = "gptj" if rng.random() < 0.2 else "neox"
    rot = D // 2 if rng.random() < 0.2 else 0
    sh = W.Shape(f"rand{i}", H, Hkv, D, T, io, kv, 1e4, rotary_dim=rot, rope_style=style,
                 max_num_tokens=1 << 16)
    ctx = [(int(rng.integers(1, 300)), T * int(rng.integers(0, 12))) for _ in range(int(rng.integers(0, 3)))]
    ng = int(rng.integers(0 if ctx else 1, 12))
    past = [int(rng.integers(0, 3000)) for _ in range(ng)]
    drafts = rng.random() < 0.5
    new = [int(rng.integers(1, 9)) if drafts else 1 for _ in range(ng)]
    tree = drafts and rng.random() < 0.5
    b = W.make_batch(sh, ctx=ctx, gen_past=past, gen_new=new, seed=9100 + i, pool_blocks_min=4,
                     label=f"rand{i}", tree=tree)
    if kv in (W.FP8_E4M3, W.INT8):
        b = W.fitted(b)
    wgs = int(rng.choice([0, 0, 0, 5, 17, 64]))        # 0: the library's own count
    return b, wgs


@pytest.fixture(scope="module")
def H():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from paged_kv_gqa_rope_amd import _lib, harness
    _lib.lib()
    return harness


@pytest.mark.parametrize("i", range(48))
def test_random_batch_matches_the_oracle(H, i):
    from paged_kv_gqa_rope_amd import _lib as L
    b, wgs = random_batch(i)
    sh = b.shape
    print("CASE random", i, sh, "ctx", list(zip(b.context_lengths.tolist(), b.past_lengths.tolist())),
          "tree", b.tree, "W", wgs, flush=True)
    old = L.pkv_set_decode_workgroups(wgs)
    try:
        st = H.PagedStep(b)
        st.step()
        torch.cuda.synchronize()
    finally:
        L.pkv_set_decode_workgroups(old)
    ref = O.run(b)
    assert_bits_equal(st.q_out_host(), ref["q_out"], f"{b.label} q_out")
    sentinel = int(np.iinfo(O.BITS[sh.kv_dtype]).max)
    assert_bits_equal(bits_of(st.pool_host()), O.expected_pool(b, sentinel), f"{b.label} pool")
    compare_attention(st.out_host(), ref["out"], sh, b.label)
