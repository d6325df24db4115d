"""GPU parity at the full workload sizes, in the launch configuration bench.py times
(one append + one attention call over the whole batch), checked on sampled requests
and heads that the oracle computes one by one."""
import time

import numpy as np
import pytest
import torch

from oracle import step as O
from parity_util import assert_bits_equal, bits_of, compare_attention
from workloads import synth as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def H():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from paged_kv_gqa_rope_amd import _lib, harness
    _lib.lib()
    return harness


def sample_requests(b, k):
    rng = np.random.default_rng(500 + k)
    B = b.num_requests
    picks = {0, B - 1}
    if b.num_contexts and b.num_contexts < B:
        picks |= {b.num_contexts - 1, b.num_contexts}          # both sides of the phase boundary
    picks |= set(rng.choice(B, size=min(2, B), replace=False).tolist())
    return sorted(picks)


def sample_heads(sh, k):
    rng = np.random.default_rng(600 + k)
    hs = {0, sh.num_heads - 1, sh.group - 1 if sh.group > 1 else 1}
    hs |= set(rng.choice(sh.num_heads, size=2, replace=False).tolist())
    return sorted(h for h in hs if h < sh.num_heads)


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_full_size_workload_sampled_parity(H, k):
    _sampled_parity(H, W.workload(k), k, f"workload {k}")


@pytest.mark.parametrize("name", ["spec4-gqa8", "tree4-gqa8", "int8kv5"])
def test_full_size_variant_sampled_parity(H, name):
    """The bench's draft-token (chain and tree) and int8-cache variants at full size."""
    import bench
    _sampled_parity(H, bench.variant_batch(name), 10 + bench.VARIANTS.index(name), f"variant {name}")


def _sampled_parity(H, b, k, what):
    sh = b.shape
    t0 = time.time()
    print(f"CASE full-size {what} ({sh.name}): building, history fill", flush=True)
    st = H.PagedStep(b, sentinel=False)
    torch.cuda.synchronize()
    print(f"  setup {time.time() - t0:.1f} s; step", flush=True)
    st.step()
    torch.cuda.synchronize()
    q_out = st.q_out_host()
    out = st.out_host()
    pool = bits_of(st.pool_host())
    off = b.token_offsets
    T = sh.tokens_per_block
    tabs = O.tables(b)
    heads = sample_heads(sh, k)
    for r in sample_requests(b, k):
        rows = slice(int(off[r]), int(off[r + 1]))
        q_ref, k_new, v_new = O.append_request(b, r, tabs)
        assert_bits_equal(q_out[rows], q_ref, f"w{k} r{r} q_out")
        # the request's whole cache in the pool (history fill + this step's append)
        k_hist, v_hist = O.history_request(b, r)
        S = int(b.sequence_lengths[r])
        pos = np.arange(S)
        blk = b.block_table[r, pos // T]
        assert_bits_equal(pool[blk, 0, pos % T], np.concatenate([k_hist, k_new]), f"w{k} r{r} K cache")
        assert_bits_equal(pool[blk, 1, pos % T], np.concatenate([v_hist, v_new]), f"w{k} r{r} V cache")
        ref = O.attention_request(b, r, tabs, heads=heads)
        stats = compare_attention(out[rows][:, heads], ref, sh, f"w{k} r{r}")
        print(f"  r{r} (n={int(b.context_lengths[r])}, S={S}) heads {heads}: {stats}", flush=True)
    del st
    torch.cuda.empty_cache()
