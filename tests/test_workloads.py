"""The seeded input generator: determinism, lengths, block tables, value formats."""
import numpy as np

from workloads import synth as W


def test_deterministic_per_seed_and_per_request():
    a, b = W.workload(2), W.workload(2)
    assert np.array_equal(a.sequence_lengths, b.sequence_lengths)
    assert np.array_equal(a.block_table, b.block_table)
    assert np.array_equal(a.hist_k(3), b.hist_k(3))
    assert not np.array_equal(a.hist_k(3)[:10], a.hist_k(4)[:10])


def test_workload_lengths_follow_their_recipes():
    w1 = W.workload(1)
    assert list(w1.request_types) == [W.CONTEXT, W.GENERATION]
    assert list(w1.context_lengths) == [37, 1] and list(w1.sequence_lengths) == [37, 51]
    assert w1.num_pool_blocks == 16
    w2 = W.workload(2)
    assert w2.num_requests == 64 and np.all(w2.context_lengths == 1)
    assert w2.past_lengths.min() >= 512 and w2.past_lengths.max() <= 4096
    w3 = W.workload(3)
    assert np.all(w3.context_lengths == 2048) and np.all(w3.past_lengths == 0)
    w4 = W.workload(4)
    assert list(w4.past_lengths[:4]) == [0, 1024, 2048, 3072] and w4.num_contexts == 4
    assert w4.num_tokens == 4224 <= w4.shape.max_num_tokens
    assert np.all(w4.past_lengths[:4] % 64 == 0)
    w5 = W.workload(5)
    assert w5.past_lengths.min() >= 16384 and w5.past_lengths.max() <= 32768


def test_block_table_is_injective_and_in_range():
    for k in W.WORKLOADS:
        b = W.workload(k)
        T = b.shape.tokens_per_block
        ids = []
        for r in range(b.num_requests):
            nb = (int(b.sequence_lengths[r]) + T - 1) // T
            row = b.block_table[r]
            assert np.all(row[:nb] >= 0) and np.all(row[nb:] == -1)
            ids.extend(row[:nb].tolist())
        assert len(set(ids)) == len(ids)
        assert min(ids) >= 0 and max(ids) < b.num_pool_blocks


def test_values_are_exact_in_the_io_format():
    b = W.small_workload(3)
    q = b.new_q(0)
    assert q.dtype == np.uint16
    f = W.make_batch(W.SHAPES[1], ctx=[(5, 0)], seed=3)
    assert f.new_q(0).dtype == np.float32
    # bf16 values are the float32 draws truncated to their upper half
    raw = W._rng(b.seed, "q", 0).standard_normal(q.shape, dtype=np.float32)
    assert np.array_equal(q, (raw.view(np.uint32) >> 16).astype(np.uint16))


def test_workload5_scales_are_fitted_to_its_values():
    """Workload 5's stored fp8 scales (and the int8 ones of its variant) are the fit of
    its drawn values: amax / 448 (int8: amax / 127) for K and V separately."""
    b = W.workload(5)
    am = W.kv_amax(b)
    assert (b.shape.k_scale, b.shape.v_scale) == W.fit_kv_scales(b, W.FP8_E4M3, am)
    assert W.W5_INT8_SCALES == W.fit_kv_scales(b, W.INT8, am)
    for s in (b.shape.k_scale, b.shape.v_scale) + W.W5_INT8_SCALES:
        assert np.frexp(s)[0] != 0.5, "a fitted scale that is a power of two tests nothing new"
    assert b.shape.k_scale != b.shape.v_scale


def test_small_fitted_scales():
    s5 = W.small_workload(5)
    ak, av = W.kv_amax(s5)
    assert s5.shape.k_scale == float(np.float32(ak / 448)) and s5.shape.v_scale == float(np.float32(av / 448))
    assert 5.0 < ak < 7.0 and 5.0 < av < 7.0
    i8 = W.fitted(W.small_workload(2), W.INT8)
    assert i8.shape.kv_dtype == W.INT8 and i8.shape.k_scale == W.fit_kv_scales(i8, W.INT8)[0]


def test_draft_tree_inputs_are_consistent():
    """The generator's tree inputs: a row's mask holds itself and its ancestors (bit i
    set, no bit at or past n), its offset is its depth (popcount - 1), a parent's mask is
    inside its child's, and context rows carry zeros."""
    b = W.make_batch(W.SHAPES[4], ctx=[(16, 0)], gen_past=[10, 300, 5], gen_new=[7, 1, 33], seed=5, tree=True)
    off, mask = b.spec_inputs()
    assert off.shape == (b.num_tokens,) and mask.shape == (b.num_tokens, 2)
    assert not off[:16].any() and not mask[:16].any()
    row = 16
    for r in range(1, b.num_requests):
        n = int(b.context_lengths[r])
        par = b.draft_parents(r)
        for i in range(n):
            m = int(mask[row + i, 0]) | (int(mask[row + i, 1]) << 32)
            assert (m >> i) & 1 and m >> n == 0
            assert int(off[row + i]) == bin(m).count("1") - 1
            if par[i] >= 0:
                pm = int(mask[row + par[i], 0]) | (int(mask[row + par[i], 1]) << 32)
                assert pm & m == pm and par[i] < i
        row += n
    assert any(b.draft_parents(3)[i] != i - 1 for i in range(1, 33))
