"""Pins of the CPU oracle against closed forms, invariants, a printed example,
library special cases and a pure-Python brute force (no GPU)."""
import math
import os
import struct

import numpy as np
import pytest

from oracle import attention as A
from oracle import codecs as C
from oracle import rope as R
from oracle import step as S
from workloads import synth as W

HERE = os.path.dirname(os.path.abspath(__file__))


# ------------------------------------------------------------------ helpers
from batch_util import Crafted, as_crafted, crafted  # noqa: E402


def rand_unit(rng, shape):
    return rng.standard_normal(shape)


# ------------------------------------------------------------------ RoPE
def test_rope_style_none_stores_the_values_as_given():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((9, 2, 64))
    cos_t, sin_t = R.neox_tables(1e4, 64, 40)
    y = R.rope_apply("none", x, rng.integers(0, 40, 9), cos_t, sin_t, 64)
    assert np.array_equal(y, x) and y is not x
    with pytest.raises(ValueError):
        R.rope_apply("rotate", x, np.zeros(9, int), cos_t, sin_t, 64)


@pytest.mark.parametrize("rot", [64, 128, 32])
def test_rope_identity_at_position_zero_and_norm_preserving(rot):
    rng = np.random.default_rng(1)
    D = 128 if rot <= 128 else rot
    x = rand_unit(rng, (50, 3, D))
    cos_t, sin_t = R.neox_tables(1e4, rot, 5000)
    y0 = R.rope_neox(x, np.zeros(50, int), cos_t, sin_t, rot)
    assert np.array_equal(y0, x)
    pos = rng.integers(0, 5000, 50)
    y = R.rope_neox(x, pos, cos_t, sin_t, rot)
    h = rot // 2
    n_in = x[..., :h] ** 2 + x[..., h:rot] ** 2
    n_out = y[..., :h] ** 2 + y[..., h:rot] ** 2
    assert np.allclose(n_out, n_in, rtol=1e-12, atol=1e-15)
    assert np.array_equal(y[..., rot:], x[..., rot:])         # dims past the rotary part pass through


def test_rope_is_complex_multiplication_on_rotate_half_pairs():
    rng = np.random.default_rng(2)
    rot, base = 128, 5e5
    x = rand_unit(rng, (40, 2, rot))
    pos = rng.integers(0, 30000, 40)
    cos_t, sin_t = R.neox_tables(base, rot, 30000)
    y = R.rope_neox(x, pos, cos_t, sin_t, rot)
    z = x[..., :64] + 1j * x[..., 64:]
    ang = pos[:, None].astype(np.float64) * R.neox_inv_freq(base, rot)[None, :]
    w = z * np.exp(1j * ang)[:, None, :]
    assert np.allclose(y[..., :64], w.real, rtol=0, atol=1e-12)
    assert np.allclose(y[..., 64:], w.imag, rtol=0, atol=1e-12)


def test_rope_pairs_are_j_and_j_plus_half():
    rot = 64
    cos_t, sin_t = R.neox_tables(1e4, rot, 10)
    for j in (0, 5, 31, 32, 40, 63):
        x = np.zeros((1, 1, rot)); x[0, 0, j] = 1.0
        y = R.rope_neox(x, np.array([7]), cos_t, sin_t, rot)
        nz = set(np.nonzero(np.abs(y[0, 0]) > 1e-15)[0].tolist())
        partner = j + 32 if j < 32 else j - 32
        assert nz <= {j, partner} and j in nz


def test_rope_relative_position_and_composition():
    rng = np.random.default_rng(3)
    rot = 128
    cos_t, sin_t = R.neox_tables(1e4, rot, 4000)
    q = rand_unit(rng, (1, 1, rot)); k = rand_unit(rng, (1, 1, rot))
    for (m, n, c) in [(10, 3, 100), (0, 500, 7), (1500, 1499, 2000)]:
        a = np.sum(R.rope_neox(q, np.array([m]), cos_t, sin_t, rot) * R.rope_neox(k, np.array([n]), cos_t, sin_t, rot))
        b = np.sum(R.rope_neox(q, np.array([m + c]), cos_t, sin_t, rot) * R.rope_neox(k, np.array([n + c]), cos_t, sin_t, rot))
        assert abs(a - b) < 1e-9
    x = rand_unit(rng, (1, 1, rot))
    ab = R.rope_neox(R.rope_neox(x, np.array([123]), cos_t, sin_t, rot), np.array([456]), cos_t, sin_t, rot)
    direct = R.rope_neox(x, np.array([579]), cos_t, sin_t, rot)
    assert np.allclose(ab, direct, atol=1e-11)


def test_rope_frequency_ladder():
    # pair 0 turns by exactly 1 radian per position; consecutive pairs slow by
    # a constant factor base^(2/R); the pair past the last would turn at 1/base.
    for base, rot in [(1e4, 64), (5e5, 128)]:
        f = R.neox_inv_freq(base, rot)
        assert f[0] == 1.0
        ratios = f[:-1] / f[1:]
        assert np.allclose(ratios, ratios[0], rtol=1e-12)
        assert np.isclose(f[-1] / ratios[0], 1.0 / base, rtol=1e-12)
        cos_t, sin_t = R.neox_tables(base, rot, 3)
        x = np.zeros((1, 1, rot)); x[0, 0, 0] = 1.0
        y = R.rope_neox(x, np.array([1]), cos_t, sin_t, rot)
        assert math.isclose(math.atan2(y[0, 0, rot // 2], y[0, 0, 0]), 1.0, rel_tol=1e-15)


@pytest.mark.parametrize("rot,D", [(128, 128), (64, 128), (32, 64)])
def test_rope_gptj_is_complex_multiplication_on_interleaved_pairs(rot, D):
    rng = np.random.default_rng(20)
    base = 1e4
    x = rand_unit(rng, (30, 2, D))
    pos = rng.integers(0, 9000, 30)
    cos_t, sin_t = R.neox_tables(base, rot, 9000)
    y = R.rope_gptj(x, pos, cos_t, sin_t, rot)
    z = x[..., 0:rot:2] + 1j * x[..., 1:rot:2]
    ang = pos[:, None].astype(np.float64) * R.neox_inv_freq(base, rot)[None, :]
    w = z * np.exp(1j * ang)[:, None, :]
    assert np.allclose(y[..., 0:rot:2], w.real, rtol=0, atol=1e-12)
    assert np.allclose(y[..., 1:rot:2], w.imag, rtol=0, atol=1e-12)
    assert np.array_equal(y[..., rot:], x[..., rot:])         # dims past the rotary part pass through
    assert np.array_equal(R.rope_gptj(x, np.zeros(30, int), cos_t, sin_t, rot), x)


def test_rope_gptj_pairs_are_2j_and_2j_plus_1():
    rot = 64
    cos_t, sin_t = R.neox_tables(1e4, rot, 10)
    for j in (0, 1, 6, 31, 32, 63):
        x = np.zeros((1, 1, rot)); x[0, 0, j] = 1.0
        y = R.rope_gptj(x, np.array([7]), cos_t, sin_t, rot)
        nz = set(np.nonzero(np.abs(y[0, 0]) > 1e-15)[0].tolist())
        assert nz <= {j, j ^ 1} and j in nz


def test_rope_gptj_is_neox_on_deinterleaved_dims():
    # reordering the rotary dims (evens first, then odds) turns interleaved pairs into
    # rotate-half pairs: the two layouts are one rotation seen through a permutation
    rng = np.random.default_rng(21)
    rot, D = 64, 128
    perm = np.concatenate([np.arange(0, rot, 2), np.arange(1, rot, 2), np.arange(rot, D)])
    x = rand_unit(rng, (25, 3, D))
    pos = rng.integers(0, 3000, 25)
    cos_t, sin_t = R.neox_tables(5e5, rot, 3000)
    a = R.rope_gptj(x, pos, cos_t, sin_t, rot)[..., perm]
    b = R.rope_neox(x[..., perm], pos, cos_t, sin_t, rot)
    assert np.array_equal(a, b)


def test_rope_gptj_relative_position():
    rng = np.random.default_rng(22)
    rot = 128
    cos_t, sin_t = R.neox_tables(1e4, rot, 4000)
    q = rand_unit(rng, (1, 1, rot)); k = rand_unit(rng, (1, 1, rot))
    for (m, n, c) in [(10, 3, 100), (0, 500, 7), (1500, 1499, 2000)]:
        a = np.sum(R.rope_gptj(q, np.array([m]), cos_t, sin_t, rot) * R.rope_gptj(k, np.array([n]), cos_t, sin_t, rot))
        b = np.sum(R.rope_gptj(q, np.array([m + c]), cos_t, sin_t, rot) * R.rope_gptj(k, np.array([n + c]), cos_t, sin_t, rot))
        assert abs(a - b) < 1e-9


def test_draft_tokens_equal_single_token_steps_with_the_earlier_drafts_cached():
    """A generation request with 1 + k new tokens (speculative-decoding verification:
    generation length and position offsets, source analysis report 1.4): token i sits
    at position p + i and sees the cache and tokens 0..i.  So its output equals that of
    a one-token generation request at position p + i whose cache already holds tokens
    0..i-1 (rotated, stored) -- built here as a separate batch."""
    from batch_util import Crafted
    sh = W.SHAPES[1]                                   # fp32 io and cache: storing is exact
    p, n = 29, 5
    A = W.make_batch(sh, gen_past=[p], gen_new=[n], seed=77)
    tabs = S.tables(A)
    outA = S.attention_request(A, 0, tabs)
    q_out, k_new, v_new = S.append_request(A, 0, tabs)
    hk, hv = A.hist_k(0), A.hist_v(0)
    for i in range(n):
        Bi = W.make_batch(sh, gen_past=[p + i], seed=78)
        Ci = Crafted(sh, Bi.seed, Bi.request_types, Bi.context_lengths, Bi.sequence_lengths,
                     Bi.block_table, Bi.num_pool_blocks, "draft-step")
        Ci.set_values([A.new_q(0)[i:i + 1]], [A.new_k(0)[i:i + 1]], [A.new_v(0)[i:i + 1]],
                      [np.concatenate([hk, k_new[:i].view(np.float32)])],
                      [np.concatenate([hv, v_new[:i].view(np.float32)])])
        outB = S.attention_request(Ci, 0, S.tables(Ci))
        assert np.allclose(outA[i], outB[0], rtol=0, atol=1e-12), i


def test_chain_shaped_tree_inputs_give_the_chain_step():
    """Position offsets 0..n-1 with lower-triangular masks (the inputs a chain of drafts
    hands over) read through the tree path give the chain step bit for bit."""
    for sh in (W.SHAPES[1], W.SHAPES[4]):
        b = W.make_batch(sh, ctx=[(20, 40)], gen_past=[29, 0, 70], gen_new=[5, 3, 1], seed=81)
        off, mask = b.spec_inputs()
        assert list(off[20:25]) == [0, 1, 2, 3, 4] and [int(m) for m in mask[20:25, 0]] == [1, 3, 7, 15, 31]
        a, t = S.run(b, tree=False), S.run(b, tree=True)
        assert np.array_equal(a["q_out"], t["q_out"]) and np.array_equal(a["out"], t["out"])
        for x, y in zip(a["k_new"], t["k_new"]):
            assert np.array_equal(x, y)


def test_tree_token_equals_one_token_step_over_its_path():
    """A draft token of a tree at depth d (position offset d, mask = itself and its
    ancestors; source analysis report 1.4) attends like a one-token generation request
    at position p + d whose cache holds the history and its ancestors' stored K/V in
    path order: the same keys, rotated at the same positions.  Its stored key is the one
    that request stores.  Built as separate batches; fp32 io and cache, so storing is
    exact."""
    from batch_util import Crafted
    sh = W.SHAPES[1]
    p, n = 29, 9
    A = W.make_batch(sh, gen_past=[p], gen_new=[n], seed=79, tree=True)
    par = A.draft_parents(0)
    assert any(par[i] != i - 1 for i in range(1, n)), "the seed must give a branching tree"
    tabs = S.tables(A)
    outA = S.attention_request(A, 0, tabs)
    _, k_new, v_new = S.append_request(A, 0, tabs)
    hk, hv = A.hist_k(0), A.hist_v(0)
    for i in range(n):
        path = []
        j = i
        while j >= 0:
            path.append(j)
            j = int(par[j])
        path = path[::-1]                       # root .. i
        d = len(path) - 1
        anc = path[:-1]
        Bi = W.make_batch(sh, gen_past=[p + d], seed=80)
        Ci = Crafted(sh, Bi.seed, Bi.request_types, Bi.context_lengths, Bi.sequence_lengths,
                     Bi.block_table, Bi.num_pool_blocks, "tree-path")
        Ci.set_values([A.new_q(0)[i:i + 1]], [A.new_k(0)[i:i + 1]], [A.new_v(0)[i:i + 1]],
                      [np.concatenate([hk, k_new[anc].view(np.float32)])],
                      [np.concatenate([hv, v_new[anc].view(np.float32)])])
        outB = S.attention_request(Ci, 0, S.tables(Ci))
        assert np.allclose(outA[i], outB[0], rtol=0, atol=1e-12), i
        _, kB, _ = S.append_request(Ci, 0, S.tables(Ci))
        assert np.array_equal(k_new[i], kB[0]), i


# ------------------------------------------------------------------ softmax / attention
def test_softmax_printed_temperature_example():
    rows = [l.split() for l in open(os.path.join(HERE, "golden", "softmax_temperature.txt"))
            if l.strip() and not l.startswith("#")]
    for r in rows:
        logits = np.array([float(v) for v in r[1:4]])
        printed = np.array([float(v) for v in r[4:7]])
        p = A.softmax_rows(logits[None, :])[0]
        matches = np.allclose(np.round(p, 2), printed, atol=1e-9)
        assert matches == (r[7] == "ok"), r


def test_softmax_invariants():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((20, 33)) * 5
    p = A.softmax_rows(x)
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-14)
    assert np.allclose(A.softmax_rows(x + 123.25), p, atol=1e-15)
    assert np.allclose(A.softmax_rows(np.full((2, 7), 3.0)), 1.0 / 7, atol=1e-16)
    xm = x.copy(); xm[:, 5:] = -np.inf
    pm = A.softmax_rows(xm)
    assert np.all(pm[:, 5:] == 0) and np.allclose(pm.sum(1), 1)


def test_attend_closed_form_zero_keys_gives_running_mean():
    L, D = 200, 16
    K = np.zeros((L, 2, D))
    V = np.broadcast_to(np.arange(L, dtype=np.float64)[:, None, None], (L, 2, D)).copy()
    pos = np.array([0, 1, 17, 63, 64, 199])
    q = np.random.default_rng(5).standard_normal((len(pos), 4, D))
    out = A.attend(q, K, V, pos)
    want = (pos / 2.0)[:, None, None]
    assert np.allclose(out, np.broadcast_to(want, out.shape), atol=1e-12)


def test_attend_single_key_and_one_hot_probe():
    rng = np.random.default_rng(6)
    D, L = 64, 60
    V = rng.standard_normal((L, 1, D))
    K = np.zeros((L, 1, D))
    for t in range(L):
        K[t, 0, t % D] = 60.0
    q = rng.standard_normal((1, 1, D))
    assert np.allclose(A.attend(q, K, V, np.array([0]))[0, 0], V[0, 0], atol=1e-15)
    for tstar in (0, 13, 59):
        qq = np.zeros((1, 1, D)); qq[0, 0, tstar % D] = 1.0
        out = A.attend(qq, K, V, np.array([L - 1]), scale=1.0)[0, 0]
        assert np.allclose(out, V[tstar, 0], atol=1e-20 + 1e-12)


def test_attend_gqa_mapping_is_contiguous_groups():
    D, L, H, Hkv = 8, 10, 8, 2
    K = np.zeros((L, Hkv, D))
    V = np.zeros((L, Hkv, D))
    for g in range(Hkv):
        V[:, g, :] = g + 1
    q = np.random.default_rng(7).standard_normal((3, H, D))
    out = A.attend(q, K, V, np.array([2, 5, 9]))
    for h in range(H):
        assert np.allclose(out[:, h], h // (H // Hkv) + 1)


def test_attend_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(8)
    H, Hkv, D, L = 12, 3, 16, 40
    q = rng.standard_normal((5, H, D)); K = rng.standard_normal((L, Hkv, D)); V = rng.standard_normal((L, Hkv, D))
    pos = np.array([0, 7, 20, 38, 39])
    a = A.attend(q, K, V, pos)
    b = A.attend(q, np.repeat(K, H // Hkv, axis=1), np.repeat(V, H // Hkv, axis=1), pos)
    assert np.allclose(a, b, atol=1e-13)


def _brute_attend(q, K, V, pos, scale):
    n, H, D = len(q), len(q[0]), len(q[0][0])
    Hkv = len(K[0]); G = H // Hkv
    out = [[[0.0] * D for _ in range(H)] for _ in range(n)]
    for i in range(n):
        for h in range(H):
            g = h // G
            s = [scale * sum(q[i][h][d] * K[t][g][d] for d in range(D)) for t in range(pos[i] + 1)]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            z = sum(e)
            for d in range(D):
                out[i][h][d] = sum(e[t] * V[t][g][d] for t in range(len(e))) / z
    return out


def test_attend_matches_pure_python_brute_force():
    rng = np.random.default_rng(9)
    H, Hkv, D, L = 4, 2, 8, 20
    q = rng.standard_normal((6, H, D)); K = rng.standard_normal((L, Hkv, D)); V = rng.standard_normal((L, Hkv, D))
    pos = np.array([0, 3, 10, 11, 19, 19])
    got = A.attend(q, K, V, pos)
    ref = np.array(_brute_attend(q.tolist(), K.tolist(), V.tolist(), pos.tolist(), 1 / math.sqrt(D)))
    assert np.allclose(got, ref, atol=1e-12)


# ------------------------------------------------------------------ step
def _f32(x):
    return struct.unpack("f", struct.pack("f", x))[0]


def test_step_matches_pure_python_brute_force_fp32():
    # tiny mixed batch: one chunked context request then two generation requests
    sh = W.Shape("t", 4, 2, 8, 4, W.FP32, W.FP32, 100.0)
    rng = np.random.default_rng(10)
    fill = lambda tag, r, rows, heads: rng.standard_normal((rows, heads, 8)).astype(np.float32)
    b = crafted(sh, ctx=[(5, 4)], gen_past=[6, 3], fill=fill)
    res = S.run(b)
    # brute force: angles with math.pow/cos/sin, rotation in Python floats, fp32 rounding via struct
    H, Hkv, D, rot = 4, 2, 8, 8
    rows_q, rows_o = [], []
    for r in range(b.num_requests):
        p = int(b.past_lengths[r]); n = int(b.context_lengths[r])
        def rot_vec(x, m):
            y = list(x)
            for j in range(rot // 2):
                a = m * math.pow(100.0, -2.0 * j / rot)
                c, s = math.cos(a), math.sin(a)
                y[j] = x[j] * c - x[j + rot // 2] * s
                y[j + rot // 2] = x[j + rot // 2] * c + x[j] * s
            return y
        K = [[[float(v) for v in b.hist_k(r)[t][g]] for g in range(Hkv)] for t in range(p)]
        Vv = [[[float(v) for v in b.hist_v(r)[t][g]] for g in range(Hkv)] for t in range(p)]
        qs = []
        for i in range(n):
            qs.append([[_f32(v) for v in rot_vec([float(v) for v in b.new_q(r)[i][h]], p + i)] for h in range(H)])
            K.append([[_f32(v) for v in rot_vec([float(v) for v in b.new_k(r)[i][g]], p + i)] for g in range(Hkv)])
            Vv.append([[float(v) for v in b.new_v(r)[i][g]] for g in range(Hkv)])
        rows_q += qs
        rows_o += _brute_attend(qs, K, Vv, [p + i for i in range(n)], 1 / math.sqrt(D))
    assert np.allclose(res["q_out"].astype(np.float64), np.array(rows_q), rtol=2 ** -23, atol=0)
    assert np.allclose(res["out"], np.array(rows_o), atol=1e-6)


def test_step_chunked_equals_unchunked():
    sh = W.Shape("c", 4, 2, 16, 8, W.FP32, W.FP32, 1e4)
    rng = np.random.default_rng(11)
    n_all, first = 29, 16                      # first chunk is a block multiple
    q = rng.standard_normal((n_all, 4, 16)).astype(np.float32)
    k = rng.standard_normal((n_all, 2, 16)).astype(np.float32)
    v = rng.standard_normal((n_all, 2, 16)).astype(np.float32)
    one = crafted(sh, ctx=[(n_all, 0)]).set_values([q], [k], [v], [k[:0]], [v[:0]])
    full = S.run(one)
    c1 = crafted(sh, ctx=[(first, 0)]).set_values([q[:first]], [k[:first]], [v[:first]], [k[:0]], [v[:0]])
    r1 = S.run(c1)
    # the second chunk sees the first chunk's stored (rotated) K and raw V as its history
    c2 = crafted(sh, ctx=[(n_all - first, first)]).set_values(
        [q[first:]], [k[first:]], [v[first:]], [r1["k_new"][0]], [r1["v_new"][0]])
    r2 = S.run(c2)
    assert np.array_equal(np.concatenate([r1["q_out"], r2["q_out"]]), full["q_out"])
    assert np.allclose(np.concatenate([r1["out"], r2["out"]]), full["out"], atol=1e-13)


def test_step_generation_row_sees_every_cached_token_including_its_own():
    # zero keys: a generation token at position p (S = p + 1 keys) must average V over 0..p
    sh = W.Shape("g", 2, 1, 8, 4, W.FP32, W.FP32, 1e4)
    def fill(tag, r, rows, heads):
        if tag in ("hv",):
            return np.broadcast_to(np.arange(rows, dtype=np.float32)[:, None, None], (rows, heads, 8)).copy()
        if tag == "v":
            return np.full((rows, heads, 8), 9.0, np.float32)       # the new token's V at position 9
        if tag == "q":
            return np.ones((rows, heads, 8), np.float32)
        return np.zeros((rows, heads, 8), np.float32)
    b = crafted(sh, gen_past=[9], fill=fill)
    out = S.run(b)["out"]
    assert np.allclose(out, 4.5, atol=1e-12)                    # mean of 0..9


def test_expected_pool_layout_and_permutation_invariance():
    sh = W.SHAPES[4]
    base = None
    for seed in (21, 22, 23):
        b = W.make_batch(sh, ctx=[(70, 64)], gen_past=[5, 130], seed=seed)
        b = W.Batch(b.shape, 99, b.request_types, b.context_lengths, b.sequence_lengths,
                    b.block_table, b.num_pool_blocks)            # same values, different table
        pool = S.expected_pool(b, sentinel=0xFFFF)
        T = sh.tokens_per_block
        tabs = S.tables(b)
        caches = []
        for r in range(b.num_requests):
            Sr = int(b.sequence_lengths[r])
            t = np.arange(Sr)
            kg = pool[b.block_table[r, t // T], 0, t % T]
            vg = pool[b.block_table[r, t // T], 1, t % T]
            kh, vh = S.history_request(b, r)
            _, kn, vn = S.append_request(b, r, tabs)
            assert np.array_equal(kg, np.concatenate([kh, kn]))
            assert np.array_equal(vg, np.concatenate([vh, vn]))
            caches.append((kg, vg))
        used = np.zeros(b.num_pool_blocks, bool)
        for r in range(b.num_requests):
            nb = (int(b.sequence_lengths[r]) + T - 1) // T
            used[b.block_table[r, :nb]] = True
        assert np.all(pool[~used] == 0xFFFF)
        if base is None:
            base = caches
        else:
            for (a1, a2), (b1, b2) in zip(base, caches):
                assert np.array_equal(a1, b1) and np.array_equal(a2, b2)


def test_fp8_cache_dequantises_what_was_quantised():
    b = W.small_workload(5)
    tabs = S.tables(b)
    q_out, K, V = S.cache_request(b, 0, tabs)
    s = b.shape.k_scale
    codes = C.f64_to_e4m3(K / s)
    assert np.array_equal(C.e4m3_to_f64(codes) * s, K)            # K holds exactly representable values
    hk = C.bf16_to_f64(b.hist_k(0))
    assert np.max(np.abs(K[: hk.shape[0]] - hk)) <= 2.0 ** -4 * np.max(np.abs(hk)) + 1e-12


def _int8_grid_batch(kv, ks, vs):
    """Generation + context batch whose cached K/V are integers times their scale (bf16
    io); new k rows are zero, so RoPE keeps them on the grid."""
    sh = W.Shape("int8-grid", 8, 2, 128, 16, W.BF16, kv, 1.0e4, k_scale=ks, v_scale=vs)

    def fill(tag, r, rows, heads):
        rng = np.random.default_rng([77, r, len(tag)])
        if tag == "q":
            x = rng.standard_normal((rows, heads, 128)).astype(np.float32)
        elif tag == "k":
            x = np.zeros((rows, heads, 128), np.float32)
        else:
            sc = ks if tag == "hk" else vs
            x = (rng.integers(-128, 128, (rows, heads, 128)) * sc).astype(np.float32)
        return (x.view(np.uint32) >> 16).astype(np.uint16)
    return crafted(sh, ctx=[(21, 40)], gen_past=[70, 33], seed=5, fill=fill)


def test_int8_cache_is_exact_on_its_grid_and_matches_bf16_cache():
    # "TensorRT-LLM 1.0 study notes", 6.4: the INT8 KV cache changes only the stored
    # format.  Values that are integers (-128 .. 127) times the scale survive the round
    # trip exactly, so the step must give the bf16 cache's results bit for bit.
    ks, vs = 2.0 ** -4, 2.0 ** -6
    b8 = _int8_grid_batch(W.INT8, ks, vs)
    b16 = as_crafted(b8, shape=W.with_shape(b8, kv_dtype=W.BF16).shape).set_values(**b8._vals)
    r8, r16 = S.run(b8), S.run(b16)
    assert np.array_equal(r8["out"], r16["out"])
    tabs = S.tables(b8)
    for r in range(b8.num_requests):
        _, K8, V8 = S.cache_request(b8, r, tabs)
        _, K16, V16 = S.cache_request(b16, r, tabs)
        assert np.array_equal(K8, K16) and np.array_equal(V8, V16)
        assert np.all(np.abs(K8) <= 128 * ks) and np.all(np.abs(V8) <= 128 * vs)
    pool = S.expected_pool(b8, 0)
    assert pool.dtype == np.uint8


def test_int8_cache_rounds_and_saturates_history():
    b = W.small_workload(5, shape=W.Shape("s5-int8", 32, 8, 128, 64, W.BF16, W.INT8, 5.0e5,
                                          k_scale=2.0 ** -5, v_scale=2.0 ** -5))
    tabs = S.tables(b)
    _, K, V = S.cache_request(b, 0, tabs)
    s = 2.0 ** -5
    c = K / s
    assert np.array_equal(c, np.round(c)) and c.min() >= -128 and c.max() <= 127
    hk = C.bf16_to_f64(b.hist_k(0))
    inside = (hk > -128.5 * s) & (hk < 127.5 * s)
    assert np.all(np.abs(K[: hk.shape[0]][inside] - hk[inside]) <= s / 2)
    assert np.all(K[: hk.shape[0]][hk >= 127.5 * s] == 127 * s)
    assert np.all(K[: hk.shape[0]][hk <= -128.5 * s] == -128 * s)
    assert np.any(~inside)                                         # the draw does reach saturation


def test_small_workload_runs_and_rows_are_convex_combinations():
    for k in (1, 3, 4):
        b = W.small_workload(k)
        res = S.run(b)
        assert res["out"].shape == (b.num_tokens, b.shape.num_heads, b.shape.head_dim)
        # each output is a convex combination of the request's V rows
        tabs = S.tables(b)
        off = b.token_offsets
        for r in range(b.num_requests):
            _, _, V = S.cache_request(b, r, tabs)
            o = res["out"][off[r]:off[r + 1]]
            G = b.shape.group
            for h in range(0, b.shape.num_heads, G):
                g = h // G
                assert np.all(o[:, h] <= V[:, g].max(axis=0) + 1e-12)
                assert np.all(o[:, h] >= V[:, g].min(axis=0) - 1e-12)


# ------------------------------------------------------------------ QK norm
from oracle import qknorm as QN  # noqa: E402


@pytest.mark.parametrize("D", [8, 64, 128])
def test_qk_norm_closed_forms(D):
    rng = np.random.default_rng(20 + D)
    x = rng.standard_normal((5, 3, D)) * rng.uniform(0.1, 10.0, (5, 3, 1))
    ones, zeros = np.ones(D), np.zeros(D)
    y = QN.qk_norm(x, "rms", ones, None, 0.0)              # unit root mean square
    assert np.max(np.abs(np.mean(y * y, axis=-1) - 1.0)) < 1e-14
    y = QN.qk_norm(x, "layer", ones, zeros, 0.0)           # zero mean, unit variance
    assert np.max(np.abs(np.mean(y, axis=-1))) < 1e-14
    assert np.max(np.abs(np.mean(y * y, axis=-1) - 1.0)) < 1e-14
    c = np.full((1, 1, D), 3.25)                           # a constant head: d = 0, y = bias
    b = rng.standard_normal(D)
    assert np.array_equal(QN.qk_norm(c, "layer", rng.standard_normal(D), b, 1e-6)[0, 0], b)
    assert np.array_equal(QN.qk_norm(x, "none", ones, None, 0.0), x)


def test_qk_norm_invariances():
    rng = np.random.default_rng(31)
    x = rng.standard_normal((4, 2, 128))
    w, b = rng.standard_normal(128), rng.standard_normal(128)
    for kind in ("rms", "layer"):
        ref = QN.qk_norm(x, kind, w, b, 0.0)
        # a power-of-two scale changes every intermediate exactly: bitwise the same
        assert np.array_equal(QN.qk_norm(x * 8.0, kind, w, b, 0.0), ref)
        assert np.allclose(QN.qk_norm(x * 0.37, kind, w, b, 0.0), ref, rtol=0, atol=1e-12)
    # layer form: shifting a head by a constant changes nothing
    ref = QN.qk_norm(x, "layer", w, b, 0.0)
    assert np.allclose(QN.qk_norm(x + 5.5, "layer", w, b, 0.0), ref, rtol=0, atol=1e-11)
    # the rms form of a zero-mean head is the layer form without bias
    xz = x - x.mean(axis=-1, keepdims=True)
    assert np.allclose(QN.qk_norm(xz, "rms", w, None, 0.0), QN.qk_norm(xz, "layer", w, np.zeros(128), 0.0),
                       rtol=0, atol=1e-13)


def test_qk_norm_matches_torch_layer_norm_and_rms_norm():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(41)
    x = rng.standard_normal((6, 4, 128))
    w, b = rng.standard_normal(128), rng.standard_normal(128)
    eps = 1e-5
    tx, tw, tb = (torch.from_numpy(a) for a in (x, w, b))
    ln = torch.nn.functional.layer_norm(tx, (128,), tw, tb, eps).numpy()
    assert np.allclose(QN.qk_norm(x, "layer", w, b, eps), ln, rtol=0, atol=1e-12)
    rms = torch.nn.functional.rms_norm(tx, (128,), tw, eps).numpy()
    assert np.allclose(QN.qk_norm(x, "rms", w, None, eps), rms, rtol=0, atol=1e-12)


def test_qk_norm_matches_pure_python_loops_bitwise():
    rng = np.random.default_rng(51)
    D = 16
    x = rng.standard_normal((3, D))
    w, b = rng.standard_normal(D), rng.standard_normal(D)
    for kind in ("rms", "layer"):
        got = QN.qk_norm(x, kind, w, b, 1e-3)
        for row in range(3):
            xs = [float(v) for v in x[row]]
            mu = 0.0
            if kind == "layer":
                s = 0.0
                for v in xs:
                    s += v
                mu = s / D
            ss = 0.0
            for v in xs:
                ss += (v - mu) * (v - mu)
            inv = 1.0 / math.sqrt(ss / D + 1e-3)
            want = [(v - mu) * inv * float(w[j]) + (float(b[j]) if kind == "layer" else 0.0)
                    for j, v in enumerate(xs)]
            assert got[row].tolist() == want


def test_step_normalises_q_and_k_before_rotating():
    """A context request's first token sits at position 0 (the rotation is the identity),
    so its stored q and k are the normalised inputs rounded once; at later positions they
    are the rotation of the normalised inputs."""
    torch = pytest.importorskip("torch")
    sh = W.Shape("qkn", 4, 2, 64, 16, W.FP32, W.FP32, 1e4, qk_norm="layer", norm_eps=1e-5)
    b = W.make_batch(sh, ctx=[(20, 0)], seed=77)
    prm = b.norm_params()
    eps = float(np.float32(sh.norm_eps))
    q = b.new_q(0).astype(np.float64)
    k = b.new_k(0).astype(np.float64)

    def tnorm(x, w, bias):
        return torch.nn.functional.layer_norm(torch.from_numpy(x), (64,), torch.from_numpy(w.astype(np.float64)),
                                              torch.from_numpy(bias.astype(np.float64)), eps).numpy()
    qn, kn = tnorm(q, prm["q_weight"], prm["q_bias"]), tnorm(k, prm["k_weight"], prm["k_bias"])
    q_out, k_store, _ = S.append_request(b, 0, S.tables(b))
    assert np.allclose(q_out[0].astype(np.float64), qn[0], rtol=2 ** -23, atol=1e-12)
    assert np.allclose(k_store[0].astype(np.float64), kn[0], rtol=2 ** -23, atol=1e-12)
    cos_t, sin_t = S.tables(b)
    pos = np.arange(20)
    assert np.allclose(q_out.astype(np.float64), R.rope_neox(qn, pos, cos_t, sin_t, 64), rtol=1e-6, atol=1e-6)
    assert np.allclose(k_store.astype(np.float64), R.rope_neox(kn, pos, cos_t, sin_t, 64), rtol=1e-6, atol=1e-6)
