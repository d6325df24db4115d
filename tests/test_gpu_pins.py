"""GPU pins beyond element-wise parity: K/V scales fitted to the data (inexact 1/scale),
the append fed the oracle's own RoPE table, a one-hot probe of the block mapping, and
every placement of a 5-block pool."""
import dataclasses
import itertools

import numpy as np
import pytest
import torch

from batch_util import as_crafted, copy_values, crafted
from oracle import codecs as C
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


def case(*a):
    print("CASE", *a, flush=True)


def sentinel(fmt):
    return int(np.iinfo(O.BITS[fmt]).max)


def check_step(H, b, label, **kw):
    """q_out and the whole sentinel-filled pool bit-exact, attention within the bars."""
    st = H.PagedStep(b, **kw)
    st.step()
    torch.cuda.synchronize()
    tabs = O.tables(b)
    ref_q = np.concatenate([O.append_request(b, r, tabs)[0] for r in range(b.num_requests)])
    assert_bits_equal(st.q_out_host(), ref_q, f"{label} q_out")
    assert_bits_equal(bits_of(st.pool_host()), O.expected_pool(b, sentinel(b.shape.kv_dtype)), f"{label} pool")
    stats = compare_attention(st.out_host(), O.run(b)["out"], b.shape, label)
    print(label, stats, flush=True)
    return st


# ------------------------------------------------------------------ fitted K/V scales
def _drafts(k, kv):
    sh = dataclasses.replace(W.SHAPES[k], max_num_tokens=1 << 16)
    return W.fitted(W.make_batch(sh, ctx=[(64, 128)], gen_past=[300, 1000, 63, 2000], gen_new=[4, 8, 2, 1],
                                 seed=3300, pool_blocks_min=4, label=f"drafts-{kv}"), kv)


FITTED_CASES = [
    # (label, batch): scales amax/448 (e4m3) or amax/127 (int8), separately for K and V
    ("s5-fp8", lambda: W.small_workload(5)),
    ("s5-int8", lambda: W.fitted(W.small_workload(5, shape=W.SHAPES[5]), W.INT8)),
    ("s4-fp8", lambda: W.fitted(W.small_workload(4), W.FP8_E4M3)),
    ("s2-int8", lambda: W.fitted(W.small_workload(2), W.INT8)),
    ("w4-drafts-fp8", lambda: _drafts(4, W.FP8_E4M3)),
    ("w4-drafts-int8", lambda: _drafts(4, W.INT8)),
    ("w1-fp32-fp8", lambda: W.fitted(W.workload(1), W.FP8_E4M3)),
    ("w1-fp32-int8", lambda: W.fitted(W.workload(1), W.INT8)),
]


@pytest.mark.parametrize("case_i", range(len(FITTED_CASES)))
def test_fitted_kv_scales(H, case_i):
    """"Scaled to fit" read as amax / code max per tensor: non-power-of-two scales, distinct
    for K and V, so the quantiser's 1/scale is inexact and a K/V scale swap shows."""
    label, make = FITTED_CASES[case_i]
    b = make()
    sh = b.shape
    assert sh.k_scale != sh.v_scale and np.frexp(sh.k_scale)[0] != 0.5 and np.frexp(sh.v_scale)[0] != 0.5
    case("fitted scales", label, sh.name, sh.kv_dtype, sh.k_scale, sh.v_scale)
    check_step(H, b, label)


# ------------------------------------------------------------------ one RoPE table
def oracle_rope_table(b):
    c, s = O.tables(b)
    return np.stack([c, s], axis=-1)          # [pos][j][cos, sin], the ABI's layout


@pytest.mark.parametrize("label", ["w1", "s3", "s4-gptj", "s5"])
def test_append_bit_exact_with_the_oracle_rope_table(H, label):
    """Both sides rotate with the same fp64 table (the oracle's numpy cos/sin, interleaved
    into the ABI's [pos][j][2] layout): the stored bits then depend on the rotation
    recipe alone, with no last-ulp table differences between device and host libm."""
    if label == "w1":
        b = W.workload(1)
    elif label == "s4-gptj":
        b = W.small_workload(4, shape=dataclasses.replace(W.SHAPES[4], rope_style="gptj", rotary_dim=64))
    else:
        b = W.small_workload(int(label[1]))
    case("oracle rope table", label, b.shape.name)
    st = check_step(H, b, label, rope_table=oracle_rope_table(b))
    assert np.array_equal(st.rope_host(), oracle_rope_table(b))


# ------------------------------------------------------------------ one-hot probe
ONEHOT_CASES = [
    # (KV heads, group, cache format, tokens per block)
    (2, 4, W.BF16, 16),
    (4, 8, W.BF16, 32),
    (4, 4, W.FP8_E4M3, 16),
    (2, 2, W.INT8, 64),
]


@pytest.mark.parametrize("case_i", range(len(ONEHOT_CASES)))
def test_one_hot_probe_finds_each_target_key(H, case_i):
    """Key t of KV head g is alpha * e_{c_g(t)} with distinct codes c_g(t) per request; each
    query is alpha * e_{c_g(t*)} for one visible target t*, so the softmax puts all its
    weight (1 - ~1e-38) on t*.  Value t is e_{v_g(t)}, again with distinct codes, so the
    output's argmax names the key the kernel found at t*: the block-table mapping of every
    block holding a target is pinned, position by position (no RoPE here, so the
    directions stay aligned)."""
    Hkv, G, kv, T = ONEHOT_CASES[case_i]
    Hq, D, alpha = Hkv * G, 128, 32.0
    sh = W.Shape(f"onehot-{case_i}", Hq, Hkv, D, T, W.BF16, kv, 1e4, rope_style="none",
                 k_scale=float(np.float32(alpha / 448)), v_scale=float(np.float32(1 / 448)))
    if kv == W.INT8:
        sh = dataclasses.replace(sh, k_scale=float(np.float32(alpha / 127)), v_scale=float(np.float32(1 / 127)))
    ctx = [(1, 0), (48, 0), (40, 2 * T if 2 * T + 40 <= 128 else T)]
    gen = [127, 100, 63, 17]
    lens = [(n, p) for n, p in ctx] + [(1, p) for p in gen]
    kcode = lambda t, g: (5 * t + 17 * g) % D          # distinct over t < 128 for each g
    vcode = lambda t, g: (3 * t + 7 * g + 1) % D

    def target(r, i, h):                              # visible key of row i, head h: the heads
        n, p = lens[r]                                # spread evenly over the visible keys
        m1 = p + i + 1
        return ((2 * h + 1) * m1 // (2 * Hq) + 13 * i + 7 * r) % m1

    def bf16(x):
        return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)

    def fill(tag, r, rows, heads):
        n, p = lens[r]
        x = np.zeros((rows, heads, D), np.float32)
        for i in range(rows):
            t = i if tag in ("hk", "hv") else p + i      # cache position of this row
            for hh in range(heads):
                if tag in ("k", "hk"):
                    x[i, hh, kcode(t, hh)] = alpha
                elif tag in ("v", "hv"):
                    x[i, hh, vcode(t, hh)] = 1.0
                else:                                    # q: head hh of KV head hh // G
                    x[i, hh, kcode(target(r, i, hh), hh // G)] = alpha
        return bf16(x)

    b = crafted(sh, ctx=ctx, gen_past=gen, seed=900 + case_i, fill=fill)
    case("one-hot probe", sh.name, kv)
    st = H.PagedStep(b)
    st.step()
    torch.cuda.synchronize()
    out = C.decode(st.out_host(), W.BF16)
    row, hit_blocks = 0, set()
    for r, (n, p) in enumerate(lens):
        for i in range(n):
            for h in range(Hq):
                t = target(r, i, h)
                g = h // G
                o = out[row, h]
                assert int(np.argmax(o)) == vcode(t, g), f"request {r} row {i} head {h}: target key {t}"
                assert abs(o[vcode(t, g)] - 1.0) <= 2 ** -7 and np.sum(np.abs(o)) <= 1.0 + 2 ** -6, (r, i, h, o.max())
                hit_blocks.add((r, t // T))
            row += 1
    all_blocks = {(r, j) for r, (n, p) in enumerate(lens) for j in range((n + p + T - 1) // T)}
    print(f"{len(hit_blocks)} of {len(all_blocks)} blocks hold a target", flush=True)
    assert len(hit_blocks) >= 0.9 * len(all_blocks)
    compare_attention(st.out_host(), O.run(b)["out"], sh, sh.name)


# ------------------------------------------------------------------ every placement
@pytest.mark.parametrize("kv", [W.BF16, W.INT8])
def test_every_placement_of_a_five_block_pool(H, kv):
    """All 120 assignments of 5 physical blocks to the batch's 5 logical blocks (a 40-token
    prompt: 3 blocks; a generation request at S = 21: 2 blocks): q_out, the output and
    each logical position's cached bits are identical in every placement."""
    sh = W.Shape("perm5", 8, 2, 128, 16, W.BF16, kv, 1e4)
    base = W.make_batch(sh, ctx=[(40, 0)], gen_past=[20], seed=55)
    assert base.num_pool_blocks == 5
    if kv == W.INT8:
        base = W.fitted(base)
    sh = base.shape
    first = None
    for pi in itertools.permutations(range(5)):
        table = np.array([[pi[0], pi[1], pi[2]], [pi[3], pi[4], -1]], np.int32)
        b = copy_values(base, as_crafted(base, table=table, pool_blocks=5))
        st = H.PagedStep(b)
        st.step()
        torch.cuda.synchronize()
        pool = bits_of(st.pool_host())
        logical = pool[np.asarray(pi)]                 # logical block order
        got = (bits_of(st.q_out_host()).copy(), bits_of(st.out_host()).copy(), logical.copy())
        if first is None:
            case("placements", kv, "first", pi)
            first = got
            assert_bits_equal(logical[[0, 1, 2, 3, 4]],
                              O.expected_pool(b, sentinel(kv))[np.asarray(pi)], "pool vs oracle")
            compare_attention(st.out_host(), O.run(b)["out"], sh, "perm5")
            continue
        for x, y, what in zip(got, first, ("q_out", "out", "cache by logical block")):
            assert np.array_equal(x, y), f"placement {pi}: {what} differs from placement (0, 1, 2, 3, 4)"
    print("120 placements bitwise identical", flush=True)
