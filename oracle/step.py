"""One step of one layer over an in-flight batch.  TEST INFRASTRUCTURE.

The step (from the pages' description of the problem):

1. lengths -- request r brings n_r new tokens on top of p_r cached ones,
   S_r = p_r + n_r ("TensorRT-LLM source analysis report", section 1.1
   sequence_length / context_lengths; the teardown's AttentionMetadata
   section); packed rows carry no padding and context requests come before
   generation requests (report, section 1.3).  A generation request brings 1
   token, or 1 + k draft tokens to verify (report, section 1.4: generation
   lengths, position offsets, packed mask); by default read as one chain, token i
   at position p_r + i, so the drafts are causal among themselves like a chunk.
   Read as a tree (``tree``), token i sits at position p_r + offset_i and sees
   the cached tokens and the new tokens j whose bit j its mask row sets, while
   its K/V still go to cache position p_r + i (the offsets move the rotation,
   not the slot);
2. append -- optionally normalise each head of the new q and k (see
   ``qknorm``), rotate them at their absolute positions p_r + i
   (RoPE, see ``rope``), round q to the io format (q_out), store the rotated k
   and the raw v in the cache format (see ``codecs``) at cache positions
   p_r .. S_r - 1 (study notes, section "KVCacheManager": the attention op
   itself writes the new K/V through the block table);
3. attention -- each new row attends over cache positions 0 .. its own
   position (see ``attention``), reading q_out and the stored K/V as decoded.

The oracle keeps each request's cache contiguous.  Only ``expected_pool``
knows the paged layout, which it writes by its definition: the pool is
[num_blocks, 2, tokens_per_block, num_kv_heads, head_dim] with K at index 0 and
V at index 1 (teardown, KV cache manager interfaces), and cache position t of
request r lives in block table[r][t // T], slot t % T (report, section 1.2
kv_cache_block_offsets; teardown, get_batch_cache_indices).

History ("already cached") values come from the workload generator as io-format
values that count as already rotated; the oracle stores them in the cache format
with the same codec as new tokens, without rotation.
"""
from __future__ import annotations

import numpy as np

from . import codecs
from .attention import attend, attend_visible
from .qknorm import qk_norm
from .rope import neox_tables, rope_apply


def io_decode(batch, bits) -> np.ndarray:
    return codecs.decode(bits, batch.shape.io_dtype)


def tables(batch, max_pos: int | None = None):
    sh = batch.shape
    if max_pos is None:
        max_pos = int(batch.sequence_lengths.max()) if batch.num_requests else 1
    return neox_tables(sh.rope_theta, sh.rot_dim, max(max_pos, 1))


def _as_tree(batch, r: int, tree) -> bool:
    """Whether request r's new tokens are read as a draft tree (generation requests of a
    tree batch, or of any batch when ``tree`` is True)."""
    use = batch.tree if tree is None else tree
    return bool(use) and int(batch.request_types[r]) == 1          # a generation request


def spec_rows(batch, r: int):
    """(offsets [n], masks [n] as Python ints) of request r's rows, from the batch's
    draft-tree inputs."""
    off, mask = batch.spec_inputs()
    a = int(batch.token_offsets[r])
    n = int(batch.context_lengths[r])
    rows = mask[a:a + n].astype(np.uint64)
    return off[a:a + n].astype(np.int64), [int(m[0]) | (int(m[1]) << 32) for m in rows]


def positions_of(batch, r: int, tree=None) -> np.ndarray:
    """Rotation positions of request r's new tokens: p_r + i, or p_r + offset_i."""
    n = int(batch.context_lengths[r])
    p = int(batch.past_lengths[r])
    if _as_tree(batch, r, tree):
        return p + spec_rows(batch, r)[0]
    return np.arange(p, p + n)


def append_request(batch, r: int, tabs, rope: bool = True, tree=None):
    """Return (q_out, k_store, v_store) of request r's new tokens, in token order (cache
    positions p_r .. S_r - 1).

    q_out is in the io representation; k_store/v_store in the cache
    representation.  ``rope=False`` stores k unrotated and skips q.
    """
    sh = batch.shape
    pos = positions_of(batch, r, tree)
    k = io_decode(batch, batch.new_k(r))
    v = io_decode(batch, batch.new_v(r))
    q_out = None
    if rope:
        cos_t, sin_t = tabs
        q = io_decode(batch, batch.new_q(r))
        if sh.qk_norm != "none":
            prm = batch.norm_params()
            eps = float(np.float32(sh.norm_eps))
            q = qk_norm(q, sh.qk_norm, prm["q_weight"], prm["q_bias"], eps)
            k = qk_norm(k, sh.qk_norm, prm["k_weight"], prm["k_bias"], eps)
        q_out = codecs.encode(rope_apply(sh.rope_style, q, pos, cos_t, sin_t, sh.rot_dim), sh.io_dtype)
        k = rope_apply(sh.rope_style, k, pos, cos_t, sin_t, sh.rot_dim)
    k_store = codecs.encode(k, sh.kv_dtype, sh.k_scale)
    v_store = codecs.encode(v, sh.kv_dtype, sh.v_scale)
    return q_out, k_store, v_store


def history_request(batch, r: int):
    """Stored cache contents of request r's p_r already-cached positions."""
    sh = batch.shape
    k = codecs.encode(io_decode(batch, batch.hist_k(r)), sh.kv_dtype, sh.k_scale)
    v = codecs.encode(io_decode(batch, batch.hist_v(r)), sh.kv_dtype, sh.v_scale)
    return k, v


def cache_request(batch, r: int, tabs, tree=None):
    """(q_out, K, V): request r's rotated q (io repr) and its whole cache after
    the append, decoded to fp64, contiguous by position [S_r, Hkv, D]."""
    sh = batch.shape
    q_out, k_new, v_new = append_request(batch, r, tabs, tree=tree)
    k_hist, v_hist = history_request(batch, r)
    K = codecs.decode(np.concatenate([k_hist, k_new], axis=0), sh.kv_dtype, sh.k_scale)
    V = codecs.decode(np.concatenate([v_hist, v_new], axis=0), sh.kv_dtype, sh.v_scale)
    return q_out, K, V


def attention_request(batch, r: int, tabs, heads=None, rows=None, tree=None) -> np.ndarray:
    """fp64 attention output of request r's new rows: [n_r (or len(rows)), H (or len(heads)), D]."""
    q_out, K, V = cache_request(batch, r, tabs, tree=tree)
    p = int(batch.past_lengths[r])
    q = io_decode(batch, q_out)
    if _as_tree(batch, r, tree):
        # row i sees cache positions 0 .. p-1 and p + j for every bit j of its mask
        masks = spec_rows(batch, r)[1]
        L = K.shape[0]
        visible = np.zeros((q.shape[0], L), dtype=bool)
        visible[:, :p] = True
        for i, m in enumerate(masks):
            for j in range(L - p):
                visible[i, p + j] = bool((m >> j) & 1)
        if rows is not None:
            rows = np.asarray(rows)
            q, visible = q[rows], visible[rows]
        return attend_visible(q, K, V, visible, heads=heads)
    positions = p + np.arange(q.shape[0])
    if rows is not None:
        rows = np.asarray(rows)
        q, positions = q[rows], positions[rows]
    return attend(q, K, V, positions, heads=heads)


def run(batch, tree=None):
    """Whole step: dict with packed q_out (io repr), out (fp64 [N, H, D]) and the
    per-request stored new K/V.  ``tree`` overrides the batch's reading of draft tokens."""
    tabs = tables(batch)
    q_outs, outs, k_new, v_new = [], [], [], []
    for r in range(batch.num_requests):
        q_out, kn, vn = append_request(batch, r, tabs, tree=tree)
        q_outs.append(q_out)
        k_new.append(kn)
        v_new.append(vn)
        outs.append(attention_request(batch, r, tabs, tree=tree))
    return {
        "q_out": np.concatenate(q_outs, axis=0),
        "out": np.concatenate(outs, axis=0),
        "k_new": k_new,
        "v_new": v_new,
    }


def output_codes(batch, out: np.ndarray) -> np.ndarray:
    """The attention output in fp8 when the batch asks for it: OCP e4m3 codes of
    out / scale, one nearest-even rounding with saturation, the convention of the KV
    scales ("TensorRT-LLM source teardown part 1", attention backends: FP8 output fused
    into the attention computation; the rounding is the reading of the fp8 cache codec)."""
    return codecs.encode(out, codecs.FP8_E4M3, batch.shape.out_fp8_scale)


BITS = {codecs.FP32: np.uint32, codecs.BF16: np.uint16, codecs.FP8_E4M3: np.uint8, codecs.INT8: np.uint8}


def expected_pool(batch, sentinel, include_new: bool = True, include_history: bool = True):
    """The whole paged pool [nb, 2, T, Hkv, D] as stored bit patterns (uint32 / uint16 /
    uint8 for fp32 / bf16 / fp8 and int8) after the history fill and the step's append; slots
    nobody writes hold the bit pattern ``sentinel``."""
    sh = batch.shape
    T = sh.tokens_per_block
    bits = BITS[sh.kv_dtype]
    pool = np.full((batch.num_pool_blocks, 2, T, sh.num_kv_heads, sh.head_dim), sentinel, dtype=bits)
    tabs = tables(batch)
    for r in range(batch.num_requests):
        p = int(batch.past_lengths[r])
        S = int(batch.sequence_lengths[r])
        parts = []
        if include_history:
            kh, vh = history_request(batch, r)
            parts.append((np.arange(0, p), kh, vh))
        if include_new:
            _, kn, vn = append_request(batch, r, tabs)
            parts.append((np.arange(p, S), kn, vn))
        for pos, ks, vs in parts:
            if pos.size == 0:
                continue
            blk = batch.block_table[r, pos // T]
            slot = pos % T
            pool[blk, 0, slot] = np.asarray(ks).view(bits)
            pool[blk, 1, slot] = np.asarray(vs).view(bits)
    return pool
