"""Seeded synthetic batches shaped like the five workloads of the hot path.

Recipe (the same for every workload):

* one ``numpy.random.Generator(PCG64(SeedSequence([seed, tag, index])))`` per
  (purpose, request), so that any single request's inputs can be regenerated
  on their own;
* request lengths are explicit or drawn with ``integers(lo, hi, endpoint=True)``;
* physical block IDs are the first ``sum(ceil(S_r / T))`` entries of
  ``permutation(pool_blocks)``, handed out to (request, logical block) in
  request order; unused table entries are -1;
* values are ``standard_normal`` drawn in float32.  For a bf16 io dtype the
  float32 draw is cut to its upper 16 bits (truncation toward zero, a pure bit
  operation), so every value is exactly representable in the io dtype and both
  sides start from the same numbers.

Values are returned in the io dtype's own representation: ``float32`` arrays
for fp32, ``uint16`` bit patterns for bf16.  History ("already cached") values
are returned the same way; they count as already rotated, and each side writes
them into its own cache representation (for an fp8 or int8 cache that means its
own quantiser).

Scales of a one-byte cache are fitted to the data (``fit_kv_scales``): for K and
for V separately, the largest magnitude over every drawn value (history and new
tokens, as drawn) divided by the largest code magnitude (448 for e4m3, 127 for
int8), rounded to float32.  Such a scale is generally not a power of two, so the
quantiser's 1/scale is inexact.

Nothing here rotates, rounds to a storage format, scatters into pages or
attends: those are the method, and each compared side implements them itself.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

FP32, BF16, FP8_E4M3, INT8 = "fp32", "bf16", "fp8_e4m3", "int8"
CONTEXT, GENERATION = 0, 1

_TAGS = {"lengths": 1, "blocks": 2, "q": 3, "k": 4, "v": 5, "hist_k": 6, "hist_v": 7, "norm": 8, "tree": 9}


def _rng(seed: int, tag: str, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _TAGS[tag], index])))


@dataclass(frozen=True)
class Shape:
    """Per-layer attention shape and storage formats."""
    name: str
    num_heads: int
    num_kv_heads: int
    head_dim: int
    tokens_per_block: int
    io_dtype: str
    kv_dtype: str
    rope_theta: float
    rotary_dim: int = 0          # 0 means head_dim
    rope_style: str = "neox"     # "neox": pairs (j, j + R/2); "gptj": pairs (2j, 2j + 1)
    k_scale: float = 1.0         # fp8 / int8 cache only: real value = scale * stored value
    v_scale: float = 1.0
    max_num_tokens: int = 8192
    qk_norm: str = "none"        # per-head norm of q and new k before RoPE: "none", "rms", "layer"
    norm_eps: float = 1e-6       # float32 value handed to both sides
    out_fp8_scale: float = 0.0   # > 0: attention output as fp8 e4m3 codes, real = scale * code value

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads

    @property
    def rot_dim(self) -> int:
        return self.rotary_dim or self.head_dim


@dataclass
class Batch:
    """One in-flight batch: lengths, block table and lazily drawn values."""
    shape: Shape
    seed: int
    request_types: np.ndarray      # int32 [B]; CONTEXT rows first
    context_lengths: np.ndarray    # int32 [B]; n_r, tokens this request brings to the step
    sequence_lengths: np.ndarray   # int32 [B]; S_r = cached + n_r
    block_table: np.ndarray        # int32 [B, max_blocks_per_seq]; -1 where unused
    num_pool_blocks: int
    label: str = ""
    tree: bool = False             # generation requests' draft tokens form random trees

    # ---- lengths -------------------------------------------------------
    @property
    def num_requests(self) -> int:
        return int(self.request_types.shape[0])

    @property
    def past_lengths(self) -> np.ndarray:
        return (self.sequence_lengths - self.context_lengths).astype(np.int32)

    @property
    def num_tokens(self) -> int:
        return int(self.context_lengths.sum())

    @property
    def num_contexts(self) -> int:
        return int((self.request_types == CONTEXT).sum())

    @property
    def token_offsets(self) -> np.ndarray:
        """int64 [B+1]: request r owns packed rows offsets[r] .. offsets[r+1]-1."""
        return np.concatenate([[0], np.cumsum(self.context_lengths.astype(np.int64))])

    @property
    def max_context_length(self) -> int:
        ctx = self.context_lengths[self.request_types == CONTEXT]
        return int(ctx.max()) if ctx.size else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    # ---- values --------------------------------------------------------
    def _draw(self, tag: str, r: int, rows: int, heads: int) -> np.ndarray:
        x = _rng(self.seed, tag, r).standard_normal((rows, heads, self.shape.head_dim), dtype=np.float32)
        if self.shape.io_dtype == BF16:
            x = (x.view(np.uint32) >> 16).astype(np.uint16)
        elif self.shape.io_dtype != FP32:
            raise ValueError(self.shape.io_dtype)
        return x

    def new_q(self, r: int) -> np.ndarray:
        return self._draw("q", r, int(self.context_lengths[r]), self.shape.num_heads)

    def new_k(self, r: int) -> np.ndarray:
        return self._draw("k", r, int(self.context_lengths[r]), self.shape.num_kv_heads)

    def new_v(self, r: int) -> np.ndarray:
        return self._draw("v", r, int(self.context_lengths[r]), self.shape.num_kv_heads)

    def hist_k(self, r: int) -> np.ndarray:
        return self._draw("hist_k", r, int(self.past_lengths[r]), self.shape.num_kv_heads)

    def hist_v(self, r: int) -> np.ndarray:
        return self._draw("hist_v", r, int(self.past_lengths[r]), self.shape.num_kv_heads)

    def norm_params(self) -> dict:
        """Synthetic per-dimension norm parameters, float32 [head_dim] each: weights
        1 + N(0, 1)/4 and biases N(0, 1)/4 for q and for k (the biases apply to the
        "layer" form only)."""
        g = _rng(self.seed, "norm").standard_normal((4, self.shape.head_dim), dtype=np.float32)
        one = np.float32(1.0)
        quarter = np.float32(0.25)
        return {"q_weight": one + quarter * g[0], "k_weight": one + quarter * g[1],
                "q_bias": quarter * g[2], "k_bias": quarter * g[3]}

    def drawn_float32(self, which: str, r: int) -> np.ndarray:
        """Request r's draw ``which`` (new_k, hist_v, ...) as the float32 values it
        stands for: for bf16 the stored upper half widened back (a bit operation)."""
        x = getattr(self, which)(r)
        if self.shape.io_dtype == BF16:
            return (x.astype(np.uint32) << 16).view(np.float32)
        return x

    # ---- draft tokens ----------------------------------------------------
    def draft_parents(self, r: int) -> np.ndarray:
        """Parent of each new token of request r in its draft tree (-1 for token 0).  A
        chain (token i - 1) unless the batch has ``tree`` and r is a generation request:
        then token i's parent is drawn uniformly from tokens 0 .. i-1 (a tree whose
        tokens are listed parents first, as verification batches list them)."""
        n = int(self.context_lengths[r])
        par = np.arange(-1, n - 1, dtype=np.int64)
        if self.tree and int(self.request_types[r]) == GENERATION and n > 1:
            g = _rng(self.seed, "tree", r)
            par[1:] = [int(g.integers(0, i)) for i in range(1, n)]
        return par

    def spec_inputs(self) -> tuple[np.ndarray, np.ndarray]:
        """The draft-tree inputs in packed row order: int32 [N] position offsets (a
        generation row's depth in its request's tree; context rows 0) and uint32 [N, 2]
        packed masks (bit j of word j // 32 at bit j % 32 set when the row's token attends
        to new token j of its request: itself and its ancestors; context rows 0)."""
        off = np.zeros(self.num_tokens, np.int32)
        mask = np.zeros((self.num_tokens, 2), np.uint32)
        row = 0
        for r in range(self.num_requests):
            n = int(self.context_lengths[r])
            if int(self.request_types[r]) == GENERATION:
                par = self.draft_parents(r)
                depth = np.zeros(n, np.int64)
                anc = [0] * n
                for i in range(n):
                    depth[i] = 0 if par[i] < 0 else depth[par[i]] + 1
                    anc[i] = (1 << i) | (0 if par[i] < 0 else anc[par[i]])
                off[row:row + n] = depth
                for i in range(n):
                    mask[row + i, 0] = anc[i] & 0xFFFFFFFF
                    mask[row + i, 1] = anc[i] >> 32
            row += n
        return off, mask

    def packed(self, which: str) -> np.ndarray:
        """Concatenate new_q / new_k / new_v over requests in packed row order."""
        parts = [getattr(self, which)(r) for r in range(self.num_requests)]
        return np.concatenate(parts, axis=0)


def make_batch(shape: Shape, ctx=(), gen_past=(), seed: int = 0, pool_blocks_min: int = 0,
               label: str = "", gen_new=None, tree: bool = False) -> Batch:
    """Build a batch from explicit lengths.

    ``ctx`` is a sequence of (n_r, past_r) for context requests (their chunk
    and the tokens already cached before it); ``gen_past`` lists the cached
    length of each generation request.  A generation request brings one new
    token, or ``gen_new[j]`` tokens (the token plus draft tokens to verify),
    which form a chain, or random trees with ``tree``.
    """
    T = shape.tokens_per_block
    types, n, s = [], [], []
    for (nr, pr) in ctx:
        types.append(CONTEXT); n.append(int(nr)); s.append(int(pr) + int(nr))
    for j, pr in enumerate(gen_past):
        nr = 1 if gen_new is None else int(gen_new[j])
        types.append(GENERATION); n.append(nr); s.append(int(pr) + nr)
    types = np.asarray(types, np.int32)
    n = np.asarray(n, np.int32)
    s = np.asarray(s, np.int32)
    need = [(int(x) + T - 1) // T for x in s]
    total = int(sum(need))
    pool = max(total, int(pool_blocks_min))
    ids = _rng(seed, "blocks").permutation(pool)[:total].astype(np.int32)
    width = max(need) if need else 1
    table = np.full((len(need), max(width, 1)), -1, np.int32)
    pos = 0
    for r, k in enumerate(need):
        table[r, :k] = ids[pos:pos + k]
        pos += k
    return Batch(shape, seed, types, n, s, table, pool, label, tree)


CODE_MAX = {FP8_E4M3: 448.0, INT8: 127.0}


def kv_amax(batch: Batch) -> tuple[float, float]:
    """Largest magnitude over every drawn key, and over every drawn value (history and
    new tokens, as drawn, before any rotation)."""
    ak = av = 0.0
    for r in range(batch.num_requests):
        for which in ("hist_k", "new_k"):
            x = batch.drawn_float32(which, r)
            if x.size:
                ak = max(ak, float(np.max(np.abs(x))))
        for which in ("hist_v", "new_v"):
            x = batch.drawn_float32(which, r)
            if x.size:
                av = max(av, float(np.max(np.abs(x))))
    return ak, av


def fit_kv_scales(batch: Batch, kv_dtype: str, amax: tuple[float, float] | None = None) -> tuple[float, float]:
    """(s_K, s_V) that fit the batch's drawn values to the codes of ``kv_dtype``:
    amax|K| / the largest code magnitude, likewise for V; computed in fp64, rounded to
    float32.  A rotated new key can exceed amax|K| by up to sqrt(2) and then saturates."""
    ak, av = kv_amax(batch) if amax is None else amax
    cm = CODE_MAX[kv_dtype]
    return float(np.float32(ak / cm)), float(np.float32(av / cm))


def fitted(batch: Batch, kv_dtype: str | None = None) -> Batch:
    """The batch with its cache format (or ``kv_dtype``) and scales fitted to its data."""
    kv = kv_dtype or batch.shape.kv_dtype
    sk, sv = fit_kv_scales(batch, kv)
    return with_shape(batch, kv_dtype=kv, k_scale=sk, v_scale=sv)


# ---- the five workloads --------------------------------------------------
SHAPES = {
    1: Shape("tiny-mixed-fp32", 4, 2, 64, 16, FP32, FP32, 1.0e4),
    2: Shape("decode-mha-bf16", 32, 32, 128, 64, BF16, BF16, 1.0e4),
    # one batch of 8 x 2048 prompt tokens: its token budget is its own size
    3: Shape("prefill-gqa4-bf16", 32, 8, 128, 64, BF16, BF16, 5.0e5, max_num_tokens=16384),
    4: Shape("mixed-gqa8-bf16", 64, 8, 128, 64, BF16, BF16, 5.0e5),
    # K/V scaled to fit: fit_kv_scales(workload(5), FP8_E4M3), stored because fitting draws
    # all 0.8 G history values (a CPU test recomputes them)
    5: Shape("longdecode-gqa4-fp8kv", 32, 8, 128, 64, BF16, FP8_E4M3, 5.0e5,
             k_scale=0.013392857275903225, v_scale=0.01311383955180645),
}
# the same fit of workload 5's values to int8 codes (amax / 127)
W5_INT8_SCALES = (0.04724409431219101, 0.046259842813014984)


def _uniform_pasts(seed: int, count: int, lo: int, hi: int) -> list[int]:
    return [int(x) for x in _rng(seed, "lengths").integers(lo, hi, size=count, endpoint=True)]


def workload(k: int) -> Batch:
    """Full-size workload k (1..5)."""
    seed = 1000 + k
    sh = SHAPES[k]
    if k == 1:
        return make_batch(sh, ctx=[(37, 0)], gen_past=[50], seed=seed, pool_blocks_min=16, label="w1")
    if k == 2:
        return make_batch(sh, gen_past=_uniform_pasts(seed, 64, 512, 4096), seed=seed, label="w2")
    if k == 3:
        return make_batch(sh, ctx=[(2048, 0)] * 8, seed=seed, label="w3")
    if k == 4:
        return make_batch(sh, ctx=[(1024, 0), (1024, 1024), (1024, 2048), (1024, 3072)],
                          gen_past=_uniform_pasts(seed, 128, 256, 4096), seed=seed, label="w4")
    if k == 5:
        return make_batch(sh, gen_past=_uniform_pasts(seed, 16, 16384, 32768), seed=seed, label="w5")
    raise KeyError(k)


def small_workload(k: int, shape: Shape | None = None) -> Batch:
    """Workload k at a size the oracle finishes in seconds: same heads,
    head_dim, block size and dtypes; several blocks and a ragged tail.  ``shape``
    replaces workload k's shape (same lengths and seeds); without it, workload 5's
    fp8 scales are fitted to the small batch's own values."""
    seed = 2000 + k
    sh = SHAPES[k] if shape is None else shape
    if k == 1:
        return make_batch(sh, ctx=[(37, 0)], gen_past=[50], seed=seed, pool_blocks_min=16, label="s1")
    if k == 2:
        return make_batch(sh, gen_past=_uniform_pasts(seed, 6, 60, 700), seed=seed, label="s2")
    if k == 3:
        return make_batch(sh, ctx=[(300, 0), (190, 0)], seed=seed, label="s3")
    if k == 4:
        return make_batch(sh, ctx=[(128, 0), (192, 128), (100, 384)],
                          gen_past=_uniform_pasts(seed, 6, 20, 500), seed=seed, label="s4")
    if k == 5:
        b = make_batch(sh, gen_past=_uniform_pasts(seed, 4, 1000, 3000), seed=seed, label="s5")
        return b if shape is not None else fitted(b)
    raise KeyError(k)


WORKLOADS = (1, 2, 3, 4, 5)
SMALL_WORKLOADS = (1, 2, 3, 4, 5)


def with_shape(batch: Batch, **changes) -> Batch:
    """Same lengths and table with a modified shape (used by invariance tests)."""
    return replace(batch, shape=replace(batch.shape, **changes))
