"""Batches with explicitly given values (shared by CPU and GPU tests)."""
from __future__ import annotations

import numpy as np

from workloads import synth as W


class Crafted(W.Batch):
    """A batch whose per-request values are given explicitly (io representation)."""

    def set_values(self, q, k, v, hk, hv):
        self._vals = dict(q=q, k=k, v=v, hk=hk, hv=hv)
        return self

    def new_q(self, r):
        return self._vals["q"][r]

    def new_k(self, r):
        return self._vals["k"][r]

    def new_v(self, r):
        return self._vals["v"][r]

    def hist_k(self, r):
        return self._vals["hk"][r]

    def hist_v(self, r):
        return self._vals["hv"][r]


def as_crafted(b: W.Batch, shape=None, table=None, pool_blocks=None) -> Crafted:
    return Crafted(shape or b.shape, b.seed, b.request_types, b.context_lengths, b.sequence_lengths,
                   b.block_table if table is None else table,
                   b.num_pool_blocks if pool_blocks is None else pool_blocks, b.label)


def crafted(shape, ctx=(), gen_past=(), seed=0, fill=None, pool_blocks_min=0) -> Crafted:
    """Lengths from make_batch; values from fill(tag, r, rows, heads) (zeros by default)."""
    b = W.make_batch(shape, ctx=ctx, gen_past=gen_past, seed=seed, pool_blocks_min=pool_blocks_min)
    cb = as_crafted(b)
    H, Hkv, D = shape.num_heads, shape.num_kv_heads, shape.head_dim
    n, p = b.context_lengths, b.past_lengths
    dt = np.float32 if shape.io_dtype == W.FP32 else np.uint16
    fill = fill or (lambda tag, r, rows, heads: np.zeros((rows, heads, D), dt))
    R = range(b.num_requests)
    return cb.set_values([fill("q", r, int(n[r]), H) for r in R], [fill("k", r, int(n[r]), Hkv) for r in R],
                         [fill("v", r, int(n[r]), Hkv) for r in R], [fill("hk", r, int(p[r]), Hkv) for r in R],
                         [fill("hv", r, int(p[r]), Hkv) for r in R])


def copy_values(src: W.Batch, dst: Crafted) -> Crafted:
    """Give dst (same lengths) the generated values of src."""
    R = range(src.num_requests)
    return dst.set_values([src.new_q(r) for r in R], [src.new_k(r) for r in R], [src.new_v(r) for r in R],
                          [src.hist_k(r) for r in R], [src.hist_v(r) for r in R])
