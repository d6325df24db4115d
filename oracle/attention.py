"""Scaled dot-product attention with GQA and a causal mask.  TEST INFRASTRUCTURE.

Follows "TensorRT-LLM 1.0 study notes", sections 6.1-6.3: a context-phase row
attends causally over its request's cached tokens and its own chunk up to and
including itself; a generation-phase query (one token) attends to every cached
token of its request, which after the step's append includes itself.  GQA
("TensorRT-LLM source analysis report", section 1.1: attention head grouping)
is read as contiguous groups: query head h uses KV head h // (H / Hkv).  The
softmax scale is 1/sqrt(head_dim) unless given.  No page gives the formula;
the plain definition O = softmax(scale * q K^T + mask) V is used, in fp64, with
the row maximum subtracted before exponentiation (an identity of softmax).
"""
from __future__ import annotations

import numpy as np


def softmax_rows(x: np.ndarray) -> np.ndarray:
    """Row-wise softmax of an fp64 matrix; -inf entries get weight 0."""
    m = np.max(x, axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, positions: np.ndarray,
           scale: float | None = None, heads=None) -> np.ndarray:
    """O[i, h] = sum_t softmax_t(scale * <q[i,h], K[t,g]>) V[t,g] over t <= positions[i].

    q: [n, H, D]; K, V: [L, Hkv, D] (contiguous, position t at index t);
    positions: [n] absolute position of each query row (L > max(positions)).
    ``heads`` optionally restricts the computed query heads (output keeps only
    those, in the given order).
    """
    L = np.asarray(K).shape[0]
    positions = np.asarray(positions, dtype=np.int64)
    visible = np.arange(L)[None, :] <= positions[:, None]        # [n, L]
    return attend_visible(q, K, V, visible, scale=scale, heads=heads)


def attend_visible(q: np.ndarray, K: np.ndarray, V: np.ndarray, visible: np.ndarray,
                   scale: float | None = None, heads=None) -> np.ndarray:
    """O[i, h] = sum over visible t of softmax_t(scale * <q[i,h], K[t,g]>) V[t,g].

    The general mask: ``visible`` [n, L] says which cache positions row i attends to
    (every row sees at least one).  Draft tokens verified as a tree ("TensorRT-LLM
    source analysis report", section 1.4: position offsets and a packed mask) see the
    cached tokens and, among the new ones, what their mask row names.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    n, H, D = q.shape
    L, Hkv, _ = K.shape
    G = H // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(np.float64(D))
    heads = list(range(H)) if heads is None else list(heads)
    masked = ~np.asarray(visible, dtype=bool)                    # [n, L]
    out = np.empty((n, len(heads), D), dtype=np.float64)
    for oi, h in enumerate(heads):
        g = h // G
        s = scale * (q[:, h, :] @ K[:, g, :].T)
        s = np.where(masked, -np.inf, s)
        out[:, oi, :] = softmax_rows(s) @ V[:, g, :]
    return out
