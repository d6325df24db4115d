"""Per-head normalisation of queries and keys before RoPE.  TEST INFRASTRUCTURE.

"TensorRT-LLM source analysis report", section 1.1, lists a "QK LayerNorm" -- layer
normalisation of the queries and keys -- among the attention features, and
"TensorRT-LLM source teardown part 1", in its listing of the kernel directory, names a
fused QK-norm + RoPE kernel (next to grouped RMSNorm kernels).  No page gives a formula.
Readings taken:

* the norm runs over the head dimension of each query head and each new key head,
  before the rotation (the fused kernel's name puts the norm first); values are not
  normalised;
* two forms: "layer" -- subtract the mean, divide by the standard deviation, then a
  per-dimension weight and bias (the report's name); "rms" -- divide by the root mean
  square, then a per-dimension weight (the RMS form of the grouped-RMSNorm kernels);
  one weight (and bias) vector of length head_dim for all query heads, another for
  all key heads;
* eps is added to the variance (mean square) under the square root;
* arithmetic, in fp64 and in this order (no fused multiply-add): mu = (sum_j x_j) / D
  for "layer" (0 for "rms"); d_j = x_j - mu; var = (sum_j d_j * d_j) / D, both sums
  accumulated in index order j = 0 .. D-1; inv = 1 / sqrt(var + eps);
  y_j = (d_j * inv) * w_j (+ b_j).  The rotation then takes y exactly as it takes x
  without the norm, and the stored value is y rotated and rounded once.
"""
from __future__ import annotations

import numpy as np


def qk_norm(x: np.ndarray, kind: str, weight: np.ndarray, bias: np.ndarray | None, eps: float) -> np.ndarray:
    """Normalise x [..., D] (fp64) over its last axis; returns fp64 of the same shape."""
    if kind == "none":
        return np.asarray(x, dtype=np.float64)
    if kind not in ("rms", "layer"):
        raise ValueError(f"unknown norm {kind!r}")
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    w = np.asarray(weight, dtype=np.float64)
    if kind == "layer":
        mu = np.cumsum(x, axis=-1)[..., -1:] / np.float64(D)      # cumsum: index-order sums
    else:
        mu = np.zeros(x.shape[:-1] + (1,), np.float64)
    d = x - mu
    var = np.cumsum(d * d, axis=-1)[..., -1:] / np.float64(D)
    inv = np.float64(1.0) / np.sqrt(var + np.float64(eps))
    y = (d * inv) * w
    if kind == "layer":
        y = y + np.asarray(bias, dtype=np.float64)
    return y
