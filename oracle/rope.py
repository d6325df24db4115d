"""Rotary position embedding: GPT-NeoX ("rotate half") and interleaved-pair forms.
TEST INFRASTRUCTURE.

"TensorRT-LLM source analysis report", section 1.1, lists rotary_embedding
among the attention parameters and names GPT-NeoX among the RoPE variants; it
gives no formula.  "TensorRT-LLM source teardown part 1", AttentionMetadata
section, defines position_ids as each token's position within its sequence.
Readings taken (no page states them):

* a token at 0-based absolute position m of its sequence is rotated by angle
  m * theta_j on the pair (x_j, x_{j + R/2}), j = 0 .. R/2 - 1, where R is the
  rotary dimension (the head dimension unless stated otherwise) and
  theta_j = base ** (-2 j / R); dimensions >= R pass through unchanged;
* rotation: y_j = x_j cos - x_{j+R/2} sin,  y_{j+R/2} = x_{j+R/2} cos + x_j sin,
  each output as two fp64 products and one fp64 add/subtract (numpy evaluates
  them as separate IEEE operations, no fused multiply-add);
* applied to every query head and every new key head; values are not rotated.

The same section lists further RoPE variants by name (ChatGLM, CogVLM) without a
formula.  The plainest layout they differ by is the pairing: the interleaved form
rotates (x_{2j}, x_{2j+1}) by the same angle m * theta_j (the GPT-J layout; applied to
a leading part of the head, R < D, it is the layout of the ChatGLM models).  Same
tables, same fp64 arithmetic.
"""
from __future__ import annotations

import numpy as np


def neox_inv_freq(base: float, rot_dim: int) -> np.ndarray:
    j = np.arange(rot_dim // 2, dtype=np.float64)
    return np.power(np.float64(base), -(2.0 * j) / np.float64(rot_dim))


def neox_tables(base: float, rot_dim: int, max_pos: int):
    """fp64 cos/sin tables [max_pos, rot_dim/2] of angle m * theta_j."""
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * neox_inv_freq(base, rot_dim)[None, :]
    return np.cos(ang), np.sin(ang)


def rope_neox(x: np.ndarray, positions: np.ndarray, cos_t: np.ndarray, sin_t: np.ndarray,
              rot_dim: int) -> np.ndarray:
    """Rotate x [n, heads, D] (fp64) at positions [n] with tables [P, rot_dim/2]."""
    x = np.asarray(x, dtype=np.float64)
    half = rot_dim // 2
    c = cos_t[positions][:, None, :]
    s = sin_t[positions][:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:rot_dim]
    y = x.copy()
    y[..., :half] = x1 * c - x2 * s
    y[..., half:rot_dim] = x2 * c + x1 * s
    return y


def rope_gptj(x: np.ndarray, positions: np.ndarray, cos_t: np.ndarray, sin_t: np.ndarray,
              rot_dim: int) -> np.ndarray:
    """Interleaved pairs: rotate (x_{2j}, x_{2j+1}) by m * theta_j, j < rot_dim/2."""
    x = np.asarray(x, dtype=np.float64)
    c = cos_t[positions][:, None, :]
    s = sin_t[positions][:, None, :]
    x1 = x[..., 0:rot_dim:2]
    x2 = x[..., 1:rot_dim:2]
    y = x.copy()
    y[..., 0:rot_dim:2] = x1 * c - x2 * s
    y[..., 1:rot_dim:2] = x2 * c + x1 * s
    return y


def rope_apply(style: str, x, positions, cos_t, sin_t, rot_dim: int):
    """style 'neox' (pairs j, j + R/2), 'gptj' (pairs 2j, 2j + 1) or 'none' (no rotation:
    the values as given)."""
    if style == "none":
        return np.array(x, dtype=np.float64)
    if style == "neox":
        return rope_neox(x, positions, cos_t, sin_t, rot_dim)
    if style == "gptj":
        return rope_gptj(x, positions, cos_t, sin_t, rot_dim)
    raise ValueError(f"unknown RoPE style {style!r}")
