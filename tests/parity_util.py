"""Shared checks for the GPU parity tests (HIP path vs the CPU oracle)."""
from __future__ import annotations

import numpy as np

from oracle import codecs

# Attention bars.  bf16 io: max-abs 2e-2 and mean-abs 2e-3; fp8 cache: max-abs 6e-2.
# fp32 io/cache is held to 1e-4.  An int8 cache (and an fp8 cache read by the fp32 io
# path) is held to the bar of the format its codes are widened to without loss (bf16
# on the bf16-io path, fp32 on the fp32 path): both sides attend over the same dequantised values, so only the attention
# arithmetic differs, as for that format.  Because outputs shrink as contexts grow,
# every case must also pass a relative L2 error <= 1e-2 and a per-row cosine >= 0.999.
BARS = {
    ("fp32", "fp32"): dict(max_abs=1e-4, mean_abs=1e-5),
    ("bf16", "bf16"): dict(max_abs=2e-2, mean_abs=2e-3),
    ("bf16", "fp8_e4m3"): dict(max_abs=6e-2, mean_abs=6e-3),
    ("bf16", "int8"): dict(max_abs=2e-2, mean_abs=2e-3),
    ("fp32", "int8"): dict(max_abs=1e-4, mean_abs=1e-5),
    ("fp32", "fp8_e4m3"): dict(max_abs=1e-4, mean_abs=1e-5),
}
REL_L2 = 1e-2
MIN_COS = 0.999


def io_values(bits: np.ndarray, io_dtype: str) -> np.ndarray:
    return codecs.decode(bits, io_dtype)


def compare_attention(got_bits: np.ndarray, ref: np.ndarray, shape, label: str = "") -> dict:
    """got_bits: GPU output in io representation [rows, heads, D]; ref: oracle fp64."""
    got = io_values(got_bits, shape.io_dtype)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{label}: non-finite GPU outputs"
    err = np.abs(got - ref)
    bars = BARS[(shape.io_dtype, shape.kv_dtype)]
    stats = dict(max_abs=float(err.max()), mean_abs=float(err.mean()),
                 rel_l2=float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)))
    g2 = got.reshape(-1, got.shape[-1])
    r2 = ref.reshape(-1, ref.shape[-1])
    cos = np.sum(g2 * r2, axis=1) / np.maximum(np.linalg.norm(g2, axis=1) * np.linalg.norm(r2, axis=1), 1e-300)
    stats["min_cos"] = float(cos.min())
    msg = f"{label}: {stats}"
    assert stats["max_abs"] <= bars["max_abs"], msg
    assert stats["mean_abs"] <= bars["mean_abs"], msg
    assert stats["rel_l2"] <= REL_L2, msg
    assert stats["min_cos"] >= MIN_COS, msg
    return stats


def bits_of(arr: np.ndarray) -> np.ndarray:
    return arr.view({4: np.uint32, 2: np.uint16, 1: np.uint8}[arr.dtype.itemsize])


def assert_bits_equal(got: np.ndarray, want: np.ndarray, label: str):
    g, w = bits_of(np.ascontiguousarray(got)), bits_of(np.ascontiguousarray(want))
    assert g.shape == w.shape, (label, g.shape, w.shape)
    bad = np.nonzero(g != w)
    n = bad[0].size
    if n:
        first = tuple(int(x[0]) for x in bad)
        raise AssertionError(f"{label}: {n} of {g.size} elements differ; first at {first}: "
                             f"got {int(g[first]):#x} want {int(w[first]):#x}")


def e4m3_ordinal(codes: np.ndarray) -> np.ndarray:
    """Position of each e4m3 code on the number line (codes are sign-magnitude)."""
    c = np.asarray(codes).astype(np.int32)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def compare_fp8_output(got_codes: np.ndarray, ref: np.ndarray, shape, label: str = "",
                       check_values: bool = True) -> dict:
    """got_codes: GPU fp8 output codes [rows, heads, D]; ref: oracle fp64 attention output.

    The GPU rounds its fp32 result, the oracle's value is fp64: the two can straddle a
    rounding boundary, and near zero the attention error spans several of the small e4m3
    steps.  So the check is that every code is the nearest-even rounding of some value
    within ``tol`` of the oracle's: the rounding is monotone, so the code must lie between
    the codes of (ref - tol) / s and (ref + tol) / s.  tol is twice the mean-abs bar of the
    io and cache formats; it bounds every element by half an e4m3 step at its magnitude
    (up to 2^-4 relative) plus tol, so no fixed absolute bar applies.  Unless the scale
    saturates outputs on purpose (``check_values=False``), the decoded output must also
    have relative L2 error <= 5e-2 (e4m3 rounding alone gives about 2^-4/sqrt(3)) and
    per-row cosine >= 0.995.
    """
    s = shape.out_fp8_scale
    bars = BARS[(shape.io_dtype, shape.kv_dtype)]
    tol = 2 * bars["mean_abs"]
    got = np.asarray(got_codes).astype(np.uint8)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert not np.any((got & 0x7F) == 0x7F), f"{label}: NaN codes"
    lo = e4m3_ordinal(codecs.encode(ref - tol, codecs.FP8_E4M3, s))
    hi = e4m3_ordinal(codecs.encode(ref + tol, codecs.FP8_E4M3, s))
    og = e4m3_ordinal(got)
    bad = np.nonzero((og < lo) | (og > hi))
    exact = float(np.mean(got == codecs.encode(ref, codecs.FP8_E4M3, s)))
    msg = f"{label}: {bad[0].size} codes outside the rounding interval; exact {exact:.4f}"
    assert bad[0].size == 0, msg + (f"; first at {tuple(int(x[0]) for x in bad)}" if bad[0].size else "")
    dec = codecs.decode(got, codecs.FP8_E4M3, s)
    err = np.abs(dec - ref)
    stats = dict(exact_codes=exact, max_abs=float(err.max()), mean_abs=float(err.mean()),
                 rel_l2=float(np.linalg.norm(dec - ref) / max(np.linalg.norm(ref), 1e-300)))
    g2, r2 = dec.reshape(-1, dec.shape[-1]), ref.reshape(-1, ref.shape[-1])
    cos = np.sum(g2 * r2, axis=1) / np.maximum(np.linalg.norm(g2, axis=1) * np.linalg.norm(r2, axis=1), 1e-300)
    stats["min_cos"] = float(cos.min())
    msg = f"{label}: {stats}"
    if check_values:
        assert stats["rel_l2"] <= 5e-2 and stats["min_cos"] >= 0.995, msg
    return stats
