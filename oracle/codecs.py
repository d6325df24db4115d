"""Storage codecs written from the public format definitions.  TEST INFRASTRUCTURE.

* bf16: the upper half of IEEE-754 binary32 -- 1 sign bit, 8 exponent bits
  (bias 127), 7 fraction bits, with subnormals, infinities and NaN.
* fp8 e4m3: the OCP 8-bit floating point "E4M3" format -- 1 sign bit,
  4 exponent bits (bias 7), 3 fraction bits, subnormals, no infinities,
  NaN only at S.1111.111, largest finite magnitude 1.75 * 2^8 = 448.
* fp32: IEEE-754 binary32; the fp64 -> fp32 step uses numpy's IEEE cast.
* int8: two's-complement 8-bit integer codes, -128 .. 127; the code's value is the
  integer itself.

Every encoder rounds an fp64 value DIRECTLY to the target format, round to
nearest, ties to even, in one step (never via an intermediate format).  The
fp8 encoder saturates finite overflow and infinities to +-448 ("satfinite"); the
int8 encoder rounds to the nearest integer (ties to even) and saturates to
-128 .. 127, storing NaN as 0.

The KV-cache quantisation follows the INT8/FP8 KV cache passage of
"TensorRT-LLM 1.0 study notes", section 6.4: values are quantised on write with
the scale kv_scale_orig_quant and dequantised on read with kv_scale_quant_orig.
Reading taken: one fp32 per-tensor scale s = kv_scale_quant_orig per K and V;
the write multiplies by 1/s computed in fp64, the read multiplies by s.  The
passage names the INT8 KV cache as the one that only compresses the stored
format (dequantised on read); the same pair of scales serves fp8 and int8.
"""
from __future__ import annotations

import numpy as np

FP32, BF16, FP8_E4M3, INT8 = "fp32", "bf16", "fp8_e4m3", "int8"


# ---------------------------------------------------------------- bf16
def bf16_to_f64(bits) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) field by field."""
    b = np.asarray(bits).astype(np.int64)
    neg = ((b >> 15) & 1) == 1
    e = (b >> 7) & 0xFF
    m = b & 0x7F
    with np.errstate(invalid="ignore"):
        val = np.where(e == 0, np.ldexp(m.astype(np.float64), -133),
                       np.ldexp((128 + m).astype(np.float64), (e - 134).astype(np.int32)))
        val = np.where(e == 255, np.where(m == 0, np.inf, np.nan), val)
    return np.where(neg, -val, val)


def f64_to_bf16(x) -> np.ndarray:
    """Round fp64 to the nearest bf16 (ties to even); returns uint16 bits."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    out = np.zeros(x.shape, dtype=np.int64)
    finite_nz = np.isfinite(a) & (a > 0)
    af = np.where(finite_nz, a, 1.0)
    _, fe = np.frexp(af)
    E = fe.astype(np.int64) - 1                      # a = 1.f * 2^E
    normal = E >= -126
    # quantum: 2^(E-7) in the normal range, 2^-133 below it
    qexp = np.where(normal, E - 7, -133)
    q = np.rint(np.ldexp(af, (-qexp).astype(np.int32))).astype(np.int64)
    carry = normal & (q == 256)
    E = np.where(carry, E + 1, E)
    q = np.where(carry, 128, q)
    bits_normal = ((E + 127) << 7) | (q - 128)
    bits_normal = np.where(E + 127 >= 255, 0x7F80, bits_normal)   # overflow -> inf
    bits_sub = q                                                  # q == 128 is the smallest normal
    out = np.where(finite_nz, np.where(normal, bits_normal, bits_sub), out)
    out = np.where(np.isinf(a), 0x7F80, out)
    out = np.where(np.isnan(a), 0x7FC0, out)
    out = np.where(np.signbit(x) & ~np.isnan(x), out | 0x8000, out)
    return out.astype(np.uint16)


# ---------------------------------------------------------------- fp8 e4m3 (OCP)
E4M3_MAX = 448.0


def e4m3_to_f64(codes) -> np.ndarray:
    """Decode OCP E4M3 codes (uint8) field by field."""
    c = np.asarray(codes).astype(np.int64)
    neg = ((c >> 7) & 1) == 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp((8 + m).astype(np.float64), (e - 10).astype(np.int32)))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return np.where(neg, -val, val)


def f64_to_e4m3(x) -> np.ndarray:
    """Round fp64 to the nearest E4M3 value (ties to even), saturating to +-448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    finite_nz = np.isfinite(a) & (a > 0)
    af = np.where(finite_nz, a, 1.0)
    _, fe = np.frexp(af)
    E = fe.astype(np.int64) - 1
    normal = E >= -6
    qexp = np.where(normal, E - 3, -9)
    q = np.rint(np.ldexp(af, (-qexp).astype(np.int32))).astype(np.int64)
    carry = normal & (q == 16)
    E = np.where(carry, E + 1, E)
    q = np.where(carry, 8, q)
    sat = normal & ((E > 8) | ((E == 8) & (q - 8 > 6)))
    code_normal = np.where(sat, 0x7E, ((E + 7) << 3) | (q - 8))
    code = np.where(normal, code_normal, q)           # subnormal: q in 0..8, 8 = smallest normal
    code = np.where(finite_nz, code, 0)
    code = np.where(np.isinf(a), 0x7E, code)
    code = np.where(np.isnan(a), 0x7F, code)
    code = np.where(np.signbit(x), code | 0x80, code)
    return code.astype(np.uint8)


# ---------------------------------------------------------------- int8
INT8_MIN, INT8_MAX = -128, 127


def int8_to_f64(codes) -> np.ndarray:
    """Decode int8 codes (int8, or their uint8 bit patterns) to their integer value."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    return np.where(c >= 128, c - 256, c).astype(np.float64)


def f64_to_int8(x) -> np.ndarray:
    """Round fp64 to the nearest integer (ties to even), saturate to -128 .. 127; NaN -> 0."""
    x = np.asarray(x, dtype=np.float64)
    r = np.rint(np.where(np.isnan(x), 0.0, x))
    return np.clip(r, INT8_MIN, INT8_MAX).astype(np.int8)


# ---------------------------------------------------------------- dispatch
def storage_dtype(fmt: str):
    return {FP32: np.float32, BF16: np.uint16, FP8_E4M3: np.uint8, INT8: np.int8}[fmt]


def encode(values, fmt: str, scale: float = 1.0) -> np.ndarray:
    """fp64 values -> stored representation of ``fmt``.

    For fp8 and int8 the value is first multiplied by 1/scale (fp64), i.e. quantised
    with kv_scale_orig_quant = 1/kv_scale_quant_orig.
    """
    v = np.asarray(values, dtype=np.float64)
    if fmt == FP32:
        return v.astype(np.float32)
    if fmt == BF16:
        return f64_to_bf16(v)
    if fmt == FP8_E4M3:
        inv = 1.0 / np.float64(np.float32(scale))
        return f64_to_e4m3(v * inv)
    if fmt == INT8:
        inv = 1.0 / np.float64(np.float32(scale))
        return f64_to_int8(v * inv)
    raise ValueError(fmt)


def decode(stored, fmt: str, scale: float = 1.0) -> np.ndarray:
    """Stored representation -> fp64 value (fp8, int8: scale * code value)."""
    if fmt == FP32:
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    if fmt == BF16:
        return bf16_to_f64(stored)
    if fmt == FP8_E4M3:
        return np.float64(np.float32(scale)) * e4m3_to_f64(stored)
    if fmt == INT8:
        return np.float64(np.float32(scale)) * int8_to_f64(stored)
    raise ValueError(fmt)
