"""Pins of the oracle's storage codecs (bf16, OCP fp8 e4m3, int8, fp32)."""
import numpy as np
import pytest
import torch

from oracle import codecs as C

ALL16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)
ALL8 = np.arange(256, dtype=np.uint16).astype(np.uint8)


def _finite16():
    v = C.bf16_to_f64(ALL16)
    return ALL16[np.isfinite(v)]


# ------------------------------------------------------------------ bf16
def test_bf16_decode_all_patterns_match_binary32_upper_half():
    # bf16 is the upper half of IEEE binary32: decode through numpy's float32.
    ref = (ALL16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    got = C.bf16_to_f64(ALL16)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_bf16_encode_roundtrip_every_finite_pattern():
    b = _finite16()
    assert np.array_equal(C.f64_to_bf16(C.bf16_to_f64(b)), b)


def test_bf16_encode_ties_to_even_and_neighbours():
    b = _finite16()
    b = b[(b & 0x7FFF) < 0x7F7F]                         # those with a finite successor in magnitude
    lo = C.bf16_to_f64(b)
    hi = C.bf16_to_f64((b + 1).astype(np.uint16))       # next magnitude, same sign
    mid = (lo + hi) / 2                                  # exact in fp64
    want = np.where((b & 1) == 0, b, (b + 1).astype(np.uint16))
    assert np.array_equal(C.f64_to_bf16(mid), want)
    above = np.nextafter(np.abs(mid), np.inf) * np.sign(mid + 0.0)
    below = np.nextafter(np.abs(mid), 0) * np.sign(mid + 0.0)
    nz = mid != 0
    assert np.array_equal(C.f64_to_bf16(above[nz]), (b + 1).astype(np.uint16)[nz])
    assert np.array_equal(C.f64_to_bf16(below[nz]), b[nz])


def test_bf16_encode_matches_torch_on_binary32_inputs():
    # torch's float32 -> bfloat16 cast rounds to nearest even; on inputs that are
    # exact binary32 values it is a direct rounding, the same as ours.
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32),
                        (rng.standard_normal(20000) * 1e-39).astype(np.float32),   # subnormals
                        (rng.standard_normal(20000) * 1e38).astype(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = C.f64_to_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_encode_is_nearest_on_random_fp64():
    rng = np.random.default_rng(8)
    x = rng.standard_normal(100000) * np.exp2(rng.integers(-140, 120, 100000))
    b = C.f64_to_bf16(x)
    y = C.bf16_to_f64(b)
    up = C.bf16_to_f64((b + 1).astype(np.uint16))
    dn = C.bf16_to_f64(np.where((b & 0x7FFF) == 0, b ^ 0x8000, b - 1).astype(np.uint16))
    err = np.abs(x - y)
    fin_up = np.isfinite(up)
    assert np.all(err[fin_up] <= np.abs(x - up)[fin_up])
    assert np.all(err <= np.abs(x - dn))


def test_bf16_special_values():
    assert C.f64_to_bf16(np.array([0.0]))[0] == 0x0000
    assert C.f64_to_bf16(np.array([-0.0]))[0] == 0x8000
    assert C.f64_to_bf16(np.array([np.inf]))[0] == 0x7F80
    assert C.f64_to_bf16(np.array([-np.inf]))[0] == 0xFF80
    assert C.f64_to_bf16(np.array([np.nan]))[0] == 0x7FC0
    big = C.bf16_to_f64(np.array([0x7F7F], np.uint16))[0]
    half_ulp = 2.0 ** (127 - 8)
    assert C.f64_to_bf16(np.array([big + half_ulp]))[0] == 0x7F80        # tie goes to even = inf
    assert C.f64_to_bf16(np.array([np.nextafter(big + half_ulp, 0)]))[0] == 0x7F7F
    assert C.f64_to_bf16(np.array([2.0 ** -134]))[0] == 0x0000          # tie to even (0)
    assert C.f64_to_bf16(np.array([3 * 2.0 ** -134]))[0] == 0x0002      # 1.5 quanta -> 2


# ------------------------------------------------------------------ fp8 e4m3
def test_e4m3_decode_matches_torch_float8_e4m3fn():
    ref = torch.from_numpy(ALL8.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = C.e4m3_to_f64(ALL8)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_e4m3_format_landmarks():
    d = C.e4m3_to_f64(ALL8)
    assert d[0x7E] == 448.0 and d[0xFE] == -448.0          # largest finite
    assert d[0x08] == 2.0 ** -6                              # smallest normal
    assert d[0x07] == 0.875 * 2.0 ** -6                      # largest subnormal
    assert d[0x01] == 2.0 ** -9                              # smallest subnormal
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])           # the only NaNs
    assert np.sum(np.isnan(d)) == 2
    assert np.all(np.diff(d[0x00:0x7F]) > 0)                 # codes ordered by value
    assert np.signbit(d[0x80]) and d[0x80] == 0


def test_e4m3_encode_roundtrip_and_ties():
    pos = np.arange(0x00, 0x7F, dtype=np.uint16).astype(np.uint8)   # 0 .. 448
    for sign in (0x00, 0x80):
        c = (pos | sign).astype(np.uint8)
        assert np.array_equal(C.f64_to_e4m3(C.e4m3_to_f64(c)), c)
    lo = C.e4m3_to_f64(pos[:-1])
    hi = C.e4m3_to_f64(pos[1:])
    mid = (lo + hi) / 2
    want = np.where((pos[:-1] & 1) == 0, pos[:-1], pos[1:])
    assert np.array_equal(C.f64_to_e4m3(mid), want)
    assert np.array_equal(C.f64_to_e4m3(np.nextafter(mid, np.inf)), pos[1:])
    assert np.array_equal(C.f64_to_e4m3(np.nextafter(mid, 0)), pos[:-1])


def test_e4m3_saturation_and_specials():
    enc = lambda v: int(C.f64_to_e4m3(np.array([v]))[0])
    assert enc(448.0) == 0x7E
    assert enc(463.99) == 0x7E and enc(464.0) == 0x7E and enc(500.0) == 0x7E
    assert enc(1e30) == 0x7E and enc(np.inf) == 0x7E and enc(-np.inf) == 0xFE
    assert enc(np.nan) & 0x7F == 0x7F
    assert enc(0.0) == 0x00 and enc(-0.0) == 0x80
    assert enc(2.0 ** -10) == 0x00        # half of the smallest subnormal: tie to even 0
    assert enc(1.5 * 2.0 ** -9) == 0x02   # tie between codes 1 and 2 -> even


def test_e4m3_encode_matches_torch_in_range():
    # torch's float32 -> float8_e4m3fn cast is round-to-nearest-even inside the
    # finite range; compare on binary32 inputs below the saturation point.
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(200000) * 60).astype(np.float32)
    x = x[np.abs(x) < 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = C.f64_to_e4m3(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_fp8_scaled_codec_is_quantise_on_write_dequantise_on_read():
    s = 2.0 ** -6
    x = np.array([0.0, 1.0, -3.25, 7.0, 100.0])
    codes = C.encode(x, C.FP8_E4M3, s)
    assert np.array_equal(codes, C.f64_to_e4m3(x * 64.0))
    back = C.decode(codes, C.FP8_E4M3, s)
    assert back[1] == 1.0 and back[2] == -3.25 and back[3] == 7.0
    assert back[4] == 448.0 * s                                    # saturated


# ------------------------------------------------------------------ int8
def test_int8_decode_matches_torch_int8_view():
    # every byte pattern read as a two's-complement int8 by torch's own dtype view
    ref = torch.from_numpy(ALL8.copy()).view(torch.int8).to(torch.float64).numpy()
    assert np.array_equal(C.int8_to_f64(ALL8), ref)
    assert np.array_equal(C.int8_to_f64(ALL8.view(np.int8)), ref)
    assert C.int8_to_f64(np.uint8(0x80)) == -128 and C.int8_to_f64(np.uint8(0x7F)) == 127


def test_int8_encode_roundtrip_ties_and_saturation():
    codes = ALL8.view(np.int8)
    assert np.array_equal(C.f64_to_int8(C.int8_to_f64(codes)), codes)
    enc = lambda v: int(C.f64_to_int8(np.array([v]))[0])
    # ties go to the even neighbour, on both signs
    assert [enc(v) for v in (0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5)] == [0, 2, 2, 0, -2, -2, 126]
    assert enc(np.nextafter(0.5, 1.0)) == 1 and enc(np.nextafter(2.5, 0.0)) == 2
    # saturation at the ends of the int8 range; NaN stores 0
    assert [enc(v) for v in (127.49, 127.5, 128.0, 1e30, np.inf)] == [127, 127, 127, 127, 127]
    assert [enc(v) for v in (-128.5, -129.0, -1e30, -np.inf)] == [-128, -128, -128, -128]
    assert enc(np.nan) == 0


def test_int8_encode_matches_torch_round_half_even_in_range():
    # torch.round rounds half to even; inside the range no saturation applies
    x = np.random.default_rng(11).uniform(-127.9, 127.4, 20000)
    x[:200] = np.round(x[:200]) + 0.5                              # exact ties
    x = x[(x > -128.5) & (x < 127.5)]
    ref = torch.round(torch.from_numpy(x)).to(torch.int8).numpy()
    assert np.array_equal(C.f64_to_int8(x), ref)


def test_int8_scaled_codec_is_quantise_on_write_dequantise_on_read():
    s = 2.0 ** -5
    x = np.array([0.0, 1.0, -3.25, 3.96875, 100.0, -100.0, 0.015625, 0.046875])
    codes = C.encode(x, C.INT8, s)
    assert codes.dtype == np.int8
    assert list(codes) == [0, 32, -104, 127, 127, -128, 0, 2]     # 0.5 and 1.5 quanta tie to even
    back = C.decode(codes, C.INT8, s)
    assert list(back) == [0.0, 1.0, -3.25, 3.96875, 3.96875, -4.0, 0.0, 0.0625]


def test_fp32_codec():
    x = np.array([1.0 + 2.0 ** -30, 1.0 + 3 * 2.0 ** -24, -2.5])
    enc = C.encode(x, C.FP32)
    assert enc.dtype == np.float32
    assert enc[0] == np.float32(1.0)
    assert enc[1] == np.float32(1.0 + 4 * 2.0 ** -24)          # tie at 1.5 ulp rounds to even
    assert np.array_equal(C.decode(enc, C.FP32), enc.astype(np.float64))
