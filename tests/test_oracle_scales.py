"""Pins for the oracle's scaled 8-bit decode and its fp32 bit decode.

The 8-bit caches (P1 "İlgili Teknikler", FP8 cache bullet: keys and values
kept in 8 bits) store a code c that means value(c) * scale, with one fp32
scale per pool or one per KV head.  These tests fix that multiply exactly:

* ``fp8.decode(c, s)`` and ``fp8.decode_e5m2(c, s)`` equal, for every code
  and for scales across the fp32 range (subnormal, tiny, inexact decimals,
  huge), the exact rational product of torch's value of the code and the
  scale rounded to fp32 by Python's ``struct`` (round to nearest even).  The
  product is exact in float64 (a 4- or 3-bit significand times a 24-bit one),
  so equality is required, not closeness.
* ``decode(quantize(x, s), s)`` returns x within half an 8-bit ulp times the
  scale (plus the fp32 rounding of x / s) for x inside the format's range.
* ``tests.parity.widen`` applies a per-head scale array along the KV-head
  axis of ``[..., Hkv, D]`` storage.
* ``numerics.f32_bits_to_f64`` equals torch's bit view and a field-by-field
  decode of IEEE binary32 (subnormals, signed zeros, infinities, NaN
  payloads).

Mutants of each (divide by the scale, the scale kept in float64 instead of
fp32, the per-head scale on the wrong axis, a value cast instead of a bit
view) must fail these pins.
"""

from __future__ import annotations

import math
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import fp8, numerics
from tests import parity

# scales across the fp32 range: exact and inexact decimals, a subnormal fp32,
# the smallest normal, large values, and amax/448-style scales
SCALES = [1.0, 0.1, 3.0, 1.0 / 448.0, 0.0117, 1e-40, 1.1754943508222875e-38, 7.5e-5, 2.5e30,
          123456.789, 3.4e38 / 448.0]


def fp32(x: float) -> float:
    """x rounded to IEEE binary32 (nearest even) by the struct module."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def torch_codes(fmt: str) -> np.ndarray:
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    dt = torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2
    return codes.view(dt).to(torch.float64).numpy()


def expected_scaled(fmt: str, scale: float) -> list:
    """Exact value of every code times fp32(scale): a Fraction, or the float
    NaN / +-inf for the special codes."""
    s = Fraction(fp32(scale))
    out = []
    for v in torch_codes(fmt):
        if math.isnan(v) or math.isinf(v):
            out.append(v * float(s))            # NaN stays NaN; inf keeps its sign (s > 0)
        else:
            out.append(Fraction(float(v)) * s)
    return out


def check_scaled_decode(decode, fmt: str):
    codes = np.arange(256, dtype=np.uint8)
    for scale in SCALES:
        got = decode(codes, scale)
        assert got.dtype == np.float64
        for c, (g, e) in enumerate(zip(got, expected_scaled(fmt, scale))):
            if isinstance(e, float):
                if math.isnan(e):
                    assert math.isnan(g), (fmt, scale, c)
                else:
                    assert g == e, (fmt, scale, c)
            else:
                assert Fraction(float(g)) == e, (fmt, scale, hex(c), g, float(e))
            if e == 0:
                assert math.copysign(1.0, g) == math.copysign(1.0, float(torch_codes(fmt)[c])), c


def test_e4m3_scaled_decode_is_the_exact_fp32_product():
    check_scaled_decode(fp8.decode, "e4m3")


def test_e5m2_scaled_decode_is_the_exact_fp32_product():
    check_scaled_decode(fp8.decode_e5m2, "e5m2")


def ulp_8bit(a: float, fmt: str) -> float:
    """Spacing of the 8-bit grid at magnitude a (mantissa bits 3 or 2,
    smallest normal exponent -6 or -14), from the format definition."""
    mbits, emin = (3, -6) if fmt == "e4m3" else (2, -14)
    if a == 0:
        return 2.0 ** (emin - mbits)
    e = max(math.frexp(a)[1] - 1, emin)
    return 2.0 ** (e - mbits)


def check_round_trip(decode, quantize, fmt: str):
    rng = np.random.default_rng(31)
    top = 448.0 if fmt == "e4m3" else 57344.0
    for scale in (1.0, 0.0117, 1.0 / 448.0, 3.0, 7.5e-5):
        s32 = fp32(scale)
        # values inside the range once divided by the scale, fp32-exact
        y = rng.uniform(-top, top, 3000) * np.exp2(rng.uniform(-12, 0, 3000))
        x = (y * s32).astype(np.float32).astype(np.float64)
        x = x[np.abs(x) / s32 <= top * 0.999]
        back = decode(quantize(x, scale), scale)
        for xi, bi in zip(x, back):
            a = abs(xi) / s32
            bound = 0.5 * ulp_8bit(a, fmt) * s32 * (1 + 2.0 ** -20) + 2.0 ** -22 * abs(xi)
            assert abs(bi - xi) <= bound, (fmt, scale, xi, bi)


def test_e4m3_round_trip_within_half_an_ulp_times_the_scale():
    check_round_trip(fp8.decode, fp8.quantize, "e4m3")


def test_e5m2_round_trip_within_half_an_ulp_times_the_scale():
    check_round_trip(fp8.decode_e5m2, fp8.quantize_e5m2, "e5m2")


def check_per_head_widen(widen, fmt: str):
    """Storage [T, Hkv, D] with T = Hkv = D = 4, so a scale broadcast along
    the wrong axis still has a valid shape and must be caught by value."""
    rng = np.random.default_rng(32)
    T = H = D = 4
    raw = rng.integers(0, 256, size=(T, H, D)).astype(np.uint8)
    table = torch_codes(fmt)
    raw[np.isnan(table[raw]) | np.isinf(table[raw])] = 0x38
    scales = np.array([0.1, 3.0, 1e-40, 2.5e30], dtype=np.float64)   # not fp32-exact on purpose
    got = widen(raw, fmt, scales)
    for t in range(T):
        for h in range(H):
            s = Fraction(fp32(float(scales[h])))
            for d in range(D):
                assert Fraction(float(got[t, h, d])) == Fraction(float(table[raw[t, h, d]])) * s, (t, h, d)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_per_head_widen_scales_the_head_axis(fmt):
    check_per_head_widen(parity.widen, fmt)


def field_decode_f32(bits: int) -> float:
    """IEEE binary32 from its fields: (-1)^s 2^(e-127) (1 + m 2^-23) for
    1 <= e <= 254, (-1)^s m 2^-149 for e = 0, +-inf or NaN for e = 255."""
    s = (bits >> 31) & 1
    e = (bits >> 23) & 0xFF
    m = bits & 0x7FFFFF
    sign = -1.0 if s else 1.0
    if e == 0xFF:
        return sign * math.inf if m == 0 else math.copysign(math.nan, sign)
    if e == 0:
        return sign * float(Fraction(m, 2 ** 149))
    return sign * float((1 + Fraction(m, 2 ** 23)) * Fraction(2) ** (e - 127))


def f32_sweep_bits() -> np.ndarray:
    rng = np.random.default_rng(33)
    specials = [0x00000000, 0x80000000, 0x00000001, 0x80000001, 0x007FFFFF, 0x00400000,
                0x00800000, 0x7F7FFFFF, 0xFF7FFFFF, 0x7F800000, 0xFF800000, 0x7FC00000,
                0xFFC00000, 0x7F800001, 0x7FBFFFFF, 0xFFFFFFFF, 0x3F800000, 0xBF800000]
    every_exponent = [(s << 31) | (e << 23) | int(m) for s in (0, 1) for e in range(256)
                      for m in rng.integers(0, 1 << 23, 4)]
    rand = rng.integers(0, 1 << 32, 20000, dtype=np.uint64).tolist()
    return np.array(specials + every_exponent + rand, dtype=np.uint64).astype(np.uint32)


def check_f32_bits(f32_bits_to_f64):
    bits = f32_sweep_bits()
    got = f32_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int32)).view(torch.float32).to(torch.float64).numpy()
    assert got.dtype == np.float64
    for b, g, r in zip(bits.tolist(), got, ref):
        f = field_decode_f32(b)
        if math.isnan(f):
            assert math.isnan(g) and math.isnan(r), hex(b)
        else:
            assert g == f == r, (hex(b), g, f, r)
            assert math.copysign(1.0, g) == math.copysign(1.0, f), hex(b)


def test_f32_bits_decode_matches_torch_and_the_field_definition():
    check_f32_bits(numerics.f32_bits_to_f64)


# ---------------------------------------------------------------- mutants

def decode_divides(codes, scale=1.0):
    return fp8.DECODE_TABLE[np.asarray(codes, dtype=np.uint8)] / np.float64(np.float32(scale))


def decode_fp64_scale(codes, scale=1.0):
    return fp8.DECODE_TABLE[np.asarray(codes, dtype=np.uint8)] * float(scale)


def decode_e5m2_fp64_scale(codes, scale=1.0):
    return fp8.DECODE_TABLE_E5M2[np.asarray(codes, dtype=np.uint8)] * float(scale)


def decode_ignores_scale(codes, scale=1.0):
    return fp8.DECODE_TABLE[np.asarray(codes, dtype=np.uint8)]


@pytest.mark.parametrize("mutant,fmt", [(decode_divides, "e4m3"), (decode_fp64_scale, "e4m3"),
                                        (decode_e5m2_fp64_scale, "e5m2"),
                                        (decode_ignores_scale, "e4m3")])
def test_scaled_decode_mutants_are_caught(mutant, fmt):
    with pytest.raises(AssertionError):
        check_scaled_decode(mutant, fmt)


def test_round_trip_catches_a_dividing_decode():
    with pytest.raises(AssertionError):
        check_round_trip(decode_divides, fp8.quantize, "e4m3")


def widen_scale_on_last_axis(raw, dtype, scale=1.0):
    per = np.asarray(scale, dtype=np.float32).astype(np.float64)
    return parity.widen(raw, dtype, 1.0) * per[None, None, :]


def widen_scale_on_first_axis(raw, dtype, scale=1.0):
    per = np.asarray(scale, dtype=np.float32).astype(np.float64)
    return parity.widen(raw, dtype, 1.0) * per[:, None, None]


def widen_scale_fp64(raw, dtype, scale=1.0):
    per = np.asarray(scale, dtype=np.float64)
    return parity.widen(raw, dtype, 1.0) * per[:, None]


@pytest.mark.parametrize("mutant", [widen_scale_on_last_axis, widen_scale_on_first_axis,
                                    widen_scale_fp64])
def test_per_head_widen_mutants_are_caught(mutant):
    with pytest.raises(AssertionError):
        check_per_head_widen(mutant, "e4m3")


def f32_value_cast(bits):
    return np.asarray(bits, dtype=np.uint32).astype(np.float64)


def f32_via_f16(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32).astype(np.float16).astype(np.float64)


@pytest.mark.parametrize("mutant", [f32_value_cast, f32_via_f16])
def test_f32_bits_mutants_are_caught(mutant):
    with pytest.raises(AssertionError):
        check_f32_bits(mutant)
