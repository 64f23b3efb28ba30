"""OCP 8-bit floating point, e4m3 ("fn") and e5m2 variants, for the oracle (test infrastructure only).

P1 "İlgili Teknikler" (FP8 cache quantisation) says only that keys and values
are stored with 8-bit precision, roughly halving cache memory against 16-bit
formats.  The concrete format read here is OCP e4m3fn: 1 sign bit, 4 exponent
bits with bias 7, 3 mantissa bits, no infinities, the two codes S.1111.111 are
NaN, largest finite magnitude 1.75 * 2**8 = 448, subnormals m * 2**-9.
Quantisation uses one fp32 scale per tensor: the stored code c means
``decode(c) * scale``.

The second flavour (P1 "İlgili Teknikler" names no flavour; e5m2 is the
other OCP format) is e5m2: 1 sign bit, 5 exponent bits with bias 15, 2
mantissa bits, IEEE-style infinities (exponent field 31, mantissa 0) and NaNs
(exponent field 31, mantissa not 0), largest finite magnitude 1.75 * 2**15 =
57344, subnormals m * 2**-16.  Its cache-write encoder rounds to nearest
even and saturates like the e4m3 one: magnitudes that round past 57344, and
+-inf, become +-57344; NaN becomes 0x7F with the NaN's sign.

Written from those definitions, not from any library's source.  Pinned in
``tests/test_oracle.py``: all 256 codes of each format against torch's
``float8_e4m3fn`` / ``float8_e5m2`` conversions (library routines),
encode(decode(c)) == c, every midpoint between neighbours rounding to the even
code, saturation and NaN handling.
"""

from __future__ import annotations

import math

import numpy as np

from .numerics import round_to_format

E4M3_BIAS = 7
E4M3_MAX = 448.0
E4M3_P = 4          # significand bits including the implicit one
E4M3_EMIN = 1 - E4M3_BIAS  # -6: exponent of the smallest normal binade


def decode_code(c: int) -> float:
    """Value of one e4m3 code, straight from the field definition."""
    s = (c >> 7) & 1
    E = (c >> 3) & 0xF
    m = c & 0x7
    sign = -1.0 if s else 1.0
    if E == 0xF and m == 0x7:
        return math.copysign(float("nan"), sign)
    if E == 0:
        return sign * m * 2.0 ** (1 - E4M3_BIAS - 3)       # subnormal: m * 2**-9
    return sign * (1.0 + m / 8.0) * 2.0 ** (E - E4M3_BIAS)


#: float64 value of each of the 256 codes
DECODE_TABLE = np.array([decode_code(c) for c in range(256)], dtype=np.float64)


def decode(codes: np.ndarray, scale: float = 1.0) -> np.ndarray:
    """uint8 codes -> float64 values times ``scale`` (fp32 scale widened exactly).

    The product is exact in float64: a 4-bit e4m3 significand times a 24-bit
    fp32 significand fits in 53 bits.
    """
    return DECODE_TABLE[np.asarray(codes, dtype=np.uint8)] * np.float64(np.float32(scale))


def round_to_e4m3(y) -> np.ndarray:
    """Nearest e4m3 value (float64), ties to even, magnitudes beyond 448 and
    +-inf saturate to +-448, NaN stays NaN."""
    return round_to_format(y, E4M3_P, E4M3_EMIN, E4M3_MAX, saturate=True)


def encode(y) -> np.ndarray:
    """float64 values -> uint8 e4m3 codes: round to nearest-even, saturate to
    +-448 (also +-inf), NaN -> 0x7F with the sign bit of the NaN kept.

    After rounding, a value r is split into its fields: in the subnormal
    binade (|r| < 2**-6) the mantissa field is |r| / 2**-9 with exponent field
    0; otherwise |r| = (1 + m/8) * 2**e gives exponent field e + 7 and
    mantissa field m.
    """
    y = np.asarray(y, dtype=np.float64)
    r = round_to_e4m3(y)
    nan = np.isnan(r)
    a = np.where(nan, 0.0, np.abs(r))
    sign = np.where(np.signbit(np.where(nan, y, r)), 0x80, 0).astype(np.int64)
    sub = a < 2.0 ** E4M3_EMIN
    m_sub = a / 2.0 ** (E4M3_EMIN - 3)
    frac, E = np.frexp(np.where(sub, 1.0, a))      # a = frac * 2**E, frac in [0.5, 1)
    e = E.astype(np.int64) - 1
    m_norm = (frac * 2.0 - 1.0) * 8.0
    mant = np.where(sub, m_sub, m_norm)
    expf = np.where(sub, 0, e + E4M3_BIAS)
    if not np.all(mant == np.floor(mant)):
        raise AssertionError("rounded value not on the e4m3 grid")
    code = sign | (expf << 3) | mant.astype(np.int64)
    code = np.where(nan, sign | 0x7F, code)
    return code.astype(np.uint8)


def quantize(x, scale: float) -> np.ndarray:
    """The cache-write quantiser: ``encode(fl32(x * fl32(1/scale)))``.

    ``x`` holds values exactly representable in fp32 (fp32, fp16 or bf16
    sources).  The reciprocal of the fp32 scale is rounded to fp32 once; the
    product is one correctly rounded fp32 multiply, then e4m3 rounding.  The
    reciprocal form (rather than a division per element) is a reading: the
    pages fix no quantiser.
    """
    inv = np.float32(1.0) / np.float32(scale)                 # fl32(1/scale)
    y = (np.asarray(x, dtype=np.float64).astype(np.float32) * inv).astype(np.float64)
    return encode(y)


# ---------------------------------------------------------------- e5m2

E5M2_BIAS = 15
E5M2_MAX = 57344.0
E5M2_P = 3
E5M2_EMIN = 1 - E5M2_BIAS   # -14


def decode_code_e5m2(c: int) -> float:
    """Value of one e5m2 code, straight from the field definition."""
    s = (c >> 7) & 1
    E = (c >> 2) & 0x1F
    m = c & 0x3
    sign = -1.0 if s else 1.0
    if E == 0x1F:
        return sign * float("inf") if m == 0 else math.copysign(float("nan"), sign)
    if E == 0:
        return sign * m * 2.0 ** (1 - E5M2_BIAS - 2)      # subnormal: m * 2**-16
    return sign * (1.0 + m / 4.0) * 2.0 ** (E - E5M2_BIAS)


#: float64 value of each of the 256 e5m2 codes
DECODE_TABLE_E5M2 = np.array([decode_code_e5m2(c) for c in range(256)], dtype=np.float64)


def decode_e5m2(codes: np.ndarray, scale: float = 1.0) -> np.ndarray:
    """uint8 e5m2 codes -> float64 values times ``scale`` (exact, as for e4m3)."""
    return DECODE_TABLE_E5M2[np.asarray(codes, dtype=np.uint8)] * np.float64(np.float32(scale))


def round_to_e5m2(y) -> np.ndarray:
    """Nearest e5m2 value, ties to even, saturating to +-57344 (also +-inf)."""
    return round_to_format(y, E5M2_P, E5M2_EMIN, E5M2_MAX, saturate=True)


def encode_e5m2(y) -> np.ndarray:
    """float64 -> uint8 e5m2 codes: nearest-even, saturating, NaN -> 0x7F
    with the NaN's sign.  Fields as for e4m3 with a 2-bit mantissa and bias
    15: subnormal binade |r| < 2**-14 has mantissa |r| / 2**-16."""
    y = np.asarray(y, dtype=np.float64)
    r = round_to_e5m2(y)
    nan = np.isnan(r)
    a = np.where(nan, 0.0, np.abs(r))
    sign = np.where(np.signbit(np.where(nan, y, r)), 0x80, 0).astype(np.int64)
    sub = a < 2.0 ** E5M2_EMIN
    m_sub = a / 2.0 ** (E5M2_EMIN - 2)
    frac, E = np.frexp(np.where(sub, 1.0, a))
    e = E.astype(np.int64) - 1
    m_norm = (frac * 2.0 - 1.0) * 4.0
    mant = np.where(sub, m_sub, m_norm)
    expf = np.where(sub, 0, e + E5M2_BIAS)
    if not np.all(mant == np.floor(mant)):
        raise AssertionError("rounded value not on the e5m2 grid")
    code = sign | (expf << 2) | mant.astype(np.int64)
    code = np.where(nan, sign | 0x7F, code)
    return code.astype(np.uint8)


def quantize_e5m2(x, scale: float) -> np.ndarray:
    """The cache-write quantiser for e5m2: ``encode_e5m2(fl32(x * fl32(1/scale)))``."""
    inv = np.float32(1.0) / np.float32(scale)
    y = (np.asarray(x, dtype=np.float64).astype(np.float32) * inv).astype(np.float64)
    return encode_e5m2(y)
