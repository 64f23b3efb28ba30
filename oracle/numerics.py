"""Storage formats <-> float64 for the oracle (test infrastructure only).

The pages fix no storage precision beyond "16-bit" caches and an "8-bit" FP8
cache (P1 "İlgili Teknikler", FP8 cache quantisation).  The path stores K/V as
IEEE binary32, IEEE binary16, bfloat16 or OCP e4m3 and accumulates in fp32; the
oracle widens every stored value to float64 exactly and does all arithmetic
there.

Decoding is exact: every fp32, fp16 and bf16 value is a float64 value.
Encoding (:func:`round_to_format`) is written from the definition of a binary
floating-point format with ``p`` significand bits and minimum normal exponent
``emin``: scale by the quantum of the value's binade, round half to even, scale
back.  Pinned in ``tests/test_oracle.py`` against NumPy's and torch's
own casts (library routines) on sweeps that include every tie.
"""

from __future__ import annotations

import numpy as np


def f32_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """uint32 bit patterns of IEEE binary32 -> float64 (exact)."""
    return np.asarray(bits, dtype=np.uint32).view(np.float32).astype(np.float64)


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of IEEE binary16 -> float64 (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of bfloat16 -> float64 (exact).

    bfloat16 is the upper half of an IEEE binary32 word, so the value is the
    binary32 whose high 16 bits are the pattern and whose low 16 bits are 0.
    """
    wide = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return wide.view(np.float32).astype(np.float64)


def round_to_format(x, p: int, emin: int, max_finite: float, saturate: bool) -> np.ndarray:
    """Round float64 values to a binary format, ties to even.

    ``p`` counts significand bits including the implicit one, ``emin`` is the
    exponent of the smallest normal binade (values below it are subnormal and
    share that binade's quantum), ``max_finite`` is the largest finite value.
    Results beyond ``max_finite`` become +-``max_finite`` when ``saturate`` is
    set and +-inf otherwise (IEEE overflow).  NaN stays NaN; +-inf saturates or
    stays inf by the same rule; signed zeros keep their sign.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    sign = np.where(np.signbit(x), -1.0, 1.0)
    a = np.abs(x)
    nan = np.isnan(x)
    finite = np.isfinite(x)
    nz = finite & (a > 0)
    # binade exponent e with 2**e <= a < 2**(e+1): frexp gives a = f*2**E, f in [0.5, 1)
    _, E = np.frexp(np.where(nz, a, 1.0))
    e = np.maximum(E.astype(np.int64) - 1, emin)
    quantum = np.ldexp(1.0, (e - (p - 1)).astype(np.int32))
    r = np.rint(np.where(nz, a, 0.0) / quantum) * quantum  # np.rint: half to even
    over = r > max_finite
    r = np.where(over, max_finite if saturate else np.inf, r)
    out[...] = np.where(nz, sign * r, np.copysign(0.0, x))  # zeros keep their sign
    inf = np.isinf(x)
    out[inf] = sign[inf] * (max_finite if saturate else np.inf)
    out[nan] = np.nan
    return out


F16_P, F16_EMIN, F16_MAX = 11, -14, 65504.0
BF16_P, BF16_EMIN, BF16_MAX = 8, -126, float.fromhex("0x1.fep127")
F32_P, F32_EMIN, F32_MAX = 24, -126, float.fromhex("0x1.fffffep127")


def round_to_f16(x) -> np.ndarray:
    """float64 -> nearest IEEE binary16 value (as float64), ties to even, overflow to inf."""
    return round_to_format(x, F16_P, F16_EMIN, F16_MAX, saturate=False)


def round_to_bf16(x) -> np.ndarray:
    """float64 -> nearest bfloat16 value (as float64), ties to even, overflow to inf."""
    return round_to_format(x, BF16_P, BF16_EMIN, BF16_MAX, saturate=False)


def round_to_f32(x) -> np.ndarray:
    """float64 -> nearest IEEE binary32 value (as float64), ties to even, overflow to inf."""
    return round_to_format(x, F32_P, F32_EMIN, F32_MAX, saturate=False)


def half_ulp(x, p: int, emin: int) -> np.ndarray:
    """Half a unit in the last place of ``x`` in a format with ``p`` significand bits.

    This is the largest error a correct round-to-nearest into that format can
    add to a value of magnitude ``|x|``; used to widen tolerances by the output
    rounding.
    """
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, E = np.frexp(np.where(a > 0, a, 1.0))
    e = np.where(a > 0, np.maximum(E.astype(np.int64) - 1, emin), emin)
    return np.ldexp(0.5, (e - (p - 1)).astype(np.int32))
