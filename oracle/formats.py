"""Number formats used by the layer (oracle side).

Definitions (format facts, not from the pages except FP4's q_max = 6, which
the SVDQuant notes page states in section 3, "Quantization Preliminary"):

* binary floating point with p significand bits and minimum normal exponent
  emin: every value is a multiple of 2^(max(E, emin) - p + 1) where
  E = floor(log2 |x|); rounding is to nearest, ties to even.
  bf16: p = 8, emin = -126.  fp16: p = 11, emin = -14, max 65504.
  fp32: p = 24, emin = -126.
* E2M1 (FP4): sign bit plus 3-bit magnitude code; magnitudes
  0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7.  Largest value 6 = q_max.
* E8M0: an unsigned byte b meaning 2^(b - 127).
* E4M3 (OCP FP8 "E4M3FN"): sign, 4-bit exponent (bias 7), 3-bit mantissa;
  exponent field 0 holds the subnormals m/8 * 2^-6; the largest finite
  magnitude is 448 (exponent 15, mantissa 6); exponent 15 with mantissa 7 is
  NaN; there is no infinity.

Pinned by: tests/test_oracle_formats.py (against numpy's float16/float32
casts and torch's bfloat16 cast, which are independent library routines,
and against the format definitions enumerated exhaustively).
"""
from __future__ import annotations

import numpy as np

E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
FP16_MAX = 65504.0
BF16_MAX = float((2.0 - 2.0 ** -7) * 2.0 ** 127)
FP32_MAX = float((2.0 - 2.0 ** -23) * 2.0 ** 127)
E4M3_MAX = 448.0


def round_binary(x, p: int, emin: int, max_finite: float) -> np.ndarray:
    """Round float64 values to the binary format (p, emin), nearest-even,
    overflowing to +-inf.  Returns float64 holding the rounded values."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                    # |x| = m 2^e, m in [0.5, 1)
    E = np.maximum(e - 1, emin)           # floor(log2|x|), clamped into the subnormal range
    q = E - (p - 1)                       # exponent of one unit in the last place
    y = np.ldexp(np.rint(np.ldexp(x, -q)), q)
    y = np.where(np.abs(y) > max_finite, np.copysign(np.inf, x), y)
    return np.where(x == 0, x, y)


def to_bf16(x) -> np.ndarray:
    return round_binary(x, 8, -126, BF16_MAX)


def to_fp16(x) -> np.ndarray:
    return round_binary(x, 11, -14, FP16_MAX)


def to_fp32(x) -> np.ndarray:
    return round_binary(x, 24, -126, FP32_MAX)


def bf16_bits(x) -> np.ndarray:
    """bf16 bit patterns of float64 values rounded once to bf16."""
    v = to_bf16(x).astype(np.float32)     # exact: a bf16 value is an fp32 value
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def bf16_value(bits) -> np.ndarray:
    """float64 values of bf16 bit patterns."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def fp16_bits(x) -> np.ndarray:
    """fp16 bit patterns of float64 values that are already fp16 values."""
    v = np.asarray(x, dtype=np.float64)
    h = v.astype(np.float16)              # exact for values already representable
    if not np.array_equal(h.astype(np.float64), v, equal_nan=True):
        raise ValueError("fp16_bits: value not representable in fp16")
    return h.view(np.uint16)


def fp16_value(bits) -> np.ndarray:
    """float64 values of fp16 bit patterns, decoded from the fields."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(b & 0x8000, -1.0, 1.0)
    ex = (b >> 10) & 0x1F
    man = (b & 0x3FF).astype(np.float64)
    normal = np.ldexp(1.0 + man / 1024.0, ex - 15)
    sub = np.ldexp(man / 1024.0, -14)
    val = np.where(ex == 0, sub, np.where(ex == 31, np.where(man == 0, np.inf, np.nan), normal))
    return sign * val


def e2m1_encode(v) -> np.ndarray:
    """Nearest E2M1 code of each value: magnitude code 0..7 of the nearest
    representable magnitude (values beyond 6 saturate to 6), ties to the even
    code; bit 3 is the sign bit of the input (so -0 encodes as 0b1000)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), 6.0)[..., None]      # beyond the largest magnitude: saturate
    d = np.abs(a - E2M1_MAGNITUDES)
    best = d.min(axis=-1, keepdims=True)
    is_best = d == best
    codes = np.arange(8)
    even_pick = np.where(is_best & (codes % 2 == 0), codes, 99).min(axis=-1)
    any_pick = np.where(is_best, codes, 99).min(axis=-1)
    mag = np.where(even_pick < 99, even_pick, any_pick)
    return (mag | (np.signbit(v).astype(np.int64) << 3)).astype(np.uint8)


def e2m1_decode(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    mag = E2M1_MAGNITUDES[c & 7]
    return np.where(c & 8, -mag, mag)


def e8m0_value(b) -> np.ndarray:
    return np.ldexp(1.0, np.asarray(b, dtype=np.int64) - 127)


def e4m3_value(b) -> np.ndarray:
    """float64 value of E4M3 bytes, decoded from the fields (NaN for S.1111.111)."""
    b = np.asarray(b, dtype=np.int64) & 0xFF
    sign = np.where(b & 0x80, -1.0, 1.0)
    ex = (b >> 3) & 0xF
    man = (b & 7).astype(np.float64)
    val = np.where(ex == 0, np.ldexp(man / 8.0, -6), np.ldexp(1.0 + man / 8.0, ex - 7))
    val = np.where((ex == 15) & (man == 7), np.nan, val)
    return sign * val


_E4M3_POS = e4m3_value(np.arange(0x7F))          # the 127 non-negative finite values, increasing


def e4m3_encode(v) -> np.ndarray:
    """E4M3 byte of each non-negative value: nearest representable value, ties
    to even (the binary rounding with 4 significand bits and minimum normal
    exponent -6), saturating at 448."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(v < 0) or np.any(np.isnan(v)):
        raise ValueError("e4m3_encode takes non-negative values")
    r = np.minimum(round_binary(v, 4, -6, np.inf), E4M3_MAX)
    idx = np.searchsorted(_E4M3_POS, r)
    if not np.array_equal(_E4M3_POS[np.minimum(idx, 126)], r):
        raise AssertionError("e4m3_encode: rounded value not in the table")
    return idx.astype(np.uint8)
