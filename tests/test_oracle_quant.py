"""Pins for oracle/quant.py: the section-3 worked example, tie rules,
idempotence, saturation, zero groups and the per-element error bound."""
import math
import os

import numpy as np
import pytest

from oracle import formats as F
from oracle import quant as Q

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.txt")


def _golden():
    d = {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, v = line.split(":", 1)
        d[k.strip()] = v.strip()
    return d


def _pad(vals, g):
    x = np.zeros((1, g), dtype=np.float32)
    x[0, :len(vals)] = np.asarray(vals, dtype=np.float32)
    return x


def test_worked_example_int4():
    d = _golden()
    vec = [float(t) for t in d["input"].split()]
    c, s = Q.int4_quantize(_pad(vec, 64))
    assert int(s[0, 0]) == int(d["int4.with_outlier.scale_bits"], 16)
    assert c[0, :6].tolist() == [int(t) for t in d["int4.with_outlier.codes"].split()]
    # the page's point: with the outlier, every small value collapses to zero
    assert np.all(c[0, :5] == 0)
    c, s = Q.int4_quantize(_pad(vec[:5], 64))
    assert int(s[0, 0]) == int(d["int4.without_outlier.scale_bits"], 16)
    assert c[0, :5].tolist() == [int(t) for t in d["int4.without_outlier.codes"].split()]
    assert len(set(c[0, :5].tolist())) == 5          # ... and without it they stay distinct


def test_worked_example_mxfp4():
    d = _golden()
    vec = [float(t) for t in d["input"].split()]
    c, s = Q.mxfp4_quantize(_pad(vec, 32))
    assert int(s[0, 0]) == int(d["mxfp4.with_outlier.scale_byte"])
    assert c[0, :6].tolist() == [int(t) for t in d["mxfp4.with_outlier.nibbles"].split()]
    assert np.all(F.e2m1_decode(c[0, :5]) == 0)
    c, s = Q.mxfp4_quantize(_pad(vec[:5], 32))
    assert int(s[0, 0]) == int(d["mxfp4.without_outlier.scale_byte"])
    assert c[0, :5].tolist() == [int(t) for t in d["mxfp4.without_outlier.nibbles"].split()]


def test_int4_half_integer_ties_to_even():
    # amax = 7 gives s = 1 exactly, so x / s is x itself.
    vals = [7.0, 2.5, 3.5, -0.5, -1.5, 0.5, 1.5, -2.5, 4.5, -6.5]
    c, s = Q.int4_quantize(_pad(vals, 64))
    assert F.fp16_value(s)[0, 0] == 1.0
    assert c[0, :10].tolist() == [7, 2, 4, 0, -2, 0, 2, -2, 4, -6]


def test_int4_zero_and_tiny_groups():
    c, s = Q.int4_quantize(np.zeros((2, 128), np.float32))
    assert np.all(c == 0) and np.all(s == 0)
    # amax / 7 below half the smallest fp16 subnormal: scale 0, all codes 0
    x = _pad([1e-8, -5e-9], 64)
    c, s = Q.int4_quantize(x)
    assert s[0, 0] == 0 and np.all(c == 0)
    # subnormal fp16 scale: precision lost, codes clamp into [-8, 7]
    x = _pad([1e-6, -1e-6, 3e-7], 64)
    c, s = Q.int4_quantize(x)
    sv = F.fp16_value(s)[0, 0]
    assert 0 < sv < 2.0 ** -14
    assert c.min() >= -8 and c.max() <= 7


def test_int4_scale_clamps_at_fp16_max():
    c, s = Q.int4_quantize(_pad([1e6, -3e5], 64))
    assert F.fp16_value(s)[0, 0] == 65504.0
    assert c[0, 0] == 7 and c[0, 1] == -5


def test_mxfp4_scale_is_floor_log2_minus_2():
    rng = np.random.default_rng(1)
    for _ in range(200):
        amax = float(np.float32(10.0 ** rng.uniform(-30, 30)))
        x = _pad([amax, -amax / 3], 32)
        _, s = Q.mxfp4_quantize(x)
        e = math.floor(math.log2(amax)) - 2
        assert int(s[0, 0]) == max(-127, min(127, e)) + 127


def test_mxfp4_zero_subnormal_and_saturation():
    x = np.zeros((1, 32), np.float32)
    x[0, 3] = -0.0
    c, s = Q.mxfp4_quantize(x)
    assert s[0, 0] == 0 and c[0, 3] == 8 and c[0, 0] == 0
    # subnormal maximum: exponent clamps at -127
    x = _pad([1e-40, -2e-41], 32)
    c, s = Q.mxfp4_quantize(x)
    assert s[0, 0] == 0
    # 7.5 * 2^e saturates to code 7 (value 6) and 4 * 2^e is code 6
    x = _pad([7.5, 4.0, -7.9], 32)
    c, s = Q.mxfp4_quantize(x)
    assert int(s[0, 0]) == 127 and c[0, :3].tolist() == [7, 6, 15]


def _data(rows, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, K)).astype(np.float32)
    x[:, rng.choice(K, 5, replace=False)] *= 50
    x[0, :64] = 0
    x[1, 64:128] *= 1e-30
    return x


@pytest.mark.parametrize("fmt", ["mxfp4", "int4"])
def test_quantize_dequantize_idempotent(fmt):
    x = _data(64, 512, 3)
    c1, s1 = Q.quantize(x, fmt)
    y = Q.dequantize(c1, s1, fmt).astype(np.float32)
    assert np.array_equal(y.astype(np.float64), Q.dequantize(c1, s1, fmt))   # exact in fp32
    c2, s2 = Q.quantize(y, fmt)
    assert np.array_equal(s1, s2)
    assert np.array_equal(Q.nibbles(c1), Q.nibbles(c2))
    z = Q.dequantize(c2, s2, fmt)
    assert np.array_equal(z, y.astype(np.float64))


def test_error_within_half_step():
    x = _data(32, 256, 4)
    # INT4: |x - q s| <= s / 2 for every element (no clamping occurs at normal scales)
    c, s = Q.int4_quantize(x)
    sv = np.repeat(F.fp16_value(s), 64, axis=1)
    err = np.abs(x - Q.int4_dequantize(c, s))
    normal = sv >= 2.0 ** -14
    assert np.all(err[normal] <= sv[normal] / 2 * (1 + 1e-6))
    # MXFP4: below 6 * 2^e the error is at most half the local spacing
    c, s = Q.mxfp4_quantize(x)
    scale = np.repeat(F.e8m0_value(s), 32, axis=1)
    v = np.abs(x) / scale
    err = np.abs(x - Q.mxfp4_dequantize(c, s)) / scale
    spacing = np.where(v < 2, 0.5, np.where(v < 4, 1.0, 2.0))
    ok = v <= 6
    assert np.all(err[ok] <= spacing[ok] / 2 + 1e-12)
    assert np.all(err[~ok] == (v[~ok] - 6))


def test_canonical_packing():
    codes = np.array([[1, 2, 3, 4, -1, -8, 7, 0]], dtype=np.int8)
    p = Q.pack_canonical(codes)
    assert p.tolist() == [[0x21, 0x43, 0x8F, 0x07]]
    assert Q.unpack_canonical(p).tolist() == [[1, 2, 3, 4, 15, 8, 7, 0]]
