"""Pins for oracle/formats.py against independent library casts and the
format definitions (E2M1, E8M0, IEEE binary16/bfloat16)."""
import math

import numpy as np
import pytest

from oracle import formats as F


def _edge_values():
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.uniform(-9, 6, 20000),
        np.array([0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 1e-8, 2.0 ** -24, 2.0 ** -25,
                  3 * 2.0 ** -26, 6.1e-5, 2.0 ** -14, 2.0 ** -126, 2.0 ** -133, 2.0 ** -149, 1e38, 3.4e38]),
    ])
    return np.concatenate([v, -v])


def test_fp16_rounding_matches_numpy_cast():
    v = _edge_values()
    ours = F.to_fp16(v)
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).astype(np.float64)   # numpy: RNE, subnormals, overflow to inf
    np.testing.assert_array_equal(ours, ref)


def test_fp16_ties_to_even():
    # 1 + 2^-11 lies halfway between 1 and 1 + 2^-10: ties to the even significand (1).
    assert F.to_fp16(1 + 2.0 ** -11) == 1.0
    assert F.to_fp16(1 + 3 * 2.0 ** -11) == 1 + 2 * 2.0 ** -10
    # halfway between the two smallest subnormals
    assert F.to_fp16(1.5 * 2.0 ** -24) == 2 * 2.0 ** -24
    assert F.to_fp16(0.5 * 2.0 ** -24) == 0.0


def test_fp32_rounding_matches_numpy_cast():
    v = _edge_values()
    ours = F.to_fp32(v)
    with np.errstate(over="ignore"):
        ref = v.astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(ours, ref)


def test_bf16_rounding_matches_torch_cast():
    torch = pytest.importorskip("torch")
    v = _edge_values()
    v32 = v.astype(np.float32).astype(np.float64)          # torch casts from fp32; compare on fp32 inputs
    ours = F.to_bf16(v32)
    ref = torch.from_numpy(v32.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)
    bits = F.bf16_bits(v32)
    np.testing.assert_array_equal(F.bf16_value(bits), ref)


def test_fp16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    ours = F.fp16_value(bits)
    finite = np.isfinite(ref)
    np.testing.assert_array_equal(ours[finite], ref[finite])
    assert np.all(np.isinf(ours[np.isinf(ref)]))
    assert np.all(np.isnan(ours[np.isnan(ref)]))


# E2M1: magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 (codes 0..7).  The table below is the
# format definition worked out by hand: every midpoint, the points just either side
# of it, saturation, and signed zero.
_MID_TABLE = [
    (0.0, 0), (0.25, 0), (0.5, 1), (0.75, 2), (1.0, 2), (1.25, 2), (1.5, 3), (1.75, 4),
    (2.0, 4), (2.5, 4), (3.0, 5), (3.5, 6), (4.0, 6), (5.0, 6), (6.0, 7), (7.0, 7), (1e30, 7),
]


@pytest.mark.parametrize("v,code", _MID_TABLE)
def test_e2m1_table(v, code):
    assert int(F.e2m1_encode(np.float64(v))) == code
    assert int(F.e2m1_encode(np.float64(-v))) == code | 8


def test_e2m1_around_midpoints():
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    below = [0, 1, 2, 3, 4, 5, 6]
    for m, lo in zip(mids, below):
        assert int(F.e2m1_encode(np.nextafter(m, 0.0))) == lo
        assert int(F.e2m1_encode(np.nextafter(m, 10.0))) == lo + 1


def test_e2m1_signed_zero_and_roundtrip():
    assert int(F.e2m1_encode(np.float64(-0.0))) == 8
    assert int(F.e2m1_encode(np.float64(0.0))) == 0
    for c in range(16):
        assert int(F.e2m1_encode(F.e2m1_decode(c))) == c
    np.testing.assert_array_equal(F.e2m1_decode(np.arange(8)), [0, .5, 1, 1.5, 2, 3, 4, 6])


def test_e8m0_value():
    assert F.e8m0_value(127) == 1.0
    assert F.e8m0_value(0) == 2.0 ** -127
    assert F.e8m0_value(254) == 2.0 ** 127
    assert math.log2(F.e8m0_value(121)) == -6
