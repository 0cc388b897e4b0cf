"""Pins of the oracle's E4M3 format and NVFP4-style quantizer (oracle/formats.py,
oracle/quant.py) against facts other than their own formulas: torch's float8
E4M3 type (an independent library routine) for every byte and for rounding,
brute force of the code choice over all 16 E2M1 codes, the group-scale choice
against torch's rounding, the tensor scale mapping the largest group onto 448,
idempotence, and a small layer brute force with exact rationals."""
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import layer as Ly
from oracle import quant as Q

torch = pytest.importorskip("torch")


def _torch_e4m3(v):
    return torch.tensor(np.asarray(v, dtype=np.float32)).to(torch.float8_e4m3fn).to(torch.float32).numpy()


def test_e4m3_decode_every_byte_matches_torch():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    ours = F.e4m3_value(np.arange(256))
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    assert np.array_equal(ref[~np.isnan(ref)], ours[~np.isnan(ours)])
    assert F.e4m3_value(0x7E) == 448.0 and F.e4m3_value(1) == 2.0 ** -9


def test_e4m3_encode_rounding_matches_torch():
    pos = F.e4m3_value(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2                     # every tie
    rng = np.random.default_rng(0)
    rand = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 20000))
    for v in (pos, mids, rand, np.nextafter(mids, 0), np.nextafter(mids, 1e9)):
        v = v.astype(np.float32).astype(np.float64)     # values torch sees exactly
        assert np.array_equal(F.e4m3_value(F.e4m3_encode(v)), _torch_e4m3(v).astype(np.float64))
    # beyond 448 the scale saturates (torch turns overflow into NaN instead)
    assert np.all(F.e4m3_encode(np.array([448.0, 470.0, 1e6])) == 0x7E)


def test_code_choice_is_nearest_over_all_codes():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((8, 64)) * rng.uniform(0.01, 50, (8, 1))).astype(np.float32)
    for gs in (np.float32(1.0), Q.nvfp4_global_scale(x)):
        codes, scales = Q.nvfp4_quantize(x, gs)
        S = (F.e4m3_value(scales).astype(np.float32) * gs).astype(np.float32)
        t = (x.reshape(8, 4, 16) / S[..., None]).astype(np.float64)
        cand = F.e2m1_decode(np.arange(16))              # every code's value
        d = np.abs(t[..., None] - cand)
        best = d.min(axis=-1)
        got = np.abs(t - F.e2m1_decode(codes.reshape(8, 4, 16)))
        assert np.array_equal(got, best)                 # no other code is closer
        # the group scale is torch's E4M3 rounding of amax / 6 / gs (all in range here)
        amax = np.abs(x.reshape(8, 4, 16)).max(axis=-1)
        u = ((amax / np.float32(6.0)).astype(np.float32) / gs).astype(np.float32)
        assert np.array_equal(F.e4m3_value(scales), _torch_e4m3(np.minimum(u, 448.0)).astype(np.float64))


def test_tensor_scale_puts_largest_group_on_448_and_idempotence():
    rng = np.random.default_rng(2)
    R = (rng.standard_normal((16, 256)) * 0.02).astype(np.float32)
    gs = Q.nvfp4_global_scale(R)
    codes, scales = Q.nvfp4_quantize(R, gs)
    r, gidx = np.unravel_index(np.abs(R).argmax(), R.shape)
    assert scales[r, gidx // 16] == 0x7E
    # a tensor that is its own dequantization (each group holds a +-6 code)
    deq = Q.nvfp4_dequantize(codes, scales, gs)
    has6 = (np.abs(F.e2m1_decode(codes)).reshape(16, 16, 16).max(axis=-1) == 6.0)
    assert has6.sum() >= 16
    c2, s2 = Q.nvfp4_quantize(deq.astype(np.float32), gs)
    keep = np.repeat(has6, 16, axis=1)
    assert np.array_equal(Q.pack_canonical(np.where(keep, c2, 0)), Q.pack_canonical(np.where(keep, codes, 0)))
    assert np.array_equal(s2[has6], scales[has6])


def test_zero_and_tiny_groups():
    x = np.zeros((1, 32), np.float32)
    x[0, 16:] = -np.float32(2.0 ** -20)          # amax / 6 rounds to an E4M3 zero
    codes, scales = Q.nvfp4_quantize(x, 1.0)
    assert np.all(scales == 0)
    assert np.all(codes[0, :16] == 0) and np.all(codes[0, 16:] == 0b1000)   # signed zeros
    assert np.all(Q.nvfp4_dequantize(codes, scales) == 0)


def test_layer_bruteforce_rational():
    """The nvfp4 layer on a small case, against exact rational arithmetic on
    the oracle's own codes and scales."""
    rng = np.random.default_rng(3)
    M, K, N, r = 3, 32, 4, 2
    X = synth.bf16_bits_from_f32(rng.standard_normal((M, K)).astype(np.float32))
    lam = rng.uniform(0.5, 2.0, K).astype(np.float32)
    R = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    L1 = synth.bf16_bits_from_f32((rng.standard_normal((K, r)) * 0.1).astype(np.float32))
    L2 = synth.bf16_bits_from_f32((rng.standard_normal((r, N)) * 0.1).astype(np.float32))
    b = synth.bf16_bits_from_f32((rng.standard_normal(N) * 0.01).astype(np.float32))
    out = Ly.forward(X, lam, L1, L2, R, b, "nvfp4")
    gs = Fraction(float(out["gsR"]))
    assert out["gsR"] == np.float32(np.abs(R).max() / np.float32(2688.0))
    xh = out["xhat"]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                xv = Fraction(float(F.e2m1_decode(out["cX"][m, k]))) * Fraction(float(F.e4m3_value(out["sX"][m, k // 16])))
                wv = Fraction(float(F.e2m1_decode(out["cR"][n, k]))) * Fraction(float(F.e4m3_value(out["sR"][n, k // 16]))) * gs
                acc += xv * wv
            for i in range(r):
                d = sum(Fraction(float(xh[m, k])) * Fraction(float(F.bf16_value(L1[k, i]))) for k in range(K))
                acc += d * Fraction(float(F.bf16_value(L2[i, n])))
            acc += Fraction(float(F.bf16_value(b[n])))
            assert abs(float(acc) - out["Y"][m, n]) <= 1e-12 * max(1.0, abs(float(acc)))
