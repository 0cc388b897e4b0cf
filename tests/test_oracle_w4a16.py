"""Pins of the W4A16 oracle (oracle/w4a16.py): exact rational brute force of
the whole product on a small case, a one-hot input reading back one weight
column, and linearity in X."""
from fractions import Fraction

import numpy as np

import synth
from oracle import formats as F
from oracle import w4a16 as W


def test_bruteforce_rational():
    rng = np.random.default_rng(3)
    M, K, N = 2, 128, 3
    X = synth.bf16_bits_from_f32(rng.standard_normal((M, K)).astype(np.float32))
    Wn = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    b = synth.bf16_bits_from_f32((rng.standard_normal(N) * 0.01).astype(np.float32))
    out = W.forward(X, Wn, b)
    cW, sW = out["cW"], out["sW"]
    xv = F.bf16_value(X)
    bv = F.bf16_value(b)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                g = k // 64
                acc += Fraction(float(xv[m, k])) * Fraction(float(F.fp16_value(sW[n, g]))) * int(cW[n, k])
            acc += Fraction(float(bv[n]))
            assert abs(float(acc) - out["Y"][m, n]) <= 1e-12 * max(1.0, abs(float(acc)))


def test_one_hot_reads_a_column_and_linearity():
    rng = np.random.default_rng(4)
    K, N = 192, 5
    Wn = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    eye = synth.bf16_bits_from_f32(np.eye(K, dtype=np.float32)[[0, 70, 191]])
    out = W.forward(eye, Wn, None)
    cW, sW = out["cW"], out["sW"]
    for row, k in enumerate([0, 70, 191]):
        col = cW[:, k].astype(np.float64) * F.fp16_value(sW[:, k // 64]).astype(np.float64)
        np.testing.assert_array_equal(out["Y"][row], col)
    a = synth.bf16_bits_from_f32(rng.integers(-4, 5, (1, K)).astype(np.float32))
    two = synth.bf16_bits_from_f32(2.0 * F.bf16_value(a).astype(np.float32))
    np.testing.assert_array_equal(W.forward(two, Wn, None)["Y"], 2.0 * W.forward(a, Wn, None)["Y"])
