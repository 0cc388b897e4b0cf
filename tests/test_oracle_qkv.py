"""Pins of the oracle's Q/K normalization and rotary embedding (oracle/qkv.py)
against facts other than their own formulas: closed forms of the RMS norm,
rotations as 2 x 2 orthogonal matrices (identity, quarter turn, composition,
length), head independence, and V passing through."""
import math

import numpy as np

from oracle import qkv as QK


def test_rms_norm_closed_forms():
    # constant vector c * 1 with unit weight: every entry c / sqrt(c^2 + eps)
    for c in (3.0, -0.25, 1e3):
        for eps in (0.0, 1e-6):
            y = QK.rms_norm(np.full(128, c), np.ones(128), eps)
            np.testing.assert_allclose(y, c / math.sqrt(c * c + eps), rtol=1e-14)
    # eps = 0: mean square of the output is 1 and the map is scale invariant
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 128))
    y = QK.rms_norm(x, np.ones(128), 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(QK.rms_norm(7.5 * x, np.ones(128), 0.0), y, rtol=1e-13)
    # the weight scales each feature: a one-hot weight keeps one coordinate
    w = np.zeros(128)
    w[17] = 2.0
    z = QK.rms_norm(x, w, 0.0)
    assert np.all(z[:, np.arange(128) != 17] == 0)
    np.testing.assert_allclose(z[:, 17], 2.0 * x[:, 17] / np.sqrt(np.mean(x * x, axis=-1)), rtol=1e-13)


def test_rotation_as_orthogonal_matrices():
    rng = np.random.default_rng(1)
    M, D = 4, 8
    x = rng.standard_normal((M, D))
    theta = rng.uniform(-math.pi, math.pi, (M, D // 2))
    # identity at angle 0
    np.testing.assert_array_equal(QK.rotate_pairs(x, np.ones((M, D // 2)), np.zeros((M, D // 2))), x)
    # a quarter turn maps (a, b) to (-b, a)
    q = QK.rotate_pairs(x, np.zeros((M, D // 2)), np.ones((M, D // 2)))
    np.testing.assert_array_equal(q[:, 0::2], -x[:, 1::2])
    np.testing.assert_array_equal(q[:, 1::2], x[:, 0::2])
    # each pair against the explicit 2 x 2 rotation matrix [[c, -s], [s, c]]
    r = QK.rotate_pairs(x, np.cos(theta), np.sin(theta))
    for m in range(M):
        for p in range(D // 2):
            c, s = math.cos(theta[m, p]), math.sin(theta[m, p])
            R = np.array([[c, -s], [s, c]])
            np.testing.assert_allclose(r[m, 2 * p:2 * p + 2], R @ x[m, 2 * p:2 * p + 2], rtol=1e-13, atol=1e-15)
    # lengths of pairs are kept; rotations compose by adding angles
    np.testing.assert_allclose(r[:, 0::2] ** 2 + r[:, 1::2] ** 2, x[:, 0::2] ** 2 + x[:, 1::2] ** 2, rtol=1e-13)
    phi = rng.uniform(-1, 1, (M, D // 2))
    two = QK.rotate_pairs(r, np.cos(phi), np.sin(phi))
    np.testing.assert_allclose(two, QK.rotate_pairs(x, np.cos(theta + phi), np.sin(theta + phi)), atol=1e-13)


def test_qkv_heads_independent_and_v_untouched():
    rng = np.random.default_rng(2)
    M, H, D = 3, 2, 8
    Y = rng.standard_normal((M, 3 * H * D))
    Y[:, D:2 * D] *= 1000.0          # second Q head much larger: normalized on its own
    wq, wk = rng.uniform(0.5, 2, D), rng.uniform(0.5, 2, D)
    cos, sin = np.ones((M, D // 2)), np.zeros((M, D // 2))
    out = QK.qkv_norm_rope(Y, D, wq, wk, 0.0, cos, sin)
    for h in range(H):
        np.testing.assert_allclose(out[:, h * D:(h + 1) * D], QK.rms_norm(Y[:, h * D:(h + 1) * D], wq, 0.0),
                                   rtol=1e-13)
        kk = slice(H * D + h * D, H * D + (h + 1) * D)
        np.testing.assert_allclose(out[:, kk], QK.rms_norm(Y[:, kk], wk, 0.0), rtol=1e-13)
    np.testing.assert_array_equal(out[:, 2 * H * D:], Y[:, 2 * H * D:])
