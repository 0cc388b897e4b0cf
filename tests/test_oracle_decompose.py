"""Pins for oracle/decompose.py: the exact smoothing identity, the balance
property that defines the smoothing factor, Eckart-Young, full rank, the
residual identity and adapter absorption."""
import numpy as np
import pytest

import synth
from oracle import decompose as Dc
from oracle import formats as F
from oracle import quant as Q


@pytest.fixture(scope="module")
def small():
    spec = synth.layer_spec("single", M=96, K=256, N=192, rank=16, x_outliers=4, w_outliers=3)
    raw = synth.draw_raw(spec, seed=11)
    return spec, raw


def test_smoothing_balances_channel_maxima(small):
    # lambda_j = sqrt(ax_j / aw_j) makes the two maxima meet: ax_j / lambda_j == lambda_j aw_j
    spec, raw = small
    lam = Dc.smoothing_factors(raw["X"], raw["W"]).astype(np.float64)
    ax = np.abs(F.bf16_value(raw["X"])).max(axis=0)
    aw = np.abs(F.bf16_value(raw["W"])).max(axis=1)
    np.testing.assert_allclose(ax / lam, lam * aw, rtol=2e-7)
    assert lam[raw["x_outliers"]].min() > np.median(lam)      # outlier channels get larger factors


def test_smoothing_zero_channels():
    X = synth.bf16_bits_from_f32(np.array([[0.0, 1.0], [0.0, -2.0]], np.float32))
    W = synth.bf16_bits_from_f32(np.array([[1.0, 1.0], [0.0, 0.0]], np.float32))
    lam = Dc.smoothing_factors(X, W)
    assert lam.tolist() == [1.0, 1.0]


def test_smoothing_identity_exact(small):
    # X W = X_hat W_hat: smoothing moves scale between operands without changing the product
    spec, raw = small
    lam = Dc.smoothing_factors(raw["X"], raw["W"])
    X = F.bf16_value(raw["X"])
    W = F.bf16_value(raw["W"])
    Xh = X / lam.astype(np.float64)[None, :]
    Wh = Dc.smoothed_weight(raw["W"], lam)
    np.testing.assert_allclose(Xh @ Wh, X @ W, rtol=1e-12, atol=1e-12 * np.abs(X @ W).max())


def test_eckart_young_and_monotone(small):
    spec, raw = small
    lam = Dc.smoothing_factors(raw["X"], raw["W"])
    Wh = Dc.smoothed_weight(raw["W"], lam)
    S = np.linalg.svd(Wh, compute_uv=False)
    prev = np.inf
    for r in (1, 4, 8, 16, 32, 64):
        d = Dc.decompose(Wh, r)
        err2 = np.linalg.norm(Wh - d["L1_64"] @ d["L2_64"]) ** 2
        np.testing.assert_allclose(err2, np.sum(S[r:] ** 2), rtol=1e-9)
        assert err2 <= prev
        prev = err2


def test_full_rank_residual_vanishes(small):
    spec, raw = small
    lam = Dc.smoothing_factors(raw["X"], raw["W"])
    Wh = Dc.smoothed_weight(raw["W"], lam)
    d = Dc.decompose(Wh, min(Wh.shape))
    assert np.linalg.norm(Wh - d["L1_64"] @ d["L2_64"]) <= 1e-12 * np.linalg.norm(Wh)


def test_residual_identity(small):
    spec, raw = small
    c = Dc.calibrate(raw["X"], raw["W"], spec.rank)
    L = F.bf16_value(c["L1"]) @ F.bf16_value(c["L2"])
    exact = c["W_hat"] - L
    # R is the single float32 rounding of W_hat - L1b L2b
    ulp = np.spacing(np.abs(c["R"]).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(c["R"] - exact) <= ulp / 2)
    # ||R|| is the Eckart-Young truncation error, up to the bf16 rounding of the factors
    tail = np.sqrt(np.sum(c["S"][spec.rank:] ** 2))
    assert abs(np.linalg.norm(c["R"]) - tail) <= 2.0 ** -7 * np.linalg.norm(c["W_hat"])


def test_quantized_reconstruction_nonincreasing_in_rank():
    spec = synth.layer_spec("single")
    raw = synth.draw_raw(spec)
    lam = Dc.smoothing_factors(raw["X"], raw["W"])
    Wh = Dc.smoothed_weight(raw["W"], lam)
    U, S, Vt = np.linalg.svd(Wh, full_matrices=False)
    prev = np.inf
    for r in (0, 8, 16, 32, 64, 128):
        L1b = F.bf16_bits(U[:, :r] * S[:r])
        L2b = F.bf16_bits(Vt[:r])
        R = F.to_fp32(Wh - F.bf16_value(L1b) @ F.bf16_value(L2b)).astype(np.float32)
        c, s = Q.int4_quantize(R.T.copy())
        e = np.linalg.norm(R.T - Q.int4_dequantize(c, s))
        assert e <= prev * (1 + 1e-9), (r, e, prev)
        prev = e


def test_adapter_absorbed_without_requantization():
    spec = synth.layer_spec("lora", M=64, K=256, N=256, rank=8, lora_rank=4, x_outliers=3, w_outliers=3)
    raw = synth.draw_raw(spec, seed=5)
    c = Dc.calibrate(raw["X"], raw["W"], spec.rank)
    L1, L2 = Dc.absorb_adapter(c["L1"], c["L2"], raw["A"], raw["B"])
    Xh = F.bf16_value(raw["X"]) / c["lam"].astype(np.float64)
    lhs = Xh @ F.bf16_value(L1) @ F.bf16_value(L2)
    rhs = Xh @ F.bf16_value(c["L1"]) @ F.bf16_value(c["L2"]) + Xh @ F.bf16_value(raw["A"]) @ F.bf16_value(raw["B"])
    np.testing.assert_allclose(lhs, rhs, rtol=1e-10, atol=1e-10 * np.abs(rhs).max())
    # the residual (and so its 4-bit codes) does not depend on the adapter
    c1, s1 = Q.mxfp4_quantize(c["R"].T.copy())
    c2, s2 = Q.mxfp4_quantize(Dc.calibrate(raw["X"], raw["W"], spec.rank)["R"].T.copy())
    assert np.array_equal(Q.pack_canonical(c1), Q.pack_canonical(c2)) and np.array_equal(s1, s2)
