"""Pins for oracle/layer.py: exact rational brute force of the whole layer,
special cases that reduce to textbook operations, the section 4.1 error
bound, GELU special values and the parity metric itself."""
import math
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import decompose as Dc
from oracle import formats as F
from oracle import layer as Ly
from oracle import quant as Q

_E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def _frac_code(code, fmt):
    c = int(code)
    if fmt == "mxfp4":
        v = _E2M1[c & 7]
        return -v if c & 8 else v
    return Fraction(c)


def _frac_scale(s, fmt):
    if fmt == "mxfp4":
        return Fraction(2) ** (int(s) - 127)
    return Fraction(float(np.uint16(s).view(np.float16)))


def _frac_bf16(bits):
    return Fraction(float(F.bf16_value(np.uint16(bits))))


@pytest.mark.parametrize("fmt", ["mxfp4", "int4"])
def test_brute_force_rational_layer(fmt):
    M = N = 8
    K, r = 128, 4
    spec = synth.layer_spec("qkv", M=M, K=K, N=N, rank=r, fmt=fmt, x_outliers=2, w_outliers=2)
    L = synth.draw_layer(spec, seed=21)
    out = Ly.forward(L["X"], L["lam"], L["L1"], L["L2"], L["R"], L["b"], fmt)
    g = Q.GROUP[fmt]
    cX, sX, cR, sR = out["cX"], out["sX"], out["cR"], out["sR"]
    xhat = out["xhat"]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += (_frac_code(cX[m, k], fmt) * _frac_scale(sX[m, k // g], fmt)
                        * _frac_code(cR[n, k], fmt) * _frac_scale(sR[n, k // g], fmt))
            for i in range(r):
                d = sum(Fraction(float(xhat[m, k])) * _frac_bf16(L["L1"][k, i]) for k in range(K))
                acc += d * _frac_bf16(L["L2"][i, n])
            acc += _frac_bf16(L["b"][n])
            y = out["Y"][m, n]
            assert abs(Fraction(float(y)) - acc) <= Fraction(1, 10 ** 9) * (1 + abs(acc)), (m, n, float(acc), y)


def test_full_rank_reduces_to_plain_matmul():
    spec = synth.layer_spec("single", M=32, K=128, N=128, rank=128, fmt="mxfp4", x_outliers=2, w_outliers=2)
    raw = synth.draw_raw(spec, seed=8)
    c = Dc.calibrate(raw["X"], raw["W"], 128)
    out = Ly.forward(raw["X"], c["lam"], c["L1"], c["L2"], c["R"].T.copy(), raw["b"], "mxfp4")
    ref = F.bf16_value(raw["X"]) @ F.bf16_value(raw["W"]) + F.bf16_value(raw["b"])[None, :]
    # At full rank the residual only holds the bf16 rounding of the factors, so the
    # layer is X W + b up to the quantized product of that small residual, which the
    # section 4.1 bound limits.
    Xm = out["xhat"].astype(np.float64)
    Rm = c["R"].astype(np.float64)
    Xq = Q.dequantize(out["cX"], out["sX"], "mxfp4")
    Rq = Q.dequantize(out["cR"], out["sR"], "mxfp4").T
    bound = Ly.quant_error_bound(Xm, Rm, Xq, Rq) + 1e-9 * np.linalg.norm(ref)
    assert np.linalg.norm(out["Y"] - ref) <= bound
    assert np.linalg.norm(Rm) < 1e-2 * np.linalg.norm(c["W_hat"])
    m = Ly.parity_metrics(out["Y"], ref)
    assert m["mean_rel"] < 1e-3, m


def test_rank0_unit_lambda_is_groupwise_w4a4():
    # Y = sum_g sX[m,g] sR[n,g] (qX[m, g] . qR[n, g]) + b  (section 3's scaled product, per group)
    rng = np.random.default_rng(2)
    M, N, K = 16, 24, 256
    X = synth.bf16_bits_from_f32(rng.standard_normal((M, K)).astype(np.float32))
    R = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    b = synth.bf16_bits_from_f32(rng.standard_normal(N).astype(np.float32))
    lam = np.ones(K, np.float32)
    for fmt in ("mxfp4", "int4"):
        g = Q.GROUP[fmt]
        out = Ly.forward(X, lam, np.zeros((K, 0), np.uint16), np.zeros((0, N), np.uint16), R, b, fmt)
        cX, sX = Q.quantize(F.bf16_value(X).astype(np.float32), fmt)
        cR, sR = Q.quantize(R, fmt)
        if fmt == "mxfp4":
            qx, qr = F.e2m1_decode(cX), F.e2m1_decode(cR)
            sx, sr = F.e8m0_value(sX), F.e8m0_value(sR)
        else:
            qx, qr = cX.astype(np.float64), cR.astype(np.float64)
            sx, sr = F.fp16_value(sX), F.fp16_value(sR)
        y = np.zeros((M, N))
        for j in range(K // g):
            y += np.outer(sx[:, j], sr[:, j]) * (qx[:, j * g:(j + 1) * g] @ qr[:, j * g:(j + 1) * g].T)
        y += F.bf16_value(b)[None, :]
        np.testing.assert_allclose(out["Y"], y, rtol=1e-12, atol=1e-12)


def test_single_group_scaled_integer_dot():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 64)).astype(np.float32)
    w = rng.standard_normal((1, 64)).astype(np.float32)
    X = synth.bf16_bits_from_f32(x)
    out = Ly.forward(X, np.ones(64, np.float32), np.zeros((64, 0), np.uint16), np.zeros((0, 1), np.uint16), w, None, "int4")
    qx, qw = out["cX"].astype(np.int64), out["cR"].astype(np.int64)
    dot = int((qx * qw).sum())                                   # exact integer dot product
    sx = float(np.uint16(out["sX"][0, 0]).view(np.float16))
    sw = float(np.uint16(out["sR"][0, 0]).view(np.float16))
    assert out["Y"][0, 0] == dot * sx * sw


def test_section41_error_bound():
    spec = synth.layer_spec("qkv", M=128, K=256, N=192, rank=16, x_outliers=3, w_outliers=3)
    L = synth.draw_layer(spec, seed=4)
    for fmt in ("mxfp4", "int4"):
        ops = Ly.quantize_operands(L["X"], L["lam"], L["R"], fmt)
        Xm = ops["xhat"].astype(np.float64)
        Wm = L["R"].T.astype(np.float64)
        Xq = Q.dequantize(ops["cX"], ops["sX"], fmt)
        Wq = Q.dequantize(ops["cR"], ops["sR"], fmt).T
        E = Ly.quant_error(Xm, Wm, Xq, Wq)
        B = Ly.quant_error_bound(Xm, Wm, Xq, Wq)
        assert 0 < E <= B


def test_lowrank_and_bias_terms_present():
    spec = synth.layer_spec("qkv", M=16, K=128, N=32, rank=8, x_outliers=2, w_outliers=2)
    L = synth.draw_layer(spec, seed=9)
    full = Ly.forward(L["X"], L["lam"], L["L1"], L["L2"], L["R"], L["b"], "mxfp4")["Y"]
    nolr = Ly.forward(L["X"], L["lam"], L["L1"], L["L2"], L["R"], L["b"], "mxfp4", with_lowrank=False)["Y"]
    nob = Ly.forward(L["X"], L["lam"], L["L1"], L["L2"], L["R"], L["b"], "mxfp4", with_bias=False)["Y"]
    xhat = Ly.smooth(L["X"], L["lam"]).astype(np.float64)
    lr = xhat @ F.bf16_value(L["L1"]) @ F.bf16_value(L["L2"])
    np.testing.assert_allclose(full - nolr, lr, rtol=1e-9, atol=1e-9 * np.abs(lr).max())
    np.testing.assert_allclose(full - nob, np.broadcast_to(F.bf16_value(L["b"]), full.shape), atol=1e-12)


def test_forward_rows_matches_forward():
    spec = synth.layer_spec("lowm", M=40, K=256, N=64, rank=8, x_outliers=3, w_outliers=2)
    L = synth.draw_layer(spec, seed=2)
    full = Ly.forward(L["X"], L["lam"], L["L1"], L["L2"], L["R"], L["b"], "mxfp4", gelu_act=True)["Y"]
    rows, cols = np.array([0, 7, 39]), np.array([1, 5, 63])
    part = Ly.forward_rows(L["X"], L["lam"], L["L1"], L["L2"], L["R"], L["b"], "mxfp4", rows, cols, gelu_act=True)
    np.testing.assert_allclose(part, full[np.ix_(rows, cols)], rtol=1e-12, atol=1e-12)


def test_gelu_special_values():
    x = np.array([-30.0, -3.0, -1.0, -1e-3, 0.0, 1e-3, 1.0, 3.0, 30.0])
    y = Ly.gelu(x)
    assert y[4] == 0.0
    np.testing.assert_allclose(y - Ly.gelu(-x), x, rtol=0, atol=1e-15)    # GELU(x) - GELU(-x) = x
    assert y[-1] == 30.0 and abs(y[0]) < 1e-100
    # GELU(1) = Phi(1) = (1 + erf(1/sqrt 2)) / 2, with erf from the standard library
    assert abs(y[6] - 0.5 * (1 + math.erf(1 / math.sqrt(2)))) < 1e-15
    np.testing.assert_allclose(Ly.gelu(1e-3) / 1e-3, 0.5, rtol=1e-3)       # slope 1/2 at 0


def test_parity_metric_detects_planted_error():
    rng = np.random.default_rng(0)
    Y = rng.standard_normal((64, 64))
    assert Ly.within_tolerance(Y, Y)
    bad = Y.copy()
    bad[3, 5] += 0.03 * np.sqrt(np.mean(Y ** 2))
    assert not Ly.within_tolerance(bad, Y)
    assert not Ly.within_tolerance(Y * 1.01, Y)
