"""Layer output, error measure and parity comparison (oracle side).

SVDQuant notes page, section 4.2, the layer identity
    X W = X_hat W_hat = X_hat L1 L2 + X_hat R ~ X_hat L1 L2 + Q(X_hat) Q(R),
and section 4.3 (Nunchaku): the down projection X_hat L1 shares the pass that
quantizes X_hat, the up projection (X_hat L1) L2 is added to the 4-bit
product's output.  With a bias b and an optional GELU:

    Y = act( deQ(Q4(X_hat)) deQ(Q4(R)) + (X_hat L1) L2 + b ).

Steps (each a plain definition, float64 unless stated):
  1. X_hat = fp32(X) / lambda                (float32 IEEE division)
  2. (cX, sX) = Q4(X_hat) per row, groups along K      -> quant.py
  3. (cR, sR) = Q4(R) per output column, groups along K -> quant.py
  4. D = X_hat L1                            (float64; X_hat exact as fp32)
  5. Y = deQ(cX, sX) deQ(cR, sR)^T + D L2 + b (float64; dequantized values are
     exact in float64)
  6. GELU, if asked: y * Phi(y) = y (1 + erf(y / sqrt 2)) / 2 (erf form).

Section 4.1's error E(X, W) = ||X W - Q(X) Q(W)||_F and its bound
||X|| ||W - Q(W)|| + ||X - Q(X)|| (||W|| + ||W - Q(W)||) (Frobenius norms)
are provided for the invariant tests.

Parity criterion (floating point): max|Y - Y_o| <= 2e-2 * rms(Y_o) and
sum|Y - Y_o| / sum|Y_o| <= 5e-3 (the mean relative error read as a ratio of
means, since a per-element ratio diverges near zero).

Pinned by: tests/test_oracle_layer.py -- exact rational brute force of the
whole layer on small shapes, reduction to a textbook matmul at full rank,
reduction to plain group-wise W4A4 at rank 0 with lambda = 1, reduction to a
scaled integer dot product at K = g, M = N = 1, the section 4.1 bound, and
GELU special values.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf

from . import formats as F
from . import quant as Q


def smooth(X_bits: np.ndarray, lam: np.ndarray) -> np.ndarray:
    """X_hat = fp32(X) / lambda, a float32 IEEE division per element."""
    x = F.bf16_value(X_bits).astype(np.float32)
    return (x / np.asarray(lam, dtype=np.float32)[None, :]).astype(np.float32)


def gelu(y: np.ndarray) -> np.ndarray:
    y = np.asarray(y, dtype=np.float64)
    return 0.5 * y * (1.0 + erf(y / math.sqrt(2.0)))


def quantize_operands(X_bits, lam, R_nk, fmt: str) -> dict:
    """Steps 1-3: smoothed activations and both quantized operands.
    R_nk is the residual in nn.Linear orientation (N x K, float32)."""
    xhat = smooth(X_bits, lam)
    R_nk = np.asarray(R_nk, dtype=np.float32)
    gsR = Q.nvfp4_global_scale(R_nk) if fmt == "nvfp4" else np.float32(1.0)
    cX, sX = Q.quantize(xhat, fmt)
    cR, sR = Q.quantize(R_nk, fmt, gsR)
    return dict(xhat=xhat, cX=cX, sX=sX, cR=cR, sR=sR, gsR=gsR)


def down_projection(xhat: np.ndarray, L1_bits: np.ndarray) -> np.ndarray:
    """Step 4: D = X_hat L1 in float64."""
    return xhat.astype(np.float64) @ F.bf16_value(L1_bits)


def forward(X_bits, lam, L1_bits, L2_bits, R_nk, b_bits, fmt: str, gelu_act: bool = False,
            with_lowrank: bool = True, with_bias: bool = True) -> dict:
    """The layer output Y_o (float64, M x N) and every intermediate."""
    ops = quantize_operands(X_bits, lam, R_nk, fmt)
    xq = Q.dequantize(ops["cX"], ops["sX"], fmt)
    rq = Q.dequantize(ops["cR"], ops["sR"], fmt, ops["gsR"])
    y = xq @ rq.T
    if with_lowrank and L1_bits is not None and np.asarray(L1_bits).shape[1] > 0:
        D = down_projection(ops["xhat"], L1_bits)
        ops["D"] = D
        y = y + D @ F.bf16_value(L2_bits)
    if with_bias and b_bits is not None:
        y = y + F.bf16_value(b_bits)[None, :]
    if gelu_act:
        y = gelu(y)
    ops["Y"] = y
    return ops


def forward_rows(X_bits, lam, L1_bits, L2_bits, R_nk, b_bits, fmt: str, rows, cols=None,
                 gelu_act: bool = False) -> np.ndarray:
    """Y_o restricted to selected rows and columns, for checks at full size.
    Quantization is per row of X_hat and per output column of R, so only the
    selected rows of X and of the N x K residual are quantized."""
    rows = np.asarray(rows)
    R_nk = np.asarray(R_nk, dtype=np.float32)
    gsR = Q.nvfp4_global_scale(R_nk) if fmt == "nvfp4" else np.float32(1.0)   # of the whole tensor
    if cols is not None:
        cols = np.asarray(cols)
        R_nk = R_nk[cols]
    cR, sR = Q.quantize(R_nk, fmt, gsR)
    rq = Q.dequantize(cR, sR, fmt, gsR)
    xhat = smooth(np.asarray(X_bits)[rows], lam)
    cX, sX = Q.quantize(xhat, fmt)
    xq = Q.dequantize(cX, sX, fmt)
    y = xq @ rq.T
    if L1_bits is not None and np.asarray(L1_bits).shape[1] > 0:
        L2 = F.bf16_value(L2_bits)
        if cols is not None:
            L2 = L2[:, cols]
        y = y + down_projection(xhat, L1_bits) @ L2
    if b_bits is not None:
        b = F.bf16_value(b_bits)
        if cols is not None:
            b = b[cols]
        y = y + b[None, :]
    return gelu(y) if gelu_act else y


def quant_error(Xm: np.ndarray, Wm: np.ndarray, Xq: np.ndarray, Wq: np.ndarray) -> float:
    """Section 4.1: E = ||X W - Q(X) Q(W)||_F (all float64 arrays, W as K x N)."""
    return float(np.linalg.norm(Xm @ Wm - Xq @ Wq))


def quant_error_bound(Xm, Wm, Xq, Wq) -> float:
    """Section 4.1's bound on E."""
    nX = np.linalg.norm(Xm)
    nW = np.linalg.norm(Wm)
    dW = np.linalg.norm(Wm - Wq)
    dX = np.linalg.norm(Xm - Xq)
    return float(nX * dW + dX * (nW + dW))


def parity_metrics(Y, Y_o) -> dict:
    Y = np.asarray(Y, dtype=np.float64)
    Y_o = np.asarray(Y_o, dtype=np.float64)
    err = np.abs(Y - Y_o)
    rms = float(np.sqrt(np.mean(Y_o ** 2)))
    return dict(max_abs=float(err.max()) if err.size else 0.0, rms=rms,
                max_over_rms=float(err.max() / rms) if err.size and rms > 0 else 0.0,
                mean_rel=float(err.sum() / np.abs(Y_o).sum()) if err.size and np.abs(Y_o).sum() > 0 else 0.0)


MAX_OVER_RMS = 2e-2
MEAN_REL = 5e-3


def within_tolerance(Y, Y_o) -> bool:
    m = parity_metrics(Y, Y_o)
    return m["max_over_rms"] <= MAX_OVER_RMS and m["mean_rel"] <= MEAN_REL
