"""Offline calibration of one layer (oracle side).

SVDQuant notes page, section 4.2 ("SVDQuant: absorbing outliers via low-rank
branch"):

1. Migrate activation outliers into the weight by a per-input-channel
   smoothing factor lambda: X_hat = X diag(lambda)^-1, W_hat = diag(lambda) W,
   so that X W = X_hat W_hat exactly (the section's identity).
2. Decompose the smoothed weight with its SVD, W_hat = U Sigma V^T, and keep
   the top r singular values: L1 = U Sigma_r (m x r, m the input-feature
   count), L2 = V_r^T (r x n).
3. The residual R = W_hat - L1 L2 is what is quantized to 4 bits; the branch
   L1 L2 stays in 16 bits.

Readings:

* The pages give no formula for lambda.  The one used is
  lambda_j = sqrt(max_m |X_mj| / max_n |W_jn|) (SmoothQuant with alpha = 1/2),
  evaluated in float64 and rounded once to float32; lambda_j = 1 when either
  maximum is zero.  For a fused QKV weight one lambda serves the concatenated
  weight.
* "16-bit" is bf16 (the Diffusers page's quantization config names bfloat16
  as the compute dtype).  The residual is taken against the rounded factors,
  R = fp32(W_hat - bf16(L1) bf16(L2)), so W_hat = L1b L2b + R holds up to
  the single float32 rounding of R.
* An adapter (LoRA) pair (A, B) is absorbed by concatenation,
  L1 <- [L1 | A], L2 <- [L2 ; B]; R is left untouched, so the packed 4-bit
  residual needs no re-quantization (SVDQuant abstract).

Weights here are in the paper orientation W (K x N, K = input channels).

Pinned by: tests/test_oracle_decompose.py -- Eckart-Young closed form for the
truncation error, monotonicity in r, zero residual at full rank, the exact
smoothing identity, the block identity of an absorbed adapter, and lambda
against its definition evaluated with the standard library.
"""
from __future__ import annotations

import numpy as np

from . import formats as F


def smoothing_factors(X_bits: np.ndarray, W_bits: np.ndarray) -> np.ndarray:
    """lambda (float32[K]) from activations X (M x K bf16) and weight W (K x N bf16)."""
    ax = np.abs(F.bf16_value(X_bits)).max(axis=0)       # per input channel over tokens
    aw = np.abs(F.bf16_value(W_bits)).max(axis=1)       # per input channel over outputs
    with np.errstate(divide="ignore", invalid="ignore"):
        lam = np.sqrt(ax / aw)
    lam = np.where((ax == 0) | (aw == 0), 1.0, lam)
    return F.to_fp32(lam).astype(np.float32)


def smoothed_weight(W_bits: np.ndarray, lam: np.ndarray) -> np.ndarray:
    """W_hat = diag(lambda) W in float64 (exact: fp32 x bf16 needs 32 bits)."""
    return np.asarray(lam, dtype=np.float64)[:, None] * F.bf16_value(W_bits)


def decompose(W_hat: np.ndarray, rank: int) -> dict:
    """Truncated SVD of the smoothed weight and the fp32 residual.

    Returns L1 (K x r bf16 bits), L2 (r x N bf16 bits), R (K x N float32),
    the float64 factors L1_64 / L2_64 and the singular values S.
    """
    U, S, Vt = np.linalg.svd(W_hat, full_matrices=False)
    L1_64 = U[:, :rank] * S[:rank]
    L2_64 = Vt[:rank, :]
    L1b = F.bf16_bits(L1_64)
    L2b = F.bf16_bits(L2_64)
    lowrank = F.bf16_value(L1b) @ F.bf16_value(L2b)
    R = F.to_fp32(W_hat - lowrank).astype(np.float32)
    return dict(L1=L1b, L2=L2b, R=R, L1_64=L1_64, L2_64=L2_64, S=S)


def absorb_adapter(L1b: np.ndarray, L2b: np.ndarray, A: np.ndarray, B: np.ndarray):
    """Concatenate an adapter pair onto the low-rank factors (bf16 bits)."""
    return (np.ascontiguousarray(np.concatenate([L1b, A], axis=1)),
            np.ascontiguousarray(np.concatenate([L2b, B], axis=0)))


def calibrate(X_bits: np.ndarray, W_bits: np.ndarray, rank: int) -> dict:
    """Smoothing factors, then the decomposition of the smoothed weight."""
    lam = smoothing_factors(X_bits, W_bits)
    W_hat = smoothed_weight(W_bits, lam)
    out = decompose(W_hat, rank)
    out["lam"] = lam
    out["W_hat"] = W_hat
    return out
