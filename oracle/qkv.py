"""Fused QKV projection with Q/K RMS normalization and rotary embedding (oracle side).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py): imported by the tests, the
smoke check and the benchmark's CPU baseline, never by the product.

The Nunchaku in Diffusers page (section "Quantizing your own model", the FLUX.1
QKV example) describes the grouped to_qkv module: one quantized linear whose
output is the concatenation [Q | K | V] along the output features, consumed by a
fused operator that applies the Q and K normalization modules (norm_q, norm_k)
and the rotary embedding together with the projection.  The page names the
pieces but does not write out their arithmetic; the readings taken here are the
standard definitions of the modules it names:

  * heads: Q, K and V each hold H heads of head_dim D consecutive features;
  * RMS normalization per head and token: n(x) = x / sqrt(mean(x^2) + eps) * w,
    with w the module's per-feature weight (bf16 values, shared by all heads);
  * rotary embedding on consecutive pairs (2p, 2p+1) of a head: the pair, read as
    the complex number x[2p] + i x[2p+1], is multiplied by cos + i sin of the
    token's angle for pair p (cos and sin given per token and pair);
  * V passes through unchanged; the rotation follows the normalization.

Everything is float64 on the layer output before its bf16 rounding.
"""
from __future__ import annotations

import numpy as np


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x (..., D) -> x / sqrt(mean over the last axis of x^2 + eps) * w."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)


def rotate_pairs(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """x (M, ..., D); cos, sin (M, D/2): pair p of every head times cos + i sin."""
    x = np.asarray(x, dtype=np.float64)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    shape = (x.shape[0],) + (1,) * (x.ndim - 2) + (x.shape[-1] // 2,)
    rot = np.asarray(cos, dtype=np.float64).reshape(shape) + 1j * np.asarray(sin, dtype=np.float64).reshape(shape)
    z = z * rot
    out = np.empty_like(x)
    out[..., 0::2] = z.real
    out[..., 1::2] = z.imag
    return out


def qkv_norm_rope(Y: np.ndarray, head_dim: int, w_q: np.ndarray, w_k: np.ndarray, eps: float,
                  cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Y (M x 3 H D) = [Q | K | V] -> [rope(n_q(Q)) | rope(n_k(K)) | V], float64."""
    Y = np.asarray(Y, dtype=np.float64)
    M, N = Y.shape
    assert N % (3 * head_dim) == 0
    hd = N // 3
    H = hd // head_dim
    out = Y.copy()
    for s, w in ((0, w_q), (1, w_k)):
        part = Y[:, s * hd:(s + 1) * hd].reshape(M, H, head_dim)
        part = rotate_pairs(rms_norm(part, w, eps), cos, sin)
        out[:, s * hd:(s + 1) * hd] = part.reshape(M, hd)
    return out
