"""4-bit weight x 16-bit activation linear (oracle side).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The Nunchaku in Diffusers page (section "Introducing Nunchaku Lite") names the
second kernel family next to the SVDQuant W4A4 layer: 4-bit weights with 16-bit
activations (AWQ) for the adaptive-normalization and modulation projections,
which are memory-bound and precision-sensitive.  The SVDQuant notes page (its
comparison of SmoothQuant and AWQ with SVDQuant) describes AWQ as
activation-aware weight quantization: the salient
channels are protected by a per-channel scale moved between weights and
activations, which is folded into the weight before quantization (and into the
producer of X), so the kernel itself computes

    Y = X . deQ(Q4(W))^T + b,

X in bf16 (not quantized), W (N x K) quantized with the INT4 rule of
oracle/quant.py (groups of 64 along K, fp16 scale), accumulation exact here
(float64), b in bf16.
"""
from __future__ import annotations

import numpy as np

from . import formats as F
from . import quant as Q


def forward(X_bits: np.ndarray, W_nk: np.ndarray, b_bits) -> dict:
    """X (M x K bf16 bits), W (N x K float32), b (N bf16 bits or None)."""
    cW, sW = Q.quantize(np.asarray(W_nk, dtype=np.float32), "int4")
    wq = Q.dequantize(cW, sW, "int4")
    x = F.bf16_value(X_bits).astype(np.float64)
    Y = x @ wq.T
    if b_bits is not None:
        Y = Y + F.bf16_value(b_bits).astype(np.float64)[None, :]
    return {"Y": Y, "cW": cW, "sW": sW}
