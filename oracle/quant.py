"""Group-wise 4-bit quantization (oracle side).

The quantizer of the SVDQuant notes page, section 3 ("Quantization
Preliminary"): Q_X = round(X / s_X) with s_X = max|X| / q_max, and the
scaled product X W ~ s_X s_W Q_X Q_W.  Here it is applied to each group of
g consecutive elements along the reduction dimension K (one scale per group),
which keeps the product factorable group by group.

Readings taken where the pages leave the step open:

* Group shape: along K, g = 32 for MXFP4 and g = 64 for INT4, for the
  activations (per row of X_hat) and for the residual (per column of R, i.e.
  per row of the N x K nn.Linear-oriented array).
* MXFP4 scale: E8M0 power of two 2^e with e = floor(log2 amax) - 2, clamped to
  [-127, 127]; e = -127 for an all-zero group.  This is the OCP MX choice of
  dividing by the largest power of two not above q_max = 6 (2^2); values that
  land above 6 saturate to 6.  Codes: nearest E2M1 magnitude of x * 2^-e,
  ties to even, sign copied from x (so -0 gives the code 0b1000).
* INT4 scale: s = fp16(fp32(amax / 7)) (q_max = 7, so the symmetric grid
  [-7, 7] is used; the notes page's worked example gives the INT4 range
  [-8, 7]), clamped to the fp16 maximum 65504.  If s == 0 every code is 0;
  otherwise q = clamp(rint(fp32(x / s)), -8, 7), rint = nearest even.
* NVFP4-style (the Nunchaku in Diffusers page names NVFP4 as the 4-bit float
  format of its Blackwell kernels; the format details are not on the pages,
  so the standard two-level NVFP4 layout is taken): groups of 16 along K,
  E2M1 codes, one E4M3 scale per group and one float32 scale gs per tensor.
  a6 = fp32(amax / 6), u = fp32(a6 / gs), the group scale byte is the nearest
  E4M3 value of u (ties to even, saturating at 448), S = fp32(E4M3(u) * gs),
  and each code is the nearest E2M1 value of t = fp32(x / S) (ties to even,
  saturating at 6, sign copied); when S == 0 every t is a zero carrying the
  sign of x.  The residual's gs is fp32(max|R| / (6 * 448)), so the largest
  group scale lands on 448; the activations use gs = 1 (their group scales are
  stored directly in E4M3; smoothing has already brought X_hat to a moderate
  range).  Dequantized value: E2M1 * E4M3 * gs.
* All of this decision arithmetic is IEEE float32 (the division x_hat = X /
  lambda, amax / 7 and x / s are correctly rounded float32 operations).

Canonical packing: two codes per byte along K, the even-K element in the low
nibble; INT4 codes are stored as their 4-bit two's complement.

Pinned by: tests/test_oracle_quant.py -- the worked example of section 3
(tests/golden/worked_example.txt), the exhaustive E2M1 tie table, INT4
half-integer ties, idempotence of quantize o dequantize, and scale edge
cases (zero groups, subnormal maxima, saturation).
"""
from __future__ import annotations

import numpy as np

from . import formats as F

GROUP = {"mxfp4": 32, "int4": 64, "nvfp4": 16}
NVFP4_GLOBAL_DIV = 6.0 * 448.0          # q_max of E2M1 times the largest E4M3 value


def _groups(x: np.ndarray, g: int) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] % g:
        raise ValueError(f"expected rows x K with K a multiple of {g}, got {x.shape}")
    return x.reshape(x.shape[0], x.shape[1] // g, g)


def mxfp4_quantize(x: np.ndarray, row_chunk: int = 1024):
    """x: float32 rows x K.  Returns (codes uint8 rows x K holding one E2M1
    nibble each, scales uint8 rows x K/32 holding E8M0 bytes)."""
    x = np.asarray(x, dtype=np.float32)
    rows, K = x.shape
    codes = np.empty((rows, K), dtype=np.uint8)
    scales = np.empty((rows, K // 32), dtype=np.uint8)
    for r0 in range(0, rows, row_chunk):
        g = _groups(x[r0:r0 + row_chunk], 32)
        amax = np.abs(g).max(axis=-1)                       # float32, exact
        _, E = np.frexp(amax.astype(np.float64))            # amax = m 2^E, m in [0.5, 1)
        e = np.where(amax == 0, -127, np.clip(E - 3, -127, 127))   # floor(log2 amax) - 2
        v = g.astype(np.float64) * np.ldexp(1.0, -e)[..., None]     # exact scaling
        codes[r0:r0 + row_chunk] = F.e2m1_encode(v).reshape(g.shape[0], K)
        scales[r0:r0 + row_chunk] = (e + 127).astype(np.uint8)
    return codes, scales


def mxfp4_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes)
    rows, K = codes.shape
    vals = F.e2m1_decode(codes).reshape(rows, K // 32, 32)
    return (vals * F.e8m0_value(scales)[..., None]).reshape(rows, K)


def int4_quantize(x: np.ndarray, row_chunk: int = 1024):
    """x: float32 rows x K.  Returns (codes int8 rows x K in [-8, 7],
    scales uint16 rows x K/64 holding fp16 bit patterns)."""
    x = np.asarray(x, dtype=np.float32)
    rows, K = x.shape
    codes = np.empty((rows, K), dtype=np.int8)
    scales = np.empty((rows, K // 64), dtype=np.uint16)
    for r0 in range(0, rows, row_chunk):
        g = _groups(x[r0:r0 + row_chunk], 64)
        amax = np.abs(g).max(axis=-1)                                   # float32
        s32 = (amax / np.float32(7.0)).astype(np.float32)               # IEEE fp32 divide
        s16 = np.minimum(F.to_fp16(s32), F.FP16_MAX)                    # fp16 RNE, clamped
        s16f = s16.astype(np.float32)                                   # exact widening
        with np.errstate(divide="ignore", invalid="ignore"):
            t = (g / s16f[..., None]).astype(np.float32)                # IEEE fp32 divide
        q = np.clip(np.rint(t), -8, 7)
        q = np.where(s16f[..., None] == 0, 0, q)
        codes[r0:r0 + row_chunk] = q.astype(np.int8).reshape(g.shape[0], K)
        scales[r0:r0 + row_chunk] = F.fp16_bits(s16)
    return codes, scales


def int4_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.int64)
    rows, K = codes.shape
    s = F.fp16_value(scales)
    return (codes.reshape(rows, K // 64, 64) * s[..., None]).reshape(rows, K).astype(np.float64)


def nvfp4_global_scale(x: np.ndarray) -> np.float32:
    """gs = fp32(max|x| / 2688) for a whole tensor (float32 IEEE division)."""
    amax = np.float32(np.abs(np.asarray(x, dtype=np.float32)).max()) if np.asarray(x).size else np.float32(0)
    return np.float32(amax / np.float32(NVFP4_GLOBAL_DIV))


def nvfp4_quantize(x: np.ndarray, gs=1.0, row_chunk: int = 1024):
    """x: float32 rows x K, gs: the tensor's float32 scale.  Returns (codes uint8
    rows x K holding one E2M1 nibble each, scales uint8 rows x K/16 holding E4M3
    bytes)."""
    x = np.asarray(x, dtype=np.float32)
    gs = np.float32(gs)
    rows, K = x.shape
    codes = np.empty((rows, K), dtype=np.uint8)
    scales = np.empty((rows, K // 16), dtype=np.uint8)
    for r0 in range(0, rows, row_chunk):
        g = _groups(x[r0:r0 + row_chunk], 16)
        amax = np.abs(g).max(axis=-1)                                   # float32
        a6 = (amax / np.float32(6.0)).astype(np.float32)                # IEEE fp32 divide
        with np.errstate(divide="ignore", invalid="ignore"):
            u = (a6 / gs).astype(np.float32) if gs != 0 else np.zeros_like(a6)
        sb = F.e4m3_encode(u.astype(np.float64))
        S = (F.e4m3_value(sb).astype(np.float32) * gs).astype(np.float32)   # one fp32 rounding
        with np.errstate(divide="ignore", invalid="ignore"):
            t = np.where(S[..., None] == 0, np.float32(0) * g, g / S[..., None]).astype(np.float32)
        codes[r0:r0 + row_chunk] = F.e2m1_encode(t.astype(np.float64)).reshape(g.shape[0], K)
        scales[r0:r0 + row_chunk] = sb
    return codes, scales


def nvfp4_dequantize(codes: np.ndarray, scales: np.ndarray, gs=1.0) -> np.ndarray:
    codes = np.asarray(codes)
    rows, K = codes.shape
    vals = F.e2m1_decode(codes).reshape(rows, K // 16, 16)
    return (vals * F.e4m3_value(scales)[..., None] * float(np.float32(gs))).reshape(rows, K)


def quantize(x: np.ndarray, fmt: str, gs=1.0):
    """Codes and scales of x; gs is the NVFP4 tensor scale (ignored otherwise)."""
    if fmt == "mxfp4":
        return mxfp4_quantize(x)
    if fmt == "int4":
        return int4_quantize(x)
    if fmt == "nvfp4":
        return nvfp4_quantize(x, gs)
    raise ValueError(fmt)


def dequantize(codes: np.ndarray, scales: np.ndarray, fmt: str, gs=1.0) -> np.ndarray:
    if fmt == "mxfp4":
        return mxfp4_dequantize(codes, scales)
    if fmt == "int4":
        return int4_dequantize(codes, scales)
    if fmt == "nvfp4":
        return nvfp4_dequantize(codes, scales, gs)
    raise ValueError(fmt)


def nibbles(codes: np.ndarray) -> np.ndarray:
    """4-bit field of each code (INT4 as two's complement)."""
    return (np.asarray(codes).astype(np.int64) & 0xF).astype(np.uint8)


def pack_canonical(codes: np.ndarray) -> np.ndarray:
    """Two codes per byte along K; element 2j in the low nibble of byte j."""
    n = nibbles(codes)
    return (n[:, 0::2] | (n[:, 1::2] << 4)).astype(np.uint8)


def unpack_canonical(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out
