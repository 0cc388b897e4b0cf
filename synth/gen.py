"""Workload recipes and seeded draws.

Five FLUX-shaped workloads are defined (sizes, rank, 4-bit format and the
outlier recipe of the activations and of the dense weight).  Two kinds of
draw are offered:

* ``draw_raw``   -- the dense tensors a calibration tool starts from:
  activations X (M x K, bf16), dense weight W (K x N, paper orientation,
  bf16), bias b (N, bf16) and, for the adapter workload, a LoRA pair
  A (K x 16), B (16 x N) in bf16.
* ``draw_layer`` -- the operands of an already calibrated SVDQuant layer,
  drawn directly: smoothing factors lambda (fp32[K]), low-rank factors
  L1 (K x r, bf16) and L2 (r x N, bf16), residual R (N x K, fp32, i.e. the
  nn.Linear orientation) and bias b.  The draw follows the structure a
  smoothed-then-decomposed weight has -- the channels whose weight rows
  are magnified by smoothing are carried by the low-rank branch and the
  residual keeps the bulk -- but it is a construction from random numbers,
  not a decomposition: nothing here runs an SVD or divides by lambda.

Random numbers come from ``numpy.random.default_rng(seed)`` (PCG64) with a
fixed draw order.  Values are drawn in float32/float64 and stored as bf16
bit patterns (round to nearest even on the float32 bits) or as float32.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

# ---------------------------------------------------------------------------
# storage helpers (representation only)
# ---------------------------------------------------------------------------


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Store float32 values as bf16 bit patterns, rounding to nearest even."""
    xf = np.ascontiguousarray(x, dtype=np.float32)
    u = xf.view(np.uint32)
    r = (u >> 16) & 1                      # no uint32 overflow for finite inputs
    r += u
    r += 0x7FFF
    r >>= 16
    out = r.astype(np.uint16)
    nan = np.isnan(xf)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# workload recipes
# ---------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    """One linear layer of a workload."""

    name: str
    M: int
    K: int
    N: int
    rank: int
    fmt: str                 # "mxfp4" or "int4"
    x_outliers: int          # number of outlier input channels in X
    x_factor: float          # their scale factor
    w_outliers: int          # number of outlier input channels of W
    w_kind: str              # "scale": N(0,.02) x w_factor ; "t3": 0.02 * Student-t(3)
    w_factor: float
    gelu: bool = False       # GELU applied after this layer (fc1 of the MLP pair)
    lora_rank: int = 0       # adapter rank concatenated onto the SVD factors


def _pct(p: float, K: int) -> int:
    return int(round(p * K))


# The five workloads.  Outlier counts are round(p * K) where the recipe gives
# a percentage.  Config 3 is a pair of layers (fc1 then fc2) in each format.
CONFIGS: Dict[str, LayerSpec] = {}


def _add(spec: LayerSpec) -> None:
    CONFIGS[spec.name] = spec


_add(LayerSpec("single", M=256, K=1024, N=1024, rank=16, fmt="int4",
               x_outliers=8, x_factor=40.0, w_outliers=4, w_kind="scale", w_factor=20.0))
_add(LayerSpec("qkv", M=4608, K=3072, N=9216, rank=32, fmt="mxfp4",
               x_outliers=_pct(0.01, 3072), x_factor=50.0,
               w_outliers=_pct(0.01, 3072), w_kind="t3", w_factor=1.0))
for _fmt in ("mxfp4", "int4", "nvfp4"):
    _add(LayerSpec(f"fc1_{_fmt}", M=4608, K=3072, N=12288, rank=32, fmt=_fmt,
                   x_outliers=_pct(0.01, 3072), x_factor=50.0,
                   w_outliers=_pct(0.01, 3072), w_kind="t3", w_factor=1.0, gelu=True))
    _add(LayerSpec(f"fc2_{_fmt}", M=4608, K=12288, N=3072, rank=32, fmt=_fmt,
                   x_outliers=_pct(0.01, 12288), x_factor=50.0,
                   w_outliers=_pct(0.01, 12288), w_kind="t3", w_factor=1.0))
_add(LayerSpec("lowm", M=1024, K=3072, N=3072, rank=128, fmt="mxfp4",
               x_outliers=_pct(0.02, 3072), x_factor=30.0,
               w_outliers=_pct(0.01, 3072), w_kind="t3", w_factor=1.0))
_add(LayerSpec("lora", M=4608, K=3072, N=12288, rank=32, fmt="mxfp4",
               x_outliers=_pct(0.01, 3072), x_factor=50.0,
               w_outliers=_pct(0.01, 3072), w_kind="t3", w_factor=1.0, lora_rank=16))

# The W4A16 (AWQ-style) modulation projection of a FLUX double block: a batch of
# conditioning vectors (M = 2 tokens) times a 3072 -> 6 x 3072 weight, INT4 g64
# weights and bf16 activations; no smoothing and no low-rank branch.
_add(LayerSpec("mod_w4a16", M=2, K=3072, N=18432, rank=0, fmt="int4",
               x_outliers=0, x_factor=1.0, w_outliers=_pct(0.01, 3072), w_kind="t3", w_factor=1.0))

# Default seeds: one per workload (the workload's position in the list, 1-based;
# the two layers of the MLP pair share seed 3 and are told apart by salt).
SEEDS = {"single": 1, "qkv": 2, "fc1_mxfp4": 3, "fc2_mxfp4": 3, "fc1_int4": 3,
         "fc2_int4": 3, "fc1_nvfp4": 3, "fc2_nvfp4": 3, "lowm": 4, "lora": 5, "mod_w4a16": 6}
_SALT = {"fc2_mxfp4": 7919, "fc2_int4": 7919, "fc2_nvfp4": 7919}


def layer_spec(name: str, **over) -> LayerSpec:
    """Spec of a named layer, optionally with sizes overridden (M, K, N, rank,
    outlier counts) for small test instances of the same recipe."""
    spec = CONFIGS[name]
    if over:
        spec = dataclasses.replace(spec, **over)
    return spec


def _seed(spec: LayerSpec, seed: Optional[int]) -> int:
    base = SEEDS.get(spec.name, 0) if seed is None else seed
    return base * 1_000_003 + _SALT.get(spec.name, 0)


# ---------------------------------------------------------------------------
# draws
# ---------------------------------------------------------------------------


def draw_activations(spec: LayerSpec, rng: np.random.Generator):
    """X (M x K) as bf16 bits: N(0,1) with `x_outliers` channels times x_factor.
    Returns (X_bits, outlier channel indices)."""
    x = rng.standard_normal((spec.M, spec.K), dtype=np.float32)
    idx = np.sort(rng.choice(spec.K, size=spec.x_outliers, replace=False)) if spec.x_outliers else np.zeros(0, np.int64)
    if idx.size:
        x[:, idx] *= np.float32(spec.x_factor)
    return bf16_bits_from_f32(x), idx


def _draw_weight(spec: LayerSpec, rng: np.random.Generator):
    w = rng.standard_normal((spec.K, spec.N), dtype=np.float32) * np.float32(0.02)
    idx = np.sort(rng.choice(spec.K, size=spec.w_outliers, replace=False)) if spec.w_outliers else np.zeros(0, np.int64)
    if idx.size:
        if spec.w_kind == "scale":
            w[idx, :] *= np.float32(spec.w_factor)
        elif spec.w_kind == "t3":
            w[idx, :] = (0.02 * rng.standard_t(3.0, size=(idx.size, spec.N))).astype(np.float32)
        else:
            raise ValueError(spec.w_kind)
    return w, idx


def draw_raw(spec: LayerSpec, seed: Optional[int] = None) -> dict:
    """Dense tensors of a workload, in the fixed draw order
    X, X-outlier channels, W, W-outlier channels, bias, LoRA pair."""
    rng = np.random.default_rng(_seed(spec, seed))
    X, x_idx = draw_activations(spec, rng)
    w, w_idx = _draw_weight(spec, rng)
    b = (rng.standard_normal(spec.N, dtype=np.float32) * np.float32(0.01))
    out = dict(X=X, W=bf16_bits_from_f32(w), b=bf16_bits_from_f32(b),
               x_outliers=x_idx, w_outliers=w_idx)
    if spec.lora_rank:
        A = rng.standard_normal((spec.K, spec.lora_rank), dtype=np.float32) * np.float32(0.02)
        B = rng.standard_normal((spec.lora_rank, spec.N), dtype=np.float32) * np.float32(0.02)
        out["A"] = bf16_bits_from_f32(A)
        out["B"] = bf16_bits_from_f32(B)
    return out


def draw_layer(spec: LayerSpec, seed: Optional[int] = None, with_lora: bool = True) -> dict:
    """Operands of a calibrated layer, drawn directly (see the module note).

    Returns X (M x K bf16 bits), lam (fp32[K]), L1 (K x r bf16 bits),
    L2 (r x N bf16 bits), R (N x K fp32), b (N bf16 bits), plus the channel
    sets used.  With a LoRA rank in the spec and ``with_lora``, the adapter
    pair is appended to the factors (L1 = [L1 | A], L2 = [L2 ; B]) while R is
    the same array as without it.
    """
    rng = np.random.default_rng(_seed(spec, seed) ^ 0x5EED)
    K, N, M, r = spec.K, spec.N, spec.M, spec.rank
    X, x_idx = draw_activations(spec, rng)
    w_idx = np.sort(rng.choice(K, size=spec.w_outliers, replace=False)) if spec.w_outliers else np.zeros(0, np.int64)
    w_idx = np.setdiff1d(w_idx, x_idx)

    # Nominal smoothing scale of a Gaussian channel pair of these sizes
    # (expected column maxima of N(0,1) over M rows and of N(0,.02) over N).
    ax = math.sqrt(2.0 * math.log(max(M, 2)))
    aw = 0.02 * math.sqrt(2.0 * math.log(max(N, 2)))
    lam_base = math.sqrt(ax / aw)
    gx = np.ones(K)
    gx[x_idx] = spec.x_factor
    gw = np.ones(K)
    w_heavy = 20.0 if spec.w_kind == "scale" else 5.0
    gw[w_idx] = spec.w_factor if spec.w_kind == "scale" else w_heavy
    jitter = np.exp(0.05 * rng.standard_normal(K))
    lam = (lam_base * np.sqrt(gx / gw) * jitter).astype(np.float32)

    # Channels whose smoothed weight rows are magnified, largest first:
    # activation-outlier channels, then weight-outlier channels.
    magnified = list(x_idx) + list(w_idx)
    n_abs = min(r, len(magnified))
    absorbed = np.array(magnified[:n_abs], dtype=np.int64)

    # Residual: bulk-level Gaussian rows; non-absorbed heavy channels keep tails.
    rho = 0.02 * lam.astype(np.float64)
    rho[absorbed] = 0.02 * lam_base
    z = rng.standard_normal((N, K), dtype=np.float32)
    heavy_left = np.setdiff1d(w_idx, absorbed)
    if heavy_left.size and spec.w_kind == "t3":
        z[:, heavy_left] = rng.standard_t(3.0, size=(N, heavy_left.size)) / math.sqrt(3.0)
    elif heavy_left.size:
        z[:, heavy_left] *= spec.w_factor
    z *= rho.astype(np.float32)[None, :]
    R = z

    # Low-rank factors: one column per absorbed channel carrying its magnified
    # row (scale = row magnitude * sqrt(N), unit-variance L2 row), then bulk
    # directions with the top bulk singular value of the residual.
    L2 = rng.standard_normal((r, N)) / math.sqrt(N)
    L1 = np.zeros((K, r))
    sig_bulk = 0.02 * lam_base * (math.sqrt(N) + math.sqrt(K))
    L1[:, :] = rng.standard_normal((K, r)) * (0.05 * sig_bulk / math.sqrt(K))
    for i, ch in enumerate(absorbed):
        mag = 0.02 * float(lam[ch]) * math.sqrt(N)
        if ch in set(w_idx.tolist()):
            mag *= (spec.w_factor if spec.w_kind == "scale" else w_heavy)
        L1[ch, i] += mag
    if n_abs < r:
        L1[:, n_abs:] = rng.standard_normal((K, r - n_abs)) * (sig_bulk / math.sqrt(K))
    b = rng.standard_normal(N).astype(np.float32) * np.float32(0.01)

    L1b = bf16_bits_from_f32(L1.astype(np.float32))
    L2b = bf16_bits_from_f32(L2.astype(np.float32))
    out = dict(X=X, lam=lam, L1=L1b, L2=L2b, R=R, b=bf16_bits_from_f32(b),
               x_outliers=x_idx, w_outliers=w_idx, absorbed=absorbed)
    if spec.lora_rank and with_lora:
        A = rng.standard_normal((K, spec.lora_rank), dtype=np.float32) * np.float32(0.02)
        B = rng.standard_normal((spec.lora_rank, N), dtype=np.float32) * np.float32(0.02)
        out["L1_svd"], out["L2_svd"] = L1b, L2b
        out["A"], out["B"] = bf16_bits_from_f32(A), bf16_bits_from_f32(B)
        out["L1"] = np.ascontiguousarray(np.concatenate([L1b, out["A"]], axis=1))
        out["L2"] = np.ascontiguousarray(np.concatenate([L2b, out["B"]], axis=0))
    return out


# ---------------------------------------------------------------------------
# inputs of the fused QKV step
# ---------------------------------------------------------------------------


def draw_w4a16(spec: LayerSpec, seed: Optional[int] = None) -> dict:
    """Operands of a W4A16 layer: X (M x K bf16 bits, N(0,1) with the spec's
    outlier channels), W (N x K fp32, the weight draw of draw_raw transposed:
    N(0, 0.02) with heavy-tailed outlier rows) and b (N bf16 bits)."""
    rng = np.random.default_rng(_seed(spec, seed))
    X, _ = draw_activations(spec, rng)
    w, _ = _draw_weight(spec, rng)
    b = rng.standard_normal(spec.N, dtype=np.float32) * np.float32(0.01)
    return dict(X=X, W=np.ascontiguousarray(w.T), b=bf16_bits_from_f32(b))


def draw_qkv_extras(M: int, head_dim: int = 128, seed: int = 2) -> dict:
    """Inputs of the Q/K normalization and rotary embedding of the fused QKV
    step: the two normalization weights (bf16[head_dim], around 1) and the
    rotary cos / sin per token and pair (fp32, M x head_dim/2).  Angles follow
    the usual rotary recipe, position times a geometric frequency ladder
    10000^(-2p / head_dim), with token positions a random permutation of 0..M-1
    (so rows do not share angles)."""
    rng = np.random.default_rng(seed * 1_000_003 + 4099)
    wq = bf16_bits_from_f32((1.0 + 0.1 * rng.standard_normal(head_dim)).astype(np.float32))
    wk = bf16_bits_from_f32((1.0 + 0.1 * rng.standard_normal(head_dim)).astype(np.float32))
    pos = rng.permutation(M).astype(np.float64)
    freq = 10000.0 ** (-2.0 * np.arange(head_dim // 2) / head_dim)
    ang = pos[:, None] * freq[None, :]
    return {"norm_q": wq, "norm_k": wk, "cos": np.cos(ang).astype(np.float32),
            "sin": np.sin(ang).astype(np.float32), "eps": 1e-6}
