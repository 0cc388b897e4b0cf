"""Calibrated operands of the workloads (test side).

Each workload layer is built the way the SVDQuant notes page, section 4.2,
describes a layer being made from a dense one, with the oracle's own
calibration (oracle/decompose.py) on the dense seeded draw (synth.draw_raw):

  lambda_j = sqrt(max_m |X_mj| / max_n |W_jn|)  (float64, rounded to float32)
  W_hat    = diag(lambda) W
  L1, L2   = top-r SVD factors of W_hat, rounded to bf16
  R        = fp32(W_hat - L1 L2), handed to the layer as N x K

The adapter workload concatenates its drawn LoRA pair onto the SVD factors
(absorb_adapter); R is the rank-32 residual, untouched by the adapter.

The second layer of the MLP pair takes as input the hidden activation of the
dense MLP it replaces: H = bf16(GELU(X W1 + b1)) with the first layer's dense
draw, in float64 (exact erf GELU).  Its smoothing factors are calibrated on
that H.

A FLUX-sized decomposition takes 10-20 s on a few host cores, so results are
kept in memory for the process and in .npy files under $SVDQ_CALIB_CACHE (or
the temp directory), keyed by the draw's seed and shape.  Nothing here runs on
the GPU, and nothing is taken from the HIP path.
"""
from __future__ import annotations

import os
import tempfile

import numpy as np

import synth
from oracle import decompose as Dc
from oracle import formats as F
from oracle import layer as Ly

_MEM: dict = {}
_KEYS = ("X", "lam", "L1", "L2", "R", "b")


def cache_dir() -> str:
    d = os.environ.get("SVDQ_CALIB_CACHE") or os.path.join(tempfile.gettempdir(), "svdq_calib")
    os.makedirs(d, exist_ok=True)
    return d


def _key(spec, seed) -> str:
    base = spec.name.split("_")[0] if spec.name.startswith(("fc1_", "fc2_")) else spec.name
    s = synth.SEEDS.get(spec.name, 0) if seed is None else seed
    return (f"{base}_s{s}_M{spec.M}_K{spec.K}_N{spec.N}_r{spec.rank}_l{spec.lora_rank}"
            f"_x{spec.x_outliers}_w{spec.w_outliers}")


def _load(key):
    d = cache_dir()
    paths = {k: os.path.join(d, f"{key}.{k}.npy") for k in _KEYS}
    if all(os.path.exists(p) for p in paths.values()):
        try:
            return {k: np.load(p) for k, p in paths.items()}
        except (OSError, ValueError):
            return None
    return None


def _store(key, L):
    d = cache_dir()
    for k in _KEYS:
        tmp = os.path.join(d, f"{key}.{k}.tmp.npy")
        np.save(tmp, np.ascontiguousarray(L[k]))
        os.replace(tmp, os.path.join(d, f"{key}.{k}.npy"))


def dense_hidden(raw1) -> np.ndarray:
    """bf16 bits of GELU(X W1 + b1) for the dense first layer of the MLP pair."""
    y = F.bf16_value(raw1["X"]) @ F.bf16_value(raw1["W"])
    y += F.bf16_value(raw1["b"])[None, :]
    return F.bf16_bits(Ly.gelu(y))


def _calibrate(spec, seed):
    if spec.name.startswith("fc2_"):
        s1 = synth.layer_spec(spec.name.replace("fc2_", "fc1_"), M=spec.M, K=synth.CONFIGS[spec.name.replace(
            "fc2_", "fc1_")].K, N=spec.K)
        raw1 = synth.draw_raw(s1, seed)
        X = dense_hidden(raw1)
        del raw1
    else:
        X = None
    raw = synth.draw_raw(spec, seed)
    if X is None:
        X = raw["X"]
    c = Dc.calibrate(X, raw["W"], spec.rank)
    L1, L2 = c["L1"], c["L2"]
    if spec.lora_rank:
        L1, L2 = Dc.absorb_adapter(L1, L2, raw["A"], raw["B"])
    return dict(X=X, lam=c["lam"], L1=L1, L2=L2, R=np.ascontiguousarray(c["R"].T), b=raw["b"])


def calibrated_layer(spec, seed=None) -> dict:
    """X (M x K bf16 bits), lam (fp32[K]), L1 (K x r bf16), L2 (r x N bf16),
    R (N x K fp32) and b (N bf16) of the workload layer `spec`, calibrated."""
    key = _key(spec, seed)
    if key in _MEM:
        return _MEM[key]
    L = _load(key)
    if L is None:
        L = _calibrate(spec, seed)
        _store(key, L)
    if len(_MEM) >= 2:
        _MEM.pop(next(iter(_MEM)))
    _MEM[key] = L
    return L
