"""SVDQuant W4A4 + low-rank linear layer on MI355X (gfx950).

A thin binding over libsvdq.so (include/svdq.h).  Functions take torch tensors
that live on the GPU, pass their addresses and the current HIP stream to the
library, and return torch tensors allocated for the outputs.  All computation
happens in the library's HIP kernels; there is no fallback path, and every
call raises if the library is not built or the device is not gfx950.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

from ._lib import (EPI_BIAS, EPI_GELU, EPI_LOWRANK, EPI_OUT_F32, INT4_G64, MXFP4, NVFP4, LIB_PATH,  # noqa: F401
                   LayerDesc, SvdqError, check, lib)

FORMATS = {"mxfp4": MXFP4, "int4": INT4_G64, "nvfp4": NVFP4}
GROUPS = {"mxfp4": 32, "int4": 64, "nvfp4": 16}


@dataclass(frozen=True)
class Layer:
    """Shape of one layer: 4-bit format, input features K, output features N, rank."""

    fmt: str
    K: int
    N: int
    rank: int

    def desc(self) -> LayerDesc:
        return LayerDesc(FORMATS[self.fmt], self.K, self.N, self.rank)

    @property
    def group(self) -> int:
        return GROUPS[self.fmt]


def _torch():
    import torch
    return torch


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _desc_ref(layer: Layer):
    d = layer.desc()
    return d, ctypes.byref(d)


def weight_bytes(layer: Layer) -> int:
    d, p = _desc_ref(layer)
    return int(lib().svdq_weight_bytes(p))


def act_bytes(layer: Layer, M: int) -> int:
    d, p = _desc_ref(layer)
    return int(lib().svdq_act_bytes(p, int(M)))


def _empty_u8(n: int, device):
    torch = _torch()
    # torch's caching allocator returns 256-byte aligned blocks for fresh tensors
    return torch.empty(int(n), dtype=torch.uint8, device=device)


def pack_weight(layer: Layer, R, L1, L2, lam, bias=None, out=None, stream=None):
    """R (N x K fp32), L1 (K x r bf16), L2 (r x N bf16), lam (K fp32), bias (N bf16 or None)."""
    d, p = _desc_ref(layer)
    if out is None:
        out = _empty_u8(lib().svdq_weight_bytes(p), R.device)
    st = lib().svdq_pack_weight(p, _ptr(R), _ptr(L1 if layer.rank else None), _ptr(L2 if layer.rank else None),
                                _ptr(lam), _ptr(bias), _ptr(out), _stream(stream))
    check("svdq_pack_weight", st)
    return out


def quantize_act(layer: Layer, w_packed, X, out=None, stream=None):
    """Launch 1: X (M x K bf16, row stride X.stride(0)) -> activation workspace."""
    d, p = _desc_ref(layer)
    M = X.shape[0]
    if out is None:
        out = _empty_u8(lib().svdq_act_bytes(p, M), X.device)
    st = lib().svdq_quantize_act(p, _ptr(w_packed), _ptr(X), M, X.stride(0), _ptr(out), _stream(stream))
    check("svdq_quantize_act", st)
    return out


def gemm(layer: Layer, w_packed, a_packed, M: int, epi: int, out=None, stream=None):
    """Launch 2: Y (M x N, bf16; fp32 with EPI_OUT_F32)."""
    torch = _torch()
    d, p = _desc_ref(layer)
    if out is None:
        dt = torch.float32 if epi & EPI_OUT_F32 else torch.bfloat16
        out = torch.empty((M, layer.N), dtype=dt, device=w_packed.device)
    st = lib().svdq_gemm(p, _ptr(w_packed), _ptr(a_packed), M, _ptr(out), out.stride(0), epi, _stream(stream))
    check("svdq_gemm", st)
    return out


def gemm_quant(layer: Layer, w_packed, a_packed, M: int, epi: int, next_layer: Layer, wn_packed, out=None,
               stream=None):
    """Launch 2 of `layer` with its bf16 output quantized for `next_layer` (fused MLP
    step): returns next_layer's activation workspace, as quantize_act would fill it."""
    d, p = _desc_ref(layer)
    dn, pn = _desc_ref(next_layer)
    if out is None:
        out = _empty_u8(lib().svdq_act_bytes(pn, M), w_packed.device)
    st = lib().svdq_gemm_quant(p, _ptr(w_packed), _ptr(a_packed), M, epi, pn, _ptr(wn_packed), _ptr(out),
                               _stream(stream))
    check("svdq_gemm_quant", st)
    return out


def gemm_qkv(layer: Layer, w_packed, a_packed, M: int, epi: int, norm_q, norm_k, eps: float, rope_cos, rope_sin,
             head_dim: int = 128, out=None, stream=None):
    """Launch 2 of a fused [Q | K | V] layer with the Q/K RMS normalization (weights
    norm_q, norm_k: bf16[head_dim]) and the rotary embedding (rope_cos, rope_sin:
    fp32 M x head_dim/2) in the epilogue; returns Y (M x N bf16)."""
    torch = _torch()
    d, p = _desc_ref(layer)
    if out is None:
        out = torch.empty((M, layer.N), dtype=torch.bfloat16, device=w_packed.device)
    st = lib().svdq_gemm_qkv(p, _ptr(w_packed), _ptr(a_packed), M, epi, head_dim, _ptr(norm_q), _ptr(norm_k),
                             float(eps), _ptr(rope_cos), _ptr(rope_sin), _ptr(out), out.stride(0), _stream(stream))
    check("svdq_gemm_qkv", st)
    return out


def gemm_w4a16(layer: Layer, w_packed, X, epi: int = 0, out=None, stream=None):
    """W4A16: Y = X deQ(Q4(W))^T (+ b) for an INT4 rank-0 blob and bf16 X (M x K);
    returns Y (M x N, bf16, or float32 with EPI_OUT_F32)."""
    torch = _torch()
    d, p = _desc_ref(layer)
    M = X.shape[0]
    if out is None:
        dt = torch.float32 if epi & EPI_OUT_F32 else torch.bfloat16
        out = torch.empty((M, layer.N), dtype=dt, device=X.device)
    st = lib().svdq_gemm_w4a16(p, _ptr(w_packed), _ptr(X), M, X.stride(0), _ptr(out), out.stride(0), epi,
                               _stream(stream))
    check("svdq_gemm_w4a16", st)
    return out


def linear(layer: Layer, w_packed, X, epi: int, out=None, workspace=None, stream=None):
    """Both launches: Y = act(deQ(Q(X/lam)) deQ(Q(R))^T + (X/lam L1) L2 + b)."""
    torch = _torch()
    d, p = _desc_ref(layer)
    M = X.shape[0]
    need = lib().svdq_act_bytes(p, M)
    if workspace is None:
        workspace = _empty_u8(need, X.device)
    if out is None:
        dt = torch.float32 if epi & EPI_OUT_F32 else torch.bfloat16
        out = torch.empty((M, layer.N), dtype=dt, device=X.device)
    st = lib().svdq_linear(p, _ptr(w_packed), _ptr(X), M, X.stride(0), _ptr(out), out.stride(0), epi,
                           _ptr(workspace), workspace.numel(), _stream(stream))
    check("svdq_linear", st)
    return out


def linear_noalloc(layer: Layer, w_packed, X, epi: int, out=None, stream=None):
    """svdq_linear with the workspace in the library's static scratch (no device
    allocation by the library; `out` is allocated here when not given)."""
    torch = _torch()
    d, p = _desc_ref(layer)
    M = X.shape[0]
    if out is None:
        dt = torch.float32 if epi & EPI_OUT_F32 else torch.bfloat16
        out = torch.empty((M, layer.N), dtype=dt, device=X.device)
    st = lib().svdq_linear_noalloc(p, _ptr(w_packed), _ptr(X), M, X.stride(0), _ptr(out), out.stride(0), epi,
                                   _stream(stream))
    check("svdq_linear_noalloc", st)
    return out


def _scales_out(torch, layer: Layer, rows: int, dev):
    """Canonical scales: one byte per group (E8M0 for MXFP4, E4M3 for NVFP4) or fp16 bits (INT4)."""
    dt = torch.int16 if layer.fmt == "int4" else torch.uint8
    return torch.empty((rows, layer.K // layer.group), dtype=dt, device=dev)


def unpack_weight(layer: Layer, w_packed, stream=None) -> dict:
    """Canonical codes (N x K/2), scales, L1, L2, lambda and bias of a packed weight."""
    torch = _torch()
    d, p = _desc_ref(layer)
    dev = w_packed.device
    K, N, r = layer.K, layer.N, layer.rank
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    scales = _scales_out(torch, layer, N, dev)
    L1 = torch.empty((K, r), dtype=torch.int16, device=dev)
    L2 = torch.empty((r, N), dtype=torch.int16, device=dev)
    lam = torch.empty(K, dtype=torch.float32, device=dev)
    bias = torch.empty(N, dtype=torch.int16, device=dev)
    st = lib().svdq_unpack_weight(p, _ptr(w_packed), _ptr(codes), _ptr(scales), _ptr(L1 if r else None),
                                  _ptr(L2 if r else None), _ptr(lam), _ptr(bias), _stream(stream))
    check("svdq_unpack_weight", st)
    return dict(codes=codes, scales=scales, L1=L1, L2=L2, lam=lam, bias=bias)


def unpack_act(layer: Layer, a_packed, M: int, stream=None) -> dict:
    """Canonical codes (M x K/2), scales and D (M x rank fp32) of an activation workspace."""
    torch = _torch()
    d, p = _desc_ref(layer)
    dev = a_packed.device
    K, r = layer.K, layer.rank
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    scales = _scales_out(torch, layer, M, dev)
    D = torch.empty((M, r), dtype=torch.float32, device=dev)
    st = lib().svdq_unpack_act(p, _ptr(a_packed), M, _ptr(codes), _ptr(scales), _ptr(D if r else None),
                               _stream(stream))
    check("svdq_unpack_act", st)
    return dict(codes=codes, scales=scales, D=D)


def device_check() -> bool:
    return lib().svdq_device_check() == 0
