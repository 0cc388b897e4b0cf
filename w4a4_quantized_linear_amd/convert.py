"""Offline conversion of a dense linear layer into the operands svdq_pack_weight takes.

SVDQuant notes page, section 4.2 ("absorbing outliers via low-rank branch"):
activation outliers are migrated into the weight by a per-input-channel
smoothing factor lambda (X_hat = X diag(lambda)^-1, W_hat = diag(lambda) W, so
the product is unchanged), the smoothed weight's top-r singular directions
become the 16-bit branch L1 L2, and what remains, R = W_hat - L1 L2, is the part
quantized to 4 bits.  The SVDQuant abstract page adds that an adapter is taken
in by extending the branch, with R left as it is.

This runs once per layer at load time, on the host, in float64:
  lambda_j = sqrt(max_m |X_mj| / max_n |W_nj|), rounded once to float32 (the
      pages give no formula; this is the square-root balance between the two
      maxima, and lambda_j = 1 when either maximum is zero);
  L1 = U_r Sigma_r and L2 = V_r^T from the thin SVD of W_hat (K x N), rounded
      to bf16 (round to nearest even);
  R = float32(W_hat - L1 L2), with the rounded factors, so W_hat = L1 L2 + R
      up to that one rounding; returned as N x K (nn.Linear orientation).

It is not part of the per-call path: svdq_quantize_act / svdq_gemm never call it.
"""
from __future__ import annotations


def _torch():
    import torch
    return torch


def smoothing_factors(x_calib, weight):
    """lambda (float32[K], CPU) from calibration activations (M x K) and the
    dense weight (N x K, nn.Linear orientation); any float dtype, any device."""
    torch = _torch()
    ax = x_calib.detach().to("cpu", torch.float64).abs().amax(dim=0)
    aw = weight.detach().to("cpu", torch.float64).abs().amax(dim=0)
    ok = (ax > 0) & (aw > 0)
    lam = torch.where(ok, torch.sqrt(ax / torch.where(ok, aw, torch.ones_like(aw))), torch.ones_like(ax))
    return lam.to(torch.float32)


def convert_linear(x_calib, weight, rank: int, bias=None, adapter=None) -> dict:
    """Operands of the 4-bit layer replacing y = x W^T + b.

    x_calib  M x K activations the smoothing is calibrated on
    weight   N x K dense weight
    rank     SVD rank r of the 16-bit branch (0 <= r <= min(K, N))
    bias     N values or None
    adapter  optional (A, B): A K x s and B s x N, bf16, concatenated onto the
             branch as [L1 | A] and [L2 ; B] (R unchanged)

    Returns CPU tensors: lam (float32[K]), L1 (bf16 K x r'), L2 (bf16 r' x N),
    R (float32 N x K) and b (bf16[N] or None), with r' = r + s.
    """
    torch = _torch()
    W = weight.detach().to("cpu", torch.float64)
    N, K = W.shape
    if not 0 <= rank <= min(K, N):
        raise ValueError(f"rank {rank} outside [0, {min(K, N)}]")
    lam = smoothing_factors(x_calib, weight)
    W_hat = lam.to(torch.float64)[:, None] * W.t()                 # K x N, exact products
    if rank > 0:
        U, S, Vh = torch.linalg.svd(W_hat, full_matrices=False)
        L1 = (U[:, :rank] * S[:rank]).to(torch.bfloat16)
        L2 = Vh[:rank, :].to(torch.bfloat16)
        R = (W_hat - L1.to(torch.float64) @ L2.to(torch.float64)).to(torch.float32)
    else:
        L1 = torch.zeros((K, 0), dtype=torch.bfloat16)
        L2 = torch.zeros((0, N), dtype=torch.bfloat16)
        R = W_hat.to(torch.float32)
    if adapter is not None:
        A, B = adapter
        L1 = torch.cat([L1, A.detach().to("cpu", torch.bfloat16)], dim=1)
        L2 = torch.cat([L2, B.detach().to("cpu", torch.bfloat16)], dim=0)
    b = None if bias is None else bias.detach().to("cpu", torch.bfloat16)
    return {"lam": lam, "L1": L1.contiguous(), "L2": L2.contiguous(), "R": R.t().contiguous(), "b": b}
