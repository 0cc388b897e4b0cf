"""The host-side conversion of a dense layer (w4a4_quantized_linear_amd.convert)
against the oracle's calibration (oracle/decompose.py) and the identities of
the SVDQuant notes page, section 4.2: identical smoothing factors, the same
rank-r branch up to the bf16 rounding of its factors, W_hat = L1 L2 + R up to
the one float32 rounding of R, and an adapter that leaves R untouched."""
import numpy as np
import pytest

import synth
from oracle import decompose as Dc
from oracle import formats as F

torch = pytest.importorskip("torch")
from w4a4_quantized_linear_amd import convert  # noqa: E402


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("name,M,K,N,rank", [("qkv", 96, 256, 384, 32), ("single", 64, 512, 128, 16),
                                             ("lowm", 40, 128, 96, 96)])
def test_convert_matches_oracle_calibration(name, M, K, N, rank):
    spec = synth.layer_spec(name, M=M, K=K, N=N, rank=rank, x_outliers=max(1, K // 50),
                            w_outliers=max(1, K // 50), lora_rank=0)
    raw = synth.draw_raw(spec)
    ref = Dc.calibrate(raw["X"], raw["W"], rank)
    c = convert.convert_linear(_bf16(raw["X"]), _bf16(raw["W"]).t(), rank, _bf16(raw["b"]))
    # smoothing factors: the same float64 formula rounded once to float32
    assert np.array_equal(c["lam"].numpy().view(np.uint32), ref["lam"].view(np.uint32))
    W_hat = ref["W_hat"]
    L1 = F.bf16_value(_bits(c["L1"]))
    L2 = F.bf16_value(_bits(c["L2"]))
    R = c["R"].numpy().T.astype(np.float64)                      # back to K x N
    # W_hat = L1 L2 + R up to the float32 rounding of R
    low = L1 @ L2
    assert np.all(np.abs(low + R - W_hat) <= 2.0 ** -24 * np.abs(W_hat - low) + 1e-300)
    # the branch equals the oracle's up to the bf16 rounding of the factors
    low_o = F.bf16_value(ref["L1"]) @ F.bf16_value(ref["L2"])
    scale = np.abs(F.bf16_value(ref["L1"])) @ np.abs(F.bf16_value(ref["L2"]))
    assert np.all(np.abs(low - low_o) <= 2.0 ** -7 * scale + 1e-12 * np.abs(W_hat).max())
    # the residual's norm is the oracle's tail energy (Eckart-Young) up to that rounding
    tail = np.sqrt(np.sum(ref["S"][rank:] ** 2))
    assert abs(np.linalg.norm(R) - tail) <= 1e-2 * np.linalg.norm(W_hat)


def test_convert_rank_zero_and_adapter():
    spec = synth.layer_spec("lora", M=32, K=256, N=128, rank=8, x_outliers=3, w_outliers=3)
    raw = synth.draw_raw(spec)
    X, Wt = _bf16(raw["X"]), _bf16(raw["W"]).t()
    c0 = convert.convert_linear(X, Wt, 0)
    lam = c0["lam"].numpy().astype(np.float64)
    # rank 0: R is the smoothed weight itself, rounded to float32
    W_hat = lam[:, None] * F.bf16_value(raw["W"])
    assert np.array_equal(c0["R"].numpy(), F.to_fp32(W_hat.T).astype(np.float32))
    assert c0["L1"].shape == (256, 0) and c0["L2"].shape == (0, 128)
    # an adapter is concatenated onto the branch; R is unchanged
    c1 = convert.convert_linear(X, Wt, 8)
    c2 = convert.convert_linear(X, Wt, 8, adapter=(_bf16(raw["A"]), _bf16(raw["B"])))
    assert torch.equal(c1["R"], c2["R"])
    assert c2["L1"].shape == (256, 8 + spec.lora_rank) and c2["L2"].shape == (8 + spec.lora_rank, 128)
    assert np.array_equal(_bits(c2["L1"][:, 8:]), raw["A"]) and np.array_equal(_bits(c2["L2"][8:]), raw["B"])
    assert np.array_equal(_bits(c2["L1"][:, :8]), _bits(c1["L1"]))
