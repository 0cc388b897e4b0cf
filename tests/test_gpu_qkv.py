"""Fused QKV step (svdq_gemm_qkv): the [Q | K | V] projection with the Q/K RMS
normalization and the rotary embedding in the GEMM epilogue, against the
oracle's layer output passed through oracle/qkv.py (float64), element by
element at a medium size and on sampled tokens (all of their heads) at the
FLUX QKV size, in every format.  The V heads must equal svdq_gemm's bf16
output bit for bit."""
import numpy as np
import pytest

import synth
import w4a4_quantized_linear_amd as sq
from oracle import layer as Ly
from oracle import qkv as QK
from oracle import formats as F

from _gpu_helpers import bf16_to_np, check_bf16_output, dev_tensor, pack

pytestmark = pytest.mark.gpu

EPI = sq.EPI_LOWRANK | sq.EPI_BIAS


@pytest.fixture(scope="module")
def torch_dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sq.lib()
    assert sq.device_check(), "current device is not gfx950"
    return torch, torch.device("cuda:0")


def _run(torch, dev, L, E, layer, M):
    w = pack(layer, L, torch, dev)
    ws = sq.quantize_act(layer, w, dev_tensor(L["X"], torch, dev))
    Yq = sq.gemm_qkv(layer, w, ws, M, EPI, dev_tensor(E["norm_q"], torch, dev), dev_tensor(E["norm_k"], torch, dev),
                     E["eps"], dev_tensor(E["cos"], torch, dev), dev_tensor(E["sin"], torch, dev))
    Yp = sq.gemm(layer, w, ws, M, EPI)
    torch.cuda.synchronize()
    return Yq, Yp


def _oracle(Y_o, E):
    return QK.qkv_norm_rope(Y_o, 128, F.bf16_value(E["norm_q"]), F.bf16_value(E["norm_k"]), E["eps"],
                            E["cos"], E["sin"])


def _random_cases(n, seed):
    """Seeded random shapes: M from 1 to 1200, K a multiple of 512 up to 2048,
    1 to 12 heads per projection, ranks 0 to 64 not all aligned to 16."""
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 1201)), 512 * int(rng.integers(1, 5)), 3 * 128 * int(rng.integers(1, 13)),
             int(rng.choice([0, 8, 16, 40, 64])), 300 + i) for i in range(n)]


# 128 x 128 tiles (a head split between two waves) in the first three; 256 x 256
# tiles (192 of them, a head per wave) in the fourth; then seeded random shapes
QKV_CASES = [(300, 1024, 768, 16, 1), (17, 512, 1536, 32, 2), (256, 512, 384, 0, 3),
             (2048, 512, 6144, 16, 4)] + _random_cases(4, 2028)
# MXFP4 only: 612 tiles of 128 x 128 with K = 1536, three workgroups per CU
QKV_CASES += [(2100, 1536, 4608, 32, 5)]


# every format: MXFP4 on all cases; INT4 and NVFP4 (their GEMMs take 128 x 128
# tiles at every size) on the first three and two of the random shapes
FMT_CASES = ([("mxfp4",) + c for c in QKV_CASES] +
             [(f,) + c for f in ("int4", "nvfp4") for c in QKV_CASES[:3] + QKV_CASES[4:6]])


@pytest.mark.parametrize("fmt,M,K,N,rank,seed", FMT_CASES)
def test_qkv_elementwise(torch_dev, fmt, M, K, N, rank, seed):
    torch, dev = torch_dev
    spec = synth.layer_spec("qkv", M=M, K=K, N=N, rank=rank, x_outliers=max(1, K // 100),
                            w_outliers=max(1, K // 100), lora_rank=0)
    L = synth.draw_layer(spec, seed=seed)
    E = synth.draw_qkv_extras(M, seed=seed)
    layer = sq.Layer(fmt, K, N, rank)
    print(f"qkv {fmt} M={M} K={K} N={N} r={rank}", flush=True)
    Yq, Yp = _run(torch, dev, L, E, layer, M)
    Y_o = Ly.forward(L["X"], L["lam"], L["L1"], L["L2"], L["R"], L["b"], fmt)["Y"]
    want = _oracle(Y_o, E)
    got = bf16_to_np(Yq)
    hd = N // 3
    check_bf16_output(got[:, :2 * hd], want[:, :2 * hd], "normalized and rotated Q | K")
    check_bf16_output(got[:, 2 * hd:], want[:, 2 * hd:], "V")
    assert torch.equal(Yq[:, 2 * hd:].view(torch.int16), Yp[:, 2 * hd:].view(torch.int16)), "V differs from svdq_gemm"


@pytest.mark.parametrize("fmt", ["mxfp4", "int4"])
def test_qkv_full_size_sampled_tokens(torch_dev, fmt):
    """FLUX QKV: M=4608, K=3072 -> N=9216 (24 heads each of Q, K, V), rank 32."""
    torch, dev = torch_dev
    spec = synth.CONFIGS["qkv"]
    L = synth.draw_layer(spec)
    E = synth.draw_qkv_extras(spec.M, seed=7)
    layer = sq.Layer(fmt, spec.K, spec.N, spec.rank)
    print(f"qkv full size {fmt}", flush=True)
    Yq, Yp = _run(torch, dev, L, E, layer, spec.M)
    rng = np.random.default_rng(99)
    rows = np.unique(np.concatenate([[0, spec.M - 1], rng.choice(spec.M, 30, replace=False)]))
    Y_o = Ly.forward_rows(L["X"], L["lam"], L["L1"], L["L2"], L["R"], L["b"], fmt, rows)
    Es = dict(E, cos=E["cos"][rows], sin=E["sin"][rows])
    want = _oracle(Y_o, Es)
    got = bf16_to_np(Yq)[rows]
    check_bf16_output(got, want, "FLUX QKV, sampled tokens")
    hd = spec.N // 3
    assert torch.equal(Yq[:, 2 * hd:].view(torch.int16), Yp[:, 2 * hd:].view(torch.int16)), "V differs from svdq_gemm"
