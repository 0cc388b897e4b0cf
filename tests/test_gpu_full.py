"""Full-size parity: every workload layer at its real shape, run the way the
benchmark runs it (svdq_linear, bf16 output, the layer's epilogue), checked on
sampled rows and columns the oracle computes one by one.

Each layer runs on its calibrated operands (lambda from the data, SVD of the
smoothed weight, residual: SVDQuant notes page, section 4.2, done by the
oracle on the dense seeded draw, tests/_calib.py), and again on directly drawn
look-alike operands (synth.draw_layer) as extra cases.

The MLP pair (fc1 -> GELU -> bf16 H -> fc2) is also checked as a chain: the
GPU's own H is handed to the oracle's fc2, whose codes and scales must equal
the GPU's bit for bit and whose output must meet the full tolerance; the
chain with each side feeding its own H is an additional, looser check."""
import numpy as np
import pytest

import synth
import w4a4_quantized_linear_amd as sq
from oracle import formats as F
from oracle import layer as Ly
from oracle import quant as Q

import _calib
from _gpu_helpers import (assert_codes_equal, assert_scales_equal, bf16_to_np, check_bf16_output,
                          check_chain_output, check_fp32_output, check_next_layer_on_gpu_h, dev_tensor, pack,
                          scales_np)

pytestmark = pytest.mark.gpu

FULL = ["single", "qkv", "fc1_mxfp4", "fc2_mxfp4", "fc1_int4", "fc2_int4", "fc1_nvfp4", "fc2_nvfp4", "lowm", "lora"]


@pytest.fixture(scope="module")
def torch_dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sq.lib()
    assert sq.device_check(), "current device is not gfx950"
    return torch, torch.device("cuda:0")


def _epi(spec):
    return sq.EPI_LOWRANK | sq.EPI_BIAS | (sq.EPI_GELU if spec.gelu else 0)


CASES = [(n, "calibrated") for n in FULL] + [(n, "drawn") for n in FULL]


def operands(spec, kind):
    return _calib.calibrated_layer(spec) if kind == "calibrated" else synth.draw_layer(spec)


@pytest.mark.parametrize("name,kind", CASES, ids=[f"{n}-{k}" for n, k in CASES])
def test_full_size_sampled(torch_dev, name, kind):
    torch, dev = torch_dev
    spec = synth.CONFIGS[name]
    print(f"full-size layer {name} ({kind} operands): M={spec.M} K={spec.K} N={spec.N} "
          f"r={spec.rank + spec.lora_rank} {spec.fmt}", flush=True)
    L = operands(spec, kind)
    layer = sq.Layer(spec.fmt, spec.K, spec.N, spec.rank + spec.lora_rank)
    w = pack(layer, L, torch, dev)
    X = dev_tensor(L["X"], torch, dev)
    Yb = sq.linear(layer, w, X, _epi(spec))
    Yf = sq.linear(layer, w, X, _epi(spec) | sq.EPI_OUT_F32)
    ws = sq.quantize_act(layer, w, X)
    ua = sq.unpack_act(layer, ws, spec.M)
    uw = sq.unpack_weight(layer, w)
    same_rounding = bool(torch.equal(Yf.to(torch.bfloat16).view(torch.int16), Yb.view(torch.int16)))
    torch.cuda.synchronize()
    assert same_rounding, "bf16 output is not the nearest-even rounding of the fp32 output"

    rng = np.random.default_rng(1234)
    rows = np.unique(np.concatenate([[0, spec.M - 1], rng.choice(spec.M, 62, replace=False)]))
    cols = np.unique(np.concatenate([[0, spec.N - 1], rng.choice(spec.N, 190, replace=False)]))
    xhat = Ly.smooth(L["X"][rows], L["lam"])
    cX, sX = Q.quantize(xhat, spec.fmt)
    assert_codes_equal(ua["codes"][rows].cpu().numpy(), cX, "activation codes (sampled rows)")
    assert_scales_equal(scales_np(ua["scales"][rows], spec.fmt), sX, "activation scales (sampled rows)")
    gsR = Q.nvfp4_global_scale(L["R"]) if spec.fmt == "nvfp4" else 1.0   # of the whole residual
    cR, sR = Q.quantize(L["R"][cols], spec.fmt, gsR)
    assert_codes_equal(uw["codes"][cols].cpu().numpy(), cR, "weight codes (sampled columns)")
    assert_scales_equal(scales_np(uw["scales"][cols], spec.fmt), sR, "weight scales (sampled columns)")

    Y_o = Ly.forward_rows(L["X"], L["lam"], L["L1"], L["L2"], L["R"], L["b"], spec.fmt, rows, cols,
                          gelu_act=spec.gelu)
    sel = np.ix_(rows, cols)
    check_fp32_output(Yf.cpu().numpy()[sel], Y_o, f"{name} fp32 output")
    check_bf16_output(bf16_to_np(Yb)[sel], Y_o, f"{name} bf16 output")


@pytest.mark.parametrize("fmt", ["mxfp4", "int4", "nvfp4"])
def test_mlp_pair_chain(torch_dev, fmt):
    """fc1 (GELU fused) -> bf16 H -> fc2 at a reduced size with several tiles.
    fc1's H against the oracle's fc1; fc2 on the GPU's H against the oracle's fc2
    on that same H (codes and scales bit-exact, full output tolerance); the chain
    with each side feeding its own H within the chain bound."""
    torch, dev = torch_dev
    s1 = synth.layer_spec(f"fc1_{fmt}", M=384, K=1024, N=4096, x_outliers=10, w_outliers=10)
    s2 = synth.layer_spec(f"fc2_{fmt}", M=384, K=4096, N=1024, x_outliers=0, w_outliers=41)
    L1 = synth.draw_layer(s1)
    L2 = synth.draw_layer(s2)
    l1 = sq.Layer(fmt, 1024, 4096, 32)
    l2 = sq.Layer(fmt, 4096, 1024, 32)
    w1, w2 = pack(l1, L1, torch, dev), pack(l2, L2, torch, dev)
    H = sq.linear(l1, w1, dev_tensor(L1["X"], torch, dev), sq.EPI_LOWRANK | sq.EPI_BIAS | sq.EPI_GELU)
    a2 = sq.quantize_act(l2, w2, H.view(torch.int16))
    Y2 = sq.gemm(l2, w2, a2, 384, sq.EPI_LOWRANK | sq.EPI_BIAS | sq.EPI_OUT_F32)
    torch.cuda.synchronize()
    Y1_o = Ly.forward(L1["X"], L1["lam"], L1["L1"], L1["L2"], L1["R"], L1["b"], fmt, gelu_act=True)["Y"]
    check_bf16_output(bf16_to_np(H), Y1_o, "fc1 + GELU")
    check_next_layer_on_gpu_h(torch, sq.unpack_act(l2, a2, 384), L2, H, Y2, fmt, np.arange(384),
                              "fc2 on the GPU's H")
    Y2_o = Ly.forward(F.bf16_bits(Y1_o), L2["lam"], L2["L1"], L2["L2"], L2["R"], L2["b"], fmt)["Y"]
    check_chain_output(Y2.cpu().numpy(), Y2_o, "MLP pair output, each side on its own H", fmt)


@pytest.mark.parametrize("fmt", ["mxfp4", "int4", "nvfp4"])
def test_mlp_pair_chain_full_size(torch_dev, fmt):
    """The FLUX MLP pair at its real size on calibrated operands, as the
    benchmark runs it: fc1 with GELU writes H (bf16), fc2 quantizes H and
    completes the layer.  On sampled rows, fc2 against the oracle's fc2 on the
    GPU's H (bit-exact codes and scales, full output tolerance)."""
    torch, dev = torch_dev
    s1, s2 = synth.CONFIGS[f"fc1_{fmt}"], synth.CONFIGS[f"fc2_{fmt}"]
    print(f"full-size MLP pair {fmt}", flush=True)
    L1 = _calib.calibrated_layer(s1)
    L2 = _calib.calibrated_layer(s2)
    l1 = sq.Layer(fmt, s1.K, s1.N, s1.rank)
    l2 = sq.Layer(fmt, s2.K, s2.N, s2.rank)
    w1, w2 = pack(l1, L1, torch, dev), pack(l2, L2, torch, dev)
    H = sq.linear(l1, w1, dev_tensor(L1["X"], torch, dev), sq.EPI_LOWRANK | sq.EPI_BIAS | sq.EPI_GELU)
    a2 = sq.quantize_act(l2, w2, H.view(torch.int16))
    Y2 = sq.gemm(l2, w2, a2, s1.M, sq.EPI_LOWRANK | sq.EPI_BIAS | sq.EPI_OUT_F32)
    torch.cuda.synchronize()
    rng = np.random.default_rng(77)
    rows = np.unique(np.concatenate([[0, s1.M - 1], rng.choice(s1.M, 30, replace=False)]))
    check_next_layer_on_gpu_h(torch, sq.unpack_act(l2, a2, s1.M), L2, H, Y2, fmt, rows,
                              f"{fmt} fc2 on the GPU's H")
