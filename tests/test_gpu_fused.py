"""Fused MLP step (svdq_gemm_quant): the first layer's GEMM quantizes its bf16
output H for the next layer instead of storing it.

The unfused path on the same GPU inputs writes H (svdq_gemm).  That H is
checked against the oracle's first layer, then handed to the oracle's next
layer: the fused workspace (and the unfused svdq_quantize_act of H) must hold
the oracle's codes and scales of H_hat bit for bit and a down projection within
the hi + lo rounding bound, and the next layer's output from either workspace
must meet the full tolerance against the oracle's on that H.  The fused and
unfused workspaces are also compared with each other (same codes and scales,
D within the bound of two fp32 sums of the same products), and the chain with
each side feeding its own H is checked under the looser chain bound."""
import numpy as np
import pytest

import _calib
import synth
import w4a4_quantized_linear_amd as sq
from oracle import formats as F
from oracle import layer as Ly

from _gpu_helpers import (bf16_to_np, check_bf16_output, check_chain_output, check_next_layer_on_gpu_h,
                          dev_tensor, pack)

pytestmark = pytest.mark.gpu

EPI1 = sq.EPI_LOWRANK | sq.EPI_BIAS | sq.EPI_GELU
EPI2 = sq.EPI_LOWRANK | sq.EPI_BIAS | sq.EPI_OUT_F32

# (M, K1, N1 = K2, rank1, N2, rank2, seed): ragged M, several tile columns of H,
# next-layer ranks 0 / 16 / 32 / 48, one row.  The fused GEMM takes the plain
# GEMM's tiles: 128 x 128 for these (fewer than 128 tiles of 256 x 256), except
# the 2048-row case (144 tiles of 256 x 256).
CASES = [
    (300, 1024, 1024, 16, 512, 32, 1),
    (513, 512, 2048, 32, 256, 48, 2),
    (64, 1024, 512, 0, 1024, 0, 3),
    (1, 512, 512, 32, 512, 16, 4),
    (2048, 512, 4608, 32, 256, 16, 6),
]


def _random_cases(n, seed):
    """Seeded random pairs: M from 1 to 900, K1 a multiple of 512 up to 2048, N1
    (the next layer's K) a multiple of 512 up to 2048, N2 a multiple of 16 up to
    1200, ranks 0 to 64 (the next layer's at most 64) not all aligned to 16."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        out.append((int(rng.integers(1, 901)), 512 * int(rng.integers(1, 5)), 512 * int(rng.integers(1, 5)),
                    int(rng.choice([0, 8, 32, 40, 64])), 16 * int(rng.integers(1, 76)),
                    int(rng.choice([0, 16, 24, 48, 64])), 200 + i))
    return out


CASES += _random_cases(4, 2027)
# more than two 128 x 128 tiles per CU with K a multiple of 1536: the three-slot
# ring (next-layer ranks 32 and 0), and the four-slot ring for a next-layer rank of 64
CASES += [(1100, 1536, 8192, 16, 512, 32, 7), (2100, 3072, 4096, 32, 256, 0, 8), (1100, 1536, 8192, 16, 512, 64, 9)]


@pytest.fixture(scope="module")
def torch_dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sq.lib()
    assert sq.device_check(), "current device is not gfx950"
    return torch, torch.device("cuda:0")


def _pair(M, K1, N1, r1, N2, r2, seed):
    s1 = synth.layer_spec("fc1_mxfp4", M=M, K=K1, N=N1, rank=r1, x_outliers=max(1, K1 // 100),
                          w_outliers=max(1, K1 // 100), lora_rank=0)
    s2 = synth.layer_spec("fc2_mxfp4", M=M, K=N1, N=N2, rank=r2, x_outliers=0, w_outliers=max(1, N1 // 100),
                          lora_rank=0)
    return synth.draw_layer(s1, seed=seed), synth.draw_layer(s2, seed=seed + 100)


def _run(torch, dev, L1, L2, M, K1, N1, r1, N2, r2, epi1=EPI1, fmt="mxfp4"):
    l1, l2 = sq.Layer(fmt, K1, N1, r1), sq.Layer(fmt, N1, N2, r2)
    w1, w2 = pack(l1, L1, torch, dev), pack(l2, L2, torch, dev)
    a1 = sq.quantize_act(l1, w1, dev_tensor(L1["X"], torch, dev))
    print(f"fused pair {fmt} M={M} {K1}->{N1}->{N2} ranks {r1}/{r2} epi {epi1}", flush=True)
    H = sq.gemm(l1, w1, a1, M, epi1)
    a2u = sq.quantize_act(l2, w2, H.view(torch.int16))
    a2f = sq.gemm_quant(l1, w1, a1, M, epi1, l2, w2)
    uu, uf = sq.unpack_act(l2, a2u, M), sq.unpack_act(l2, a2f, M)
    Y2u = sq.gemm(l2, w2, a2u, M, EPI2)
    Y2f = sq.gemm(l2, w2, a2f, M, EPI2)
    torch.cuda.synchronize()
    return dict(H=H, uu=uu, uf=uf, Y2u=Y2u, Y2f=Y2f, fmt=fmt)


def _check_against_oracle(torch, r, L1, L2, M, what, rows=None, epi1=EPI1):
    """The GPU's H against the oracle's first layer, then the oracle's next layer
    on that H against both workspaces and both outputs: the second layer is
    judged on the input it actually received."""
    rows = np.arange(M) if rows is None else rows
    gelu = (epi1 & sq.EPI_GELU) != 0
    fmt = r["fmt"]
    Y1_o = Ly.forward_rows(L1["X"], L1["lam"], L1["L1"], L1["L2"], L1["R"], L1["b"] if epi1 & sq.EPI_BIAS else None,
                           fmt, rows, gelu_act=gelu)
    check_bf16_output(bf16_to_np(r["H"])[rows], Y1_o, f"{what}: first layer's H")
    ref = check_next_layer_on_gpu_h(torch, r["uf"], L2, r["H"], r["Y2f"], fmt, rows, f"{what}: fused")
    check_next_layer_on_gpu_h(torch, r["uu"], L2, r["H"], r["Y2u"], fmt, rows, f"{what}: unfused")
    return ref


def _check_against_unfused(torch, r, L2, r2, what):
    uu, uf = r["uu"], r["uf"]
    assert torch.equal(uu["codes"], uf["codes"]), f"{what}: codes differ from quantize_act(H)"
    assert torch.equal(uu["scales"], uf["scales"]), f"{what}: scales differ from quantize_act(H)"
    if r2:
        # both are fp32 sums of the bf16 hi + lo products of x_hat with L1', each within
        # 2^-14 of the exact sum relative to sum |x_hat| |L1'|
        h = bf16_to_np(r["H"]).astype(np.float32)
        xhat = (h / L2["lam"].astype(np.float32)).astype(np.float64)
        bound = np.abs(xhat) @ np.abs(F.bf16_value(L2["L1"]))
        diff = np.abs(uf["D"].cpu().numpy().astype(np.float64) - uu["D"].cpu().numpy().astype(np.float64))
        assert np.all(diff <= 2.0 ** -13 * bound + 1e-30), f"{what}: down projection"
    yu = r["Y2u"].cpu().numpy().astype(np.float64)
    yf = r["Y2f"].cpu().numpy().astype(np.float64)
    rms = float(np.sqrt(np.mean(yu ** 2)))
    assert np.abs(yf - yu).max() <= 1e-4 * rms, f"{what}: next layer's output moved by {np.abs(yf - yu).max():.3e}"


# MXFP4 on every case; INT4 (128 x 128 tiles at every size) on the fixed cases
# and two of the random ones
FMT_CASES = [("mxfp4", c) for c in CASES] + [("int4", c) for c in CASES[:5] + CASES[5:7]]


@pytest.mark.parametrize("fmt,case", FMT_CASES,
                         ids=[f"{f}-M{c[0]}-{c[1]}-{c[2]}-{c[4]}-r{c[3]}-{c[5]}" for f, c in FMT_CASES])
def test_fused_equals_unfused_and_oracle_chain(torch_dev, fmt, case):
    torch, dev = torch_dev
    M, K1, N1, r1, N2, r2, seed = case
    L1, L2 = _pair(*case)
    r = _run(torch, dev, L1, L2, M, K1, N1, r1, N2, r2, fmt=fmt)
    _check_against_oracle(torch, r, L1, L2, M, f"case {case}")
    _check_against_unfused(torch, r, L2, r2, f"case {case}")
    # the chain through the oracle, which forms and quantizes its own H
    Y1_o = Ly.forward(L1["X"], L1["lam"], L1["L1"], L1["L2"], L1["R"], L1["b"], fmt, gelu_act=True)["Y"]
    Y2_o = Ly.forward(F.bf16_bits(Y1_o), L2["lam"], L2["L1"], L2["L2"], L2["R"], L2["b"], fmt)["Y"]
    check_chain_output(r["Y2f"].cpu().numpy(), Y2_o, "fused MLP output", fmt)


@pytest.mark.parametrize("case", [(300, 1024, 1024, 16, 512, 32, 11), (2048, 512, 4608, 32, 256, 16, 12)],
                         ids=["128x128-tiles", "256x256-tiles"])
def test_fused_without_gelu(torch_dev, case):
    """The fused step with the bias and low-rank term but no activation: the
    codes and scales still equal quantize_act's of the stored output."""
    torch, dev = torch_dev
    L1, L2 = _pair(*case)
    epi1 = sq.EPI_LOWRANK | sq.EPI_BIAS
    r = _run(torch, dev, L1, L2, *case[:6], epi1=epi1)
    _check_against_oracle(torch, r, L1, L2, case[0], f"no GELU, case {case}", epi1=epi1)
    _check_against_unfused(torch, r, L2, case[5], f"no GELU, case {case}")


@pytest.mark.parametrize("fmt", ["mxfp4", "int4"])
def test_fused_ieee_division_path(torch_dev, fmt):
    """A next-layer lambda outside [2^-32, 2^32] sends the whole layer to IEEE
    division; the fused codes still equal quantize_act's."""
    torch, dev = torch_dev
    case = (200, 512, 1024, 16, 256, 32, 5)
    L1, L2 = _pair(*case)
    lam = L2["lam"].copy()
    lam[3] = np.float32(2.0 ** 40)
    lam[700] = np.float32(2.0 ** -35)
    L2["lam"] = lam
    r = _run(torch, dev, L1, L2, *case[:6], fmt=fmt)
    _check_against_oracle(torch, r, L1, L2, case[0], "lambda outside the fast range")
    _check_against_unfused(torch, r, L2, case[5], "lambda outside the fast range")


@pytest.mark.parametrize("fmt,kind", [("mxfp4", "calibrated"), ("mxfp4", "drawn"), ("int4", "calibrated")])
def test_fused_full_size_flux_mlp(torch_dev, fmt, kind):
    """The FLUX MLP pair at its real size (fc1 4608 x 3072 -> 12288, GELU; fc2
    12288 -> 3072; rank 32), as the benchmark's fused step runs it, on the
    calibrated operands and on drawn ones: on sampled rows, H against the
    oracle's fc1 and the fused workspace and fc2's output against the oracle's
    fc2 on the GPU's H; on every row, codes and scales equal quantize_act's and
    D and fc2's output lie within bounds of the unfused path."""
    torch, dev = torch_dev
    s1, s2 = synth.CONFIGS[f"fc1_{fmt}"], synth.CONFIGS[f"fc2_{fmt}"]
    print(f"fused FLUX MLP pair, {fmt}, {kind} operands", flush=True)
    if kind == "calibrated":
        L1, L2 = _calib.calibrated_layer(s1), _calib.calibrated_layer(s2)
    else:
        L1, L2 = synth.draw_layer(s1), synth.draw_layer(s2)
    r = _run(torch, dev, L1, L2, s1.M, s1.K, s1.N, s1.rank, s2.N, s2.rank, fmt=fmt)
    rng = np.random.default_rng(78)
    rows = np.unique(np.concatenate([[0, s1.M - 1], rng.choice(s1.M, 30, replace=False)]))
    _check_against_oracle(torch, r, L1, L2, s1.M, f"FLUX MLP pair ({kind})", rows=rows)
    _check_against_unfused(torch, r, L2, s2.rank, f"FLUX MLP pair ({kind})")
