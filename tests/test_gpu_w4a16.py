"""W4A16 GEMM (svdq_gemm_w4a16) against the oracle (oracle/w4a16.py), element by
element, through the C ABI.

Bars, from the arithmetic: the kernel sums exact bf16 products (a code q enters
as 128 + q + 8, corrected by 136 times the group's sum of X) in fp32.  Each
term passes at most K/256 + 40 fp32 roundings (the MFMA's internal additions,
the per-group correction and scaling, the sequential sum over a wave's groups,
the three cross-wave additions and the bias), each of relative size 2^-24 of a
partial sum bounded by sum_k 144 s |x|; so |Y - Y_o| <= 2^-24 (K/256 + 40)
sum_k 144 s_g(k) |x_k| (+ |b| 2^-24).  On inputs where every product and sum is
an integer multiple of the scale below 2^24 (integer X, W a power of two times
integers with a 7 in each group) the result is exact and must equal the oracle
bit for bit.  The bf16 output is the fp32 result rounded to nearest even."""
import numpy as np
import pytest

import synth
import w4a4_quantized_linear_amd as sq
from oracle import formats as F
from oracle import quant as Q
from oracle import w4a16 as W

from _gpu_helpers import bf16_to_np, check_bf16_output, dev_tensor, scales_np

pytestmark = pytest.mark.gpu

# (M, K, N, seed): one token, the modulation batch, a ragged second 16-token
# block, an odd number of 128-K steps per wave (K = 1536: three), N not a
# multiple of 32 (16-row workgroups) or of 256, a single 16-row tile, many token
# blocks, the largest M whose X fits the kernel's LDS copy at K = 3072 (6) next
# to the smallest that does not (7), and a wide layer whose workgroups take two
# 16-row tiles (X from global memory, N / 32 >= 512)
CASES = [
    (1, 512, 16, 1),
    (2, 3072, 272, 2),
    (17, 1536, 512, 3),
    (40, 1024, 1040, 4),
    (300, 512, 256, 5),
    (6, 3072, 544, 6),
    (7, 3072, 256, 7),
    (17, 512, 16384, 8),
]


def _random_cases(n, seed):
    """Seeded random shapes: M from 1 to 64 (both the LDS and the direct path),
    K a multiple of 512 up to 4096, N a multiple of 16 up to 8192."""
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 65)), 512 * int(rng.integers(1, 9)), 16 * int(rng.integers(1, 513)), 400 + i)
            for i in range(n)]


CASES += _random_cases(4, 2029)


@pytest.fixture(scope="module")
def torch_dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sq.lib()
    assert sq.device_check(), "current device is not gfx950"
    return torch, torch.device("cuda:0")


def _pack(torch, dev, K, N, Wn, b):
    layer = sq.Layer("int4", K, N, 0)
    w = sq.pack_weight(layer, dev_tensor(Wn, torch, dev), None, None,
                       dev_tensor(np.ones(K, np.float32), torch, dev),
                       dev_tensor(b, torch, dev) if b is not None else None)
    return layer, w


def _bound(X_bits, sW, K, bias_bits):
    """2^-24 (K/256 + 40) sum_k 144 s_g(k) |x_k| + 2^-24 |b| per output."""
    ax = np.abs(F.bf16_value(X_bits).astype(np.float64))
    s = np.repeat(F.fp16_value(sW).astype(np.float64), 64, axis=1)   # N x K
    lim = 2.0 ** -24 * (K / 256 + 40) * (ax @ (144.0 * s).T)
    if bias_bits is not None:
        lim = lim + 2.0 ** -24 * np.abs(F.bf16_value(bias_bits))[None, :]
    return lim


def _run_and_check(torch, dev, X, Wn, b, what, exact=False):
    M, K = X.shape
    N = Wn.shape[0]
    print(f"w4a16 {what}: M={M} K={K} N={N}", flush=True)
    layer, w = _pack(torch, dev, K, N, Wn, b)
    o = W.forward(X, Wn, b)
    # the packed weight holds the oracle's codes and scales
    u = sq.unpack_weight(layer, w)
    assert np.array_equal(u["codes"].cpu().numpy(), Q.pack_canonical(o["cW"])), what
    assert np.array_equal(scales_np(u["scales"], "int4"), o["sW"]), what
    epi = sq.EPI_BIAS if b is not None else 0
    Xd = dev_tensor(X, torch, dev)
    y32 = sq.gemm_w4a16(layer, w, Xd, epi | sq.EPI_OUT_F32)
    y16 = sq.gemm_w4a16(layer, w, Xd, epi)
    torch.cuda.synchronize()
    y = y32.cpu().numpy().astype(np.float64)
    if exact:
        np.testing.assert_array_equal(y, o["Y"], err_msg=f"{what}: exact case")
    else:
        err = np.abs(y - o["Y"])
        lim = _bound(X, o["sW"], K, b)
        assert np.all(err <= lim), f"{what}: {int((err > lim).sum())} outputs beyond the fp32 bound"
        assert err.sum() <= 1e-4 * np.abs(o["Y"]).sum(), f"{what}: mean error {err.mean():.3e}"
    # bf16 output: the fp32 result rounded once, and within the layer tolerance
    want16 = F.bf16_bits(y32.cpu().numpy().astype(np.float64))
    got16 = y16.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got16, want16), f"{what}: bf16 output is not the rounded fp32 output"
    check_bf16_output(bf16_to_np(y16), o["Y"], what)


@pytest.mark.parametrize("case", CASES, ids=[f"M{c[0]}-K{c[1]}-N{c[2]}" for c in CASES])
def test_w4a16_matches_oracle(torch_dev, case):
    torch, dev = torch_dev
    M, K, N, seed = case
    spec = synth.layer_spec("mod_w4a16", M=M, K=K, N=N, w_outliers=max(1, K // 100))
    d = synth.draw_w4a16(spec, seed=seed)
    _run_and_check(torch, dev, d["X"], d["W"], d["b"], f"case {case}")


def test_w4a16_no_bias_and_exact_integers(torch_dev):
    """Integer X in [-3, 3] and W = 2^e (integers in [-7, 7], a +-7 in every
    64-group), so the scale is 2^e, every code is the integer and the fp32 sums
    are exact: the GPU equals the oracle exactly, without bias and with one."""
    torch, dev = torch_dev
    rng = np.random.default_rng(11)
    M, K, N = 19, 1024, 48
    q = rng.integers(-7, 8, (N, K))
    q[:, ::64] = rng.choice([-7, 7], (N, K // 64))
    e = rng.integers(-12, -4, (N, K // 64))
    Wn = (q * np.ldexp(1.0, np.repeat(e, 64, axis=1))).astype(np.float32)
    X = synth.bf16_bits_from_f32(rng.integers(-3, 4, (M, K)).astype(np.float32))
    _run_and_check(torch, dev, X, Wn, None, "exact, no bias", exact=True)
    b = synth.bf16_bits_from_f32((rng.integers(-64, 65, N) * 2.0 ** -6).astype(np.float32))
    _run_and_check(torch, dev, X, Wn, b, "exact, bias", exact=True)
    # few tokens: X read from the kernel's LDS copy
    _run_and_check(torch, dev, np.ascontiguousarray(X[:5]), Wn, b, "exact, bias, 5 tokens", exact=True)


def test_w4a16_zero_tokens(torch_dev):
    torch, dev = torch_dev
    K, N = 512, 32
    layer, w = _pack(torch, dev, K, N, np.zeros((N, K), np.float32), None)
    y = sq.gemm_w4a16(layer, w, torch.empty((0, K), dtype=torch.int16, device=dev))
    assert y.shape == (0, N)


def test_w4a16_full_size_modulation(torch_dev):
    """The FLUX modulation projection at its real size (2 tokens, 3072 -> 18432),
    every output element, in the launch configuration the benchmark times."""
    torch, dev = torch_dev
    spec = synth.CONFIGS["mod_w4a16"]
    d = synth.draw_w4a16(spec)
    _run_and_check(torch, dev, d["X"], d["W"], d["b"], "mod_w4a16 full size")
