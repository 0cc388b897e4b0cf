"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Element by element on seeded inputs at sizes the oracle finishes in seconds
(several tiles, ragged M and N tails, rank 0 / 48 / 256, strided X, tiny and
zero rows), and on sampled rows and columns at the full workload sizes in the
launch configuration the benchmark times.  Codes and scales must be bit-exact;
outputs within max|Y - Y_o| <= 2e-2 rms(Y_o) and mean relative error <= 5e-3
(fp32 output), bf16 output adds half a bf16 ulp per value and must equal the
round-to-nearest-even of the fp32 output.
"""
import numpy as np
import pytest

import synth
import w4a4_quantized_linear_amd as sq
from oracle import formats as F
from oracle import layer as Ly
from oracle import quant as Q

from _gpu_helpers import (assert_codes_equal, assert_scales_equal, bf16_to_np, check_bf16_output,
                          check_fp32_output, dev_tensor, pack, scales_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sq.lib()
    assert sq.device_check(), "current device is not gfx950"
    return torch, torch.device("cuda:0")


# (name, fmt, M, K, N, rank, seed): ragged M/N tails, rank 0 .. 256, one row, minimum N
MEDIUM = [
    ("qkv", "mxfp4", 300, 1024, 512, 16, 1),
    ("single", "int4", 300, 1024, 512, 16, 2),
    ("qkv", "mxfp4", 1, 512, 256, 32, 3),
    ("single", "int4", 17, 1536, 272, 0, 4),
    ("lora", "mxfp4", 513, 2048, 784, 48, 5),
    ("lowm", "mxfp4", 64, 512, 16, 256, 6),
    ("lowm", "int4", 130, 512, 48, 128, 7),
    ("qkv", "nvfp4", 300, 1024, 512, 16, 8),
    ("lowm", "nvfp4", 1, 512, 48, 0, 9),
    ("lora", "nvfp4", 513, 2048, 784, 48, 10),
]


def _random_cases(n, seed):
    """Seeded random shapes on top of the hand-picked ones: every format, M from
    1 to 900, K a multiple of 512 up to 2048, N a multiple of 16 up to 1600, ranks
    0 to 128 including ones that are not multiples of 16."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        fmt = ("mxfp4", "int4", "nvfp4")[i % 3]
        M = int(rng.integers(1, 901))
        K = 512 * int(rng.integers(1, 5))
        N = 16 * int(rng.integers(1, 101))
        rank = int(rng.choice([0, 8, 16, 24, 32, 40, 64, 100, 128]))
        out.append(("qkv", fmt, M, K, N, rank, 100 + i))
    return out


MEDIUM += _random_cases(12, 2026)


def _medium_layer(name, fmt, M, K, N, rank, seed, edge=False):
    spec = synth.layer_spec(name, M=M, K=K, N=N, rank=rank, fmt=fmt, x_outliers=max(1, K // 100),
                            w_outliers=max(1, K // 100), lora_rank=0)
    L = synth.draw_layer(spec, seed=seed)
    if edge and M >= 4:
        # edge rows: all zero, tiny (subnormal after smoothing), negative zeros, huge
        X = L["X"].copy()
        X[0] = 0
        X[1] = synth.bf16_bits_from_f32(np.full(K, 3e-38, np.float32) * np.sign(np.arange(K) % 3 - 1))
        X[2] = 0x8000
        X[3, :7] = synth.bf16_bits_from_f32(np.array([3e37, -1e30, 1.0, -2.5, 0.0, 5e-39, 7.0], np.float32))
        L["X"] = X
    if edge and N >= 32:
        R = L["R"].copy()
        R[0] = 0.0
        R[1, :5] = np.array([1e-40, -1e-41, 2e-39, 0.0, -0.0], np.float32)
        L["R"] = R
    return spec, L


@pytest.mark.parametrize("case", MEDIUM, ids=[f"{c[1]}-M{c[2]}-K{c[3]}-N{c[4]}-r{c[5]}" for c in MEDIUM])
def test_layer_elementwise(torch_dev, case):
    torch, dev = torch_dev
    name, fmt, M, K, N, rank, seed = case
    spec, L = _medium_layer(*case)
    layer = sq.Layer(fmt, K, N, rank)
    print(f"case {case}", flush=True)
    w = pack(layer, L, torch, dev)
    X = dev_tensor(L["X"], torch, dev)
    ws = sq.quantize_act(layer, w, X)
    uw = sq.unpack_weight(layer, w)
    ua = sq.unpack_act(layer, ws, M)
    Yf = sq.gemm(layer, w, ws, M, sq.EPI_LOWRANK | sq.EPI_BIAS | sq.EPI_OUT_F32)
    Yb = sq.gemm(layer, w, ws, M, sq.EPI_LOWRANK | sq.EPI_BIAS)
    Yg = sq.gemm(layer, w, ws, M, sq.EPI_LOWRANK | sq.EPI_BIAS | sq.EPI_GELU | sq.EPI_OUT_F32)
    Yl = sq.linear(layer, w, X, sq.EPI_LOWRANK | sq.EPI_BIAS)
    torch.cuda.synchronize()

    ref = Ly.forward(L["X"], L["lam"], L["L1"], L["L2"], L["R"], L["b"], fmt)
    # weights: codes and scales bit-exact, the 16-bit operands round-trip exactly
    assert_codes_equal(uw["codes"].cpu().numpy(), ref["cR"], "weight codes")
    assert_scales_equal(scales_np(uw["scales"], fmt), ref["sR"], "weight scales")
    if rank:
        assert np.array_equal(uw["L1"].cpu().numpy().view(np.uint16), L["L1"])
        assert np.array_equal(uw["L2"].cpu().numpy().view(np.uint16), L["L2"])
    assert np.array_equal(uw["lam"].cpu().numpy(), L["lam"])
    assert np.array_equal(uw["bias"].cpu().numpy().view(np.uint16), L["b"])
    # activations: codes and scales bit-exact
    assert_codes_equal(ua["codes"].cpu().numpy(), ref["cX"], "activation codes")
    assert_scales_equal(scales_np(ua["scales"], fmt), ref["sX"], "activation scales")
    # down projection: hi/lo bf16 split of X_hat, fp32 accumulation
    if rank:
        Dg = ua["D"].cpu().numpy().astype(np.float64)
        bound = np.abs(ref["xhat"].astype(np.float64)) @ np.abs(F.bf16_value(L["L1"]))
        assert np.all(np.abs(Dg - ref["D"]) <= 2.0 ** -14 * bound + 1e-30), "down projection"
    # outputs
    Y_o = ref["Y"]
    check_fp32_output(Yf.cpu().numpy(), Y_o, "fp32 output")
    check_bf16_output(bf16_to_np(Yb), Y_o, "bf16 output")
    # bf16 output is exactly the round-to-nearest-even of the fp32 output
    assert np.array_equal(Yb.cpu().view(torch.int16).numpy().view(np.uint16), F.bf16_bits(Yf.cpu().numpy()))
    # the two-launch entry point gives the same bytes
    assert torch.equal(Yl.view(torch.int16), Yb.view(torch.int16))
    check_fp32_output(Yg.cpu().numpy(), Ly.gelu(Y_o), "GELU output")


def test_tile_schedules_elementwise(torch_dev):
    """The MXFP4 GEMM picks its tiles by the size of the output: 256-wide tiles
    for 128 up to one round of 256 x 256 ones, else 128 x 128 tiles; both walk
    the output in groups of 8 tile columns.  Each schedule, element by element
    against the oracle, with a last raster group narrower than 8: 2048 x 4352
    (136 big tiles, 17 columns: 187 tiles of 256 x 192), 2048 x 8448 (264 big
    tiles: 128 x 128 tiles, 66 columns), 1024 x 512 (8 big tiles: 128 x 128
    tiles, 4 columns)."""
    torch, dev = torch_dev
    for (M, N, seed) in [(2048, 4352, 43), (2048, 8448, 41), (1024, 512, 42)]:
        K = 512
        spec, L = _medium_layer("qkv", "mxfp4", M, K, N, 16, seed)
        layer = sq.Layer("mxfp4", K, N, 16)
        print(f"tile schedule M={M} N={N}", flush=True)
        w = pack(layer, L, torch, dev)
        Y = sq.linear(layer, w, dev_tensor(L["X"], torch, dev), sq.EPI_LOWRANK | sq.EPI_BIAS | sq.EPI_OUT_F32)
        torch.cuda.synchronize()
        ref = Ly.forward(L["X"], L["lam"], L["L1"], L["L2"], L["R"], L["b"], "mxfp4")
        check_fp32_output(Y.cpu().numpy(), ref["Y"], f"M={M} N={N}")


@pytest.mark.parametrize("fmt", ["int4", "nvfp4"])
def test_int4_nvfp4_tile_sizes(torch_dev, fmt):
    """INT4 and NVFP4 layers with fewer 128 x 128 output tiles than CUs take
    64 x 64 tiles.  2048 x 1024 -> 4352 (544 tiles of 128 x 128) against the
    oracle element by element, with and without the low-rank branch; at rank 0
    the rows are independent, so its first 200 rows computed as a 200-row layer
    (68 tiles of 128 x 128: the 64 x 64 schedule) must give the same bits, in
    fp32 and in bf16 with GELU."""
    torch, dev = torch_dev
    M, K, N = 2048, 1024, 4352
    for rank in (0, 32):
        spec, L = _medium_layer("qkv", fmt, M, K, N, rank, 60 + rank)
        layer = sq.Layer(fmt, K, N, rank)
        print(f"{fmt} tile sizes rank {rank}", flush=True)
        w = pack(layer, L, torch, dev)
        X = dev_tensor(L["X"], torch, dev)
        epi = sq.EPI_LOWRANK | sq.EPI_BIAS | sq.EPI_OUT_F32
        Yf = sq.linear(layer, w, X, epi)
        Yg = sq.linear(layer, w, X, sq.EPI_LOWRANK | sq.EPI_BIAS | sq.EPI_GELU)
        torch.cuda.synchronize()
        ref = Ly.forward(L["X"], L["lam"], L["L1"], L["L2"], L["R"], L["b"], fmt)
        check_fp32_output(Yf.cpu().numpy(), ref["Y"], f"{fmt} M={M} rank {rank}")
        if rank == 0:
            Xs = dev_tensor(L["X"][:200], torch, dev)
            Ysf = sq.linear(layer, w, Xs, epi)
            Ysg = sq.linear(layer, w, Xs, sq.EPI_LOWRANK | sq.EPI_BIAS | sq.EPI_GELU)
            torch.cuda.synchronize()
            assert torch.equal(Ysf.view(torch.int32), Yf[:200].view(torch.int32)), "fp32 rows differ by tile size"
            assert torch.equal(Ysg.view(torch.int16), Yg[:200].view(torch.int16)), "bf16 GELU rows differ by tile size"


def test_short_tiles_elementwise(torch_dev):
    """256-wide tiles shorter than 256 rows, chosen when they fill more CUs in
    one round: 4600 x 3072 (12 tile columns: 252 tiles of 224 rows, the last
    one past the padded rows) and 2048 x 4352 (17 columns: 187 tiles of 192
    rows).  fp32, bf16 and GELU outputs element by element against the oracle;
    bf16 must be the round-to-nearest-even of fp32 (the odd last block of a
    224-row tile goes through the store staging alone)."""
    torch, dev = torch_dev
    for (M, N, seed) in [(4600, 3072, 44), (2048, 4352, 45)]:
        K = 512
        spec, L = _medium_layer("qkv", "mxfp4", M, K, N, 32, seed)
        layer = sq.Layer("mxfp4", K, N, 32)
        print(f"short tiles M={M} N={N}", flush=True)
        w = pack(layer, L, torch, dev)
        ws = sq.quantize_act(layer, w, dev_tensor(L["X"], torch, dev))
        Yf = sq.gemm(layer, w, ws, M, sq.EPI_LOWRANK | sq.EPI_BIAS | sq.EPI_OUT_F32)
        Yb = sq.gemm(layer, w, ws, M, sq.EPI_LOWRANK | sq.EPI_BIAS)
        Yg = sq.gemm(layer, w, ws, M, sq.EPI_LOWRANK | sq.EPI_BIAS | sq.EPI_GELU)
        torch.cuda.synchronize()
        ref = Ly.forward(L["X"], L["lam"], L["L1"], L["L2"], L["R"], L["b"], "mxfp4")
        check_fp32_output(Yf.cpu().numpy(), ref["Y"], f"M={M} N={N} fp32")
        check_bf16_output(bf16_to_np(Yb), ref["Y"], f"M={M} N={N} bf16")
        assert np.array_equal(Yb.cpu().view(torch.int16).numpy().view(np.uint16), F.bf16_bits(Yf.cpu().numpy()))
        check_bf16_output(bf16_to_np(Yg), Ly.gelu(ref["Y"]), f"M={M} N={N} GELU bf16")


@pytest.mark.parametrize("M,K,N,rank,seed", [(1000, 3072, 1008, 128, 46), (257, 4096, 400, 32, 47),
                                              (2048, 1024, 2048, 16, 48), (33, 2048, 3072, 100, 49)],
                         ids=["64-tiles-K3072-r128", "12-tiles-K4096", "256-tiles-K1024", "24-tiles-K2048-r100"])
def test_one_tile_per_cu_elementwise(torch_dev, M, K, N, rank, seed):
    """MXFP4 grids of at most one 128 x 128 tile per CU (the low-M shape's
    schedule) with long K: 24 to 32 K steps, ragged M and N, ranks up to 128,
    exactly 256 tiles.  fp32, bf16 and GELU outputs element by element against
    the oracle; bf16 must be the round-to-nearest-even of fp32."""
    torch, dev = torch_dev
    spec, L = _medium_layer("lowm", "mxfp4", M, K, N, rank, seed)
    layer = sq.Layer("mxfp4", K, N, rank)
    print(f"one tile per CU M={M} K={K} N={N} rank={rank}", flush=True)
    w = pack(layer, L, torch, dev)
    ws = sq.quantize_act(layer, w, dev_tensor(L["X"], torch, dev))
    Yf = sq.gemm(layer, w, ws, M, sq.EPI_LOWRANK | sq.EPI_BIAS | sq.EPI_OUT_F32)
    Yb = sq.gemm(layer, w, ws, M, sq.EPI_LOWRANK | sq.EPI_BIAS)
    Yg = sq.gemm(layer, w, ws, M, sq.EPI_LOWRANK | sq.EPI_BIAS | sq.EPI_GELU | sq.EPI_OUT_F32)
    torch.cuda.synchronize()
    ref = Ly.forward(L["X"], L["lam"], L["L1"], L["L2"], L["R"], L["b"], "mxfp4")
    check_fp32_output(Yf.cpu().numpy(), ref["Y"], f"M={M} K={K} N={N} fp32")
    check_bf16_output(bf16_to_np(Yb), ref["Y"], f"M={M} K={K} N={N} bf16")
    assert np.array_equal(Yb.cpu().view(torch.int16).numpy().view(np.uint16), F.bf16_bits(Yf.cpu().numpy()))
    check_fp32_output(Yg.cpu().numpy(), Ly.gelu(ref["Y"]), f"M={M} K={K} N={N} GELU")


@pytest.mark.parametrize("M,K,N,rank,seed", [(2100, 1536, 4000, 48, 50), (1100, 3072, 8208, 32, 51)],
                         ids=["544-tiles-K1536-r48", "585-tiles-K3072"])
def test_three_per_cu_elementwise(torch_dev, M, K, N, rank, seed):
    """MXFP4 grids of more than two 128 x 128 tiles per CU with K a multiple of
    1536 take a three-slot ring (blocks of twelve 128-K steps whose last two
    loads read nothing): 256 x 128 tiles at two workgroups per CU without GELU
    (the fp32, bf16 and bias-free outputs), 128 x 128 tiles at three per CU with
    it (the GELU output); one and two blocks, ragged M and N.  Every output
    element by element against the oracle; bf16 must be the round-to-nearest-even
    of fp32 (the bf16 stores are staged through the ring after the loop)."""
    torch, dev = torch_dev
    spec, L = _medium_layer("qkv", "mxfp4", M, K, N, rank, seed)
    layer = sq.Layer("mxfp4", K, N, rank)
    print(f"three per CU M={M} K={K} N={N} rank={rank}", flush=True)
    w = pack(layer, L, torch, dev)
    ws = sq.quantize_act(layer, w, dev_tensor(L["X"], torch, dev))
    Yf = sq.gemm(layer, w, ws, M, sq.EPI_LOWRANK | sq.EPI_BIAS | sq.EPI_OUT_F32)
    Yb = sq.gemm(layer, w, ws, M, sq.EPI_LOWRANK | sq.EPI_BIAS)
    Yn = sq.gemm(layer, w, ws, M, sq.EPI_LOWRANK)
    Yg = sq.gemm(layer, w, ws, M, sq.EPI_LOWRANK | sq.EPI_BIAS | sq.EPI_GELU)
    torch.cuda.synchronize()
    ref = Ly.forward(L["X"], L["lam"], L["L1"], L["L2"], L["R"], L["b"], "mxfp4")
    check_fp32_output(Yf.cpu().numpy(), ref["Y"], f"M={M} K={K} N={N} fp32")
    check_bf16_output(bf16_to_np(Yb), ref["Y"], f"M={M} K={K} N={N} bf16")
    assert np.array_equal(Yb.cpu().view(torch.int16).numpy().view(np.uint16), F.bf16_bits(Yf.cpu().numpy()))
    ref_nb = Ly.forward(L["X"], L["lam"], L["L1"], L["L2"], L["R"], L["b"], "mxfp4", with_bias=False)
    check_bf16_output(bf16_to_np(Yn), ref_nb["Y"], f"M={M} K={K} N={N} bf16 without bias")
    check_bf16_output(bf16_to_np(Yg), Ly.gelu(ref["Y"]), f"M={M} K={K} N={N} GELU bf16")


def test_gelu_epilogue_pointwise(torch_dev):
    """The GEMM's GELU against the exact erf form, value by value: with R = 0,
    rank 0 and lambda = 1 the output is GELU(b), so the bias carries the test
    values (2032 points spread over [-12, 12], rounded to bf16, and special values)."""
    torch, dev = torch_dev
    K, N, M = 512, 2048, 8
    spec, L = _medium_layer("qkv", "mxfp4", M, K, N, 0, 31)
    vals = np.concatenate([np.linspace(-12.0, 12.0, N - 16),
                           [0.0, -0.0, 1e-30, -1e-30, 5e-39, 3e38, -3e38, 40.0, -40.0, 0.5, -0.5,
                            1.0, -1.0, 6.0, -6.0, 9.0]]).astype(np.float32)
    assert vals.size == N
    L["b"] = synth.bf16_bits_from_f32(vals)
    L["R"] = np.zeros_like(L["R"])
    L["lam"] = np.ones_like(L["lam"])
    layer = sq.Layer("mxfp4", K, N, 0)
    w = pack(layer, L, torch, dev)
    ws = sq.quantize_act(layer, w, dev_tensor(L["X"], torch, dev))
    Y = sq.gemm(layer, w, ws, M, sq.EPI_BIAS | sq.EPI_GELU | sq.EPI_OUT_F32)
    torch.cuda.synchronize()
    b = F.bf16_value(L["b"]).astype(np.float64)
    want = Ly.gelu(b)
    got = Y.cpu().numpy().astype(np.float64)
    assert np.all(got == got[0]), "every row sees the same bias"
    err = np.abs(got[0] - want)
    assert np.all(err <= 1e-6 * np.maximum(1.0, np.abs(b))), f"max GELU error {err.max():.3e}"


@pytest.mark.parametrize("fmt", ["mxfp4", "int4", "nvfp4"])
def test_edge_values_bit_exact(torch_dev, fmt):
    """Zero rows, signed zeros, subnormal inputs after smoothing, huge values:
    codes and scales still match the oracle bit for bit."""
    torch, dev = torch_dev
    spec, L = _medium_layer("qkv", fmt, 40, 1024, 64, 16, 21, edge=True)
    layer = sq.Layer(fmt, 1024, 64, 16)
    w = pack(layer, L, torch, dev)
    ws = sq.quantize_act(layer, w, dev_tensor(L["X"], torch, dev))
    uw, ua = sq.unpack_weight(layer, w), sq.unpack_act(layer, ws, 40)
    Y = sq.gemm(layer, w, ws, 40, sq.EPI_LOWRANK | sq.EPI_BIAS | sq.EPI_OUT_F32)
    torch.cuda.synchronize()
    ref = Ly.forward(L["X"], L["lam"], L["L1"], L["L2"], L["R"], L["b"], fmt)
    assert_codes_equal(uw["codes"].cpu().numpy(), ref["cR"], "weight codes")
    assert_scales_equal(scales_np(uw["scales"], fmt), ref["sR"], "weight scales")
    assert_codes_equal(ua["codes"].cpu().numpy(), ref["cX"], "activation codes")
    assert_scales_equal(scales_np(ua["scales"], fmt), ref["sX"], "activation scales")
    rows = np.arange(4, 40)                      # ordinary rows keep the stated tolerance
    check_fp32_output(Y.cpu().numpy()[rows], ref["Y"][rows], "ordinary rows")
    assert np.all(np.isfinite(Y.cpu().numpy()))


def test_int4_largest_group_sums(torch_dev):
    """INT4 operands whose every row is one value up to sign (codes all 7 in
    magnitude): each 64-group's integer sum reaches the largest magnitude the
    quantizer can give, 64 * 49, or cancels to 0.  The GEMM's int8 operands hold
    16 times the codes, so its int32 sums are 256 times these; the codes and the
    output still match the oracle."""
    torch, dev = torch_dev
    M, K, N = 64, 1024, 64
    spec = synth.layer_spec("single", M=M, K=K, N=N, rank=0, fmt="int4", x_outliers=1, w_outliers=1, lora_rank=0)
    L = synth.draw_layer(spec, seed=31)
    k = np.arange(K)
    alt = np.where(k % 2 == 0, 1.0, -1.0)
    # X rows: +c, -c, or c alternating in sign along K; R rows likewise
    X = np.empty((M, K), np.float32)
    for m in range(M):
        pat = (np.ones(K), -np.ones(K), alt)[m % 3]
        X[m] = pat * (0.5 + 0.25 * m)
    R = np.empty((N, K), np.float32)
    for n in range(N):
        pat = (np.ones(K), alt, -alt)[n % 3]
        R[n] = pat * (1.0 + 0.125 * n)
    L["X"] = synth.bf16_bits_from_f32(X)
    L["R"] = R
    L["lam"] = np.ones(K, np.float32)
    layer = sq.Layer("int4", K, N, 0)
    w = pack(layer, L, torch, dev)
    ws = sq.quantize_act(layer, w, dev_tensor(L["X"], torch, dev))
    ua = sq.unpack_act(layer, ws, M)
    Y = sq.gemm(layer, w, ws, M, sq.EPI_BIAS | sq.EPI_OUT_F32)
    torch.cuda.synchronize()
    ref = Ly.forward(L["X"], L["lam"], L["L1"], L["L2"], L["R"], L["b"], "int4")
    assert np.abs(ref["cX"].astype(np.int64)).max() == 7, "codes of the largest magnitude"
    assert_codes_equal(ua["codes"].cpu().numpy(), ref["cX"], "activation codes")
    check_fp32_output(Y.cpu().numpy(), ref["Y"], "largest INT4 group sums")


@pytest.mark.parametrize("fmt", ["mxfp4", "int4", "nvfp4"])
@pytest.mark.parametrize("lam_edge", ["inside", "outside"])
def test_division_range_edges_bit_exact(torch_dev, fmt, lam_edge):
    """Smoothing quotients at the edges of the range the activation kernel's
    fast division accepts: |x| near 2^-40 and 2^60 with lambda at 2^-32 and
    2^32 ("inside"), and a layer with some lambda outside [2^-32, 2^32], which
    takes IEEE division everywhere ("outside").  Codes and scales must match the
    oracle's IEEE fp32 quotients bit for bit."""
    torch, dev = torch_dev
    M, K, N, r = 48, 1024, 64, 16
    spec, L = _medium_layer("qkv", fmt, M, K, N, r, 31)
    rng = np.random.default_rng(77)
    lam = L["lam"].copy()
    if lam_edge == "inside":
        lam[0], lam[1], lam[2], lam[3] = 2.0 ** -32, 2.0 ** 32, np.float32(2.0 ** -32 * 1.75), np.float32(2.0 ** 31 * 1.5)
        lam[4:64] = np.exp2(rng.uniform(-32, 32, 60)).astype(np.float32)
    else:
        lam[5], lam[9] = 2.0 ** 40, 2.0 ** -40
    L["lam"] = lam
    X = L["X"].copy()
    vals = np.array([2.0 ** -40, -(2.0 ** -40) * 1.5, 2.0 ** 60 * 0.99, -(2.0 ** 59) * 1.875, 2.0 ** -39,
                     1.0, -3.0, 2.0 ** 59], np.float32)
    X[0:8, 0:64] = synth.bf16_bits_from_f32(np.resize(vals, (8, 64)))
    X[8:16] = synth.bf16_bits_from_f32(rng.standard_normal((8, K)).astype(np.float32)
                                       * np.exp2(rng.integers(-38, 58, (8, K))).astype(np.float32))
    L["X"] = X
    layer = sq.Layer(fmt, K, N, r)
    w = pack(layer, L, torch, dev)
    ws = sq.quantize_act(layer, w, dev_tensor(L["X"], torch, dev))
    ua = sq.unpack_act(layer, ws, M)
    torch.cuda.synchronize()
    cX, sX = Q.quantize(Ly.smooth(L["X"], L["lam"]), fmt)
    assert_codes_equal(ua["codes"].cpu().numpy(), cX, f"activation codes ({lam_edge})")
    assert_scales_equal(scales_np(ua["scales"], fmt), sX, f"activation scales ({lam_edge})")


def test_epilogue_flags_separately(torch_dev):
    torch, dev = torch_dev
    spec, L = _medium_layer("qkv", "mxfp4", 96, 1024, 256, 32, 11)
    layer = sq.Layer("mxfp4", 1024, 256, 32)
    w = pack(layer, L, torch, dev)
    ws = sq.quantize_act(layer, w, dev_tensor(L["X"], torch, dev))
    out = {e: sq.gemm(layer, w, ws, 96, e | sq.EPI_OUT_F32).cpu().numpy()
           for e in (0, sq.EPI_LOWRANK, sq.EPI_BIAS, sq.EPI_LOWRANK | sq.EPI_BIAS)}
    base = Ly.forward(L["X"], L["lam"], L["L1"], L["L2"], L["R"], L["b"], "mxfp4", with_lowrank=False,
                      with_bias=False)["Y"]
    lr = Ly.forward(L["X"], L["lam"], L["L1"], L["L2"], L["R"], L["b"], "mxfp4", with_bias=False)["Y"]
    check_fp32_output(out[0], base, "4-bit branch only")
    check_fp32_output(out[sq.EPI_LOWRANK], lr, "with low-rank")
    diff = out[sq.EPI_BIAS].astype(np.float64) - out[0]
    np.testing.assert_allclose(diff, np.broadcast_to(F.bf16_value(L["b"]), diff.shape), rtol=0,
                               atol=2.0 ** -23 * np.abs(out[0]).max())


def test_pack_without_bias_and_strided_x(torch_dev):
    torch, dev = torch_dev
    spec, L = _medium_layer("single", "int4", 50, 1024, 128, 16, 12)
    layer = sq.Layer("int4", 1024, 128, 16)
    w = pack(layer, L, torch, dev, bias=False)
    wide = torch.zeros((50, 1024 + 64), dtype=torch.int16, device=dev)
    wide[:, 32:32 + 1024] = dev_tensor(L["X"], torch, dev)
    Xs = wide[:, 32:32 + 1024]                      # row stride 1088, 64-byte offset
    Y = sq.linear(layer, w, Xs, sq.EPI_LOWRANK | sq.EPI_BIAS | sq.EPI_OUT_F32)
    torch.cuda.synchronize()
    ref = Ly.forward(L["X"], L["lam"], L["L1"], L["L2"], L["R"], None, "int4")["Y"]
    check_fp32_output(Y.cpu().numpy(), ref, "no bias, strided X")


def test_empty_batch_is_a_noop(torch_dev):
    torch, dev = torch_dev
    spec, L = _medium_layer("qkv", "mxfp4", 8, 512, 64, 16, 13)
    layer = sq.Layer("mxfp4", 512, 64, 16)
    w = pack(layer, L, torch, dev)
    X = torch.empty((0, 512), dtype=torch.int16, device=dev)
    Y = sq.linear(layer, w, X, sq.EPI_LOWRANK | sq.EPI_BIAS)
    torch.cuda.synchronize()
    assert Y.shape == (0, 64)


def test_deterministic(torch_dev):
    torch, dev = torch_dev
    spec, L = _medium_layer("lora", "mxfp4", 700, 2048, 512, 48, 14)
    layer = sq.Layer("mxfp4", 2048, 512, 48)
    w = pack(layer, L, torch, dev)
    X = dev_tensor(L["X"], torch, dev)
    a = sq.linear(layer, w, X, sq.EPI_LOWRANK | sq.EPI_BIAS | sq.EPI_OUT_F32)
    b = sq.linear(layer, w, X, sq.EPI_LOWRANK | sq.EPI_BIAS | sq.EPI_OUT_F32)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_adapter_needs_no_requantization(torch_dev):
    torch, dev = torch_dev
    spec = synth.layer_spec("lora", M=256, K=1024, N=512)
    L = synth.draw_layer(spec)
    L0 = dict(L, L1=L["L1_svd"], L2=L["L2_svd"])
    l48 = sq.Layer("mxfp4", 1024, 512, 48)
    l32 = sq.Layer("mxfp4", 1024, 512, 32)
    w48 = pack(l48, L, torch, dev)
    w32 = pack(l32, L0, torch, dev)
    u48, u32 = sq.unpack_weight(l48, w48), sq.unpack_weight(l32, w32)
    assert torch.equal(u48["codes"], u32["codes"]) and torch.equal(u48["scales"], u32["scales"])
    nbytes = 512 * 1024 // 2 + 512 * 1024 // 32       # code and scale sections lead the blob
    assert torch.equal(w48[:nbytes], w32[:nbytes])
    Y = sq.linear(l48, w48, dev_tensor(L["X"], torch, dev), sq.EPI_LOWRANK | sq.EPI_BIAS | sq.EPI_OUT_F32)
    torch.cuda.synchronize()
    ref = Ly.forward(L["X"], L["lam"], L["L1"], L["L2"], L["R"], L["b"], "mxfp4")["Y"]
    check_fp32_output(Y.cpu().numpy(), ref, "adapter-stacked layer")


def test_device_error_path_on_gpu(torch_dev):
    torch, dev = torch_dev
    layer = sq.Layer("mxfp4", 512, 64, 16)
    w = torch.zeros(sq.weight_bytes(layer), dtype=torch.uint8, device=dev)
    ws = torch.zeros(sq.act_bytes(layer, 4), dtype=torch.uint8, device=dev)
    Y = torch.full((4, 64), 7, dtype=torch.int16, device=dev)
    sq.lib().svdq_test_force_device_error(1)
    try:
        with pytest.raises(sq.SvdqError) as e:
            sq.gemm(layer, w, ws, 4, 0, out=Y)
        assert e.value.status == 6
    finally:
        sq.lib().svdq_test_force_device_error(0)
    torch.cuda.synchronize()
    assert bool((Y == 7).all())                      # outputs untouched on error
    with pytest.raises(sq.SvdqError) as e:
        sq.linear(layer, w, torch.zeros((4, 512), dtype=torch.int16, device=dev), 0,
                  workspace=ws[:ws.numel() - 256])
    assert e.value.status == 5
