"""svdq_linear_noalloc (the workspace in the library's static scratch) against
svdq_linear on the same inputs: the same kernels, so the same output bits.  Two
calls in a row, the second with fewer rows and a smaller layer, so the scratch
still holds the first call's larger contents; plus a FLUX-sized layer."""
import numpy as np
import pytest

import synth
import w4a4_quantized_linear_amd as sq

from _gpu_helpers import dev_tensor, pack

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sq.lib()
    assert sq.device_check(), "current device is not gfx950"
    return torch, torch.device("cuda:0")


def _layer(name, fmt, M, K, N, rank, seed):
    spec = synth.layer_spec(name, M=M, K=K, N=N, rank=rank, fmt=fmt, x_outliers=max(1, K // 100),
                            w_outliers=max(1, K // 100), lora_rank=0)
    return synth.draw_layer(spec, seed=seed)


@pytest.mark.parametrize("fmt", ["mxfp4", "int4", "nvfp4"])
def test_noalloc_equals_linear(torch_dev, fmt):
    torch, dev = torch_dev
    epi = sq.EPI_LOWRANK | sq.EPI_BIAS | sq.EPI_GELU
    for (M, K, N, rank, seed) in [(700, 2048, 1040, 48, 11), (130, 1024, 512, 16, 12)]:
        print(f"noalloc {fmt} M={M} K={K} N={N} r={rank}", flush=True)
        L = _layer("qkv", fmt, M, K, N, rank, seed)
        layer = sq.Layer(fmt, K, N, rank)
        w = pack(layer, L, torch, dev)
        X = dev_tensor(L["X"], torch, dev)
        Yn = sq.linear_noalloc(layer, w, X, epi)
        Yr = sq.linear(layer, w, X, epi)
        Yn32 = sq.linear_noalloc(layer, w, X, epi | sq.EPI_OUT_F32)
        Yr32 = sq.linear(layer, w, X, epi | sq.EPI_OUT_F32)
        torch.cuda.synchronize()
        assert torch.equal(Yn.view(torch.int16), Yr.view(torch.int16)), f"{fmt} M={M}: bf16 output differs"
        assert torch.equal(Yn32.view(torch.int32), Yr32.view(torch.int32)), f"{fmt} M={M}: fp32 output differs"


def test_noalloc_flux_fc2_shape(torch_dev):
    """The largest FLUX layer (fc2: 4608 x 12288 -> 3072, K split in the
    activation kernel) through the static scratch, then a small layer."""
    torch, dev = torch_dev
    spec = synth.CONFIGS["fc2_mxfp4"]
    L = synth.draw_layer(spec)
    layer = sq.Layer("mxfp4", spec.K, spec.N, spec.rank)
    w = pack(layer, L, torch, dev)
    X = dev_tensor(L["X"], torch, dev)
    epi = sq.EPI_LOWRANK | sq.EPI_BIAS
    Yn = sq.linear_noalloc(layer, w, X, epi)
    Yr = sq.linear(layer, w, X, epi)
    torch.cuda.synchronize()
    assert torch.equal(Yn.view(torch.int16), Yr.view(torch.int16))
    L2 = _layer("qkv", "mxfp4", 33, 512, 256, 32, 13)
    l2 = sq.Layer("mxfp4", 512, 256, 32)
    w2 = pack(l2, L2, torch, dev)
    X2 = dev_tensor(L2["X"], torch, dev)
    Yn2 = sq.linear_noalloc(l2, w2, X2, epi)
    Yr2 = sq.linear(l2, w2, X2, epi)
    torch.cuda.synchronize()
    assert torch.equal(Yn2.view(torch.int16), Yr2.view(torch.int16))
