"""The seeded generator: determinism, shapes, the adapter rule, and that the
directly drawn calibrated layer has the statistics the oracle's real
calibration (smoothing + SVD + residual) gives on the raw recipe."""
import numpy as np
import pytest

import synth
from oracle import decompose as Dc
from oracle import formats as F
from oracle import layer as Ly


def test_deterministic_and_shapes():
    spec = synth.layer_spec("lora", M=64, K=256, N=512)
    a = synth.draw_layer(spec)
    b = synth.draw_layer(spec)
    for k in ("X", "lam", "L1", "L2", "R", "b"):
        assert np.array_equal(a[k], b[k])
    r = spec.rank + spec.lora_rank
    assert a["X"].shape == (64, 256) and a["X"].dtype == np.uint16
    assert a["lam"].shape == (256,) and a["lam"].dtype == np.float32 and np.all(a["lam"] > 0)
    assert a["L1"].shape == (256, r) and a["L2"].shape == (r, 512)
    assert a["R"].shape == (512, 256) and a["R"].dtype == np.float32
    assert a["b"].shape == (512,)
    c = synth.draw_layer(spec, with_lora=False)
    assert np.array_equal(a["R"], c["R"]) and c["L1"].shape == (256, spec.rank)
    assert np.array_equal(a["L1"][:, :spec.rank], c["L1"])


def test_configs_cover_the_five_workloads():
    names = set(synth.CONFIGS)
    assert {"single", "qkv", "fc1_mxfp4", "fc2_mxfp4", "fc1_int4", "fc2_int4", "lowm", "lora"} <= names
    s = synth.CONFIGS["fc1_mxfp4"]
    assert (s.M, s.K, s.N, s.rank, s.gelu) == (4608, 3072, 12288, 32, True)
    assert synth.CONFIGS["fc2_int4"].K == 12288 and synth.CONFIGS["lowm"].rank == 128
    assert synth.CONFIGS["lora"].rank + synth.CONFIGS["lora"].lora_rank == 48
    assert synth.CONFIGS["qkv"].x_outliers == 31 and synth.CONFIGS["lowm"].x_outliers == 61


def test_bf16_storage_rounds_to_nearest_even():
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 0.0], np.float32)
    b = synth.bf16_bits_from_f32(x)
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(b), F.to_bf16(x.astype(np.float64)))


def _stats(lam, L1, L2, R_nk, X):
    xh = Ly.smooth(X, lam).astype(np.float64)
    lr = xh @ F.bf16_value(L1) @ F.bf16_value(L2)
    res = xh @ R_nk.T.astype(np.float64)
    rms = lambda a: float(np.sqrt(np.mean(np.square(a, dtype=np.float64))))
    return dict(lam_med=float(np.median(lam)), lam_max=float(lam.max()), R=rms(R_nk),
                lowrank=rms(lr), residual=rms(res), xhat=rms(xh))


@pytest.mark.parametrize("name,over", [("single", {}), ("qkv", dict(M=576, K=1024, N=1152, x_outliers=10, w_outliers=10))])
def test_direct_draw_matches_calibrated_statistics(name, over):
    spec = synth.layer_spec(name, **over)
    raw = synth.draw_raw(spec)
    c = Dc.calibrate(raw["X"], raw["W"], spec.rank)
    L = synth.draw_layer(spec)
    a = _stats(c["lam"], c["L1"], c["L2"], c["R"].T, raw["X"])
    b = _stats(L["lam"], L["L1"], L["L2"], L["R"], L["X"])
    for k in a:
        assert 1 / 1.5 < b[k] / a[k] < 1.5, (k, a[k], b[k])
