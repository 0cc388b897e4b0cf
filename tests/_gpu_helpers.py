"""Helpers shared by the GPU tests: move seeded inputs to the device, run the
layer through the C ABI, and compare with the oracle."""
from __future__ import annotations

import numpy as np

import w4a4_quantized_linear_amd as sq
from oracle import formats as F
from oracle import layer as Ly
from oracle import quant as Q


def dev_tensor(a, torch, device):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def pack(layer, L, torch, device, bias=True):
    return sq.pack_weight(layer, dev_tensor(L["R"], torch, device), dev_tensor(L["L1"], torch, device),
                          dev_tensor(L["L2"], torch, device), dev_tensor(L["lam"], torch, device),
                          dev_tensor(L["b"], torch, device) if bias else None)


def scales_np(t, fmt):
    a = t.cpu().numpy()
    return a.view(np.uint16) if fmt == "int4" else a.view(np.uint8)


def bf16_to_np(t):
    return F.bf16_value(t.cpu().view(__import__("torch").int16).numpy().view(np.uint16))


def assert_codes_equal(got_packed, ref_codes, what):
    ref = Q.pack_canonical(ref_codes)
    if not np.array_equal(got_packed, ref):
        bad = np.argwhere(got_packed != ref)
        r, j = bad[0]
        raise AssertionError(f"{what}: {len(bad)} code bytes differ; first at row {r} byte {j}: "
                             f"got {got_packed[r, j]:#04x} want {ref[r, j]:#04x}")


def assert_scales_equal(got, ref, what):
    if not np.array_equal(got, ref):
        bad = np.argwhere(got != ref)
        r, j = bad[0]
        raise AssertionError(f"{what}: {len(bad)} scales differ; first at row {r} group {j}: "
                             f"got {got[r, j]} want {ref[r, j]}")


def bf16_half_ulp(y):
    """Half a bf16 unit in the last place at each |y| (the output rounding allowance)."""
    a = np.abs(np.asarray(y, dtype=np.float64))
    _, e = np.frexp(np.maximum(a, 2.0 ** -126))
    return np.ldexp(1.0, e - 1 - 8)


def check_fp32_output(Y, Y_o, what):
    m = Ly.parity_metrics(Y, Y_o)
    assert m["max_over_rms"] <= Ly.MAX_OVER_RMS and m["mean_rel"] <= Ly.MEAN_REL, f"{what}: {m}"
    return m


def check_bf16_output(Yb, Y_o, what):
    """bf16 output: the stated tolerance plus the output format's own rounding
    (half a bf16 ulp of each value), and the mean relative error bound."""
    Yb = np.asarray(Yb, dtype=np.float64)
    err = np.abs(Yb - Y_o)
    rms = float(np.sqrt(np.mean(Y_o ** 2)))
    lim = Ly.MAX_OVER_RMS * rms + bf16_half_ulp(Y_o)
    assert np.all(err <= lim), f"{what}: max excess {(err - lim).max():.3e} (rms {rms:.3e})"
    mean_rel = float(err.sum() / np.abs(Y_o).sum())
    assert mean_rel <= Ly.MEAN_REL, f"{what}: mean rel {mean_rel:.3e}"
    return mean_rel


def check_chain_output(Y, Y_o, what, fmt="mxfp4"):
    """Output of a chain of layers where each side feeds its own intermediate
    (GPU H vs oracle H) to the next 4-bit quantizer.  Intermediates that differ
    by rounding flip a few 4-bit codes, and one flip moves a product term by a
    whole quantization step, so the per-element max bound does not carry over;
    the mean relative error bound does.  Checked: mean relative error <= 5e-3,
    at most 0.1% of elements beyond 2e-2 rms (0.2% for INT4, whose uniform grid
    of 15 steps per group puts more decision boundaries in the bulk of the
    values than E2M1's, so the same differences in H flip more codes), none
    beyond 0.25 rms."""
    Y = np.asarray(Y, dtype=np.float64)
    err = np.abs(Y - Y_o)
    rms = float(np.sqrt(np.mean(Y_o ** 2)))
    mean_rel = float(err.sum() / np.abs(Y_o).sum())
    frac = float(np.mean(err > Ly.MAX_OVER_RMS * rms))
    frac_max = 2e-3 if fmt == "int4" else 1e-3
    assert mean_rel <= Ly.MEAN_REL and frac <= frac_max and err.max() <= 0.25 * rms, \
        f"{what}: mean rel {mean_rel:.2e}, fraction over 2e-2 rms {frac:.2e}, max/rms {err.max() / rms:.3f}"
    return mean_rel, frac


def check_next_layer_on_gpu_h(torch, ua, L2, H, Y2f, fmt, rows, what):
    """The oracle's next layer on the GPU's own bf16 H (its rows `rows`): `ua`
    (the GPU's unpacked activation workspace of that layer for H) must hold the
    oracle's codes and scales of H_hat bit for bit, and a down projection within
    the bound of a bf16 hi + lo split summed in fp32; the layer's fp32 output
    Y2f must meet the full tolerance against the oracle's on the same H."""
    Hb = H.view(torch.int16).cpu().numpy().view(np.uint16)[rows]
    ref = Ly.forward(Hb, L2["lam"], L2["L1"], L2["L2"], L2["R"], L2["b"], fmt)
    assert_codes_equal(ua["codes"].cpu().numpy()[rows], ref["cX"], f"{what}: codes of H_hat")
    assert_scales_equal(scales_np(ua["scales"], fmt)[rows], ref["sX"], f"{what}: scales of H_hat")
    if np.asarray(L2["L1"]).shape[1]:
        Dg = ua["D"].cpu().numpy()[rows].astype(np.float64)
        bound = np.abs(ref["xhat"].astype(np.float64)) @ np.abs(F.bf16_value(L2["L1"]))
        assert np.all(np.abs(Dg - ref["D"]) <= 2.0 ** -14 * bound + 1e-30), f"{what}: down projection"
    check_fp32_output(Y2f.cpu().numpy()[rows], ref["Y"], f"{what}: output")
    return ref
