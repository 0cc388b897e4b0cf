"""The C ABI on the host: the library loads, exports every symbol the header
declares, answers size queries, and rejects every invalid call with the
documented status before touching a device.  The device-error hook is switched
on for calls that would pass validation, so no fake pointer reaches a launch
even on a machine with a GPU."""
import ctypes
import os
import re

import pytest

import w4a4_quantized_linear_amd as sq
from w4a4_quantized_linear_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "svdq.h")


@pytest.fixture(scope="module")
def L():
    return sq.lib()


@pytest.fixture
def forced_device_error(L):
    L.svdq_test_force_device_error(1)
    yield
    L.svdq_test_force_device_error(0)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(svdq_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
        assert n in _lib.SIGNATURES, f"binding lacks {n}"
    assert set(_lib.SIGNATURES) == set(names)


def test_version_and_status_strings(L):
    assert L.svdq_version() == 107
    for s in range(9):
        assert L.svdq_status_str(s)
    assert L.svdq_status_str(99) == b"unknown status"


def D(fmt=1, K=1024, N=512, rank=16):
    return _lib.LayerDesc(fmt, K, N, rank)


def test_size_queries(L):
    wb = L.svdq_weight_bytes(ctypes.byref(D()))
    assert wb >= 512 * 1024 // 2 + 512 * 1024 // 32 + 1024 * 32 * 2 + 512 * 32 * 2 + 1024 * 8 + 512 * 2
    assert wb % 256 == 0
    # MXFP4 and INT4 use the same bytes (E8M0 per 32 vs fp16 per 64); NVFP4 one
    # more scale byte per 32 (E4M3 per 16), rows padded to 512 here
    assert L.svdq_weight_bytes(ctypes.byref(D(fmt=2))) == wb
    assert L.svdq_weight_bytes(ctypes.byref(D(fmt=3))) == wb + 512 * 1024 // 32
    assert L.svdq_act_bytes(ctypes.byref(D(fmt=3)), 4608) > L.svdq_act_bytes(ctypes.byref(D()), 4608)
    a1 = L.svdq_act_bytes(ctypes.byref(D()), 1)
    a2 = L.svdq_act_bytes(ctypes.byref(D()), 4608)
    assert 0 < a1 < a2 and a2 >= 4608 * 1024 // 2 + 4608 * 1024 // 32 + 4608 * 32 * 4
    assert L.svdq_act_bytes(ctypes.byref(D()), 0) > 0
    # invalid descriptors or rows give 0
    assert L.svdq_weight_bytes(None) == 0
    assert L.svdq_weight_bytes(ctypes.byref(D(K=1000))) == 0
    assert L.svdq_weight_bytes(ctypes.byref(D(N=24))) == 0
    assert L.svdq_weight_bytes(ctypes.byref(D(rank=257))) == 0
    assert L.svdq_weight_bytes(ctypes.byref(D(fmt=7))) == 0
    assert L.svdq_act_bytes(ctypes.byref(D()), -1) == 0


P = 0x100000  # a 256-aligned fake device address; never dereferenced (validation fails first)


def test_pack_weight_validation(L, forced_device_error):
    f = L.svdq_pack_weight
    assert f(None, P, P, P, P, P, P, None) == 1
    assert f(ctypes.byref(D()), None, P, P, P, P, P, None) == 1           # R
    assert f(ctypes.byref(D()), P, None, P, P, P, P, None) == 1           # L1 with rank > 0
    assert f(ctypes.byref(D(rank=0)), P, None, None, P, None, P, None) == 6  # rank 0: factors may be NULL
    assert f(ctypes.byref(D(K=768)), P, P, P, P, P, P, None) == 2
    assert f(ctypes.byref(D(fmt=0)), P, P, P, P, P, P, None) == 3
    assert f(ctypes.byref(D()), P + 8, P, P, P, P, P, None) == 4          # R not 16-byte aligned
    assert f(ctypes.byref(D()), P, P, P, P, P, P + 16, None) == 4         # blob not 256-byte aligned
    assert f(ctypes.byref(D()), P, P, P, P, None, P, None) == 6           # valid (bias NULL) -> device


def test_quantize_act_validation(L, forced_device_error):
    f = L.svdq_quantize_act
    d = ctypes.byref(D())
    assert f(d, P, None, 4, 1024, P, None) == 1
    assert f(d, P, None, 0, 1024, P, None) == 6       # M = 0: X may be NULL
    assert f(d, None, P, 4, 1024, P, None) == 1
    assert f(d, P, P, -1, 1024, P, None) == 2
    assert f(d, P, P, 4, 1000, P, None) == 2          # ldx < K
    assert f(d, P, P, 4, 1028, P, None) == 4          # ldx not a multiple of 8
    assert f(d, P, P, 4, (1 << 24) + 8, P, None) == 2  # ldx beyond 2^24 (32-bit row offsets)
    assert f(d, P, P, 4, 1 << 24, P, None) == 6
    assert f(d, P, P + 2, 4, 1024, P, None) == 4
    assert f(ctypes.byref(D(fmt=9)), P, P, 4, 1024, P, None) == 3
    assert f(d, P, P, 4, 1024, P, None) == 6


def test_gemm_and_linear_validation(L, forced_device_error):
    g, lin = L.svdq_gemm, L.svdq_linear
    d = ctypes.byref(D())
    assert g(d, P, P, 4, None, 512, 3, None) == 1
    assert g(d, P, P, 4, P, 500, 3, None) == 2        # ldy < N
    assert g(d, P, P, 4, P, 512, 16, None) == 3       # unknown flag
    assert g(d, P, P, 4, P, 516, 3, None) == 4
    assert g(d, P, P, 4, P, 512, 15, None) == 6
    need = L.svdq_act_bytes(d, 4)
    assert lin(d, P, P, 4, 1024, P, 512, 3, P, need - 1, None) == 5
    assert lin(d, P, P, 4, 1024, P, 512, 3, P, need, None) == 6
    assert lin(d, P, P, 4, 1024, P, 512, 3, None, need, None) == 1
    assert lin(d, P, P, 4, (1 << 24) + 8, P, 512, 3, P, need, None) == 2


def test_linear_noalloc_validation(L, forced_device_error):
    f = L.svdq_linear_noalloc
    d = ctypes.byref(D())
    assert f(d, P, P, 4, 1024, P, 512, 3, None) == 6                  # valid -> device check
    assert f(d, P, None, 0, 1024, None, 512, 3, None) == 6            # M = 0: X and Y may be NULL
    assert f(None, P, P, 4, 1024, P, 512, 3, None) == 1
    assert f(d, None, P, 4, 1024, P, 512, 3, None) == 1
    assert f(d, P, P, 4, 1024, None, 512, 3, None) == 1
    assert f(d, P, P, 4, 1000, P, 512, 3, None) == 2                  # ldx < K
    assert f(d, P, P, 4, 1024, P, 500, 3, None) == 2                  # ldy < N
    assert f(d, P, P, 4, 1024, P, 512, 16, None) == 3                 # unknown flag
    assert f(d, P + 64, P, 4, 1024, P, 512, 3, None) == 4             # blob 256-aligned
    # the workspace of the FLUX shapes fits the 64 MiB scratch; a larger one is refused
    assert f(ctypes.byref(D(K=12288, N=3072, rank=32)), P, P, 4608, 12288, P, 3072, 3, None) == 6
    assert f(ctypes.byref(D(K=65536, N=512, rank=16)), P, P, 4096, 65536, P, 512, 3, None) == 8
    assert b"64 MiB" in L.svdq_status_str(8)


def test_gemm_quant_validation(L, forced_device_error):
    q = L.svdq_gemm_quant
    d = ctypes.byref(D(K=1024, N=512, rank=16))          # this layer: 1024 -> 512
    dn = ctypes.byref(D(K=512, N=256, rank=32))          # next layer: 512 -> 256
    assert q(None, P, P, 4, 7, dn, P, P, None) == 1
    assert q(d, P, P, 4, 7, None, P, P, None) == 1
    assert q(d, P, P, 4, 7, dn, P, None, None) == 1
    assert q(d, P, P, 4, 7, ctypes.byref(D(K=1024, N=256)), P, P, None) == 2      # next K != N
    assert q(d, P, P, 4, 7, ctypes.byref(D(K=512, N=256, rank=80)), P, P, None) == 2  # next rank > 64
    assert q(d, P, P, -1, 7, dn, P, P, None) == 2
    assert q(ctypes.byref(D(fmt=2, K=1024, N=512)), P, P, 4, 7, dn, P, P, None) == 3   # INT4 into MXFP4
    assert q(d, P, P, 4, 7, ctypes.byref(D(fmt=2, K=512, N=256)), P, P, None) == 3      # MXFP4 into INT4
    assert q(ctypes.byref(D(fmt=3, K=1024, N=512)), P, P, 4, 7, ctypes.byref(D(fmt=3, K=512, N=256)), P, P,
             None) == 3                                                                 # NVFP4 pairs
    assert q(ctypes.byref(D(fmt=2, K=1024, N=512)), P, P, 4, 7, ctypes.byref(D(fmt=2, K=512, N=256, rank=32)),
             P, P, None) == 6                                                           # INT4 pair served
    assert q(d, P, P, 4, 15, dn, P, P, None) == 3        # fp32 output flag
    assert q(d, P, P, 4, 7, dn, P, P + 16, None) == 4    # workspace not 256-aligned
    assert q(d, P, P, 4, 7, dn, P, P, None) == 6         # valid -> device check
    assert q(d, P, P, 0, 7, dn, P, P, None) == 6


def test_gemm_qkv_validation(L, forced_device_error):
    f = L.svdq_gemm_qkv
    d = ctypes.byref(D(K=1024, N=768, rank=16))          # [Q | K | V], two heads of 128 each
    ok = (P, P, 4, 3, 128, P, P, ctypes.c_float(1e-6), P, P, P, 768, None)
    assert f(d, *ok) == 6                                 # valid -> device check
    assert f(None, *ok) == 1
    assert f(d, P, P, 4, 3, 128, None, P, ctypes.c_float(1e-6), P, P, P, 768, None) == 1    # norm_q
    assert f(d, P, P, 4, 3, 128, P, P, ctypes.c_float(1e-6), None, P, P, 768, None) == 1    # rope_cos
    assert f(d, P, P, 4, 3, 64, P, P, ctypes.c_float(1e-6), P, P, P, 768, None) == 2       # head_dim
    assert f(ctypes.byref(D(K=1024, N=512)), P, P, 4, 3, 128, P, P, ctypes.c_float(1e-6), P, P, P, 512, None) == 2
    assert f(d, P, P, 4, 3, 128, P, P, ctypes.c_float(-1.0), P, P, P, 768, None) == 2       # eps
    assert f(d, P, P, 4, 7, 128, P, P, ctypes.c_float(1e-6), P, P, P, 768, None) == 3       # GELU flag
    assert f(ctypes.byref(D(fmt=2, K=1024, N=768)), *ok) == 6                                 # INT4 served
    assert f(ctypes.byref(D(fmt=3, K=1024, N=768)), *ok) == 6                                 # NVFP4 served
    assert f(ctypes.byref(D(fmt=4, K=1024, N=768)), *ok) == 3                                 # no such format
    assert f(d, P, P, 4, 3, 128, P + 8, P, ctypes.c_float(1e-6), P, P, P, 768, None) == 4   # norm_q aligned
    assert f(d, P, P, 4, 3, 128, P, P, ctypes.c_float(1e-6), P, P, P + 8, 768, None) == 4   # Y aligned


def test_gemm_w4a16_validation(L, forced_device_error):
    f = L.svdq_gemm_w4a16
    d = ctypes.byref(D(fmt=2, K=1024, N=512, rank=0))
    assert f(d, P, P, 4, 1024, P, 512, 10, None) == 6         # valid (bias, fp32 out) -> device check
    assert f(d, P, None, 0, 1024, None, 512, 2, None) == 6    # M = 0: X and Y may be NULL
    assert f(None, P, P, 4, 1024, P, 512, 2, None) == 1
    assert f(d, P, None, 4, 1024, P, 512, 2, None) == 1
    assert f(d, P, P, 4, 1000, P, 512, 2, None) == 2          # ldx < K
    assert f(d, P, P, 4, 1024, P, 500, 2, None) == 2          # ldy < N
    assert f(d, P, P, 4, (1 << 24) + 8, P, 512, 2, None) == 2  # ldx beyond 2^24
    assert f(ctypes.byref(D(fmt=2, K=1000, N=512, rank=0)), P, P, 4, 1024, P, 512, 2, None) == 2
    assert f(ctypes.byref(D(fmt=1, K=1024, N=512, rank=0)), P, P, 4, 1024, P, 512, 2, None) == 3  # MXFP4
    assert f(ctypes.byref(D(fmt=2, K=1024, N=512, rank=16)), P, P, 4, 1024, P, 512, 2, None) == 3  # rank
    assert f(d, P, P, 4, 1024, P, 512, 1, None) == 3          # low-rank flag
    assert f(d, P, P, 4, 1024, P, 512, 6, None) == 3          # GELU flag
    assert f(d, P, P + 8, 4, 1024, P, 512, 2, None) == 4      # X aligned
    assert f(d, P, P, 4, 1028, P, 512, 2, None) == 4          # ldx multiple of 8
    assert f(d, P, P, 4, 1024, P + 8, 512, 2, None) == 4      # Y aligned
    assert f(d, P + 64, P, 4, 1024, P, 512, 2, None) == 4     # blob 256-aligned


def test_unpack_validation(L, forced_device_error):
    d = ctypes.byref(D())
    assert L.svdq_unpack_weight(d, None, P, P, P, P, P, P, None) == 1
    assert L.svdq_unpack_weight(d, P + 64, P, P, P, P, P, P, None) == 4
    assert L.svdq_unpack_act(d, P, -5, P, P, P, None) == 2
    assert L.svdq_unpack_act(d, P, 4, P, P, P, None) == 6


def test_device_hook_and_python_errors(L):
    L.svdq_test_force_device_error(1)
    try:
        assert L.svdq_device_check() == 6
        with pytest.raises(sq.SvdqError) as e:
            sq.check("svdq_gemm", 6)
        assert "SVDQ_ERR_DEVICE" in str(e.value) and e.value.status == 6
    finally:
        L.svdq_test_force_device_error(0)


def test_binding_refuses_missing_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError):
        _lib.lib()
