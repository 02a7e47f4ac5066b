"""The C-ABI library loads and exports every entry point declared in
include/fq.h; host-side argument validation rejects bad shapes before any
launch (no GPU needed for these calls)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fq.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:fq_status|const char\*|void)\s+(fq_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_five_calls():
    names = _declared()
    for n in ("fq_quantize", "fq_dequant_gemm", "fq_decode_attention", "fq_layer_step", "fq_generate"):
        assert n in names


def test_library_exports_every_declared_symbol():
    fq = pytest.importorskip("bit_weight_kv_amd")
    lib = ctypes.CDLL(fq.LIB_PATH)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing
    assert set(_declared()) == set(fq.EXPORTED)


def test_version_and_error_strings():
    fq = pytest.importorskip("bit_weight_kv_amd")
    assert "gfx950" in fq.fq_version()
    assert fq.fq_last_error() == ""


def test_host_validation_without_launch():
    fq = pytest.importorskip("bit_weight_kv_amd")
    lib = fq._lib
    p = fq.fq_packed(ctypes.c_void_p(16), ctypes.c_void_p(16), 4, 100, 64)
    assert lib.fq_quantize(ctypes.c_void_p(16), 4, 100, 100, ctypes.byref(p), None) == fq.FQ_ERR_INVALID
    assert "multiple of 64" in fq.fq_last_error()
    p.group = 32
    p.cols = 128
    assert lib.fq_quantize(ctypes.c_void_p(16), 4, 128, 128, ctypes.byref(p), None) == fq.FQ_ERR_UNSUPPORTED
    # zero rows is a no-op that succeeds without touching memory
    p.group, p.rows = 64, 0
    assert lib.fq_quantize(None, 0, 128, 128, ctypes.byref(p), None) == fq.FQ_OK
    kv = fq.fq_kv_layer(ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16),
                        2, 4, 128, 10, 64)
    # positions beyond capacity are rejected
    assert lib.fq_kv_append(ctypes.byref(kv), ctypes.c_void_p(16), ctypes.c_void_p(16), 1536, 0, 2, 4, 8,
                            None) == fq.FQ_ERR_INVALID
    assert "capacity" in fq.fq_last_error()
    assert lib.fq_decode_attention(ctypes.c_void_p(16), 512, ctypes.byref(kv), 0, 3, 5, ctypes.c_void_p(16), 512,
                                   None) == fq.FQ_ERR_INVALID
    kv.head_dim = 96
    assert lib.fq_decode_attention(ctypes.c_void_p(16), 512, ctypes.byref(kv), 0, 1, 5, ctypes.c_void_p(16), 512,
                                   None) == fq.FQ_ERR_UNSUPPORTED
    w = fq.fq_weight(fq.FQ_WEIGHT_PACKED4, fq.fq_packed(ctypes.c_void_p(16), ctypes.c_void_p(16), 64, 100, 64),
                     None, 64, 100)
    assert lib.fq_dequant_gemm(ctypes.c_void_p(16), 4, 128, ctypes.byref(w), None, None, 0, 0, 1.0, 0,
                               ctypes.c_void_p(16), 64, None) == fq.FQ_ERR_INVALID
    assert "K must be a multiple of 64" in fq.fq_last_error()
