"""The C-ABI library: loads, exports every entry point include/if4.h
declares, and rejects bad arguments on the host before any HIP call (so
these run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "if4.h")
LIB = os.path.join(ROOT, "adaptive_block_scaled_amd", "libif4.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libif4.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(if4_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    from adaptive_block_scaled_amd import if4
    return if4.lib


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert names == sorted(["if4_version", "if4_status_string", "if4_quantize",
                            "if4_quantize_mode", "if4_quantize_t", "if4_quantize_rht",
                            "if4_quantize_ifn", "if4_dequantize", "if4_dequantize_ifn",
                            "if4_gemm"])
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings(L):
    assert L.if4_version() >= 100
    for st in range(7):
        assert L.if4_status_string(st)
    assert L.if4_status_string(99) == b"unknown status"


FAKE = 0x100000  # 16-byte aligned fake device address; never dereferenced


def q(L, x=FAKE, dt=1, rows=4, cols=32, ld=32, codes=FAKE, scales=FAKE, e=0, mode=0):
    return L.if4_quantize_mode(x, dt, rows, cols, ld, codes, scales, e, mode, None)


def test_quantize_validation(L):
    assert q(L, dt=7) == 4
    assert q(L, mode=3) == 4
    assert q(L, cols=24, ld=24) == 2
    assert q(L, rows=-1) == 2
    assert q(L, ld=16) == 2
    assert q(L, e=65) == 5 and q(L, e=-65) == 5
    assert q(L, x=None) == 1 and q(L, codes=None) == 1 and q(L, scales=None) == 1
    assert q(L, x=FAKE + 2) == 3
    assert q(L, codes=FAKE + 4) == 3
    assert q(L, dt=1, ld=36) == 3      # 72 B rows: not a multiple of 16
    # empty inputs are valid and launch nothing
    assert q(L, rows=0) == 0 and q(L, rows=3, cols=0, ld=0) == 0
    assert L.if4_quantize(FAKE, 1, 0, 32, 32, FAKE, FAKE, 0, None) == 0


def qt(L, x=FAKE, dt=1, rows=32, cols=8, ld=8, codes=FAKE, scales=FAKE, e=0, mode=0):
    return L.if4_quantize_t(x, dt, rows, cols, ld, codes, scales, e, mode, None)


def test_quantize_t_validation(L):
    # every call below has exactly one bad argument, so none launches
    assert qt(L, dt=7) == 4
    assert qt(L, mode=3) == 4
    assert qt(L, rows=20) == 2         # groups run down the rows
    assert qt(L, rows=-16) == 2
    assert qt(L, ld=4) == 2
    assert qt(L, e=65) == 5
    assert qt(L, x=None) == 1 and qt(L, codes=None) == 1 and qt(L, scales=None) == 1
    assert qt(L, x=FAKE + 1, dt=1) == 3  # bf16 needs 2-byte alignment
    assert qt(L, x=FAKE + 2, dt=0) == 3  # fp32 needs 4-byte alignment
    assert qt(L, codes=FAKE + 4) == 3
    assert qt(L, rows=0) == 0 and qt(L, cols=0, ld=0) == 0


def qr(L, x=FAKE, dt=1, rows=4, cols=32, ld=32, mask=0x1234, codes=FAKE, scales=FAKE, e=0,
       mode=0):
    return L.if4_quantize_rht(x, dt, rows, cols, ld, mask, codes, scales, e, mode, None)


def test_quantize_rht_validation(L):
    # every call below has exactly one bad argument, so none launches
    assert qr(L, mask=0x10000) == 5 and qr(L, mask=0xFFFFFFFF) == 5
    assert qr(L, dt=7) == 4
    assert qr(L, mode=3) == 4
    assert qr(L, cols=40, ld=40) == 2  # groups run along the rows
    assert qr(L, ld=16) == 2
    assert qr(L, rows=-1) == 2
    assert qr(L, e=-65) == 5
    assert qr(L, x=None) == 1 and qr(L, codes=None) == 1 and qr(L, scales=None) == 1
    assert qr(L, x=FAKE + 2) == 3
    assert qr(L, ld=36) == 3           # 72-byte rows break 16-byte alignment
    assert qr(L, codes=FAKE + 4) == 3
    assert qr(L, rows=0) == 0 and qr(L, cols=0, ld=0) == 0


def qn(L, bits=6, x=FAKE, dt=1, rows=4, cols=32, ld=32, codes=FAKE, scales=FAKE, e=0, mode=0):
    return L.if4_quantize_ifn(bits, x, dt, rows, cols, ld, codes, scales, e, mode, None)


def dn(L, bits=6, codes=FAKE, scales=FAKE, rows=4, cols=32, e=0, y=FAKE, dt=1, ld=32):
    return L.if4_dequantize_ifn(bits, codes, scales, rows, cols, e, y, dt, ld, None)


def test_ifn_validation(L):
    # every call below has exactly one bad argument, so none launches
    for b in (0, 4, 5, 8):
        assert qn(L, bits=b) == 4 and dn(L, bits=b) == 4
    assert qn(L, dt=2) == 4 and qn(L, mode=3) == 4
    assert qn(L, cols=40, ld=40) == 2 and qn(L, ld=16) == 2
    assert qn(L, e=65) == 5
    assert qn(L, x=None) == 1 and qn(L, codes=None) == 1
    assert qn(L, x=FAKE + 2) == 3 and qn(L, codes=FAKE + 4) == 3
    assert qn(L, rows=0) == 0 and qn(L, bits=3, cols=0, ld=0) == 0
    assert dn(L, dt=5) == 4 and dn(L, cols=20, ld=32) == 2 and dn(L, ld=16) == 2
    assert dn(L, e=-65) == 5 and dn(L, y=None) == 1 and dn(L, scales=None) == 1
    assert dn(L, y=FAKE + 8) == 3 and dn(L, codes=FAKE + 4) == 3
    assert dn(L, rows=0) == 0


def test_dequantize_validation(L):
    d = L.if4_dequantize
    assert d(FAKE, FAKE, 4, 32, 0, FAKE, 5, 32, None) == 4
    assert d(FAKE, FAKE, 4, 20, 0, FAKE, 0, 32, None) == 2
    assert d(FAKE, FAKE, 4, 32, 0, FAKE, 0, 16, None) == 2
    assert d(FAKE, FAKE, 4, 32, 99, FAKE, 0, 32, None) == 5
    assert d(None, FAKE, 4, 32, 0, FAKE, 0, 32, None) == 1
    assert d(FAKE, FAKE, 4, 32, 0, FAKE + 8, 0, 32, None) == 3
    assert d(FAKE, FAKE, 0, 32, 0, FAKE, 0, 32, None) == 0


def test_gemm_validation(L):
    g = L.if4_gemm
    assert g(FAKE, FAKE, 0, FAKE, FAKE, 0, 8, 8, 24, FAKE, 8, None) == 2
    assert g(FAKE, FAKE, 0, FAKE, FAKE, 0, 8, 8, 32, FAKE, 4, None) == 2
    assert g(FAKE, FAKE, 0, FAKE, FAKE, 0, -1, 8, 32, FAKE, 8, None) == 2
    assert g(FAKE, FAKE, 70, FAKE, FAKE, 0, 8, 8, 32, FAKE, 8, None) == 5
    assert g(FAKE, FAKE, 0, None, FAKE, 0, 8, 8, 32, FAKE, 8, None) == 1
    assert g(FAKE, FAKE, 0, FAKE, FAKE, 0, 8, 8, 32, None, 8, None) == 1
    assert g(FAKE + 4, FAKE, 0, FAKE, FAKE, 0, 8, 8, 32, FAKE, 8, None) == 3
    assert g(FAKE, FAKE, 0, FAKE, FAKE, 0, 0, 8, 32, FAKE, 8, None) == 0


def test_python_binding_raises_without_gpu_tensors():
    import torch
    from adaptive_block_scaled_amd import if4
    with pytest.raises(ValueError):
        if4.quantize(torch.zeros(4, 32))
