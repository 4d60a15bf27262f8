"""ctypes binding of the C oracle (liboracle.so), numpy in and out.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and
bench.py's CPU-baseline leg, never by the product path.
"""
import ctypes
import os

import numpy as np

from .build import LIB, build_oracle

ADAPTIVE, FORCE_FP4, FORCE_INT4 = 0, 1, 2
GROUP = 16

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build_oracle()
        L = ctypes.CDLL(LIB)
        c_u8p = ctypes.POINTER(ctypes.c_uint8)
        c_f32p = ctypes.POINTER(ctypes.c_float)
        c_f64p = ctypes.POINTER(ctypes.c_double)
        c_i64p = ctypes.POINTER(ctypes.c_int64)
        c_u16p = ctypes.POINTER(ctypes.c_uint16)
        i64, i32 = ctypes.c_int64, ctypes.c_int32
        L.if4o_e4m3_value.restype = ctypes.c_double
        L.if4o_e4m3_value.argtypes = [ctypes.c_uint]
        L.if4o_e2m1_value.restype = ctypes.c_double
        L.if4o_e2m1_value.argtypes = [ctypes.c_uint]
        L.if4o_scale_code.restype = ctypes.c_uint
        L.if4o_scale_code.argtypes = [ctypes.c_double]
        L.if4o_fp4_index.restype = ctypes.c_uint
        L.if4o_fp4_index.argtypes = [ctypes.c_double, ctypes.c_double]
        L.if4o_int4_mag.restype = ctypes.c_uint
        L.if4o_int4_mag.argtypes = [ctypes.c_double, ctypes.c_double]
        L.if4o_quantize.restype = None
        L.if4o_quantize.argtypes = [c_f32p, i64, i64, i64, i32, ctypes.c_int, c_u8p,
                                    c_u8p, c_f32p, c_f32p, ctypes.c_int]
        L.if4o_dequantize.restype = None
        L.if4o_dequantize.argtypes = [c_u8p, c_u8p, i64, i64, i32, c_f32p, i64,
                                      ctypes.c_int]
        L.if4o_f32_to_bf16.restype = None
        L.if4o_f32_to_bf16.argtypes = [c_f32p, i64, c_u16p]
        L.if4o_decode_f64.restype = None
        L.if4o_decode_f64.argtypes = [c_u8p, c_u8p, i64, i64, i32, c_f64p, ctypes.c_int]
        L.if4o_gemm_sample_f64.restype = None
        L.if4o_gemm_sample_f64.argtypes = [c_u8p, c_u8p, i32, c_u8p, c_u8p, i32, i64,
                                           c_i64p, i64, c_i64p, i64, c_f64p,
                                           ctypes.c_int]
        L.if4o_rht16.restype = None
        L.if4o_rht16.argtypes = [c_f32p, i64, i64, i64, ctypes.c_uint32, ctypes.c_int, c_f32p,
                                 i64, ctypes.c_int]
        L.if4o_quantize_rht.restype = None
        L.if4o_quantize_rht.argtypes = [c_f32p, i64, i64, i64, ctypes.c_uint32, ctypes.c_int,
                                        i32, ctypes.c_int, c_u8p, c_u8p, ctypes.c_int]
        L.if4o_ifn_fp_value.restype = ctypes.c_double
        L.if4o_ifn_fp_value.argtypes = [ctypes.c_int, ctypes.c_uint]
        L.if4o_ifn_scale_code.restype = ctypes.c_uint
        L.if4o_ifn_scale_code.argtypes = [ctypes.c_int, ctypes.c_double]
        L.if4o_ifn_fp_index.restype = ctypes.c_uint
        L.if4o_ifn_fp_index.argtypes = [ctypes.c_int, ctypes.c_double, ctypes.c_double]
        L.if4o_ifn_int_mag.restype = ctypes.c_uint
        L.if4o_ifn_int_mag.argtypes = [ctypes.c_int, ctypes.c_double, ctypes.c_double]
        L.if4o_ifn_quantize.restype = ctypes.c_int
        L.if4o_ifn_quantize.argtypes = [ctypes.c_int, c_f32p, i64, i64, i64, i32, ctypes.c_int,
                                        c_u8p, c_u8p, c_f32p, c_f32p, ctypes.c_int]
        L.if4o_ifn_dequantize.restype = ctypes.c_int
        L.if4o_ifn_dequantize.argtypes = [ctypes.c_int, c_u8p, c_u8p, i64, i64, i32, c_f32p, i64,
                                          ctypes.c_int]
        _lib = L
    return _lib


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def e4m3_value(code7: int) -> float:
    return lib().if4o_e4m3_value(code7)


def e2m1_value(idx: int) -> float:
    return lib().if4o_e2m1_value(idx)


def scale_code(a_scaled: float) -> int:
    return lib().if4o_scale_code(float(a_scaled))


def fp4_index(ax: float, s: float) -> int:
    return lib().if4o_fp4_index(float(ax), float(s))


def int4_mag(ax: float, s: float) -> int:
    return lib().if4o_int4_mag(float(ax), float(s))


def quantize(x, scale_exp: int = 0, mode: int = ADAPTIVE, with_errors: bool = False,
             nthreads: int = 0):
    """x: float32 [rows, cols] (bf16 inputs widened exactly). Returns codes
    uint8 [rows, cols/2], scales uint8 [rows, cols/16] (and the fp32 error
    sums [rows, cols/16] x2 when with_errors)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x.shape
    assert cols % GROUP == 0
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // GROUP), np.uint8)
    ef = np.zeros((rows, cols // GROUP), np.float32) if with_errors else None
    ei = np.zeros((rows, cols // GROUP), np.float32) if with_errors else None
    lib().if4o_quantize(_ptr(x, ctypes.c_float), rows, cols, cols, scale_exp, mode,
                        _ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8),
                        _ptr(ef, ctypes.c_float) if with_errors else None,
                        _ptr(ei, ctypes.c_float) if with_errors else None, nthreads)
    if with_errors:
        return codes, scales, ef, ei
    return codes, scales


def dequantize(codes, scales, scale_exp: int = 0, nthreads: int = 0):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, half = codes.shape
    cols = 2 * half
    assert scales.shape == (rows, cols // GROUP)
    y = np.zeros((rows, cols), np.float32)
    lib().if4o_dequantize(_ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8),
                          rows, cols, scale_exp, _ptr(y, ctypes.c_float), cols, nthreads)
    return y


def f32_to_bf16_bits(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.zeros(x.shape, np.uint16)
    lib().if4o_f32_to_bf16(_ptr(x, ctypes.c_float), x.size, _ptr(out, ctypes.c_uint16))
    return out


def decode_f64(codes, scales, scale_exp: int = 0, nthreads: int = 0):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, half = codes.shape
    cols = 2 * half
    y = np.zeros((rows, cols), np.float64)
    lib().if4o_decode_f64(_ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8),
                          rows, cols, scale_exp, _ptr(y, ctypes.c_double), nthreads)
    return y


def gemm_sample_f64(a_codes, a_scales, a_exp, w_codes, w_scales, w_exp, rows=None,
                    cols=None, nthreads: int = 0):
    """fp64 C[rows, cols] = A_dec[rows] @ W_dec[cols]^T (A [M,K], W [N,K])."""
    a_codes = np.ascontiguousarray(a_codes, dtype=np.uint8)
    a_scales = np.ascontiguousarray(a_scales, dtype=np.uint8)
    w_codes = np.ascontiguousarray(w_codes, dtype=np.uint8)
    w_scales = np.ascontiguousarray(w_scales, dtype=np.uint8)
    M, K = a_codes.shape[0], 2 * a_codes.shape[1]
    N = w_codes.shape[0]
    assert w_codes.shape[1] * 2 == K
    rows = np.arange(M, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    cols = np.arange(N, dtype=np.int64) if cols is None else np.asarray(cols, np.int64)
    rows = np.ascontiguousarray(rows)
    cols = np.ascontiguousarray(cols)
    c = np.zeros((rows.size, cols.size), np.float64)
    lib().if4o_gemm_sample_f64(_ptr(a_codes, ctypes.c_uint8), _ptr(a_scales, ctypes.c_uint8),
                               a_exp, _ptr(w_codes, ctypes.c_uint8),
                               _ptr(w_scales, ctypes.c_uint8), w_exp, K,
                               _ptr(rows, ctypes.c_int64), rows.size,
                               _ptr(cols, ctypes.c_int64), cols.size,
                               _ptr(c, ctypes.c_double), nthreads)
    return c


def rht16(x, sign_mask: int, round_to_bf16: bool = False, nthreads: int = 0):
    """Per-group random-sign Hadamard rotation along dim 1 (fp32 butterflies;
    bit i of sign_mask negates element i of every group).  Returns fp32
    [rows, cols]; with round_to_bf16 every value is bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x.shape
    assert cols % GROUP == 0
    y = np.zeros((rows, cols), np.float32)
    lib().if4o_rht16(_ptr(x, ctypes.c_float), rows, cols, cols, sign_mask & 0xFFFF,
                     int(round_to_bf16), _ptr(y, ctypes.c_float), cols, nthreads)
    return y


def quantize_rht(x, sign_mask: int, scale_exp: int = 0, mode: int = ADAPTIVE,
                 round_to_bf16: bool = False, nthreads: int = 0):
    """IF4 of rht16(x, sign_mask, round_to_bf16): (codes, scales)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x.shape
    assert cols % GROUP == 0
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // GROUP), np.uint8)
    lib().if4o_quantize_rht(_ptr(x, ctypes.c_float), rows, cols, cols, sign_mask & 0xFFFF,
                            int(round_to_bf16), scale_exp, mode, _ptr(codes, ctypes.c_uint8),
                            _ptr(scales, ctypes.c_uint8), nthreads)
    return codes, scales


def ifn_fp_value(bits: int, idx: int) -> float:
    return lib().if4o_ifn_fp_value(bits, idx)


def ifn_scale_code(bits: int, a_scaled: float) -> int:
    return lib().if4o_ifn_scale_code(bits, float(a_scaled))


def ifn_fp_index(bits: int, ax: float, s: float) -> int:
    return lib().if4o_ifn_fp_index(bits, float(ax), float(s))


def ifn_int_mag(bits: int, ax: float, s: float) -> int:
    return lib().if4o_ifn_int_mag(bits, float(ax), float(s))


def quantize_ifn(x, bits: int, scale_exp: int = 0, mode: int = ADAPTIVE,
                 with_errors: bool = False, nthreads: int = 0):
    """IF3 (bits=3) or IF6 (bits=6) of float32 x [rows, cols]: codes uint8
    [rows, cols/16 * 2*bits], scales uint8 [rows, cols/16] (and the fp32
    error sums when with_errors)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x.shape
    assert cols % GROUP == 0 and bits in (3, 6)
    codes = np.zeros((rows, cols // GROUP * 2 * bits), np.uint8)
    scales = np.zeros((rows, cols // GROUP), np.uint8)
    ef = np.zeros((rows, cols // GROUP), np.float32) if with_errors else None
    ei = np.zeros((rows, cols // GROUP), np.float32) if with_errors else None
    st = lib().if4o_ifn_quantize(bits, _ptr(x, ctypes.c_float), rows, cols, cols, scale_exp, mode,
                                 _ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8),
                                 _ptr(ef, ctypes.c_float) if with_errors else None,
                                 _ptr(ei, ctypes.c_float) if with_errors else None, nthreads)
    assert st == 0
    if with_errors:
        return codes, scales, ef, ei
    return codes, scales


def dequantize_ifn(codes, scales, bits: int, scale_exp: int = 0, nthreads: int = 0):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, gpr = scales.shape
    cols = gpr * GROUP
    assert codes.shape == (rows, gpr * 2 * bits)
    y = np.zeros((rows, cols), np.float32)
    st = lib().if4o_ifn_dequantize(bits, _ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8),
                                   rows, cols, scale_exp, _ptr(y, ctypes.c_float), cols, nthreads)
    assert st == 0
    return y
