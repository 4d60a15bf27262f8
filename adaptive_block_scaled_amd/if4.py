"""Thin Python binding of libif4 (include/if4.h).

Argument marshalling only: device pointers, sizes and the current HIP stream
cross the boundary; every step of quantize / dequantize / GEMM runs in the
HIP kernels of libif4.so.  PyTorch is used for device memory and streams.
There is no fallback: if the library is missing the import of this module
raises.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# IF4_LIB selects another build of the same sources (the sanitizer build)
LIB_PATH = os.environ.get("IF4_LIB") or os.path.join(HERE, "libif4.so")

IF4_OK, IF4_ERR_NULL, IF4_ERR_SHAPE, IF4_ERR_ALIGN, IF4_ERR_DTYPE, IF4_ERR_RANGE, IF4_ERR_HIP = range(7)
IF4_F32, IF4_BF16 = 0, 1
MODE_ADAPTIVE, MODE_FORCE_FP4, MODE_FORCE_INT4 = 0, 1, 2
GROUP = 16

EXPORTS = ("if4_version", "if4_status_string", "if4_quantize", "if4_quantize_mode",
           "if4_quantize_t", "if4_quantize_rht", "if4_quantize_ifn", "if4_dequantize",
           "if4_dequantize_ifn", "if4_gemm")


class IF4Error(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn}: status {status} ({status_string(status)})")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libif4.so not found at {LIB_PATH}; build it with "
            "`python -m adaptive_block_scaled_amd.build` (or __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
    L.if4_version.restype = ci
    L.if4_version.argtypes = []
    L.if4_status_string.restype = ctypes.c_char_p
    L.if4_status_string.argtypes = [ci]
    L.if4_quantize.restype = ci
    L.if4_quantize.argtypes = [vp, ci, i64, i64, i64, vp, vp, i32, vp]
    L.if4_quantize_mode.restype = ci
    L.if4_quantize_mode.argtypes = [vp, ci, i64, i64, i64, vp, vp, i32, ci, vp]
    L.if4_quantize_t.restype = ci
    L.if4_quantize_t.argtypes = [vp, ci, i64, i64, i64, vp, vp, i32, ci, vp]
    L.if4_quantize_ifn.restype = ci
    L.if4_quantize_ifn.argtypes = [ci, vp, ci, i64, i64, i64, vp, vp, i32, ci, vp]
    L.if4_dequantize_ifn.restype = ci
    L.if4_dequantize_ifn.argtypes = [ci, vp, vp, i64, i64, i32, vp, ci, i64, vp]
    L.if4_quantize_rht.restype = ci
    L.if4_quantize_rht.argtypes = [vp, ci, i64, i64, i64, ctypes.c_uint32, vp, vp, i32, ci, vp]
    L.if4_dequantize.restype = ci
    L.if4_dequantize.argtypes = [vp, vp, i64, i64, i32, vp, ci, i64, vp]
    L.if4_gemm.restype = ci
    L.if4_gemm.argtypes = [vp, vp, i32, vp, vp, i32, i64, i64, i64, vp, i64, vp]
    return L


lib = _load()


def status_string(status: int) -> str:
    return lib.if4_status_string(status).decode()


def version() -> int:
    return lib.if4_version()


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _check(fn, st):
    if st != IF4_OK:
        raise IF4Error(fn, st)


def _dtype_code(dt) -> int:
    if dt == torch.bfloat16:
        return IF4_BF16
    if dt == torch.float32:
        return IF4_F32
    raise TypeError(f"IF4 supports float32 and bfloat16 tensors, not {dt}")


def _need(t, name, shape, dtype, device, dense=True):
    """Check a tensor handed to a kernel as a bare pointer: CUDA, on `device`,
    of `shape` and `dtype`, and contiguous (dense) or at least with unit
    stride along dim 1 and rows that do not overlap (an output with a row
    stride).  The kernels trust these sizes, so a mismatch must stop here."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, not {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    if dense:
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    elif t.dim() != 2 or t.stride(1) != 1 or (t.shape[0] > 1 and t.stride(0) < t.shape[1]):
        raise ValueError(f"{name} must have unit stride along dim 1 and non-overlapping rows")


def _input(x):
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or not x.is_cuda or x.stride(1) != 1 or \
            (x.shape[0] > 1 and x.stride(0) < x.shape[1]):
        raise ValueError("x must be a 2-D CUDA tensor with unit stride along dim 1")


def _outputs(out, device, codes_shape, scales_shape):
    if out is None:
        return (torch.empty(codes_shape, dtype=torch.uint8, device=device),
                torch.empty(scales_shape, dtype=torch.uint8, device=device))
    codes, scales = out
    _need(codes, "codes", codes_shape, torch.uint8, device)
    _need(scales, "scales", scales_shape, torch.uint8, device)
    return codes, scales


def quantize(x: torch.Tensor, scale_exp: int = 0, mode: int = MODE_ADAPTIVE, out=None):
    """Quantize a 2-D [rows, cols] CUDA tensor (fp32 or bf16, unit stride
    along dim 1) to IF4.  Returns (codes uint8 [rows, cols/2], scales uint8
    [rows, cols/16]); `out` may pass preallocated (codes, scales)."""
    _input(x)
    rows, cols = x.shape
    codes, scales = _outputs(out, x.device, (rows, cols // 2), (rows, cols // GROUP))
    st = lib.if4_quantize_mode(x.data_ptr(), _dtype_code(x.dtype), rows, cols, x.stride(0),
                               codes.data_ptr(), scales.data_ptr(), int(scale_exp), int(mode),
                               _stream(x.device))
    _check("if4_quantize_mode", st)
    return codes, scales


def quantize_t(x: torch.Tensor, scale_exp: int = 0, mode: int = MODE_ADAPTIVE, out=None):
    """IF4 of x^T for a 2-D [rows, cols] CUDA tensor (unit stride along dim
    1): groups of 16 consecutive rows of each column.  Returns (codes uint8
    [cols, rows/2], scales uint8 [cols, rows/16])."""
    _input(x)
    rows, cols = x.shape
    codes, scales = _outputs(out, x.device, (cols, rows // 2), (cols, rows // GROUP))
    st = lib.if4_quantize_t(x.data_ptr(), _dtype_code(x.dtype), rows, cols, x.stride(0),
                            codes.data_ptr(), scales.data_ptr(), int(scale_exp), int(mode),
                            _stream(x.device))
    _check("if4_quantize_t", st)
    return codes, scales


def quantize_rht(x: torch.Tensor, sign_mask: int, scale_exp: int = 0, mode: int = MODE_ADAPTIVE,
                 out=None):
    """IF4 of x after a random-sign 16-point Hadamard rotation of every group
    along dim 1 (bit i of sign_mask negates element i of each group first).
    Same layout and return as quantize(); the rotated values never reach
    memory."""
    _input(x)
    rows, cols = x.shape
    codes, scales = _outputs(out, x.device, (rows, cols // 2), (rows, cols // GROUP))
    st = lib.if4_quantize_rht(x.data_ptr(), _dtype_code(x.dtype), rows, cols, x.stride(0),
                              int(sign_mask), codes.data_ptr(), scales.data_ptr(),
                              int(scale_exp), int(mode), _stream(x.device))
    _check("if4_quantize_rht", st)
    return codes, scales


def quantize_ifn(x: torch.Tensor, bits: int, scale_exp: int = 0, mode: int = MODE_ADAPTIVE,
                 out=None):
    """IF3 (bits=3) or IF6 (bits=6) of a 2-D CUDA tensor (groups of 16 along
    dim 1).  Returns (codes uint8 [rows, cols/16 * 2*bits], scales uint8
    [rows, cols/16])."""
    _input(x)
    rows, cols = x.shape
    codes, scales = _outputs(out, x.device, (rows, cols // GROUP * 2 * bits),
                             (rows, cols // GROUP))
    st = lib.if4_quantize_ifn(int(bits), x.data_ptr(), _dtype_code(x.dtype), rows, cols,
                              x.stride(0), codes.data_ptr(), scales.data_ptr(), int(scale_exp),
                              int(mode), _stream(x.device))
    _check("if4_quantize_ifn", st)
    return codes, scales


def dequantize_ifn(codes: torch.Tensor, scales: torch.Tensor, bits: int, scale_exp: int = 0,
                   dtype=torch.float32, out=None) -> torch.Tensor:
    if not isinstance(scales, torch.Tensor) or scales.dim() != 2:
        raise ValueError("scales must be a 2-D tensor [rows, cols/16]")
    rows, gpr = scales.shape
    cols = gpr * GROUP
    _need(codes, "codes", (rows, gpr * 2 * bits), torch.uint8, codes.device)
    _need(scales, "scales", (rows, gpr), torch.uint8, codes.device)
    if out is None:
        y = torch.empty((rows, cols), dtype=dtype, device=codes.device)
    else:
        y = out
        _need(y, "out", (rows, cols), y.dtype, codes.device, dense=False)
    st = lib.if4_dequantize_ifn(int(bits), codes.data_ptr(), scales.data_ptr(), rows, cols,
                                int(scale_exp), y.data_ptr(), _dtype_code(y.dtype), y.stride(0),
                                _stream(codes.device))
    _check("if4_dequantize_ifn", st)
    return y


def dequantize(codes: torch.Tensor, scales: torch.Tensor, scale_exp: int = 0,
               dtype=torch.float32, out=None) -> torch.Tensor:
    if not isinstance(codes, torch.Tensor) or codes.dim() != 2:
        raise ValueError("codes must be a 2-D tensor [rows, cols/2]")
    rows, half = codes.shape
    cols = 2 * half
    _need(codes, "codes", (rows, half), torch.uint8, codes.device)
    _need(scales, "scales", (rows, cols // GROUP), torch.uint8, codes.device)
    if out is None:
        y = torch.empty((rows, cols), dtype=dtype, device=codes.device)
    else:
        y = out
        _need(y, "out", (rows, cols), y.dtype, codes.device, dense=False)
    st = lib.if4_dequantize(codes.data_ptr(), scales.data_ptr(), rows, cols, int(scale_exp),
                            y.data_ptr(), _dtype_code(y.dtype), y.stride(0),
                            _stream(codes.device))
    _check("if4_dequantize", st)
    return y


def gemm(a_codes, a_scales, a_exp, w_codes, w_scales, w_exp, out=None) -> torch.Tensor:
    """C[M, N] = A[M, K] W[N, K]^T for IF4 operands; fp32 result."""
    for name, t in (("a_codes", a_codes), ("w_codes", w_codes)):
        if not isinstance(t, torch.Tensor) or t.dim() != 2:
            raise ValueError(f"{name} must be a 2-D tensor [rows, K/2]")
    M, K = a_codes.shape[0], 2 * a_codes.shape[1]
    N = w_codes.shape[0]
    if w_codes.shape[1] * 2 != K:
        raise ValueError("A and W must share K")
    dev = a_codes.device
    _need(a_codes, "a_codes", (M, K // 2), torch.uint8, dev)
    _need(a_scales, "a_scales", (M, K // GROUP), torch.uint8, dev)
    _need(w_codes, "w_codes", (N, K // 2), torch.uint8, dev)
    _need(w_scales, "w_scales", (N, K // GROUP), torch.uint8, dev)
    if out is None:
        c = torch.empty((M, N), dtype=torch.float32, device=dev)
    else:
        c = out
        _need(c, "out", (M, N), torch.float32, dev, dense=False)
    st = lib.if4_gemm(a_codes.data_ptr(), a_scales.data_ptr(), int(a_exp), w_codes.data_ptr(),
                      w_scales.data_ptr(), int(w_exp), M, N, K, c.data_ptr(), c.stride(0),
                      _stream(a_codes.device))
    _check("if4_gemm", st)
    return c
