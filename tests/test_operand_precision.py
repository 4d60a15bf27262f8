"""Why the GEMM decodes IF4 operands to fp16 rather than bf16 (CPU only).

FP4 values c*s' have at most 6 significant bits and are exact in either
16-bit type; INT4 values 6|q|s'/7 are not.  This simulates both operand
types on a C4-shaped sample (activations with outlier columns, N(0, 0.02)
weights, K = 4096), quantized by the oracle, against the exact fp64 product
of the decoded operands, and checks the 1e-3 relative Frobenius budget.
The fp16 simulation follows the kernel's decode exactly: every operand is
the decoded value times 2^-9 in fp16 (subnormals included), FP4 c*s' exact,
INT4 fl16(|q| * fl16(fl32(s' * fl32(6/7))) * 2^-9); products accumulated in
fp64 (the MFMA accumulates the exact fp16 products in fp32).
"""
import numpy as np

from adaptive_block_scaled_amd import workloads as wl

E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float64)


def e4m3(code7):
    code7 = np.asarray(code7, np.int64)
    e, m = code7 >> 3, code7 & 7
    return np.where(e == 0, m * 2.0 ** -9, (1 + m / 8) * 2.0 ** (e - 7))


def unpack(codes):
    lo, hi = codes & 0xF, codes >> 4
    return np.stack([lo, hi], -1).reshape(codes.shape[0], -1)


def decode_kernel_fp16(codes, scales):
    """The GPU decode (without 2^E), as fp16 values widened to fp64."""
    nib = unpack(codes).astype(np.int64)
    mag, neg = nib & 7, (nib >> 3) & 1
    b = np.repeat(scales.astype(np.int64), 16, axis=1)
    sp = e4m3(b & 0x7F)
    int4 = (b & 0x80) != 0
    sig_int = (sp.astype(np.float32) * np.float32(6.0 / 7.0)).astype(np.float16)
    v_int = (mag * sig_int.astype(np.float64) * 2.0**-9).astype(np.float16).astype(np.float64)
    v_int = v_int * 2.0**9
    v_fp = (E2M1[mag] * sp * 2.0**-9).astype(np.float16).astype(np.float64) * 2.0**9  # exact
    v = np.where(int4, v_int, v_fp)
    return np.where(neg == 1, -v, v)


def decode_bf16(codes, scales):
    import torch
    nib = unpack(codes).astype(np.int64)
    mag, neg = nib & 7, (nib >> 3) & 1
    b = np.repeat(scales.astype(np.int64), 16, axis=1)
    sp = e4m3(b & 0x7F)
    exact = np.where((b & 0x80) != 0, 6.0 * mag * sp / 7.0, E2M1[mag] * sp)
    v = torch.from_numpy(exact).to(torch.bfloat16).double().numpy()
    return np.where(neg == 1, -v, v)


def test_fp16_operands_meet_tolerance_bf16_do_not(oracle_mod):
    a = wl.to_bf16_f32(wl.outlier_activations(256, 4096, 0))
    w = wl.to_bf16_f32(wl.normal_weights(256, 4096, 1))
    ea = wl.tensor_scale_exp(float(np.abs(a).max()))
    ew = wl.tensor_scale_exp(float(np.abs(w).max()))
    ac, as_ = oracle_mod.quantize(a, ea)
    wc, ws = oracle_mod.quantize(w, ew)
    ref = oracle_mod.gemm_sample_f64(ac, as_, ea, wc, ws, ew)
    scale = 2.0 ** (ea + ew)
    c16 = (decode_kernel_fp16(ac, as_) @ decode_kernel_fp16(wc, ws).T) * scale
    cbf = (decode_bf16(ac, as_) @ decode_bf16(wc, ws).T) * scale
    e16 = np.linalg.norm(c16 - ref) / np.linalg.norm(ref)
    ebf = np.linalg.norm(cbf - ref) / np.linalg.norm(ref)
    print(f"predicted rel. Frobenius error: fp16 operands {e16:.3e}, bf16 operands {ebf:.3e}")
    assert e16 < 5e-4
    assert ebf > 1e-3
