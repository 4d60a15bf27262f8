"""Exact-rational brute-force statement of IF3 and IF6 quantization, for
pinning the C oracle.  Written independently of oracle/: the grids come from
their bit layouts, every rounding is an argmin over all candidates with exact
Fractions (ties to the even code), and the two errors are exact sums of
squares in the original units.

Pages: "Adaptive Block-Scaled Data Types for FP4 Training" (podcast
companion), "It Generalizes: IF3 and IF6"; gist.science summary, section 2
("Extensoes"): the same per-group choice between a float and a pre-scaled
integer encoding, at 3 and 6 bits.  The grids are readings (the pages define
none): IF6 = FP6 E2M3 vs INT6 (magnitudes 0..31, top 31 -> 7.5); IF3 = FP3
E2M0 (0, 1, 2, 4) vs INT3 (0..3, top 3 -> 4).
"""
from fractions import Fraction as F
import math

from exact_if4 import E4M3, argmin_even


def e2m3():
    """FP6 E2M3 magnitudes by bit layout: 2 exponent bits (bias 1), 3 mantissa bits."""
    out = []
    for c in range(32):
        e, m = c >> 3, c & 7
        v = F(m, 8) if e == 0 else (1 + F(m, 8)) * F(2) ** (e - 1)
        out.append((c, v))
    return out


def e2m0():
    """FP3 E2M0 magnitudes by bit layout: 2 exponent bits (bias 1), no mantissa
    (exponent 0 is the subnormal zero)."""
    return [(c, F(0) if c == 0 else F(2) ** (c - 1)) for c in range(4)]


FORMATS = {
    6: dict(fp=e2m3(), qmax=31),
    3: dict(fp=e2m0(), qmax=3),
}


def top(bits):
    return FORMATS[bits]["fp"][-1][1]


def quantize_group(xs, bits, scale_exp=0):
    fmt = FORMATS[bits]
    T = top(bits)
    qmax = fmt["qmax"]
    if any(not math.isfinite(v) for v in xs):
        return dict(byte=0x7F, nonfinite=True)
    ax = [abs(F(v)) for v in xs]
    a = max(ax)
    code, sp = argmin_even(a * F(2) ** (-scale_exp) / T, E4M3)
    if code == 0:
        return dict(byte=0, zero=True)
    s = sp * F(2) ** scale_exp
    step = T / qmax  # INT value per unit of |q|
    fidx, fval, qmag = [], [], []
    for v in ax:
        c, cv = argmin_even(v / s, fmt["fp"])
        fidx.append(c)
        fval.append(cv)
        q, _ = argmin_even(v / (step * s), [(k, F(k)) for k in range(qmax + 1)])
        qmag.append(q)
    sse_fp = sum((v - cv * s) ** 2 for v, cv in zip(ax, fval))
    sse_int = sum((v - q * step * s) ** 2 for v, q in zip(ax, qmag))
    signs = [1 if math.copysign(1.0, v) < 0 else 0 for v in xs]
    return dict(code=code, s=s, fidx=fidx, qmag=qmag, signs=signs, sse_fp=sse_fp,
                sse_int=sse_int)


def unpack(field, bits):
    """16 codes from a group's little-endian bit field (bytes)."""
    acc = int.from_bytes(bytes(field), "little")
    return [(acc >> (bits * i)) & ((1 << bits) - 1) for i in range(16)]


def decode(code, byte, bits, scale_exp=0):
    """Exact value of one code under scale byte `byte`."""
    fmt = FORMATS[bits]
    sp = dict(E4M3)[byte & 0x7F]
    mag = code & ((1 << (bits - 1)) - 1)
    if byte & 0x80:
        v = mag * (top(bits) / fmt["qmax"]) * sp
    else:
        v = fmt["fp"][mag][1] * sp
    v *= F(2) ** scale_exp
    return -v if code >> (bits - 1) else v
