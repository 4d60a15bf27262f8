"""Exact-rational brute-force statement of IF4 quantization, for pinning the
C oracle.  Written independently of oracle/: every rounding is an argmin over
all candidates with exact Fractions (ties to the even code), and the two
errors are exact sums of squares in the original units.

Pages: "Adaptive Block-Scaled Data Types" (gist.science summary), section 2
"Metodologia" -- quantize each group of 16 both as FP4 (E2M1) and as INT4
pre-scaled by 7/6 (descaled by 6/7), compute each encoding's MSE, keep the
lower, flag the choice in the E4M3 scale's sign bit (0 = FP4, 1 = INT4).
"""
from fractions import Fraction as F
import math
import struct


def f32_fraction(v: float) -> F:
    """Exact value of a float (python float holds any fp32 exactly)."""
    return F(v)


def e4m3_candidates():
    """(code, value) for the 127 finite non-negative E4M3 codes, from the bit
    layout (4 exponent bits, bias 7, 3 mantissa bits, subnormals)."""
    out = []
    for code in range(127):
        e, m = code >> 3, code & 7
        if e == 0:
            v = F(m, 8) * F(2) ** (1 - 7)
        else:
            v = (1 + F(m, 8)) * F(2) ** (e - 7)
        out.append((code, v))
    return out


E4M3 = e4m3_candidates()
# E2M1 by its bit layout: e = code >> 1, m = code & 1, bias 1.
E2M1 = [(c, (F(c & 1, 2) if (c >> 1) == 0 else (1 + F(c & 1, 2)) * F(2) ** ((c >> 1) - 1)))
        for c in range(8)]


def argmin_even(target: F, cands):
    """cands: list of (code, value).  Nearest value to target, ties -> even code."""
    best = None
    for code, v in cands:
        d = abs(target - v)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0 and best[1] % 2 == 1):
            best = (d, code, v)
    return best[1], best[2]


def quantize_group(xs, scale_exp=0):
    """xs: 16 python floats (fp32/bf16 values).  Returns dict with the scale
    code, flag, nibbles and exact SSE of each encoding."""
    assert len(xs) == 16
    if any(not math.isfinite(v) for v in xs):
        return dict(byte=0x7F, nibbles=[0] * 16, sse_fp=F(0), sse_int=F(0), nonfinite=True)
    ax = [abs(f32_fraction(v)) for v in xs]
    a = max(ax)
    code, sp = argmin_even(a * F(2) ** (-scale_exp) / 6, E4M3)
    if code == 0:
        return dict(byte=0, nibbles=[0] * 16, sse_fp=F(0), sse_int=F(0), zero=True)
    s = sp * F(2) ** scale_exp
    fidx, fval, qmag = [], [], []
    for v in ax:
        c, cv = argmin_even(v / s, E2M1)
        fidx.append(c)
        fval.append(cv)
        q, _ = argmin_even(F(7) * v / (6 * s), [(k, F(k)) for k in range(8)])
        qmag.append(q)
    sse_fp = sum((v - cv * s) ** 2 for v, cv in zip(ax, fval))
    sse_int = sum((v - F(6, 7) * q * s) ** 2 for v, q in zip(ax, qmag))
    signs = [1 if math.copysign(1.0, v) < 0 else 0 for v in xs]
    return dict(code=code, s=s, fidx=fidx, qmag=qmag, signs=signs, sse_fp=sse_fp,
                sse_int=sse_int)


def nibbles_for(res, use_int4):
    mags = res["qmag"] if use_int4 else res["fidx"]
    return [(sg << 3) | m for sg, m in zip(res["signs"], mags)]


def pack(nibbles):
    return bytes((nibbles[2 * j] | (nibbles[2 * j + 1] << 4)) for j in range(len(nibbles) // 2))


def bf16_round(v: float) -> float:
    """Round-to-nearest-even of a python float to bf16, via fp32 bits."""
    u = struct.unpack("<I", struct.pack("<f", v))[0]
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return struct.unpack("<f", struct.pack("<I", u))[0]
