"""Pins of the oracle's IF3 / IF6 against things other than the oracle: the
grids from their bit layouts and the OCP FP6 E2M3 facts (top 7.5, smallest
step 1/8), exhaustive brute force of every rounding in exact rationals, an
independent exact-rational statement of whole groups (tests/exact_ifn.py),
and invariants.  CPU only."""
from fractions import Fraction as F
import math
import struct

import numpy as np
import pytest

import exact_ifn as ex


def bf16_nonneg():
    return [struct.unpack("<f", struct.pack("<I", h << 16))[0] for h in range(0, 0x7F80)]


@pytest.mark.parametrize("bits", [3, 6])
def test_float_grid_closed_form(oracle_mod, bits):
    grid = [oracle_mod.ifn_fp_value(bits, i) for i in range(1 << (bits - 1))]
    assert grid == [float(v) for _, v in ex.FORMATS[bits]["fp"]]
    assert grid == sorted(grid) and len(set(grid)) == len(grid)
    if bits == 6:
        # OCP microscaling FP6 E2M3: largest normal 7.5, subnormal step 0.125
        assert grid[-1] == 7.5 and grid[1] == 0.125 and grid[8] == 1.0
    else:
        assert grid == [0.0, 1.0, 2.0, 4.0]


@pytest.mark.parametrize("bits", [3, 6])
def test_scale_code_every_bf16_amax(oracle_mod, bits):
    T = ex.top(bits)
    vals = bf16_nonneg()[::7]  # a seventh of all finite bf16 magnitudes, every binade
    for v in vals:
        want, _ = ex.argmin_even(F(v) / T, ex.E4M3)
        assert oracle_mod.ifn_scale_code(bits, v) == want, (bits, v)


@pytest.mark.parametrize("bits", [3, 6])
@pytest.mark.parametrize("scode", [1, 7, 8, 0x23, 0x38, 0x3E, 0x55, 0x7E])
def test_codes_bruteforce(oracle_mod, bits, scode):
    fmt = ex.FORMATS[bits]
    s = dict(ex.E4M3)[scode]
    T = ex.top(bits)
    ints = [(k, F(k)) for k in range(fmt["qmax"] + 1)]
    # every bf16 |x| from s/64 to 1.2 T s, plus the fp32 values at and next to
    # the midpoints of both grids (the float midpoints are exact in fp32; the
    # INT ones, multiples of T/qmax = 4/3 or 15/62, are not, so those are
    # near-ties)
    lo, hi = float(s) / 64, float(1.2 * T * s)
    xs = [v for v in bf16_nonneg() if lo <= v <= hi]
    fpv = [v for _, v in fmt["fp"]]
    mids = [(fpv[k] + fpv[k + 1]) / 2 * s for k in range(len(fpv) - 1)]
    mids += [(k + F(1, 2)) * T / fmt["qmax"] * s for k in range(fmt["qmax"])]
    for m in mids:
        m32 = np.float32(float(m))
        xs += [float(m32), float(np.nextafter(m32, np.float32(0))),
               float(np.nextafter(m32, np.float32(np.inf)))]
    for x in xs:
        fx = F(x)
        want_f, _ = ex.argmin_even(fx / s, fmt["fp"])
        want_q, _ = ex.argmin_even(fx / (T / fmt["qmax"] * s), ints)
        assert oracle_mod.ifn_fp_index(bits, x, float(s)) == want_f, (bits, scode, x)
        assert oracle_mod.ifn_int_mag(bits, x, float(s)) == want_q, (bits, scode, x)


def _groups(n, seed, kind):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        x = rng.standard_normal((n, 16))
    elif kind == "uniform":
        x = rng.uniform(-1, 1, (n, 16))
    else:
        x = rng.standard_t(4, (n, 16)) * 0.02
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).view(np.float32)  # bf16 values


@pytest.mark.parametrize("bits", [3, 6])
@pytest.mark.parametrize("kind", ["normal", "uniform", "t4"])
def test_whole_groups_against_exact_statement(oracle_mod, bits, kind):
    x = _groups(300, bits * 10 + len(kind), kind)
    e = -8 if kind == "t4" else 0
    codes, scales, ef, ei = oracle_mod.quantize_ifn(x.reshape(1, -1), bits, e, with_errors=True)
    cb = 2 * bits
    mismatched_choice = 0
    for g in range(x.shape[0]):
        r = ex.quantize_group([float(v) for v in x[g]], bits, e)
        byte = int(scales[0, g])
        assert (byte & 0x7F) == r["code"]
        got = ex.unpack(codes[0, g * cb:(g + 1) * cb], bits)
        use_int = bool(byte & 0x80)
        mags = r["qmag"] if use_int else r["fidx"]
        want = [(sg << (bits - 1)) | m for sg, m in zip(r["signs"], mags)]
        assert got == want, (g, got, want)
        # the fp32 errors are the exact SSE scaled into the oracle's domain,
        # up to their rounding; the choice agrees with exact arithmetic except
        # at near-ties
        exact_int = r["sse_int"] < r["sse_fp"]
        if exact_int != use_int:
            mismatched_choice += 1
            assert abs(r["sse_int"] - r["sse_fp"]) <= F(1, 10**5) * max(r["sse_int"], r["sse_fp"])
    assert mismatched_choice <= 2


@pytest.mark.parametrize("bits", [3, 6])
def test_dequantize_every_code_exact(oracle_mod, bits):
    # one group per (flag, scale code) with every magnitude of both signs spread over rows
    rows = []
    nm = 1 << (bits - 1)
    for flag in (0, 1):
        for sc in (1, 5, 8, 0x2B, 0x38, 0x51, 0x7E):
            for start in range(0, 2 * nm, 16):
                cs = [(start + i) % (2 * nm) for i in range(16)]
                field = sum(c << (bits * i) for i, c in enumerate(cs)).to_bytes(2 * bits, "little")
                rows.append((list(field), sc | (flag << 7), cs))
    codes = np.array([r[0] for r in rows], np.uint8)
    scales = np.array([[r[1]] for r in rows], np.uint8)
    for e in (0, -20, 9):
        y = oracle_mod.dequantize_ifn(codes, scales, bits, e)
        for i, (_, byte, cs) in enumerate(rows):
            for j, c in enumerate(cs):
                want = ex.decode(c, byte, bits, e)
                w32 = float(np.float32(float(want)))  # the fp32 nearest the exact value
                # exact ties between fp32 neighbours do not occur (at most 13-bit numerators)
                assert y[i, j] == w32 or (want == 0 and y[i, j] == 0), (bits, byte, c, e)
                if want == 0:
                    assert math.copysign(1, y[i, j]) == (-1 if c >> (bits - 1) else 1)


@pytest.mark.parametrize("bits", [3, 6])
def test_invariants(oracle_mod, bits):
    x = _groups(400, 77 + bits, "normal").reshape(20, -1)
    c0, s0, ef, ei = oracle_mod.quantize_ifn(x, bits, 0, with_errors=True)
    # kept error is the minimum of the two; the flag is bit 7 only
    use_int = (s0 & 0x80) != 0
    assert np.all(np.where(use_int, ei, ef) == np.minimum(ef, ei))
    for mode in (1, 2):
        _, sm = oracle_mod.quantize_ifn(x, bits, 0, mode)
        assert np.array_equal(sm & 0x7F, s0 & 0x7F)
        assert np.all((sm >> 7) == (1 if mode == 2 else 0))
    # sign symmetry: negating x flips exactly the sign bit of every code
    c1, s1 = oracle_mod.quantize_ifn(-x, bits, 0)
    assert np.array_equal(s1, s0)
    y0 = oracle_mod.dequantize_ifn(c0, s0, bits)
    y1 = oracle_mod.dequantize_ifn(c1, s1, bits)
    assert np.array_equal(y0, -y1)
    # exponent shift: quantize(x, E) == quantize(x 2^-E, 0)
    c2, s2 = oracle_mod.quantize_ifn(x * np.float32(2.0 ** 12), bits, 12)
    assert np.array_equal(c2, c0) and np.array_equal(s2, s0)
    # zero group, non-finite group
    z = np.zeros((1, 32), np.float32)
    z[0, 20] = np.nan
    cz, sz = oracle_mod.quantize_ifn(z, bits, 0)
    assert list(sz[0]) == [0, 0x7F] and not cz.any()
    # storage: bits per value plus one byte per 16
    assert c0.shape[1] * 8 == x.shape[1] * bits
    # requantization: for groups with a normal, unsaturated scale whose
    # largest code is the top of its grid (so the decoded amax is top * s'
    # and gives back the same scale), dequantize -> quantize reproduces the
    # decoded values; the flag may only flip where both errors are equal
    c3, s3, ef3, ei3 = oracle_mod.quantize_ifn(y0, bits, 0, with_errors=True)
    y3 = oracle_mod.dequantize_ifn(c3, s3, bits)
    cb, nm = 2 * bits, (1 << (bits - 1)) - 1
    checked = 0
    for r in range(x.shape[0]):
        for g in range(x.shape[1] // 16):
            sc, flag = int(s0[r, g]) & 0x7F, int(s0[r, g]) >> 7
            top_mag = ex.FORMATS[bits]["qmax"] if flag else len(ex.FORMATS[bits]["fp"]) - 1
            mags = [c & nm for c in ex.unpack(c0[r, g * cb:(g + 1) * cb], bits)]
            if not (0x08 <= sc < 0x7E and max(mags) == top_mag):
                continue
            checked += 1
            assert np.array_equal(y3[r, 16 * g:16 * (g + 1)], y0[r, 16 * g:16 * (g + 1)]), (r, g)
            if (int(s3[r, g]) ^ int(s0[r, g])) & 0x80:
                assert ef3[r, g] == ei3[r, g]
    assert checked > 0.5 * x.size / 16


def test_if6_error_below_if3(oracle_mod):
    x = _groups(512, 5, "normal").reshape(32, -1)
    mse = {}
    for bits in (3, 6):
        c, s = oracle_mod.quantize_ifn(x, bits, 0)
        mse[bits] = float(np.mean((oracle_mod.dequantize_ifn(c, s, bits) - x) ** 2))
    assert mse[6] < mse[3] / 20
