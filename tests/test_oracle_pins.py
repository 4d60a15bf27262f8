"""Pins of the CPU oracle against things other than itself: closed forms,
facts the pages state, exhaustive brute force with exact rationals,
hand-worked groups and invariants.  CPU only."""
from fractions import Fraction as F
import json
import math
import os
import struct

import numpy as np
import pytest

import exact_if4 as ex
from adaptive_block_scaled_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_groups.json")


def bf16_values_nonneg():
    """All finite non-negative bf16 values, as python floats."""
    out = []
    for hi in range(0, 0x7F80):
        out.append(struct.unpack("<f", struct.pack("<I", hi << 16))[0])
    return out


# --------------------------------------------------------------------------
# Grids


def test_e2m1_closed_form(oracle_mod):
    # FP4 E2M1 (sign, 2 exponent bits bias 1, 1 mantissa bit): the grid the
    # pages quantize to -- values 0, 0.5, 1, 1.5, 2, 3, 4, 6, top value 6.
    expect = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert [oracle_mod.e2m1_value(i) for i in range(8)] == expect
    for c, v in ex.E2M1:
        assert float(v) == expect[c]


def test_e4m3_table_matches_page_facts(oracle_mod):
    # E4M3 (fugumt page, "FP8 Formats for Deep Learning"): no infinities and a
    # single NaN mantissa pattern, so S.1111.111 is NaN and 0x7E = 448 the max.
    vals = [oracle_mod.e4m3_value(c) for c in range(128)]
    assert math.isnan(vals[0x7F])
    finite = vals[:0x7F]
    assert all(math.isfinite(v) for v in finite)
    assert max(finite) == 448.0 and vals[0x7E] == 448.0
    assert vals[0x01] == 2.0 ** -9 and vals[0x08] == 2.0 ** -6
    assert all(finite[i] < finite[i + 1] for i in range(126))
    for c, v in ex.E4M3:
        assert float(v) == finite[c]


# --------------------------------------------------------------------------
# Exhaustive brute force of the three roundings


def test_scale_code_all_bf16_amax(oracle_mod):
    """RNE(a/6) on E4M3 for every finite non-negative bf16 a: argmin over all
    127 finite magnitudes, ties to the even code, saturation at 448."""
    cands = [(c, v * 6) for c, v in ex.E4M3]  # compare a with 6*g exactly
    vals = bf16_values_nonneg()
    bad = []
    for a in vals:
        fa = F(a)
        best = None
        for c, v6 in cands:
            d = abs(fa - v6)
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                best = (d, c)
        if oracle_mod.scale_code(a) != best[1]:
            bad.append((a, best[1]))
    assert not bad, bad[:5]


def test_scale_code_fp32_near_ties(oracle_mod):
    """fp32 a exactly on 6*midpoint and one ulp either side."""
    grid = [float(v) for _, v in ex.E4M3]
    for k in range(126):
        mid = 3.0 * (grid[k] + grid[k + 1])  # 6 * midpoint, exact
        for a in (np.nextafter(np.float32(mid), np.float32(0)), np.float32(mid),
                  np.nextafter(np.float32(mid), np.float32(1e9))):
            a = float(a)
            code, _ = ex.argmin_even(F(a) / 6, ex.E4M3)
            assert oracle_mod.scale_code(a) == code, (k, a)


@pytest.mark.parametrize("scode", list(range(1, 127, 5)) + [0x7E, 0x38, 0x01, 0x07, 0x08])
def test_fp4_and_int4_codes_bruteforce(oracle_mod, scode):
    """For a scale s', every bf16 |x| in [2^-4 s', 9 s']: FP4 index =
    argmin over the 8 E2M1 magnitudes of |x - c s'|, INT4 = argmin over
    0..7 of |7x - 6 q s'|, ties to the even code."""
    s = ex.E4M3[scode][1]
    lo, hi = float(s) / 16.0, float(s) * 9.0
    xs = [v for v in bf16_values_nonneg() if lo <= v <= hi]
    ints = [(k, F(k)) for k in range(8)]
    for x in xs:
        fx = F(x)
        c, _ = ex.argmin_even(fx / s, ex.E2M1)
        q, _ = ex.argmin_even(F(7) * fx / (6 * s), ints)
        assert oracle_mod.fp4_index(x, float(s)) == c, (x, float(s))
        assert oracle_mod.int4_mag(x, float(s)) == q, (x, float(s))


# --------------------------------------------------------------------------
# Hand-worked groups


def _group(vals):
    x = np.zeros((1, 16), np.float32)
    x[0, :len(vals)] = vals
    return x


def test_hand_worked_groups(oracle_mod):
    with open(GOLDEN) as f:
        groups = json.load(f)["groups"]
    assert len(groups) >= 12
    for g in groups:
        codes, scales, ef, ei = oracle_mod.quantize(_group(g["x"]), 0, with_errors=True)
        assert scales[0, 0] == g["byte"], g["name"]
        assert list(codes[0]) == g["codes"], g["name"]
        assert float(ef[0, 0]) == g["err_fp"], g["name"]
        assert float(ei[0, 0]) == g["err_int"], g["name"]


# --------------------------------------------------------------------------
# Whole groups against the exact-rational statement


def _exact_group_check(oracle_mod, x, scale_exp=0):
    codes, scales, ef, ei = oracle_mod.quantize(x, scale_exp, with_errors=True)
    rows, cols = x.shape
    near_ties = 0
    for r in range(rows):
        for g in range(cols // 16):
            xs = [float(v) for v in x[r, 16 * g:16 * g + 16]]
            res = ex.quantize_group(xs, scale_exp)
            byte = int(scales[r, g])
            got = bytes(codes[r, 8 * g:8 * g + 8])
            if res.get("zero"):
                assert byte == 0 and got == bytes(8)
                continue
            assert byte & 0x7F == res["code"], (r, g)
            # fp32 error sums are 49 * SSE up to rounding
            for e32, sse in ((ef[r, g], res["sse_fp"]), (ei[r, g], res["sse_int"])):
                exact = float(49 * sse)
                assert abs(float(e32) - exact) <= 1e-5 * exact + 1e-300, (r, g)
            exact_int4 = res["sse_int"] < res["sse_fp"]
            got_int4 = bool(byte & 0x80)
            if exact_int4 != got_int4:
                # allowed only where the two exact errors agree to fp32 rounding
                d = abs(res["sse_int"] - res["sse_fp"]) / max(res["sse_int"], res["sse_fp"])
                assert d < F(1, 10 ** 5), (r, g, float(d))
                near_ties += 1
            assert got == ex.pack(ex.nibbles_for(res, got_int4)), (r, g)
    return near_ties


def test_exact_rational_random_groups(oracle_mod):
    rng = np.random.default_rng(123)
    blocks = [
        rng.standard_normal((8, 64), dtype=np.float32),
        rng.uniform(-1, 1, (8, 64)).astype(np.float32),
        wl.outlier_activations(8, 4096, 5)[:, :64],
        wl.rht_gradient(8, 64, 6),
        (rng.standard_t(4, (8, 64)) * 0.02).astype(np.float32),
    ]
    ties = 0
    for b in blocks:
        xb = wl.to_bf16_f32(b)
        ties += _exact_group_check(oracle_mod, xb, 0)
        e = wl.tensor_scale_exp(float(np.abs(xb).max()))
        ties += _exact_group_check(oracle_mod, xb, e)
    # fp32 near-ties between the two encodings are rare
    assert ties <= 2


def test_exact_rational_fp32_inputs(oracle_mod):
    c1 = wl.c1_mixed_fp32(0).values
    assert _exact_group_check(oracle_mod, c1[::16, :64].copy(), 0) <= 1
    assert _exact_group_check(oracle_mod, c1[1::16, 64:128].copy(), -9) <= 1


# --------------------------------------------------------------------------
# Invariants


def _rand_bf16(rows, cols, seed, kind="normal"):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        x = rng.standard_normal((rows, cols), dtype=np.float32)
    else:
        x = rng.uniform(-1, 1, (rows, cols)).astype(np.float32)
    return wl.to_bf16_f32(x)


def test_invariant_min_error_and_flag_only_in_sign_bit(oracle_mod):
    x = _rand_bf16(64, 256, 1)
    c0, s0, ef, ei = oracle_mod.quantize(x, 0, oracle_mod.ADAPTIVE, with_errors=True)
    c1, s1 = oracle_mod.quantize(x, 0, oracle_mod.FORCE_FP4)
    c2, s2 = oracle_mod.quantize(x, 0, oracle_mod.FORCE_INT4)
    # I3: bits 6..0 depend only on the amax; forced modes set the flag
    assert np.array_equal(s0 & 0x7F, s1 & 0x7F) and np.array_equal(s0 & 0x7F, s2 & 0x7F)
    assert not (s1 & 0x80).any() and ((s2 & 0x80) | (s2 == 0)).all()
    # I1: the kept encoding has the lower error; ties keep FP4
    use_int = (s0 & 0x80) != 0
    assert np.array_equal(use_int, ei < ef)
    # the kept codes are those of the forced mode that matches the flag
    gsel = np.repeat(use_int, 8, axis=1)
    assert np.array_equal(c0, np.where(gsel, c2, c1))
    # IF4 mixes formats on Gaussian data
    assert 0.2 < use_int.mean() < 0.9


def test_invariant_zero_and_nonfinite_groups(oracle_mod):
    x = np.zeros((2, 48), np.float32)
    x[1, 16] = np.inf
    x[1, 40] = np.nan
    x[0, 20] = -0.0
    codes, scales = oracle_mod.quantize(x)
    assert list(scales[0]) == [0, 0, 0] and not codes[0].any()
    assert list(scales[1]) == [0, 0x7F, 0x7F] and not codes[1].any()
    y = oracle_mod.dequantize(codes, scales)
    assert np.isnan(y[1, 16:48]).all() and (y[:, :16] == 0).all()


def test_invariant_sign_symmetry(oracle_mod):
    x = _rand_bf16(32, 128, 2)
    c, s = oracle_mod.quantize(x)
    cn, sn = oracle_mod.quantize(-x)
    assert np.array_equal(s, sn)
    nz = np.repeat(s != 0, 8, axis=1)
    assert np.array_equal(np.where(nz, c ^ 0x88, c), cn)


def test_invariant_exponent_shift(oracle_mod):
    # I5: quantize(x, E) == quantize(x * 2^-E, 0)
    x = _rand_bf16(32, 128, 3, "uniform")
    for e in (-20, -9, -1, 3, 17):
        a = oracle_mod.quantize(x, e)
        b = oracle_mod.quantize(np.ldexp(x, -e).astype(np.float32), 0)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_invariant_size_and_bound(oracle_mod):
    x = _rand_bf16(16, 256, 4)
    codes, scales = oracle_mod.quantize(x)
    # I6: 4.5 bits per value, the same storage as NVFP4
    assert (codes.nbytes + scales.nbytes) * 8 / x.size == 4.5
    # I7: |dequantized| <= 6 s' for every group
    y = oracle_mod.dequantize(codes, scales)
    sp = np.array([oracle_mod.e4m3_value(int(b) & 0x7F) for b in scales.ravel()]).reshape(scales.shape)
    bound = np.repeat(6 * sp, 16, axis=1)
    assert (np.abs(y) <= bound).all()


def test_invariant_fp4_grid_inputs_stay_fp4(oracle_mod):
    # I9: inputs on the FP4 grid with group max 6 s have zero FP4 error
    rng = np.random.default_rng(5)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float32)
    x = grid[rng.integers(0, 8, (32, 64))] * np.where(rng.random((32, 64)) < 0.5, -1, 1)
    x[:, ::16] = 6.0
    x = (x * np.float32(0.25)).astype(np.float32)
    codes, scales, ef, ei = oracle_mod.quantize(x, 0, with_errors=True)
    assert (ef == 0).all() and not (scales & 0x80).any()
    assert np.array_equal(oracle_mod.dequantize(codes, scales), x)


def test_invariant_requantization(oracle_mod):
    """I8: with normal unsaturated scales and each group's largest code
    reaching the top of its grid, dequantize -> quantize gives back the same
    decoded values; the flag may only differ where both errors are equal."""
    x = _rand_bf16(64, 256, 6)
    codes, scales = oracle_mod.quantize(x)
    y = oracle_mod.dequantize(codes, scales)
    c2, s2, ef, ei = oracle_mod.quantize(y, 0, with_errors=True)
    y2 = oracle_mod.dequantize(c2, s2)
    sc = scales & 0x7F
    ok = (sc >= 0x08) & (sc < 0x7E)
    mags = np.stack([codes & 7, codes >> 4 & 7], -1).reshape(codes.shape[0], -1, 16).max(-1)
    ok &= mags == 7
    okx = np.repeat(ok, 16, axis=1)
    assert ok.mean() > 0.9
    assert np.array_equal(np.where(okx, y2, 0), np.where(okx, y, 0))
    flip = ((scales ^ s2) & 0x80) != 0
    assert (ef[flip & ok] == ei[flip & ok]).all()


def test_results_independent_of_thread_count(oracle_mod):
    x = _rand_bf16(128, 512, 7)
    a = oracle_mod.quantize(x, 0, nthreads=1)
    b = oracle_mod.quantize(x, 0, nthreads=5)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# --------------------------------------------------------------------------
# Dequantize and decode


def test_dequantize_all_codes_exact(oracle_mod):
    """Every (flag, scale, nibble): FP4 decodes to +-c s' exactly, INT4 to the
    fp32 nearest (ties even) to 6 |q| s'/7 ([gist] 'Metodo 6/7': INT4 values
    are descaled by 6/7)."""
    rows = []
    for flag in (0, 1):
        for sc in range(1, 127):
            rows.append((flag << 7) | sc)
    scales = np.array(rows, np.uint8).reshape(-1, 1)
    nib = np.arange(16, dtype=np.uint8)
    codes = np.tile((nib[0::2] | (nib[1::2] << 4)).reshape(1, 8), (len(rows), 1))
    y = oracle_mod.dequantize(codes, scales)
    y64 = oracle_mod.decode_f64(codes, scales)
    for i, b in enumerate(rows):
        sp = ex.E4M3[b & 0x7F][1]
        for n in range(16):
            mag, neg = n & 7, n >> 3
            if b & 0x80:
                exact = F(6 * mag, 7) * sp
            else:
                exact = ex.E2M1[mag][1] * sp
            v = float(y[i, n])
            assert math.copysign(1.0, v) == (-1.0 if neg else 1.0)
            v = abs(v)
            # nearest fp32 to exact, no ties possible (6 q s'/7 is exact or
            # has a repeating binary expansion)
            lo = float(np.nextafter(np.float32(v), np.float32(0)))
            hi = float(np.nextafter(np.float32(v), np.float32(np.inf)))
            assert abs(F(v) - exact) < abs(F(lo) - exact) or exact == 0
            assert abs(F(v) - exact) < abs(F(hi) - exact)
            assert abs(F(abs(float(y64[i, n]))) - exact) <= exact * F(1, 2 ** 52)


def test_bf16_rounding_matches_torch(oracle_mod):
    import torch
    rng = np.random.default_rng(8)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1e-40, 3.4e38, np.inf, -np.inf], np.float32)])
    ours = oracle_mod.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(wl.to_bf16_f32(x).view(np.uint32) >> 16, ref.astype(np.uint32))


# --------------------------------------------------------------------------
# GEMM oracle


def test_gemm_sample_matches_numpy_fp64(oracle_mod):
    a = _rand_bf16(24, 256, 9)
    w = wl.to_bf16_f32(wl.normal_weights(40, 256, 10))
    ea = wl.tensor_scale_exp(float(np.abs(a).max()))
    ew = wl.tensor_scale_exp(float(np.abs(w).max()))
    ac, as_ = oracle_mod.quantize(a, ea)
    wc, ws = oracle_mod.quantize(w, ew)
    ad = oracle_mod.decode_f64(ac, as_, ea)
    wd = oracle_mod.decode_f64(wc, ws, ew)
    ref = ad @ wd.T  # library routine, different summation
    rows, cols = [0, 5, 23], [1, 2, 39, 17]
    c = oracle_mod.gemm_sample_f64(ac, as_, ea, wc, ws, ew, rows, cols)
    assert np.allclose(c, ref[np.ix_(rows, cols)], rtol=1e-12, atol=1e-12)
    full = oracle_mod.gemm_sample_f64(ac, as_, ea, wc, ws, ew)
    assert np.allclose(full, ref, rtol=1e-12, atol=1e-12)


def test_gemm_exact_small_k(oracle_mod):
    """K = 16 and 32 with power-of-two scales and FP4-only groups: every
    product and sum is a small dyadic number, so fp64 is exact; compare
    with exact integer arithmetic."""
    rng = np.random.default_rng(11)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float32)
    for k in (16, 32):
        a = grid[rng.integers(0, 8, (8, k))] * np.where(rng.random((8, k)) < .5, -1, 1)
        w = grid[rng.integers(0, 8, (6, k))] * np.where(rng.random((6, k)) < .5, -1, 1)
        a[:, ::16] = 6
        w[:, ::16] = -6
        a = a.astype(np.float32)
        w = w.astype(np.float32)
        ac, as_ = oracle_mod.quantize(a)
        wc, ws = oracle_mod.quantize(w)
        c = oracle_mod.gemm_sample_f64(ac, as_, 0, wc, ws, 0)
        exact = [[sum(F(float(a[i, t])) * F(float(w[j, t])) for t in range(k))
                  for j in range(6)] for i in range(8)]
        assert all(F(float(c[i, j])) == exact[i][j] for i in range(8) for j in range(6))
