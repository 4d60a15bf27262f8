"""Host check of the bound behind the quantize kernels' INT clamp elision
(adaptive_block_scaled_amd/csrc/quantize.hip: fast_group; csrc/ifn.hip:
fast_group_bf16).

A wave skips the per-element clamp |q| <= qmax when none of its groups has a
subnormal E4M3 scale (codes 1-7) or, for IF4, an fp32 quotient
q6 = fl(fl(a 2^-E) fl(1/6)) of 448 or more (IF3: the 448 code).  The claim is
that for every other group the largest element's INT quotient stays below
qmax + 1/2, so that rounding it can never exceed qmax: 7 a'/(6 s') < 7.5 for
IF4 and 3 a'/(4 s') < 3.5 for IF3, with a' = a 2^-E and s' the scale the
oracle picks.  This test checks that with exact rationals for every finite
positive bf16 absmax at several exponents, and that the excluded cases are
needed: a subnormal scale and a saturated one each give a quotient of 7.5
(3.5) or more somewhere.  The kernels round an approximation of the quotient
snapped to a 2^-18 (IF3: 2^-19) grid, within 2^-20 of the exact value; the
largest exact quotient found, 7.4375 (3.1875), leaves 1/16 to the rounding
boundary.
"""
from fractions import Fraction as F

import numpy as np
import pytest

EXPS = [0, -3, -18, 9, 20]


def _bf16_positive_finite():
    bits = np.arange(1, 0x7F80, dtype=np.uint32) << 16
    return bits.view(np.float32)


@pytest.mark.parametrize("E", EXPS)
def test_if4_int_quotient_below_clamp_without_subnormal_or_saturated_scale(oracle_mod, E):
    amax = _bf16_positive_finite()
    with np.errstate(over="ignore"):
        # exact scaling by a power of two, or infinite where a 2^-E leaves the
        # fp32 range: the kernel's quotient q6 is then infinite too, which
        # takes the clamped loop
        ap = (amax.astype(np.float64) * 2.0 ** -E).astype(np.float32)
        q6 = ap * np.float32(1.0 / 6.0)  # the kernel's fp32 quotient
    worst, checked, need = F(0), 0, [False, False]
    for a_s, q in zip(ap.tolist(), q6.tolist()):
        if a_s == float("inf"):
            continue
        code = oracle_mod.scale_code(a_s)
        if code == 0 or a_s == 0.0:
            continue
        s = F(oracle_mod.e4m3_value(code))
        ratio = 7 * F(a_s) / (6 * s)
        if 1 <= code <= 7 or q >= 448.0:
            if ratio >= F(15, 2):
                need[0 if code <= 7 else 1] = True
            continue
        checked += 1
        worst = max(worst, ratio)
        assert ratio < F(15, 2), (a_s, code, ratio)
    print(f"E={E}: {checked} groups, largest 7a'/(6s') = {float(worst):.6f}")
    assert worst <= F(119, 16)  # 7 * 1.0625
    if E == 0:
        assert need[0] and need[1], need  # both exclusions are needed somewhere


@pytest.mark.parametrize("E", EXPS)
def test_if3_int_quotient_below_clamp_without_subnormal_or_top_scale(oracle_mod, E):
    amax = _bf16_positive_finite()
    with np.errstate(over="ignore"):
        ap = (amax.astype(np.float64) * 2.0 ** -E).astype(np.float32)
    worst, checked, need = F(0), 0, [False, False]
    for a_s in ap.tolist():
        if a_s == float("inf"):  # the kernel's scale is then the 448 code
            continue
        code = oracle_mod.ifn_scale_code(3, a_s)
        if code == 0 or a_s == 0.0:
            continue
        s = F(oracle_mod.e4m3_value(code))
        ratio = 3 * F(a_s) / (4 * s)
        if 1 <= code <= 7 or code >= 126:
            if ratio >= F(7, 2):
                need[0 if code <= 7 else 1] = True
            continue
        checked += 1
        worst = max(worst, ratio)
        assert ratio < F(7, 2), (a_s, code, ratio)
    print(f"E={E}: {checked} groups, largest 3a'/(4s') = {float(worst):.6f}")
    assert worst <= F(51, 16)  # 3 * 1.0625
    if E == 0:
        assert need[0] and need[1], need
