"""Where the fp32 selection rule and exact arithmetic choose differently.

The encoding of each group is chosen by comparing two fp32 error sums (the
oracle's rule, fixed in its order).  This script recomputes both sums of
squared errors EXACTLY for every group of a tensor and counts the groups
whose flag would differ under exact arithmetic ("Adaptive Block-Scaled Data
Types", gist.science summary, section 2 "Mecanismo de Selecao": compute each
encoding's MSE, keep the lower).  It is informational: the fp32 rule is the
contract, and a flip is only possible where the two errors agree to fp32
rounding.

How the exact comparison is made: the codes come from the oracle run in its
forced modes (the FP4 index and the INT4 magnitude of every element do not
depend on the error arithmetic), the grid values from the oracle's own E2M1
and E4M3 tables.  In the x7 domain every difference 7|x| - 7 c s and
7|x| - 6 |q| s is exact in fp64 (a 24-bit x and a 9-bit product, exponents
at most a few binades apart wherever the code is non-zero; checked: no
group's amax exceeds 8 s).  Their squares
and the 16-term sums are rounded in fp64, so each sum is within 20 * 2^-53
of its exact value (relative); a group whose two sums are further apart than
that is decided by the fp64 comparison, and any closer pair is settled with
exact rationals.

Run: python tests/flag_flips.py   (all workloads, full tensors)
"""
from fractions import Fraction
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402

REL_BOUND = 20 * 2.0 ** -53


def _nibbles(codes):
    """[rows, cols/2] bytes -> [rows, cols] nibbles, element 2j = low nibble."""
    n = np.empty((codes.shape[0], codes.shape[1] * 2), np.uint8)
    n[:, 0::2] = codes & 0xF
    n[:, 1::2] = codes >> 4
    return n


def _tables():
    e2m1 = np.array([oracle.e2m1_value(i) for i in range(8)], np.float64)
    e4m3 = np.array([oracle.e4m3_value(c) for c in range(127)] + [np.nan], np.float64)
    return e2m1, e4m3


def exact_choice(x, scale_exp, nthreads=0):
    """x: fp32 [rows, cols].  Returns (live, exact_int4, got_int4, near):
    per group, whether it has a finite non-zero scale, whether INT4 has the
    strictly lower exact squared error, whether the oracle's fp32 rule chose
    INT4, and whether the pair was close enough to need exact rationals."""
    x = np.ascontiguousarray(x, np.float32)
    e2m1, e4m3 = _tables()
    cf, sf = oracle.quantize(x, scale_exp, oracle.FORCE_FP4, nthreads=nthreads)
    ci, _ = oracle.quantize(x, scale_exp, oracle.FORCE_INT4, nthreads=nthreads)
    _, sa = oracle.quantize(x, scale_exp, oracle.ADAPTIVE, nthreads=nthreads)
    rows, cols = x.shape
    g = cols // 16
    live = ((sf & 0x7F) != 0) & ((sf & 0x7F) != 0x7F)  # zero and non-finite groups excluded
    s = e4m3[sf & 0x7F] * 2.0 ** scale_exp                         # [rows, g]
    ax = np.abs(x.astype(np.float64)).reshape(rows, g, 16)
    c = e2m1[_nibbles(cf) & 7].reshape(rows, g, 16)
    q = (_nibbles(ci) & 7).astype(np.float64).reshape(rows, g, 16)
    # the exactness argument needs |x| within a few binades of s wherever a
    # code is non-zero: true unless the scale saturates far below the amax
    assert np.all(ax.max(axis=2)[live] <= 8.0 * s[live])
    s3 = s[:, :, None]
    df = 7.0 * ax - 7.0 * c * s3
    di = 7.0 * ax - 6.0 * q * s3
    sse_f = (df * df).sum(axis=2)
    sse_i = (di * di).sum(axis=2)
    with np.errstate(invalid="ignore"):
        exact_int4 = sse_i < sse_f
        near = live & (np.abs(sse_f - sse_i) <= REL_BOUND * np.maximum(sse_f, sse_i))
    for r, k in zip(*np.nonzero(near)):
        xs = [Fraction(float(v)) for v in x[r, 16 * k:16 * k + 16]]
        sk = Fraction(float(s[r, k]))
        ef = sum((7 * abs(v) - 7 * Fraction(float(cv)) * sk) ** 2
                 for v, cv in zip(xs, c[r, k]))
        ei = sum((7 * abs(v) - 6 * int(qv) * sk) ** 2 for v, qv in zip(xs, q[r, k]))
        exact_int4[r, k] = ei < ef
    return live, exact_int4, (sa & 0x80) != 0, near


def count_flips(x, scale_exp, nthreads=0):
    """Returns (groups compared, flips, near ties settled exactly)."""
    live, exact_int4, got_int4, near = exact_choice(x, scale_exp, nthreads)
    flips = int(np.count_nonzero(live & (got_int4 != exact_int4)))
    return int(np.count_nonzero(live)), flips, int(np.count_nonzero(near))


def count_flips_chunked(x, scale_exp, rows_per_chunk=2048):
    tot = [0, 0, 0]
    for r0 in range(0, x.shape[0], rows_per_chunk):
        res = count_flips(x[r0:r0 + rows_per_chunk], scale_exp)
        tot = [a + b for a, b in zip(tot, res)]
    return tuple(tot)


def main():
    from adaptive_block_scaled_amd import workloads as wl
    cases = []
    c1 = wl.c1_mixed_fp32(0)
    cases += [("C1 fp32 256x256", c1.values, 0), ("C1 fp32 256x256", c1.values, c1.scale_exp)]
    c2 = wl.c2_activations()
    cases.append(("C2 activations 8192x4096", c2.values, c2.scale_exp))
    del c2
    c3 = wl.c3_rht_gradient()
    cases += [("C3 gradient 16384x4096", c3.values, c3.scale_exp),
              ("C3 gradient 16384x4096", c3.values, 0)]
    del c3
    a4, w4 = wl.c4_gemm()
    cases += [("C4 A 4096x4096", a4.values, a4.scale_exp),
              ("C4 W 4096x4096", w4.values, w4.scale_exp)]
    print("| Tensor | E | groups compared | flips | near ties settled exactly |")
    print("|---|---|---|---|---|")
    for name, v, e in cases:
        n, f, t = count_flips_chunked(v, e)
        print(f"| {name} | {e} | {n} | {f} | {t} |", flush=True)
    del cases, a4, w4
    a5, w5 = wl.c5_ffn()
    for name, t in (("C5 A 8192x8192", a5), ("C5 W 28672x8192", w5)):
        e = t.scale_exp
        n, f, nt = count_flips_chunked(t.values, e)
        print(f"| {name} | {e} | {n} | {f} | {nt} |", flush=True)


if __name__ == "__main__":
    main()
