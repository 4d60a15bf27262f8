"""Host checks of constructions in the IF3 and IF6 bf16 fast paths
(adaptive_block_scaled_amd/csrc/ifn.hip: fast_group_bf16, if6_pair_bf16), run
on the CPU.

* The float index: the kernel moves each midpoint of the FP3 E2M0 grid
  {0, 1, 2, 4} by less than the distance of the nearest non-tie quotient, and
  reads the index from one fp32 exponent.  tests/if3_index_host.c models the
  kernel's fp32 steps with the host's correctly rounded fma / frexp / ldexp
  and compares them with the oracle's IF3 rounding for every bf16 |x|, every
  E4M3 scale and several exponents, with the reciprocal moved by up to two
  ulp.  A margin constant that is too small or too large, or a missing cap on
  overflowing products, must make it fail.
* The packing: the magnitudes go into the 48-bit field with the INT ones as
  whole magic-number floats (the constant part subtracted once per word), and
  the sign bits come from the bf16 words through v_perm sign-fill selectors.
  IF6 packs its INT magnitudes the same way into 96-bit fields.
  The constants are read from the kernel source and checked against the field
  layout (element i at bits 3i .. 3i+2, sign at 3i + 2) on random words.

The GPU tests (tests/test_gpu_ifn.py) sweep the kernel itself over every
(bf16 x, E4M3 s') pair; these tests pin the derivation independently of it.
"""
import os
import random
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "adaptive_block_scaled_amd", "csrc", "ifn.hip")


@pytest.fixture(scope="module")
def index_check():
    out_dir = os.path.join(ROOT, "tests", "_build")
    os.makedirs(out_dir, exist_ok=True)
    exe = os.path.join(out_dir, "if3_index_host")
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off",
                    "-I", os.path.join(ROOT, "oracle"), "-o", exe,
                    os.path.join(ROOT, "tests", "if3_index_host.c"),
                    os.path.join(ROOT, "oracle", "if4_oracle.c"), "-lm"], check=True)

    def run(*args):
        p = subprocess.run([exe, *map(str, args)], capture_output=True, text=True, timeout=600)
        m = re.search(r"checked (\d+) mismatches (\d+)", p.stdout)
        assert m, p.stdout + p.stderr
        return int(m.group(1)), int(m.group(2))
    return run


def test_if3_binade_index_matches_oracle(index_check):
    checked, bad = index_check()
    assert checked == 185068800
    assert bad == 0


@pytest.mark.parametrize("margin", ["0", "0x1p-13"])
def test_if3_index_check_rejects_wrong_margin(index_check, margin):
    # ties at 1.5 (margin 0) or at 3 (margin too large) go to the wrong side
    _, bad = index_check(margin, 1, 2)
    assert bad > 0


def test_if3_index_check_rejects_missing_cap(index_check):
    # at extreme exponents |x| * ra overflows; frexp of infinity is 0
    _, bad = index_check("0x1p-15", 0, 9)
    assert bad > 0


def _perm(s0, s1, sel):
    """v_perm_b32 on the bytes {s0 : s1} (s1 the low four), including the
    selectors 8-11 (a byte of copies of bit 15, 31, 47 or 63), 12 (zero) and
    13 and up (0xff)."""
    data = (s0 << 32) | s1
    out = 0
    for k in range(4):
        b = (sel >> (8 * k)) & 0xFF
        if b >= 13:
            v = 0xFF
        elif b == 12:
            v = 0
        elif b >= 8:
            v = 0xFF if (data >> (15 + 16 * (b - 8))) & 1 else 0
        else:
            v = (data >> (8 * b)) & 0xFF
        out |= v << (8 * k)
    return out


def test_if3_sign_gather_layout():
    src = open(SRC).read()
    calls = re.findall(r"sgn\(xw\[(\d)\], xw\[(\d)\], (0x[0-9A-Fa-f]+)u, (0x[0-9A-Fa-f]+)u\)", src)
    assert len(calls) == 8
    words = [0] * 5 + [1] * 3   # the first five calls build word 0, the rest word 1
    rng = random.Random(3)
    for _ in range(5000):
        xw = [rng.getrandbits(32) for _ in range(8)]
        want = [0, 0]
        for i in range(16):
            sign = (xw[i // 2] >> (15 if i % 2 == 0 else 31)) & 1
            want[(3 * i + 2) // 32] |= sign << ((3 * i + 2) % 32)
        got = [0, 0]
        for w, (hi, lo, sel, mask) in zip(words, calls):
            got[w] |= _perm(xw[int(hi)], xw[int(lo)], int(sel, 16)) & int(mask, 16)
        assert got == want


def test_if3_int_bias():
    # what 1.5 * 2^23 + |q| shifted into place adds beyond |q| (mod 2^32),
    # restated from the layout: elements 0-10 in word 0, 11-15 in word 1
    bias = [0, 0]
    for i in range(16):
        w = 0 if i <= 10 else 1
        bias[w] = (bias[w] + ((0x4B400000 << (3 * i - 32 * w)) & 0xFFFFFFFF)) & 0xFFFFFFFF
    src = open(SRC).read()
    assert "0x4B400000u << (3 * i - 32 * w)" in src and "i <= 10 ? 0 : 1" in src
    rng = random.Random(5)
    for _ in range(5000):
        q = [rng.randrange(4) for _ in range(16)]
        acc = [0, 0]
        for i in range(16):
            w = 0 if i <= 10 else 1
            acc[w] = (acc[w] + (((0x4B400000 + q[i]) << (3 * i - 32 * w)) & 0xFFFFFFFF)) & 0xFFFFFFFF
        field = sum(q[i] << (3 * i) for i in range(16))
        assert (acc[0] - bias[0]) & 0xFFFFFFFF == field & 0xFFFFFFFF
        assert (acc[1] - bias[1]) & 0xFFFFFFFF == field >> 32


def test_if6_int_bias():
    # IF6's INT magnitudes: 1.5 * 2^23 + |q| (|q| <= 31) shifted into 6-bit fields
    # whole, a straddling field's upper bits into the next word; the constant
    # part, restated from the layout, must come out exactly
    src = open(SRC).read()
    assert "0x4B400000u >> (32 - (bit & 31))" in src and "mq[h][bit >> 5] += rb << (bit & 31);" in src
    bias = [0, 0, 0]
    for i in range(16):
        bit = 6 * i
        bias[bit >> 5] = (bias[bit >> 5] + ((0x4B400000 << (bit & 31)) & 0xFFFFFFFF)) & 0xFFFFFFFF
        if (bit & 31) + 6 > 32:
            w = (bit >> 5) + 1
            bias[w] = (bias[w] + (0x4B400000 >> (32 - (bit & 31)))) & 0xFFFFFFFF
    rng = random.Random(7)
    for _ in range(5000):
        q = [rng.randrange(32) for _ in range(16)]
        acc = [0, 0, 0]
        for i in range(16):
            rb, bit = 0x4B400000 + q[i], 6 * i
            acc[bit >> 5] = (acc[bit >> 5] + ((rb << (bit & 31)) & 0xFFFFFFFF)) & 0xFFFFFFFF
            if (bit & 31) + 6 > 32:
                acc[(bit >> 5) + 1] = (acc[(bit >> 5) + 1] + (rb >> (32 - (bit & 31)))) & 0xFFFFFFFF
        field = sum(q[i] << (6 * i) for i in range(16))
        for w in range(3):
            assert (acc[w] - bias[w]) & 0xFFFFFFFF == (field >> (32 * w)) & 0xFFFFFFFF

