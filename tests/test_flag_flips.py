"""The exact flag-flip count (tests/flag_flips.py) checked against the
independent exact-rational statement of IF4 (tests/exact_if4.py): for every
sampled group, the fast exact decision (fp64 with an error bound, exact
rationals on near ties) equals the comparison of the two exact sums of
squared errors, and the oracle's fp32 choice differs from it only on groups
whose exact errors agree to fp32 rounding."""
from fractions import Fraction as F

import numpy as np

import exact_if4 as ex
import flag_flips as ff
from adaptive_block_scaled_amd import workloads as wl


def _blocks():
    rng = np.random.default_rng(77)
    return [
        (wl.c1_mixed_fp32(0).values[::8, :96].copy(), None),
        (wl.to_bf16_f32(rng.standard_normal((16, 64), dtype=np.float32)), None),
        (wl.to_bf16_f32(wl.outlier_activations(16, 4096, 9)[:, :64]), None),
        (wl.to_bf16_f32(wl.rht_gradient(16, 64, 4)), None),
        (wl.to_bf16_f32((rng.standard_t(4, (16, 64)) * 0.02).astype(np.float32)), None),
    ]


def test_exact_choice_matches_exact_rationals(oracle_mod):
    checked = 0
    for x, _ in _blocks():
        for e in (0, wl.tensor_scale_exp(float(np.abs(x).max()))):
            live, exact_int4, got_int4, _ = ff.exact_choice(x, e)
            for r in range(x.shape[0]):
                for k in range(x.shape[1] // 16):
                    res = ex.quantize_group([float(v) for v in x[r, 16 * k:16 * k + 16]], e)
                    if "code" not in res:
                        assert not live[r, k]
                        continue
                    assert live[r, k]
                    assert bool(exact_int4[r, k]) == (res["sse_int"] < res["sse_fp"]), (r, k, e)
                    if bool(got_int4[r, k]) != bool(exact_int4[r, k]):
                        d = abs(res["sse_int"] - res["sse_fp"]) / max(res["sse_int"],
                                                                      res["sse_fp"])
                        assert d < F(1, 10 ** 5)
                    checked += 1
    assert checked > 500


def test_count_flips_sees_a_wrong_flag(oracle_mod, monkeypatch):
    """A planted mistake: an oracle whose adaptive flag is inverted on one
    group must show up as exactly one flip."""
    x = wl.to_bf16_f32(np.random.default_rng(5).standard_normal((8, 64), dtype=np.float32))
    base = ff.count_flips(x, 0)
    real = ff.oracle.quantize

    def planted(v, e, mode=0, **kw):
        c, s = real(v, e, mode, **kw)
        if mode == ff.oracle.ADAPTIVE:
            s = s.copy()
            s[2, 1] ^= 0x80
        return c, s

    monkeypatch.setattr(ff.oracle, "quantize", planted)
    n, flips, _ = ff.count_flips(x, 0)
    assert n == base[0] and flips == base[1] + 1
