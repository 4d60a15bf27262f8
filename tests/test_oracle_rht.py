"""Pins of the oracle's random-sign Hadamard rotation (rht16) and of the
rotate-then-quantize composition, against things other than the oracle:
scipy's Sylvester Hadamard matrix on inputs where every sum is exact, the
rounding-error bound of a depth-4 summation, the transform's own inverse,
hand-worked fp32 groups whose values depend on the butterfly order, and
torch's bf16 rounding.  CPU only."""
import json
import os

import numpy as np
import pytest
import scipy.linalg
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rht_groups.json")
H16 = scipy.linalg.hadamard(16).astype(np.float64)


def signs(mask: int) -> np.ndarray:
    return np.array([-1.0 if (mask >> i) & 1 else 1.0 for i in range(16)])


def exact_rotation(x: np.ndarray, mask: int) -> np.ndarray:
    """fp64 H16 (d .* x_g) / 4 per group of 16 along dim 1."""
    rows, cols = x.shape
    g = x.astype(np.float64).reshape(rows, cols // 16, 16) * signs(mask)
    return (g @ H16.T).reshape(rows, cols) / 4.0


@pytest.mark.parametrize("mask", [0, 0xFFFF, 0x8001, 0x1234, 0xBEEF])
def test_rht_matches_sylvester_matrix_on_exact_inputs(oracle_mod, mask):
    # integers below 2^10: every butterfly sum is exact in fp32, so the
    # oracle must equal scipy's Sylvester matrix product exactly (order of
    # the matrix, sign-mask bit order and the 1/4 normalisation)
    rng = np.random.default_rng(mask)
    x = rng.integers(-1023, 1024, (7, 64)).astype(np.float32)
    y = oracle_mod.rht16(x, mask)
    np.testing.assert_array_equal(y.astype(np.float64), exact_rotation(x, mask))


def test_rht_is_its_own_inverse_up_to_signs(oracle_mod):
    # H16/4 is symmetric orthonormal: rotating with mask 0 after rotating
    # with d returns d .* x; exact for inputs that are multiples of 4
    rng = np.random.default_rng(1)
    x = (4 * rng.integers(-255, 256, (5, 48))).astype(np.float32)
    for mask in (0, 0x5A5A, 0xFFFF):
        y = oracle_mod.rht16(x, mask)
        back = oracle_mod.rht16(y, 0)
        np.testing.assert_array_equal(back, x * np.tile(signs(mask), 3).astype(np.float32))


@pytest.mark.parametrize("kind", ["normal", "t4", "wide"])
def test_rht_within_summation_error_bound(oracle_mod, kind):
    # four rounded adds per output: |y - exact| <= gamma_4 * sum|x_i| / 4
    rng = np.random.default_rng(7)
    if kind == "normal":
        x = rng.standard_normal((64, 256)).astype(np.float32)
    elif kind == "t4":
        x = rng.standard_t(4, (64, 256)).astype(np.float32)
    else:
        x = (rng.standard_normal((64, 256)) * np.exp2(rng.integers(-30, 30, (64, 256)))).astype(
            np.float32)
    mask = 0x3C96
    y = oracle_mod.rht16(x, mask).astype(np.float64)
    ex = exact_rotation(x, mask)
    u = 2.0 ** -24
    gamma4 = 4 * u / (1 - 4 * u)
    bound = gamma4 * np.repeat(np.abs(x.astype(np.float64)).reshape(64, 16, 16).sum(2) / 4, 16,
                               axis=1)
    assert np.all(np.abs(y - ex) <= bound)
    # and the rounding is not the trivial one: most outputs differ from the
    # once-rounded exact value somewhere in a tensor this size
    assert np.any(y != ex.astype(np.float32).astype(np.float64))


def test_rht_hand_worked_stage_order(oracle_mod):
    fx = json.load(open(GOLDEN))
    for g in fx["groups"]:
        x = np.zeros((1, 16), np.float32)
        x[0, :4] = np.array(g["x_u"], np.float64) * 2.0 ** -24
        y = oracle_mod.rht16(x, g["sign_mask"])[0].astype(np.float64)
        want = np.tile(np.array(g["y4_u"], np.float64) * 2.0 ** -26, 4)
        np.testing.assert_array_equal(y, want, err_msg=g["name"])
        # the fixture's alternatives really are different answers
        assert g["y4_u"] != g["reversed_order_y4_u"]
        assert g["y4_u"] != g["exact_product_y4_u"]


def test_rht_bf16_rounding_matches_torch(oracle_mod):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((32, 128)).astype(np.float32)
    y32 = oracle_mod.rht16(x, 0x0F0F)
    yb = oracle_mod.rht16(x, 0x0F0F, round_to_bf16=True)
    want = torch.from_numpy(y32).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(yb, want)


def test_rht_nonfinite_spreads_to_its_group(oracle_mod):
    x = np.ones((2, 32), np.float32)
    x[0, 3] = np.inf
    x[1, 20] = np.nan
    y = oracle_mod.rht16(x, 0)
    assert not np.isfinite(y[0, :16]).any() and np.isfinite(y[0, 16:]).all()
    assert np.isfinite(y[1, :16]).all() and np.isnan(y[1, 16:]).all()
    codes, scales = oracle_mod.quantize_rht(x, 0)
    # a group of ones rotates to [4, 0, ..., 0]: scale RNE_E4M3(4/6) =
    # 1.375 * 2^-1 = code 0x33, FP4 index 6 (4/0.6875 = 5.8 -> 6) in nibble 0
    assert list(scales[0]) == [0x7F, 0x33] and list(scales[1]) == [0x33, 0x7F]
    assert list(codes[0, 8:]) == [7, 0, 0, 0, 0, 0, 0, 0] and not codes[0, :8].any()


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_quantize_rht_is_rotation_then_quantize(oracle_mod, bf16, mode):
    rng = np.random.default_rng(11)
    x = (rng.standard_t(4, (40, 96)) * 0.02).astype(np.float32)
    if bf16:
        x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    mask = 0xA5C3
    y = oracle_mod.rht16(x, mask, round_to_bf16=bf16)
    c0, s0 = oracle_mod.quantize(y, -9, mode)
    c1, s1 = oracle_mod.quantize_rht(x, mask, -9, mode, round_to_bf16=bf16)
    np.testing.assert_array_equal(c0, c1)
    np.testing.assert_array_equal(s0, s1)


def test_rotation_raises_int4_share_on_heavy_tails(oracle_mod):
    # the pages' motivation: a Hadamard rotation makes heavy-tailed groups
    # more uniform, where the INT4 encoding wins more often
    rng = np.random.default_rng(5)
    x = torch.from_numpy((rng.standard_t(4, (256, 1024)) * 0.02).astype(np.float32))
    x = x.to(torch.bfloat16).float().numpy()
    _, s_plain = oracle_mod.quantize(x, -8)
    _, s_rot = oracle_mod.quantize_rht(x, 0x6D2B, -7, round_to_bf16=True)
    share_plain = (s_plain >= 0x80).mean()
    share_rot = (s_rot >= 0x80).mean()
    assert share_rot > share_plain + 0.1, (share_plain, share_rot)
