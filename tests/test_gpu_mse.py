"""Quantization error of IF4 against its fixed encodings, through the GPU
path (libif4 quantize in the three modes + libif4 dequantize).  Per group,
the adaptive choice must never end worse than the better of FP4 and INT4
beyond the fp32 selection's rounding (a near-tie can flip; 1e-5 relative),
and over each tensor IF4's MSE must not exceed either fixed format's."""
import pytest

from adaptive_block_scaled_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def check(r):
    print(f"[mse] {r['tensor']} E={r['scale_exp']} IF4 {r['mse_if4']:.4e} FP4 {r['mse_fp4']:.4e} "
          f"INT4 {r['mse_int4']:.4e} INT4 share {r['int4_share']:.3f} worse {r['groups_if4_above_best_fixed']}",
          flush=True)
    assert r["groups_if4_above_best_fixed"] == 0
    assert r["mse_if4"] <= r["mse_fp4"] * (1 + 1e-12)
    assert r["mse_if4"] <= r["mse_int4"] * (1 + 1e-12)


@pytest.mark.parametrize("e", [0, None])
def test_c1(e):
    from adaptive_block_scaled_amd.mse_report import report_tensor
    check(report_tensor(wl.c1_mixed_fp32(), e))


def test_c2_activations():
    from adaptive_block_scaled_amd.mse_report import report_tensor
    r = report_tensor(wl.c2_activations())
    check(r)
    assert r["mse_if4"] < r["mse_fp4"] and r["mse_if4"] < r["mse_int4"]


def test_c3_rotated_gradient():
    from adaptive_block_scaled_amd.mse_report import report_tensor
    r = report_tensor(wl.c3_rht_gradient(rows=2048))
    check(r)
    assert r["mse_if4"] < r["mse_fp4"] and r["mse_if4"] < r["mse_int4"]


def test_rotation_makes_heavy_tails_prefer_int4():
    """The pages: after a random Hadamard rotation data look more uniform and
    INT4 wins more often.  Student-t(4) weights (heavy tails) choose INT4 in
    fewer groups than Gaussian data; rotated by the per-group random-sign
    Hadamard they become near-Gaussian and INT4's share rises."""
    import numpy as np
    from adaptive_block_scaled_amd.mse_report import report_tensor
    x = wl.student_t_weights(2048, 4096, seed=5)
    plain = report_tensor(wl.Tensor("t4", wl.to_bf16_f32(x), "bf16"))
    rot = report_tensor(wl.Tensor("t4_rht", wl.to_bf16_f32(
        wl.rht16(x, wl.random_signs(np.random.default_rng(6)))), "bf16"))
    check(plain)
    check(rot)
    assert rot["int4_share"] > plain["int4_share"] + 0.1


@pytest.mark.parametrize("bits", [3, 6])
def test_ifn_error_not_above_either_fixed_format(bits):
    """IF3 / IF6 keep the lower-error encoding per group, so their MSE is at
    most that of the forced float and forced INT formats (the pages' claim
    that the adaptive pattern holds across bit widths)."""
    from adaptive_block_scaled_amd import mse_report
    for t in (wl.c2_activations(rows=1024), wl.c3_rht_gradient(rows=1024)):
        r = mse_report.report_tensor_ifn(t, bits)
        print(r, flush=True)
        assert r["mse_if"] <= r["mse_fp"] and r["mse_if"] <= r["mse_int"]
        assert r["groups_if_above_best_fixed"] <= 2
        assert 0.0 < r["int_share"] < 1.0
