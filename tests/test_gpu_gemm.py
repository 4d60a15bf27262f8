"""GPU IF4 x IF4 GEMM (through the C ABI) against the fp64 oracle on the
decoded operands: relative Frobenius error <= 1e-3, and exact equality where
every product and sum is exact in fp32."""
from fractions import Fraction as F

import numpy as np
import pytest

from adaptive_block_scaled_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TOL = 1e-3


def gpu_gemm(ac, as_, ea, wc, ws, ew, ldc=None):
    from adaptive_block_scaled_amd import if4
    M, N = ac.shape[0], wc.shape[0]
    t = [torch.from_numpy(np.ascontiguousarray(v)).cuda() for v in (ac, as_, wc, ws)]
    if ldc is not None:
        big = torch.full((M, ldc), 7.0, dtype=torch.float32, device="cuda")
        c = if4.gemm(t[0], t[1], ea, t[2], t[3], ew, out=big[:, :N])
        torch.cuda.synchronize()
        bigc = big.cpu().numpy()
        assert (bigc[:, N:] == 7.0).all()  # nothing written past N
        return bigc[:, :N]
    c = if4.gemm(t[0], t[1], ea, t[2], t[3], ew)
    torch.cuda.synchronize()
    return c.cpu().numpy()


def rel_fro(got, ref):
    return float(np.linalg.norm(got.astype(np.float64) - ref) / np.linalg.norm(ref))


def quantized_pair(oracle_mod, M, N, K, seed):
    a = wl.to_bf16_f32(wl.outlier_activations(M, K, seed))
    w = wl.to_bf16_f32(wl.normal_weights(N, K, seed + 1))
    ea = wl.tensor_scale_exp(float(np.abs(a).max()))
    ew = wl.tensor_scale_exp(float(np.abs(w).max()))
    ac, as_ = oracle_mod.quantize(a, ea)
    wc, ws = oracle_mod.quantize(w, ew)
    return ac, as_, ea, wc, ws, ew


@pytest.mark.parametrize("mnk", [(1, 1, 16), (7, 5, 32), (200, 136, 272), (128, 128, 64),
                                 (257, 383, 1040), (64, 512, 4096)])
def test_ragged_shapes(oracle_mod, mnk):
    M, N, K = mnk
    print(f"[gemm] ragged M={M} N={N} K={K}", flush=True)
    ac, as_, ea, wc, ws, ew = quantized_pair(oracle_mod, M, N, K, M + N + K)
    got = gpu_gemm(ac, as_, ea, wc, ws, ew, ldc=N + 3)
    ref = oracle_mod.gemm_sample_f64(ac, as_, ea, wc, ws, ew)
    err = rel_fro(got, ref)
    print(f"    rel fro {err:.3e}", flush=True)
    assert err <= TOL


def test_exact_when_products_exact(oracle_mod):
    """FP4-only operands with power-of-two scales: products are small dyadic
    numbers and partial sums stay exact in fp32, so C must equal the exact
    result bit for bit."""
    rng = np.random.default_rng(12)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float32)
    for K in (16, 32, 48, 160):
        M, N = 70, 90
        a = grid[rng.integers(0, 8, (M, K))] * np.where(rng.random((M, K)) < .5, -1, 1)
        w = grid[rng.integers(0, 8, (N, K))] * np.where(rng.random((N, K)) < .5, -1, 1)
        a[:, ::16] = 6
        w[:, ::16] = -6
        a = (a * 0.5).astype(np.float32)
        w = (w * 2.0).astype(np.float32)
        ac, as_ = oracle_mod.quantize(a, 0)
        wc, ws = oracle_mod.quantize(w, 0)
        assert not (as_ & 0x80).any() and not (ws & 0x80).any()
        for ea, ew in ((0, 0), (-3, 5)):
            got = gpu_gemm(ac, as_, ea, wc, ws, ew)
            ref = (a.astype(np.float64) @ w.T.astype(np.float64)) * 2.0 ** (ea + ew)
            assert np.array_equal(got.astype(np.float64), ref), (K, ea, ew)


def test_k_zero_writes_zeros():
    from adaptive_block_scaled_amd import if4
    c = torch.full((5, 7), 3.0, device="cuda")
    e = torch.empty((5, 0), dtype=torch.uint8, device="cuda")
    f = torch.empty((7, 0), dtype=torch.uint8, device="cuda")
    if4.gemm(e, e, 0, f, f, 0, out=c)
    torch.cuda.synchronize()
    assert (c.cpu() == 0).all()


def test_nan_scale_propagates(oracle_mod):
    ac, as_, ea, wc, ws, ew = quantized_pair(oracle_mod, 64, 64, 64, 3)
    as_ = as_.copy()
    as_[5, 2] = 0x7F
    got = gpu_gemm(ac, as_, ea, wc, ws, ew)
    assert np.isnan(got[5]).all()
    assert np.isfinite(np.delete(got, 5, axis=0)).all()


@pytest.mark.parametrize("mnk", [(5965, 4040, 512), (4452, 4645, 768), (2560, 7000, 1024)])
def test_more_tiles_than_compute_units(oracle_mod, mnk):
    """Shapes with more 256x256 tiles than the chip has compute units (384,
    342 and 280 tiles), ragged in M and N: the workgroups each run several
    tiles in turn, some more than others.  One row in every M-tile (and the
    last row) is checked against all N columns, so every tile is covered."""
    M, N, K = mnk
    print(f"[gemm] multi-tile M={M} N={N} K={K}", flush=True)
    ac, as_, ea, wc, ws, ew = quantized_pair(oracle_mod, M, N, K, 11 + K)
    got = gpu_gemm(ac, as_, ea, wc, ws, ew)
    tiles_m = (M + 255) // 256
    rows = sorted({min(M - 1, t * 256 + (t * 37) % 256) for t in range(tiles_m)} | {M - 1, 0})
    ref = oracle_mod.gemm_sample_f64(ac, as_, ea, wc, ws, ew, rows=np.array(rows))
    err = rel_fro(got[rows], ref)
    print(f"    rel fro on {len(rows)} rows x {N} cols: {err:.3e}", flush=True)
    assert err <= TOL
    # every tile individually: each sampled row's 256-column blocks
    g, r_ = got[rows].astype(np.float64), ref
    for j in range(0, N, 256):
        blk = np.linalg.norm(g[:, j:j + 256] - r_[:, j:j + 256]) / np.linalg.norm(r_[:, j:j + 256])
        assert blk <= 4 * TOL, (j, blk)


def test_c4_full_size(oracle_mod):
    a, w = wl.c4_gemm()
    ea, ew = a.scale_exp, w.scale_exp
    print(f"[gemm] c4 4096^3 E_A={ea} E_W={ew}", flush=True)
    ac, as_ = oracle_mod.quantize(a.values, ea)
    wc, ws = oracle_mod.quantize(w.values, ew)
    got = gpu_gemm(ac, as_, ea, wc, ws, ew)
    rows = np.sort(np.random.default_rng(7).choice(4096, 256, replace=False))
    ref = oracle_mod.gemm_sample_f64(ac, as_, ea, wc, ws, ew, rows=rows)
    err = rel_fro(got[rows], ref)
    print(f"    rel fro on 256 sampled rows x 4096 cols: {err:.3e}", flush=True)
    assert err <= TOL


def test_c5_full_size(oracle_mod):
    a, w = wl.c5_ffn()
    ea, ew = a.scale_exp, w.scale_exp
    print(f"[gemm] c5 M=8192 N=28672 K=8192 E_A={ea} E_W={ew}", flush=True)
    ac, as_ = oracle_mod.quantize(a.values, ea)
    wc, ws = oracle_mod.quantize(w.values, ew)
    del a, w
    got = gpu_gemm(ac, as_, ea, wc, ws, ew)
    rng = np.random.default_rng(8)
    rows = np.sort(rng.choice(8192, 48, replace=False))
    ref = oracle_mod.gemm_sample_f64(ac, as_, ea, wc, ws, ew, rows=rows)
    err = rel_fro(got[rows], ref)
    print(f"    rel fro on 48 sampled rows x 28672 cols: {err:.3e}", flush=True)
    assert err <= TOL
