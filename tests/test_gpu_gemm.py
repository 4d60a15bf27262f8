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


@pytest.mark.parametrize("mn_ld", [(261, 77, 80), (9, 300, (1 << 21) + 40)])
def test_stores_stay_inside_c(oracle_mod, mn_ld):
    """Partial tiles on the bottom and right edges, C a view into a larger
    buffer: every output of C[:M, :N] is right, and the columns past N and
    the three rows past M of the buffer keep their sentinel.  A row stride
    above 2^21 floats takes the kernel's general store path."""
    M, N, ldc = mn_ld
    K = 256
    print(f"[gemm] edges M={M} N={N} K={K} ldc={ldc}", flush=True)
    from adaptive_block_scaled_amd import if4
    ac, as_, ea, wc, ws, ew = quantized_pair(oracle_mod, M, N, K, 11)
    t = [torch.from_numpy(np.ascontiguousarray(v)).cuda() for v in (ac, as_, wc, ws)]
    big = torch.full((M + 3, ldc), 7.0, dtype=torch.float32, device="cuda")
    if4.gemm(t[0], t[1], ea, t[2], t[3], ew, out=big[:M, :N])
    torch.cuda.synchronize()
    assert bool((big[M:] == 7.0).all()), "a store landed in a row past M"
    assert bool((big[:M, N:] == 7.0).all()), "a store landed in a column past N"
    got = big[:M, :N].cpu().numpy()
    ref = oracle_mod.gemm_sample_f64(ac, as_, ea, wc, ws, ew)
    err = rel_fro(got, ref)
    print(f"    rel fro {err:.3e}", flush=True)
    assert err <= TOL


# (a_exp, w_exp) pairs and the power of two the operands are scaled by so
# that every exact result is a normal fp32 number: the sums of products lie in
# [2^-18, 2^23] times the operand scale squared, and C = sum * 2^(a_exp + w_exp)
EXP_CASES = [((0, 0), 0), ((-3, 5), 0), ((64, 64), -8), ((55, 55), -4), ((64, -64), 0),
             ((-64, 64), 0), ((-64, -64), 4)]


def _fp4_grid_operands(rng, M, N, K, scale_pow):
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float32)
    a = grid[rng.integers(0, 8, (M, K))] * np.where(rng.random((M, K)) < .5, -1, 1)
    w = grid[rng.integers(0, 8, (N, K))] * np.where(rng.random((N, K)) < .5, -1, 1)
    a[:, ::16] = 6
    w[:, ::16] = -6
    a = (a * 0.5 * 2.0 ** scale_pow).astype(np.float32)
    w = (w * 2.0 * 2.0 ** scale_pow).astype(np.float32)
    a[3] = 0.0  # an all-zero row of A: its row of C must be +0
    return a, w


@pytest.mark.parametrize("K", [16, 32, 48, 160, 256, 512, 1024])
def test_exact_when_products_exact(oracle_mod, K):
    """FP4-only operands with power-of-two scales: products are small dyadic
    numbers and partial sums stay exact in fp32, so C must equal the exact
    result bit for bit, at every exponent pair the C ABI accepts the extremes
    of.  K = 256, 512 and 1024 (multiples of 256, rows 16-byte aligned in
    fresh allocations) take the wide-fetch path the benchmark runs; the others
    the per-word path.  Row 3 of A is zero and must give +0 (not -0 or NaN)."""
    rng = np.random.default_rng(12 + K)
    M, N = 70, 90
    for (ea, ew), pw in EXP_CASES:
        a, w = _fp4_grid_operands(rng, M, N, K, pw)
        ac, as_ = oracle_mod.quantize(a, 0)
        wc, ws = oracle_mod.quantize(w, 0)
        assert not (as_ & 0x80).any() and not (ws & 0x80).any()
        got = gpu_gemm(ac, as_, ea, wc, ws, ew)
        exact = a.astype(np.float64) @ w.T.astype(np.float64)
        ref = exact * 2.0 ** (ea + ew)
        nz = ref != 0
        assert np.all(np.abs(ref[nz]) >= 2.0 ** -126) and np.all(np.abs(ref) < 2.0 ** 128)
        assert np.array_equal(got.astype(np.float64), ref), (K, ea, ew)
        # the oracle's fp64 GEMM of the same codes agrees with the exact product
        assert np.array_equal(oracle_mod.gemm_sample_f64(ac, as_, ea, wc, ws, ew), ref)
        assert (got[3] == 0).all() and not np.signbit(got[3]).any(), (K, ea, ew)


@pytest.mark.parametrize("exps", [(64, 64), (55, 55), (64, -64), (-64, -64)])
@pytest.mark.parametrize("K", [512, 528])
def test_extreme_exponents_against_oracle(oracle_mod, exps, K):
    """Adaptive (FP4 and INT4) operands at the largest and smallest exponent
    pairs the C ABI accepts, drawn so that C is representable: scale bytes
    small for (64, 64) and (55, 55), large for (-64, -64).  The output is
    2^(a_exp + w_exp + 18) times the fp32 sums, applied per output, so it
    must meet the same tolerance as at E = 0, with no inf and no NaN; an
    all-zero row of A comes back +0.  K = 512 runs the wide path, 528 the
    per-word path."""
    ea, ew = exps
    rng = np.random.default_rng(ea * 3 + ew + K)
    M, N = 96, 320
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    wc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    # E4M3 codes 0x01-0x08 (2^-9 .. 2^-6) at (64, 64), 0x01-0x30 (up to 0.5)
    # at (55, 55), 0x60-0x7E (32 .. 448) at (-64, -64), any finite code at
    # (64, -64); bit 7 (INT4) random
    lo, hi = {(64, 64): (1, 0x08), (55, 55): (1, 0x30), (64, -64): (1, 0x7E),
              (-64, -64): (0x60, 0x7E)}[exps]
    as_ = (rng.integers(lo, hi + 1, (M, K // 16)) | (rng.integers(0, 2, (M, K // 16)) << 7)
           ).astype(np.uint8)
    ws = (rng.integers(lo, hi + 1, (N, K // 16)) | (rng.integers(0, 2, (N, K // 16)) << 7)
          ).astype(np.uint8)
    ac[5] = 0
    as_[5] = 0
    print(f"[gemm] exponents {exps} K={K} INT4 share {((as_ & 0x80) != 0).mean():.2f}",
          flush=True)
    got = gpu_gemm(ac, as_, ea, wc, ws, ew)
    ref = oracle_mod.gemm_sample_f64(ac, as_, ea, wc, ws, ew)
    assert np.isfinite(ref).all() and np.abs(ref).max() < 2.0 ** 127
    assert np.isfinite(got).all(), exps
    assert (got[5] == 0).all() and not np.signbit(got[5]).any()
    err = rel_fro(got, ref)
    print(f"    rel fro {err:.3e}", flush=True)
    assert err <= TOL


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
    """The 4096^3 workload, every one of the 16.8 M outputs against the fp64
    oracle: the relative Frobenius error over all of C, and over each
    256 x 256 output tile (the unit one workgroup computes)."""
    a, w = wl.c4_gemm()
    ea, ew = a.scale_exp, w.scale_exp
    print(f"[gemm] c4 4096^3 E_A={ea} E_W={ew}", flush=True)
    ac, as_ = oracle_mod.quantize(a.values, ea)
    wc, ws = oracle_mod.quantize(w.values, ew)
    got = gpu_gemm(ac, as_, ea, wc, ws, ew).astype(np.float64)
    ref = oracle_mod.gemm_sample_f64(ac, as_, ea, wc, ws, ew)
    err = rel_fro(got, ref)
    print(f"    rel fro on all 4096 x 4096 outputs: {err:.3e}", flush=True)
    assert err <= TOL
    d = (got - ref).reshape(16, 256, 16, 256)
    r = ref.reshape(16, 256, 16, 256)
    tile_err = np.sqrt((d ** 2).sum(axis=(1, 3)) / (r ** 2).sum(axis=(1, 3)))
    print(f"    worst 256x256 tile {tile_err.max():.3e}", flush=True)
    assert tile_err.max() <= TOL


def test_c5_full_size(oracle_mod):
    """The FFN workload (M=8192, N=28672, K=8192): one seeded row in every
    256-row M-tile plus the first and last rows, each against all 28672
    columns; the error is checked over the sample and over every 256-column
    block of it, so each of the 3584 output tiles is compared on its own."""
    a, w = wl.c5_ffn()
    ea, ew = a.scale_exp, w.scale_exp
    print(f"[gemm] c5 M=8192 N=28672 K=8192 E_A={ea} E_W={ew}", flush=True)
    ac, as_ = oracle_mod.quantize(a.values, ea)
    wc, ws = oracle_mod.quantize(w.values, ew)
    del a, w
    got = gpu_gemm(ac, as_, ea, wc, ws, ew)
    rng = np.random.default_rng(8)
    rows = sorted({t * 256 + int(rng.integers(0, 256)) for t in range(32)} | {0, 8191})
    ref = oracle_mod.gemm_sample_f64(ac, as_, ea, wc, ws, ew, rows=np.array(rows))
    g = got[rows].astype(np.float64)
    err = rel_fro(g, ref)
    print(f"    rel fro on {len(rows)} rows (every M-tile) x 28672 cols: {err:.3e}", flush=True)
    assert err <= TOL
    worst = 0.0
    for t in range(32):  # the sampled rows of M-tile t, each 256-column block
        sel = [i for i, r in enumerate(rows) if r // 256 == t]
        assert sel, t
        for j in range(0, 28672, 256):
            blk = np.linalg.norm(g[sel, j:j + 256] - ref[sel, j:j + 256]) / np.linalg.norm(
                ref[sel, j:j + 256])
            worst = max(worst, blk)
            assert blk <= 4 * TOL, (t, j, blk)
    print(f"    worst tile block {worst:.3e}", flush=True)
