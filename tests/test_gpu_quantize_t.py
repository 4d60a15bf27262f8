"""GPU if4_quantize_t (groups along dim 0) against its definition: the
oracle's quantize of the transposed array, bit for bit; and the backward
products of a W4A4G4 linear layer built from it with the IF4 GEMM
(dgrad = dY W, wgrad = dY^T X) against the fp64 oracle on the same
operands."""
import numpy as np
import pytest

from adaptive_block_scaled_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def gpu_qt(x, e, mode=0, dtype="bf16", ld=None, offset=0):
    """x on the GPU as a [rows, cols] view with leading dimension ld, starting
    `offset` elements into its allocation (offset 1 breaks 16-byte alignment)."""
    from adaptive_block_scaled_amd import if4
    rows, cols = x.shape
    t = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    if ld is not None or offset:
        ld = cols if ld is None else ld
        big = torch.zeros((rows, ld + offset), dtype=t.dtype, device="cuda")
        big[:, offset:offset + cols] = t
        t = big[:, offset:offset + cols]
    c, s = if4.quantize_t(t, e, mode)
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy()


def oracle_qt(oracle_mod, x, e, mode=0):
    return oracle_mod.quantize(np.ascontiguousarray(x.T), e, mode=mode)


@pytest.mark.parametrize("shape", [(16, 1), (32, 300), (272, 1000), (512, 64)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_matches_quantize_of_transpose(oracle_mod, shape, dtype):
    rows, cols = shape
    x = wl.outlier_activations(rows, cols, rows + cols)
    if dtype == "bf16":
        x = wl.to_bf16_f32(x)
    e = wl.tensor_scale_exp(float(np.abs(x).max()))
    print(f"[quantize_t] {dtype} {rows}x{cols} E={e}", flush=True)
    for mode in (0, 1, 2):
        rc, rs = oracle_qt(oracle_mod, x, e, mode)
        gc, gs = gpu_qt(x, e, mode, dtype)
        assert np.array_equal(gc, rc) and np.array_equal(gs, rs), (mode, shape, dtype)
    gc, gs = gpu_qt(x, e, 0, dtype, ld=cols + 24)
    rc, rs = oracle_qt(oracle_mod, x, e, 0)
    assert np.array_equal(gc, rc) and np.array_equal(gs, rs)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape,ld,offset", [
    ((144, 130), 136, 0),   # 16-byte rows: LDS-tiled kernel, ragged last tile both ways
    ((256, 200), 200, 0),   # whole row tiles: the aligned 16-byte column stores
    ((48, 3), 8, 0),        # a single partial 16-byte chunk per row
    ((400, 270), 272, 0),   # several tiles, 2-element tail chunk
    ((144, 130), 136, 1),   # misaligned start: per-element kernel
    ((32, 300), 300, 0),    # bf16 rows of 600 bytes: per-element kernel
])
def test_tiled_and_per_element_paths(oracle_mod, dtype, shape, ld, offset):
    rows, cols = shape
    x = wl.outlier_activations(rows, cols, 7 * rows + cols)
    if dtype == "bf16":
        x = wl.to_bf16_f32(x)
    e = wl.tensor_scale_exp(float(np.abs(x).max()))
    print(f"[quantize_t] {dtype} {rows}x{cols} ld={ld} offset={offset} E={e}", flush=True)
    for mode in (0, 2):
        gc, gs = gpu_qt(x, e, mode, dtype, ld=ld, offset=offset)
        rc, rs = oracle_qt(oracle_mod, x, e, mode)
        assert np.array_equal(gc, rc) and np.array_equal(gs, rs), (mode, shape, ld, offset)


def test_full_size_weight(oracle_mod):
    """W 4096x4096 (C4's weight) along dim 0 against the GPU's own row quantize
    of the transposed tensor (itself bit-exact against the oracle) and the
    oracle on a sample of columns."""
    from adaptive_block_scaled_amd import if4
    x = wl.to_bf16_f32(wl.normal_weights(4096, 4096, 1))
    e = wl.tensor_scale_exp(float(np.abs(x).max()))
    gc, gs = gpu_qt(x, e)
    xt = torch.from_numpy(np.ascontiguousarray(x.T)).cuda().to(torch.bfloat16)
    rc, rs = if4.quantize(xt, e)
    assert np.array_equal(gc, rc.cpu().numpy()) and np.array_equal(gs, rs.cpu().numpy())
    cols = np.random.default_rng(3).choice(4096, 64, replace=False)
    oc, os_ = oracle_mod.quantize(np.ascontiguousarray(x.T[cols]), e)
    assert np.array_equal(gc[cols], oc) and np.array_equal(gs[cols], os_)


def rel_fro(got, ref):
    return float(np.linalg.norm(got.astype(np.float64) - ref) / np.linalg.norm(ref))


def test_backward_products(oracle_mod):
    """dgrad[M,K] = dY[M,N] W[N,K]: A = dY grouped along N (row quantize),
    B = W^T grouped along N (quantize_t of W).  wgrad[N,K] = dY^T X: A = dY^T
    and B = X^T, both grouped along M (quantize_t)."""
    from adaptive_block_scaled_amd import if4
    M, N, K = 256, 384, 320
    dy = wl.to_bf16_f32(wl.normal_weights(M, N, 11, std=1e-3))
    w = wl.to_bf16_f32(wl.normal_weights(N, K, 12))
    x = wl.to_bf16_f32(wl.outlier_activations(M, K, 13))
    e_dy = wl.tensor_scale_exp(float(np.abs(dy).max()))
    e_w = wl.tensor_scale_exp(float(np.abs(w).max()))
    e_x = wl.tensor_scale_exp(float(np.abs(x).max()))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda().to(torch.bfloat16)
    # dgrad
    a_c, a_s = if4.quantize(dev(dy), e_dy)
    b_c, b_s = if4.quantize_t(dev(w), e_w)
    got = if4.gemm(a_c, a_s, e_dy, b_c, b_s, e_w).cpu().numpy()
    ref = oracle_mod.gemm_sample_f64(a_c.cpu().numpy(), a_s.cpu().numpy(), e_dy,
                                     b_c.cpu().numpy(), b_s.cpu().numpy(), e_w)
    err = rel_fro(got, ref)
    print(f"[backward] dgrad rel fro {err:.3e}; vs unquantized "
          f"{rel_fro(got, dy.astype(np.float64) @ w.astype(np.float64)):.3e}", flush=True)
    assert err <= 1e-3
    # wgrad
    a_c, a_s = if4.quantize_t(dev(dy), e_dy)
    b_c, b_s = if4.quantize_t(dev(x), e_x)
    got = if4.gemm(a_c, a_s, e_dy, b_c, b_s, e_x).cpu().numpy()
    ref = oracle_mod.gemm_sample_f64(a_c.cpu().numpy(), a_s.cpu().numpy(), e_dy,
                                     b_c.cpu().numpy(), b_s.cpu().numpy(), e_x)
    err = rel_fro(got, ref)
    print(f"[backward] wgrad rel fro {err:.3e}; vs unquantized "
          f"{rel_fro(got, dy.T.astype(np.float64) @ x.astype(np.float64)):.3e}", flush=True)
    assert err <= 1e-3
