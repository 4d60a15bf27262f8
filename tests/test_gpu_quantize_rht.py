"""GPU parity of if4_quantize_rht (random-sign 16-point Hadamard rotation
fused into the IF4 quantize, called through the C ABI) against the CPU
oracle's rotate-then-quantize: codes and scale bytes must match bit for bit.
Also checks that a GEMM of two operands rotated with the same signs matches
the oracle and approximates the unrotated product."""
import numpy as np
import pytest

from adaptive_block_scaled_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _if4():
    from adaptive_block_scaled_amd import if4
    return if4


def to_dev(x_np, dtype, ld=None):
    rows, cols = x_np.shape
    t = torch.from_numpy(np.ascontiguousarray(x_np))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t.float()
    if ld is not None and ld != cols:
        big = torch.zeros((rows, ld), dtype=t.dtype)
        big[:, :cols] = t
        return big.cuda()[:, :cols]
    return t.cuda()


def rot_exp(oracle_mod, x_np, mask, dtype):
    y = oracle_mod.rht16(x_np, mask, round_to_bf16=(dtype == "bf16"))
    a = float(np.abs(y).max()) if y.size else 0.0
    return wl.tensor_scale_exp(a)


def check(oracle_mod, x_np, dtype, mask, e=None, mode=0, ld=None, label=""):
    if e is None:
        e = rot_exp(oracle_mod, x_np, mask, dtype)
    print(f"[quantize_rht] {label} shape={x_np.shape} dtype={dtype} mask={mask:#06x} E={e} "
          f"mode={mode} ld={ld}", flush=True)
    codes, scales = _if4().quantize_rht(to_dev(x_np, dtype, ld), mask, e, mode)
    torch.cuda.synchronize()
    gc, gs = codes.cpu().numpy(), scales.cpu().numpy()
    oc, os_ = oracle_mod.quantize_rht(x_np, mask, e, mode, round_to_bf16=(dtype == "bf16"))
    bad = np.nonzero(gs != os_)
    assert np.array_equal(gs, os_), (label, bad[0][:5], bad[1][:5], gs[bad][:5], os_[bad][:5])
    assert np.array_equal(gc, oc), label
    return gs


def draw(shape, kind, seed, dtype):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        x = rng.standard_normal(shape).astype(np.float32)
    elif kind == "t4":
        x = (rng.standard_t(4, shape) * 0.02).astype(np.float32)
    else:  # wide: exponents across most of the fp32 range, subnormals included
        x = (rng.standard_normal(shape) * np.exp2(rng.integers(-140, 120, shape))).astype(
            np.float32)
    return wl.to_bf16_f32(x) if dtype == "bf16" else x


@pytest.mark.parametrize("shape", [(1, 16), (3, 48), (37, 4144), (513, 272)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mask", [0x0000, 0xFFFF, 0x9A3C])
def test_shapes_dtypes_masks(oracle_mod, shape, dtype, mask):
    x = draw(shape, "t4", shape[0] * 7 + mask, dtype)
    check(oracle_mod, x, dtype, mask, label="t4")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("kind", ["normal", "wide"])
@pytest.mark.parametrize("e", [None, 0, -64, 64])
def test_distributions_and_exponents(oracle_mod, dtype, kind, e):
    x = draw((129, 1024), kind, 3, dtype)
    check(oracle_mod, x, dtype, 0x5AC3, e=e, label=kind)


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forced_modes(oracle_mod, mode, dtype):
    x = draw((200, 512), "normal", 4, dtype)
    check(oracle_mod, x, dtype, 0x1234, mode=mode, label="forced")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_strided_input(oracle_mod, dtype):
    x = draw((77, 320), "t4", 5, dtype)
    check(oracle_mod, x, dtype, 0xF00F, ld=320 + 64, label="strided")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_edge_groups(oracle_mod, dtype):
    g = np.zeros((12, 16), np.float32)
    g[1, :] = -0.0                               # all negative zeros
    g[2, 5] = np.inf                             # infinity -> whole group non-finite
    g[3, 9] = np.nan
    g[4, :] = 3.0e38                             # the butterflies overflow to inf
    g[5, :8] = 3.0e38
    g[5, 8:] = -3.0e38                           # inf - inf = NaN in a stage
    g[6, :] = 1e-40                              # subnormal inputs
    g[7, 0] = 1.0
    g[7, 1:] = 2.0 ** -24                        # order-sensitive fp32 sums
    g[8, :] = np.arange(16) - 7.5                # exact sums
    g[9, :] = 6.0                                # rotates to [24, 0, ..., 0]
    g[10, ::2] = 1.0
    g[10, 1::2] = -1.0
    g[11, :] = np.float32(2.0 ** -130)
    x = g.reshape(3, 64)
    if dtype == "bf16":
        x = wl.to_bf16_f32(x)
    for mask in (0, 0xFFFF, 0x0001, 0x8000):
        for e in (0, -20, 30):
            check(oracle_mod, x, dtype, mask, e=e, label="edge")


def test_empty_and_zero_rows(oracle_mod):
    if4 = _if4()
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    c, s = if4.quantize_rht(x, 0x1, 0)
    assert c.shape == (0, 32) and s.shape == (0, 4)
    x = torch.zeros((5, 0), dtype=torch.bfloat16, device="cuda")
    c, s = if4.quantize_rht(x, 0x1, 0)
    assert c.shape == (5, 0) and s.shape == (5, 0)


def test_rejects_mask_above_16_bits():
    if4 = _if4()
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(if4.IF4Error):
        if4.quantize_rht(x, 0x10000, 0)


def test_gradient_full_size(oracle_mod):
    """The gradient workload (16384 x 4096 bf16, N(0, 1e-3)) at full size, in
    the benchmark's launch configuration, rotated and quantized in one pass,
    compared with the oracle on every group."""
    t, mask = wl.c3_raw_gradient()
    x = t.values
    gs = check(oracle_mod, x, "bf16", mask, label=t.name)
    share_rot = float(((gs & 0x80) != 0).mean())
    print(f"    int4 share after rotation {share_rot:.3f}", flush=True)
    assert (gs == 0).mean() < 0.01


def test_rotated_operands_gemm(oracle_mod):
    """Rotating A and W along K with the same signs leaves A W^T unchanged
    (H16/4 is orthogonal), so the IF4 GEMM of the rotated operands must match
    the oracle's product of the same codes and approximate the unrotated
    product to within the quantization error."""
    if4 = _if4()
    rng = np.random.default_rng(21)
    M, N, K = 256, 320, 1024
    a = wl.to_bf16_f32(rng.standard_normal((M, K)).astype(np.float32))
    w = wl.to_bf16_f32((rng.standard_t(4, (N, K)) * 0.02).astype(np.float32))
    mask = 0x3E51
    ea = rot_exp(oracle_mod, a, mask, "bf16")
    ew = rot_exp(oracle_mod, w, mask, "bf16")
    ac, as_ = if4.quantize_rht(to_dev(a, "bf16"), mask, ea)
    wc, ws = if4.quantize_rht(to_dev(w, "bf16"), mask, ew)
    c = if4.gemm(ac, as_, ea, wc, ws, ew)
    torch.cuda.synchronize()
    c = c.cpu().numpy().astype(np.float64)
    ref = oracle_mod.gemm_sample_f64(ac.cpu().numpy(), as_.cpu().numpy(), ea,
                                     wc.cpu().numpy(), ws.cpu().numpy(), ew)
    rel = np.linalg.norm(c - ref) / np.linalg.norm(ref)
    exact = a.astype(np.float64) @ w.astype(np.float64).T
    rel_q = np.linalg.norm(ref - exact) / np.linalg.norm(exact)
    print(f"[rotated gemm] rel fro vs oracle {rel:.3e}; vs unrotated product {rel_q:.3e}",
          flush=True)
    assert rel <= 1e-3
    assert rel_q < 0.2


def test_weight_full_size_sampled(oracle_mod):
    """Rotate + quantize of the FFN weight (28672 x 8192 bf16) with the sign
    mask and exponent bench.py uses: the whole tensor through the kernel, 64
    rows (the first two, the last, 61 seeded) against the oracle."""
    _, t = wl.c5_ffn()
    x = t.values
    n = x.shape[0]
    mask = wl.sign_mask(wl.random_signs(np.random.default_rng(0)))
    e = t.scale_exp + 2
    rows = np.unique(np.concatenate([[0, 1, n - 1],
                                     np.random.default_rng(8).choice(n, 61, replace=False)]))
    print(f"[quantize_rht] {t.name} mask={mask:#06x} E={e} sampled rows {len(rows)}", flush=True)
    codes, scales = _if4().quantize_rht(to_dev(x, "bf16"), mask, e)
    torch.cuda.synchronize()
    idx = torch.from_numpy(rows).cuda()
    gc, gs = codes[idx].cpu().numpy(), scales[idx].cpu().numpy()
    oc, os_ = oracle_mod.quantize_rht(x[rows], mask, e, 0, round_to_bf16=True)
    assert np.array_equal(gs, os_)
    assert np.array_equal(gc, oc)
