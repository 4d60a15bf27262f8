"""GPU parity of if4_dequantize against the CPU oracle, bit for bit (fp32
and bf16 outputs; NaN groups compared as NaN)."""
import numpy as np
import pytest

from adaptive_block_scaled_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def gpu_deq(codes, scales, e, dtype, ld=None):
    from adaptive_block_scaled_amd import if4
    rows, half = codes.shape
    cols = 2 * half
    c = torch.from_numpy(codes).cuda()
    s = torch.from_numpy(scales).cuda()
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    if ld is not None:
        big = torch.empty((rows, ld), dtype=tdt, device="cuda")
        y = if4.dequantize(c, s, e, tdt, out=big[:, :cols])
    else:
        y = if4.dequantize(c, s, e, tdt)
    torch.cuda.synchronize()
    if dtype == "bf16":
        return y.view(torch.int16).cpu().numpy().view(np.uint16)
    return y.cpu().numpy()


def compare(oracle_mod, codes, scales, e, label, ld=None):
    print(f"[dequantize] {label} shape={codes.shape} E={e}", flush=True)
    ref = oracle_mod.dequantize(codes, scales, e)
    got = gpu_deq(codes, scales, e, "f32", ld)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), label
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32)), label
    refb = oracle_mod.f32_to_bf16_bits(ref)
    gotb = gpu_deq(codes, scales, e, "bf16", ld)
    nanb = (refb & 0x7FFF) > 0x7F80
    assert np.array_equal((gotb & 0x7FFF) > 0x7F80, nanb), label
    assert np.array_equal(gotb[~nanb], refb[~nanb]), label


def test_every_scale_byte_and_nibble(oracle_mod):
    # 256 scale bytes (both flags, NaN patterns, zero) x all 16 nibbles
    scales = np.arange(256, dtype=np.uint8).reshape(64, 4)
    nib = np.arange(16, dtype=np.uint8)
    group = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)
    codes = np.tile(group, (64, 4))
    for e in (0, -64, -20, 9, 64):
        compare(oracle_mod, codes, scales, e, f"all codes E={e}")


@pytest.mark.parametrize("shape", [(1, 16), (5, 80), (129, 4112), (256, 256)])
def test_random_codes(oracle_mod, shape):
    rng = np.random.default_rng(shape[0] + shape[1])
    rows, cols = shape
    codes = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, (rows, cols // 16), dtype=np.uint8)
    compare(oracle_mod, codes, scales, 0, "random")
    compare(oracle_mod, codes, scales, -3, "random strided", ld=cols + 16)


def test_roundtrip_c1(oracle_mod):
    c1 = wl.c1_mixed_fp32(0)
    for e in (0, c1.scale_exp):
        codes, scales = oracle_mod.quantize(c1.values, e)
        compare(oracle_mod, codes, scales, e, f"c1 E={e}")


def test_full_size_c2(oracle_mod):
    t = wl.c2_activations()
    codes, scales = oracle_mod.quantize(t.values, t.scale_exp)
    compare(oracle_mod, codes, scales, t.scale_exp, t.name)


def test_full_size_weight_sampled(oracle_mod):
    """The FFN weight (28672 x 8192) dequantized to bf16 in the launch
    configuration bench.py times: the whole tensor through the kernel, 64
    rows (the first two, the last, 61 seeded) against the oracle's dequantize
    of the same codes."""
    from adaptive_block_scaled_amd import if4
    _, t = wl.c5_ffn()
    n = t.values.shape[0]
    rows = np.unique(np.concatenate([[0, 1, n - 1],
                                     np.random.default_rng(7).choice(n, 61, replace=False)]))
    print(f"[dequantize] {t.name} E={t.scale_exp} sampled rows {len(rows)}", flush=True)
    x = torch.from_numpy(t.values).to(torch.bfloat16).cuda()
    codes, scales = if4.quantize(x, t.scale_exp)
    y = if4.dequantize(codes, scales, t.scale_exp, torch.bfloat16)
    torch.cuda.synchronize()
    idx = torch.from_numpy(rows).cuda()
    c, s = codes[idx].cpu().numpy(), scales[idx].cpu().numpy()
    want = oracle_mod.f32_to_bf16_bits(oracle_mod.dequantize(c, s, t.scale_exp))
    got = y[idx].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want)
