"""GPU parity of if4_quantize (through the C ABI) against the CPU oracle:
codes and scale bytes must match bit for bit."""
import struct
import sys

import numpy as np
import pytest

from adaptive_block_scaled_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _if4():
    from adaptive_block_scaled_amd import if4
    return if4


def gpu_quant(x_np, dtype, scale_exp=0, mode=0, ld=None):
    """Quantize on the GPU; x_np holds values exactly representable in dtype."""
    if4 = _if4()
    rows, cols = x_np.shape
    t = torch.from_numpy(np.ascontiguousarray(x_np))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t.float()
    if ld is not None and ld != cols:
        big = torch.zeros((rows, ld), dtype=t.dtype)
        big[:, :cols] = t
        t = big.cuda()[:, :cols]
    else:
        t = t.cuda()
    codes, scales = if4.quantize(t, scale_exp, mode)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def check(oracle_mod, x_np, dtype, scale_exp=0, mode=0, ld=None, label=""):
    print(f"[quantize] {label} shape={x_np.shape} dtype={dtype} E={scale_exp} mode={mode}",
          flush=True)
    gc, gs = gpu_quant(x_np, dtype, scale_exp, mode, ld)
    oc, os_ = oracle_mod.quantize(x_np, scale_exp, mode)
    bad_s = np.argwhere(gs != os_)
    assert bad_s.size == 0, (label, bad_s[:5], gs[tuple(bad_s[0])], os_[tuple(bad_s[0])])
    bad_c = np.argwhere(gc != oc)
    assert bad_c.size == 0, (label, bad_c[:5])
    return gs


def test_c1_fp32_both_exponents(oracle_mod):
    c1 = wl.c1_mixed_fp32(0)
    check(oracle_mod, c1.values, "f32", 0, label="c1 E=0")
    check(oracle_mod, c1.values, "f32", c1.scale_exp, label="c1 E=rule")


@pytest.mark.parametrize("shape", [(1, 16), (3, 48), (37, 4144), (513, 272), (64, 4096)])
@pytest.mark.parametrize("kind", ["normal", "uniform", "outlier", "rht", "t4"])
def test_bf16_shapes_and_distributions(oracle_mod, shape, kind):
    rows, cols = shape
    rng = np.random.default_rng(rows * 7919 + cols)
    if kind == "normal":
        x = rng.standard_normal(shape, dtype=np.float32)
    elif kind == "uniform":
        x = rng.uniform(-1, 1, shape).astype(np.float32)
    elif kind == "outlier":
        x = wl.outlier_activations(rows, cols, 3)
    elif kind == "rht":
        x = wl.rht_gradient(rows, cols, 4)
    else:
        x = (rng.standard_t(4, shape) * 0.02).astype(np.float32)
    x = wl.to_bf16_f32(x)
    e = wl.tensor_scale_exp(float(np.abs(x).max()))
    check(oracle_mod, x, "bf16", 0, label=kind)
    check(oracle_mod, x, "bf16", e, label=kind + " rule-E")


@pytest.mark.parametrize("mode", [1, 2])
def test_forced_modes(oracle_mod, mode):
    x = wl.to_bf16_f32(np.random.default_rng(1).standard_normal((128, 512), dtype=np.float32))
    gs = check(oracle_mod, x, "bf16", 0, mode, label=f"mode{mode}")
    assert ((gs & 0x80) != 0).all() if mode == 2 else not (gs & 0x80).any()


def test_strided_input(oracle_mod):
    x = wl.to_bf16_f32(np.random.default_rng(2).standard_normal((50, 96), dtype=np.float32))
    check(oracle_mod, x, "bf16", 0, ld=104, label="bf16 ld=104")
    xf = np.random.default_rng(3).standard_normal((50, 96), dtype=np.float32)
    check(oracle_mod, xf, "f32", 0, ld=100, label="f32 ld=100")


def _bf16(bits):
    return struct.unpack("<f", struct.pack("<I", bits << 16))[0]


def test_every_bf16_amax_sets_the_scale(oracle_mod):
    """All 32640 finite positive bf16 values as the group maximum (plus 0),
    alone and with a random tail below it, at E = 0 and E = -20, 20."""
    amax = np.array([_bf16(b) for b in range(0, 0x7F80)], np.float32)
    n = amax.size
    rng = np.random.default_rng(4)
    x = np.zeros((n, 16), np.float32)
    x[:, 0] = amax
    tail = wl.to_bf16_f32((rng.uniform(-1, 1, (n, 15)) * amax[:, None]).astype(np.float32))
    x2 = x.copy()
    x2[:, 1:] = tail
    for e in (0, -20, 20):
        check(oracle_mod, x.reshape(-1, 64), "bf16", e, label=f"amax alone E={e}")
        check(oracle_mod, x2.reshape(-1, 64), "bf16", e, label=f"amax+tail E={e}")


@pytest.mark.parametrize("e", [0, -3, 5])
def test_int4_clamp_only_where_needed(oracle_mod, e):
    """The row kernel runs the INT4 loop without its clamp in waves whose 64
    groups all have ordinary scales.  Groups whose largest element sits at
    the bound of that elision (a/6 = 2^k * 1.0625 exactly, a tie that rounds
    the scale down to 2^k, so 7a/(6s) = 7.4375) fill every wave; in every
    other wave one group has an E4M3 subnormal scale (a = 2^-6 * 2^e: 7a/(6s)
    = 9.33, which only the clamp brings back to 7) or one a saturating scale
    (a/6 = 600 * 2^e).  Codes and scale bytes must match the oracle in
    every wave, adaptively and with INT4 forced (where a missing clamp would
    show in the codes of the groups that need it whatever the selection)."""
    rng = np.random.default_rng(11)
    waves, gpw = 96, 64
    k = rng.integers(-4, 6, waves * gpw)
    amax = (6.375 * 2.0 ** k).astype(np.float32)  # 6 * 1.0625 * 2^k, exact in bf16
    x = np.empty((waves * gpw, 16), np.float32)
    x[:, 0] = amax
    tail = rng.uniform(-1, 1, (waves * gpw, 15)) * amax[:, None]
    x[:, 1:] = wl.to_bf16_f32(tail.astype(np.float32))
    for w in range(1, waves, 2):
        g = w * gpw + int(rng.integers(0, gpw))
        big = 2.0 ** -6 if w % 4 == 1 else 3600.0
        x[g, 0] = big
        x[g, 1:] = wl.to_bf16_f32((rng.uniform(0.9, 1.0, 15) * big).astype(np.float32))
    x = (x * np.float32(2.0 ** e)).astype(np.float32)
    for mode in (0, 2):
        check(oracle_mod, x.reshape(-1, 64 * 16), "bf16", e, mode,
              label=f"clamp elision E={e}")


def test_exhaustive_element_codes(oracle_mod):
    """Every (bf16 |x| <= 6 s', E4M3 scale s') pair: groups [6 s', x, ...]
    fix the scale at s', so each element's FP4 and INT4 codes and both error
    sums are exercised for every representable input (both signs)."""
    positive = np.array([_bf16(b) for b in range(0, 0x7F80)], np.float32)
    rows = []
    for sc in range(1, 127):
        e, m = sc >> 3, sc & 7
        sp = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        xs = positive[positive <= 6 * sp]
        vals = np.concatenate([xs, -xs])
        pad = (-vals.size) % 15
        vals = np.concatenate([vals, np.zeros(pad, np.float32)]).reshape(-1, 15)
        grp = np.empty((vals.shape[0], 16), np.float32)
        grp[:, 0] = 6 * sp
        grp[:, 1:] = vals
        rows.append(grp)
    allg = np.concatenate(rows)
    pad = (-allg.shape[0]) % 64
    allg = np.concatenate([allg, np.zeros((pad, 16), np.float32)])
    x = allg.reshape(-1, 64 * 16)
    print(f"[quantize] exhaustive element sweep: {allg.shape[0]} groups", flush=True)
    check(oracle_mod, x, "bf16", 0, label="exhaustive E=0")
    check(oracle_mod, np.ldexp(x, 7).astype(np.float32), "bf16", 7, label="exhaustive E=7")


def test_edge_groups(oracle_mod):
    big = _bf16(0x7F7F)  # largest finite bf16
    tiny = _bf16(0x0001)  # smallest subnormal bf16
    g = np.zeros((12, 16), np.float32)
    g[1, 3] = -0.0
    g[2, 5] = np.nan
    g[3, 0] = np.inf
    g[4, 7] = -np.inf
    g[5, :] = tiny
    g[6, :] = big
    g[6, 1::2] = -big
    g[7, 0] = 3072.0  # saturating scale
    g[7, 1] = -2000.0
    g[8, :] = np.linspace(-1, 1, 16, dtype=np.float32)
    g[9, 0] = 6.0
    g[9, 1:] = -1e-30  # negative values that round to zero
    g[10, :] = _bf16(0x0080)  # smallest normal bf16
    g[11, 0] = 3 * 2.0 ** -9  # scale ties to zero
    x = wl.to_bf16_f32(g).reshape(3, 64)
    for e in (0, -64, 64, -9):
        check(oracle_mod, x, "bf16", e, label=f"edges E={e}")
        check(oracle_mod, g.reshape(3, 64), "f32", e, label=f"edges f32 E={e}")


def test_fp32_near_tie_inputs(oracle_mod):
    """fp32 inputs one ulp around every FP4/INT4/scale midpoint."""
    rng = np.random.default_rng(5)
    out = []
    for sc in rng.integers(1, 127, 40):
        e, m = sc >> 3, sc & 7
        sp = np.float32(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
        mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0] + [3 * (2 * k + 1) / 7 for k in range(7)]
        vals = []
        for md in mids:
            v = np.float32(md * sp)
            vals += [np.nextafter(v, np.float32(0)), v, np.nextafter(v, np.float32(1e30))]
        vals = np.array(vals, np.float32)
        vals = np.concatenate([vals, -vals])
        pad = (-vals.size) % 15
        vals = np.concatenate([vals, np.zeros(pad, np.float32)]).reshape(-1, 15)
        grp = np.empty((vals.shape[0], 16), np.float32)
        grp[:, 0] = 6 * sp
        grp[:, 1:] = vals
        out.append(grp)
    allg = np.concatenate(out)
    allg = np.concatenate([allg, np.zeros(((-allg.shape[0]) % 4, 16), np.float32)])
    check(oracle_mod, allg.reshape(-1, 64), "f32", 0, label="fp32 near ties")


@pytest.mark.parametrize("cfg", ["c2", "c3", "c3_e0", "c4", "c5"])
def test_full_size_configs(oracle_mod, cfg):
    """The benchmark workloads at full size, in the benchmark's launch
    configuration, compared with the oracle on every group (c5: on a seeded
    sample of 2048 rows of each operand)."""
    if cfg == "c2":
        ts = [wl.c2_activations()]
    elif cfg in ("c3", "c3_e0"):
        ts = [wl.c3_rht_gradient()]
    elif cfg == "c4":
        ts = list(wl.c4_gemm())
    else:
        ts = list(wl.c5_ffn())
    for t in ts:
        e = 0 if cfg == "c3_e0" else t.scale_exp
        x = t.values
        print(f"[quantize] {t.name} E={e}", flush=True)
        gc, gs = gpu_quant(x, "bf16", e)
        if cfg == "c5":
            rows = np.sort(np.random.default_rng(6).choice(x.shape[0], 2048, replace=False))
            oc, os_ = oracle_mod.quantize(x[rows], e)
            gc, gs = gc[rows], gs[rows]
        else:
            oc, os_ = oracle_mod.quantize(x, e)
        assert np.array_equal(gs, os_), t.name
        assert np.array_equal(gc, oc), t.name
        frac_int4 = float(((gs & 0x80) != 0).mean())
        frac_zero = float((gs == 0).mean())
        print(f"    int4 share {frac_int4:.3f}, zero-scale share {frac_zero:.3f}", flush=True)
        if cfg == "c3_e0":
            assert frac_zero > 0.99  # sigma = 1e-3 underflows the E4M3 scale at E = 0
        else:
            assert frac_zero < 0.01


def test_fp32_grid_stride_beyond_one_pass(oracle_mod):
    """The fp32 kernel caps its grid at 65536 workgroups of 256 groups
    (16,777,216 groups) and strides over the rest.  A 4096 x 65600 fp32
    tensor has 16,793,600 groups: every group from row 4092, column-group 16
    on is quantized by the loop's second pass.  The input is drawn on the GPU
    (seeded), and rows on both sides of that boundary, plus the first row,
    are checked against the oracle in full."""
    if4 = _if4()
    rows, cols = 4096, 65600
    gen = torch.Generator(device="cuda").manual_seed(31)
    x = torch.randn((rows, cols), generator=gen, device="cuda", dtype=torch.float32)
    x[4094] *= 1e-3  # a row at a different exponent
    e = 0
    print(f"[quantize] fp32 grid stride rows={rows} cols={cols} groups={rows * cols // 16}",
          flush=True)
    codes, scales = if4.quantize(x, e)
    torch.cuda.synchronize()
    sample = [0, 2047, 4091, 4092, 4093, 4094, 4095]
    assert rows * (cols // 16) > 65536 * 256 > 4092 * (cols // 16)
    xs = x[sample].cpu().numpy()
    oc, os_ = oracle_mod.quantize(xs, e)
    gc, gs = codes[sample].cpu().numpy(), scales[sample].cpu().numpy()
    assert np.array_equal(gs, os_)
    assert np.array_equal(gc, oc)
