"""GPU parity of IF3 / IF6 (if4_quantize_ifn, if4_dequantize_ifn through the
C ABI) against the CPU oracle: codes, scale bytes and decoded values bit for
bit."""
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


def check_q(oracle_mod, x, bits, dtype, e, mode=0, ld=None, label=""):
    print(f"[ifn] {label} IF{bits} {dtype} {x.shape} E={e} mode={mode} ld={ld}", flush=True)
    c, s = _if4().quantize_ifn(to_dev(x, dtype, ld), bits, e, mode)
    torch.cuda.synchronize()
    gc, gs = c.cpu().numpy(), s.cpu().numpy()
    oc, os_ = oracle_mod.quantize_ifn(x, bits, e, mode)
    bad = np.nonzero(gs != os_)
    assert np.array_equal(gs, os_), (label, bad[0][:4], bad[1][:4], gs[bad][:4], os_[bad][:4])
    assert np.array_equal(gc, oc), label
    return c, s


def check_dq(oracle_mod, c, s, bits, e, label=""):
    want = oracle_mod.dequantize_ifn(c.cpu().numpy(), s.cpu().numpy(), bits, e)
    y32 = _if4().dequantize_ifn(c, s, bits, e, torch.float32)
    yb = _if4().dequantize_ifn(c, s, bits, e, torch.bfloat16)
    torch.cuda.synchronize()
    got = y32.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)) or \
        np.array_equal(np.isnan(got), np.isnan(want)) and \
        np.array_equal(np.where(np.isnan(got), 0, got).view(np.uint32),
                       np.where(np.isnan(want), 0, want).view(np.uint32)), label
    wb = torch.from_numpy(want).to(torch.bfloat16).float().numpy()
    gb = yb.float().cpu().numpy()
    assert np.array_equal(np.isnan(gb), np.isnan(wb))
    assert np.array_equal(np.where(np.isnan(gb), 0, gb).view(np.uint32),
                          np.where(np.isnan(wb), 0, wb).view(np.uint32)), label


def draw(shape, kind, seed, dtype):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        x = rng.standard_normal(shape)
    elif kind == "t4":
        x = rng.standard_t(4, shape) * 0.02
    elif kind == "uniform":
        x = rng.uniform(-1, 1, shape)
    else:  # wide exponents, subnormals included
        x = rng.standard_normal(shape) * np.exp2(rng.integers(-140, 120, shape))
    x = x.astype(np.float32)
    return wl.to_bf16_f32(x) if dtype == "bf16" else x


@pytest.mark.parametrize("bits", [3, 6])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(1, 16), (7, 48), (129, 1040)])
@pytest.mark.parametrize("kind", ["normal", "t4", "uniform"])
def test_parity_shapes_and_distributions(oracle_mod, bits, dtype, shape, kind):
    x = draw(shape, kind, shape[0] + bits, dtype)
    e = wl.tensor_scale_exp(float(np.abs(x).max()) * (6.0 / (7.5 if bits == 6 else 4.0)))
    c, s = check_q(oracle_mod, x, bits, dtype, e, label=kind)
    check_dq(oracle_mod, c, s, bits, e, label=kind)


@pytest.mark.parametrize("bits", [3, 6])
@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forced_modes(oracle_mod, bits, mode, dtype):
    x = draw((64, 256), "normal", 9, dtype)
    c, s = check_q(oracle_mod, x, bits, dtype, 0, mode, label="forced")
    check_dq(oracle_mod, c, s, bits, 0)


@pytest.mark.parametrize("bits", [3, 6])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("e", [-64, -20, 0, 30, 64])
def test_wide_values_and_exponents(oracle_mod, bits, dtype, e):
    x = draw((33, 512), "wide", 11, dtype)
    c, s = check_q(oracle_mod, x, bits, dtype, e, label="wide")
    check_dq(oracle_mod, c, s, bits, e)


@pytest.mark.parametrize("bits", [3, 6])
@pytest.mark.parametrize("tdt", ["f32", "bf16"])
def test_dequantize_strided_output_ragged(oracle_mod, bits, tdt):
    """Dequantize into rows of a wider buffer: 129 x 4112 is 33153 groups (519
    one-wave workgroups for IF3: 32 full runs of 16 for the XCD pairing and a
    remainder of 7), the padding past each row left untouched."""
    x = draw((129, 4112), "normal", 21, "bf16")
    c, s = check_q(oracle_mod, x, bits, "bf16", -3, label="dq strided")
    want = oracle_mod.dequantize_ifn(c.cpu().numpy(), s.cpu().numpy(), bits, -3)
    dt = torch.float32 if tdt == "f32" else torch.bfloat16
    big = torch.full((129, 4112 + 16), 7.0, dtype=dt, device="cuda")
    _if4().dequantize_ifn(c, s, bits, -3, out=big[:, :4112])
    torch.cuda.synchronize()
    got = big[:, :4112].float().cpu().numpy()
    wantt = torch.from_numpy(want).to(dt).float().numpy()
    assert np.array_equal(got.view(np.uint32), wantt.view(np.uint32))
    assert bool((big[:, 4112:] == 7.0).all())


@pytest.mark.parametrize("bits", [3, 6])
def test_edge_groups_and_strided_input(oracle_mod, bits):
    g = np.zeros((10, 16), np.float32)
    g[1, :] = -0.0
    g[2, 3] = np.inf
    g[3, 9] = np.nan
    g[4, :] = 3.0e38
    g[5, 0] = 1e-40
    g[6, :] = np.linspace(-7.5, 7.5, 16)
    g[7, :] = np.linspace(-4, 4, 16)
    g[8, :] = 2.0 ** -12
    g[9, ::2] = 1.0
    x = g.reshape(5, 32)
    for dtype in ("bf16", "f32"):
        xx = wl.to_bf16_f32(x) if dtype == "bf16" else x
        for e in (0, -12, 20):
            c, s = check_q(oracle_mod, xx, bits, dtype, e, label="edge")
            check_dq(oracle_mod, c, s, bits, e)
        check_q(oracle_mod, draw((20, 96), "t4", 3, dtype), bits, dtype, -8, ld=96 + 32,
                label="strided")


@pytest.mark.parametrize("bits", [3, 6])
@pytest.mark.parametrize("e", [0, -40, 40, -64, 64])
def test_ties_and_near_ties(oracle_mod, bits, e):
    """fp32 values at and next to every rounding boundary of both grids, in
    groups whose first element (top * s') pins the scale: exercises the
    rounding decisions themselves (ties to the even index, saturation)."""
    top, qmax = (7.5, 31) if bits == 6 else (4.0, 3)
    fp = sorted({float(v) for v in oracle_mod_grid(oracle_mod, bits)})
    vals = []
    for sc in (0x08, 0x23, 0x38, 0x3B, 0x55, 0x7E):
        s = (1 + (sc & 7) / 8) * 2.0 ** ((sc >> 3) - 7) * 2.0 ** e
        bounds = [(fp[k] + fp[k + 1]) / 2 * s for k in range(len(fp) - 1)]
        bounds += [(k + 0.5) * top / qmax * s for k in range(qmax)]
        cand = []
        for b in bounds:
            b32 = np.float32(b)
            cand += [b32, np.nextafter(b32, np.float32(0)), np.nextafter(b32, np.float32(np.inf))]
        cand = np.array(cand, np.float32)
        cand[1::2] *= -1
        for i in range(0, len(cand), 15):
            chunk = cand[i:i + 15]
            g = np.zeros(16, np.float32)
            g[0] = np.float32(top * s)
            g[1:1 + len(chunk)] = chunk
            vals.append(g)
    x = np.stack(vals).reshape(-1, 64) if len(vals) % 4 == 0 else np.stack(vals).reshape(1, -1)
    c, s_ = check_q(oracle_mod, x, bits, "f32", e, label="ties")
    check_dq(oracle_mod, c, s_, bits, e)
    assert (s_.cpu().numpy() & 0x7F).min() > 0


def oracle_mod_grid(oracle_mod, bits):
    return [oracle_mod.ifn_fp_value(bits, i) for i in range(1 << (bits - 1))]


@pytest.mark.parametrize("bits", [3, 6])
def test_dequantize_every_code(oracle_mod, bits):
    # every code under both flags and a spread of scale bytes (NaN scale included)
    nm = 1 << bits
    rows = []
    for flag in (0, 0x80):
        for sc in (0, 1, 7, 8, 0x2B, 0x38, 0x51, 0x7E, 0x7F):
            for start in range(0, nm, 16):
                cs = [(start + i) % nm for i in range(16)]
                field = sum(c << (bits * i) for i, c in enumerate(cs)).to_bytes(2 * bits, "little")
                rows.append((list(field), sc | flag))
    codes = torch.tensor([r[0] for r in rows], dtype=torch.uint8).cuda()
    scales = torch.tensor([[r[1]] for r in rows], dtype=torch.uint8).cuda()
    for e in (0, -30, 17):
        check_dq(oracle_mod, codes, scales, bits, e, label="all codes")


def test_full_size_activation(oracle_mod):
    """The activation workload (8192 x 4096 bf16 with outlier columns) in IF6
    and IF3, every group against the oracle."""
    t = wl.c2_activations()
    x = t.values
    for bits in (6, 3):
        e = wl.tensor_scale_exp(float(np.abs(x).max()) * (6.0 / (7.5 if bits == 6 else 4.0)))
        c, s = check_q(oracle_mod, x, bits, "bf16", e, label=t.name)
        gs = s.cpu().numpy()
        print(f"    IF{bits} int share {float((gs >= 0x80).mean()):.3f}", flush=True)


def test_full_size_weight_sampled(oracle_mod):
    """The FFN weight (28672 x 8192 bf16, Student-t) in IF6 and IF3 at the
    exponent and in the launch configuration bench.py times: the whole tensor
    goes through the kernels; 64 rows (the first two, the last, 61 seeded)
    are checked against the oracle, codes, scale bytes and the bf16
    dequantized values."""
    _, t = wl.c5_ffn()
    x = t.values
    n = x.shape[0]
    rows = np.unique(np.concatenate([[0, 1, n - 1],
                                     np.random.default_rng(5).choice(n, 61, replace=False)]))
    xd = to_dev(x, "bf16")
    for bits in (6, 3):
        print(f"[ifn] {t.name} IF{bits} E={t.scale_exp} sampled rows {len(rows)}", flush=True)
        c, s = _if4().quantize_ifn(xd, bits, t.scale_exp)
        y = _if4().dequantize_ifn(c, s, bits, t.scale_exp, torch.bfloat16)
        torch.cuda.synchronize()
        idx = torch.from_numpy(rows).cuda()
        gc, gs = c[idx].cpu().numpy(), s[idx].cpu().numpy()
        oc, os_ = oracle_mod.quantize_ifn(x[rows], bits, t.scale_exp, 0)
        assert np.array_equal(gs, os_), bits
        assert np.array_equal(gc, oc), bits
        want = torch.from_numpy(oracle_mod.dequantize_ifn(oc, os_, bits, t.scale_exp))
        assert torch.equal(y[idx].cpu(), want.to(torch.bfloat16)), bits
        del c, s, y


@pytest.mark.parametrize("bits", [3, 6])
def test_exhaustive_bf16_element_codes(oracle_mod, bits):
    """Every (bf16 |x| <= top s', E4M3 scale s') pair, both signs: groups
    [top s', x, ...] pin the scale at s', so each element's float and INT
    codes and both error sums are exercised for every representable bf16
    input (the bf16 kernel's snapped-quotient roundings against the oracle's
    exact ones), at E = 0 and, shifted, at E = 7 and E = -30."""
    top = 7.5 if bits == 6 else 4.0
    positive = np.arange(0, 0x7F80, dtype=np.uint32) << 16
    positive = positive.view(np.float32)
    rows = []
    for sc in range(1, 127):
        e, m = sc >> 3, sc & 7
        sp = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        xs = positive[positive <= top * sp * 1.0625]
        vals = np.concatenate([xs, -xs])
        pad = (-vals.size) % 15
        vals = np.concatenate([vals, np.zeros(pad, np.float32)]).reshape(-1, 15)
        grp = np.empty((vals.shape[0], 16), np.float32)
        grp[:, 0] = np.float32(top * sp)
        grp[:, 1:] = vals
        rows.append(grp)
    allg = np.concatenate(rows)
    pad = (-allg.shape[0]) % 64
    allg = np.concatenate([allg, np.zeros((pad, 16), np.float32)])
    x = allg.reshape(-1, 64 * 16)
    assert np.array_equal(wl.to_bf16_f32(x), x)
    print(f"[ifn] exhaustive bf16 sweep IF{bits}: {allg.shape[0]} groups", flush=True)
    for e in (0, 7, -30):
        # (the shift down by 2^30 rounds the smallest values to bf16 again)
        xe = wl.to_bf16_f32(np.ldexp(x, e).astype(np.float32))
        c, s_ = check_q(oracle_mod, xe, bits, "bf16", e, label=f"exhaustive E={e}")
        sc_seen = np.unique(s_.cpu().numpy() & 0x7F)
        assert sc_seen.size >= 126


@pytest.mark.parametrize("e", [0, -3, 5])
def test_if3_int_clamp_only_where_needed(oracle_mod, e):
    """IF3 runs its INT3 loop without the clamp in waves whose 64 groups all
    have ordinary scales.  Groups at that elision's bound (a/4 = 2^k * 1.0625
    exactly: the scale rounds down to 2^k and 3a/(4s) = 3.1875) fill every
    wave; every other wave also holds one group with an E4M3 subnormal scale
    (a = 5 * 2^-9 * 2^e: 3a/(4s) = 3.75) or one at the 448 code (a = 2304 *
    2^e: 3.86), which only the clamp brings back to 3.  Adaptive and with
    INT3 forced."""
    rng = np.random.default_rng(12)
    waves, gpw = 96, 64
    k = rng.integers(-4, 6, waves * gpw)
    amax = (4.25 * 2.0 ** k).astype(np.float32)  # 4 * 1.0625 * 2^k, exact in bf16
    x = np.empty((waves * gpw, 16), np.float32)
    x[:, 0] = amax
    tail = rng.uniform(-1, 1, (waves * gpw, 15)) * amax[:, None]
    x[:, 1:] = wl.to_bf16_f32(tail.astype(np.float32))
    for w in range(1, waves, 2):
        g = w * gpw + int(rng.integers(0, gpw))
        big = 5 * 2.0 ** -9 if w % 4 == 1 else 2304.0
        x[g, 0] = big
        x[g, 1:] = wl.to_bf16_f32((rng.uniform(0.9, 1.0, 15) * big).astype(np.float32))
    x = (x * np.float32(2.0 ** e)).astype(np.float32)
    for mode in (0, 2):
        check_q(oracle_mod, x.reshape(-1, 64 * 16), 3, "bf16", e, mode,
                label=f"IF3 clamp elision E={e}")
