"""The Python binding hands tensors to the C ABI as bare pointers and sizes,
so it must refuse any tensor whose shape, dtype, device or layout the kernel
would not expect -- before a kernel runs.  Each case below raises ValueError
(or TypeError for an unsupported dtype) with no launch."""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def if4():
    from adaptive_block_scaled_amd import if4
    return if4


@pytest.fixture(scope="module")
def operands(if4):
    g = torch.Generator().manual_seed(0)
    a = torch.randn(64, 128, generator=g).to(torch.bfloat16).cuda()
    w = torch.randn(96, 128, generator=g).to(torch.bfloat16).cuda()
    ac, as_ = if4.quantize(a)
    wc, ws = if4.quantize(w)
    torch.cuda.synchronize()
    return a, ac, as_, wc, ws


def test_quantize_outputs_checked(if4, operands):
    a, ac, as_, _, _ = operands
    u8 = dict(dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="codes"):
        if4.quantize(a, out=(torch.empty(64, 63, **u8), torch.empty(64, 8, **u8)))
    with pytest.raises(ValueError, match="scales"):
        if4.quantize(a, out=(torch.empty(64, 64, **u8), torch.empty(64, 9, **u8)))
    with pytest.raises(ValueError, match="codes"):
        if4.quantize(a, out=(torch.empty(64, 64, dtype=torch.int32, device="cuda"),
                             torch.empty(64, 8, **u8)))
    with pytest.raises(ValueError, match="contiguous"):
        if4.quantize(a, out=(torch.empty(64, 128, **u8)[:, :64], torch.empty(64, 8, **u8)))
    with pytest.raises(ValueError, match="CUDA"):
        if4.quantize(a, out=(torch.empty(64, 64, dtype=torch.uint8), torch.empty(64, 8, **u8)))
    with pytest.raises(ValueError, match="codes"):
        if4.quantize_ifn(a, 6, out=(torch.empty(64, 8 * 11, **u8), torch.empty(64, 8, **u8)))
    with pytest.raises(ValueError, match="codes"):
        if4.quantize_t(a, out=(torch.empty(64, 64, **u8), torch.empty(128, 4, **u8)))
    with pytest.raises(ValueError, match="x must"):
        if4.quantize(a.cpu())


def test_dequantize_and_gemm_inputs_checked(if4, operands):
    _, ac, as_, wc, ws = operands
    with pytest.raises(ValueError, match="scales"):
        if4.dequantize(ac, as_[:, :7])
    with pytest.raises(ValueError, match="contiguous"):
        if4.dequantize(ac[:, ::2], as_[:, :4])
    with pytest.raises(ValueError, match="out"):
        if4.dequantize(ac, as_, out=torch.empty(64, 127, device="cuda"))
    with pytest.raises(TypeError):
        if4.dequantize(ac, as_, out=torch.empty(64, 128, dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError, match="a_scales"):
        if4.gemm(ac, as_[:32], 0, wc, ws, 0)
    with pytest.raises(ValueError, match="w_codes"):
        if4.gemm(ac, as_, 0, wc.float(), ws, 0)
    with pytest.raises(ValueError, match="out"):
        if4.gemm(ac, as_, 0, wc, ws, 0, out=torch.empty(64, 95, device="cuda"))
    with pytest.raises(ValueError, match="out"):
        if4.gemm(ac, as_, 0, wc, ws, 0, out=torch.empty(64, 96, dtype=torch.bfloat16,
                                                         device="cuda"))


def test_strided_outputs_accepted(if4, operands):
    # an output with a row stride (unit stride along dim 1) is allowed and
    # written only in its own columns
    a, ac, as_, wc, ws = operands
    want_y = if4.dequantize(ac, as_)
    big = torch.full((64, 160), 7.0, device="cuda")
    y = if4.dequantize(ac, as_, out=big[:, :128])
    want_c = if4.gemm(ac, as_, 0, wc, ws, 0)
    bigc = torch.full((64, 100), 7.0, device="cuda")
    c = if4.gemm(ac, as_, 0, wc, ws, 0, out=bigc[:, :96])
    ifn = {}
    for bits in (6, 3):
        nc, ns = if4.quantize_ifn(a, bits)
        bign = torch.full((64, 144), 7.0, dtype=torch.bfloat16, device="cuda")
        ifn[bits] = (if4.dequantize_ifn(nc, ns, bits, 0, torch.bfloat16),
                     if4.dequantize_ifn(nc, ns, bits, 0, out=bign[:, :128]), bign)
    torch.cuda.synchronize()
    assert torch.equal(y, want_y) and bool((big[:, 128:] == 7.0).all())
    assert torch.equal(c, want_c) and bool((bigc[:, 96:] == 7.0).all())
    for bits, (want_n, got_n, bign) in ifn.items():
        assert torch.equal(got_n, want_n), bits
        assert bool((bign[:, 128:] == 7.0).all()), bits


def test_runs_on_the_callers_stream(if4, operands):
    # every entry point enqueues on torch's current stream: the same path on
    # a side stream (default priority) gives the default stream's results
    a, ac, as_, wc, ws = operands
    want = (if4.quantize(a), if4.dequantize(ac, as_, 0, torch.bfloat16),
            if4.gemm(ac, as_, 0, wc, ws, 0), if4.quantize_ifn(a, 6), if4.quantize_t(a),
            if4.quantize_rht(a, 0x1234))
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = (if4.quantize(a), if4.dequantize(ac, as_, 0, torch.bfloat16),
               if4.gemm(ac, as_, 0, wc, ws, 0), if4.quantize_ifn(a, 6), if4.quantize_t(a),
               if4.quantize_rht(a, 0x1234))
    side.synchronize()
    torch.cuda.synchronize()
    flat = lambda r: [t for x in r for t in (x if isinstance(x, tuple) else (x,))]
    for g, w in zip(flat(got), flat(want)):
        assert torch.equal(g, w)
