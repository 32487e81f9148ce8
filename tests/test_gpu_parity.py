"""Bit-exact parity of the HIP path (through the C ABI) with the CPU oracle.

Small and ragged shapes, every finite bf16 pattern and arbitrary code and
scale bytes are compared element by element (the full-size workloads, whole
tensors, are in test_gpu_full.py).  Every comparison is bytewise: codes,
scales, the AXS-6 config plane, and dequantized / fake-quantized values
(exact power-of-two products).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import assert_bytes_equal, to_dev, to_host

pytestmark = pytest.mark.gpu

FMTS = [0, 1, 2, 3, 4]
FMT_NAMES = {0: "e2m3", 1: "e3m2", 2: "e2m1", 3: "e4m3", 4: "axs6"}
BPB = oracle.BYTES_PER_BLOCK


@pytest.fixture(scope="module")
def mx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_bit_amd as m
    return m


def _special_input(rng, rows, cols, dtype):
    x = (rng.standard_t(3, (rows, cols)) * np.exp2(rng.integers(-40, 40, (rows, 1)))).astype(np.float32)
    flat = x.reshape(-1)
    nb = flat.size // 32
    blocks = flat.reshape(nb, 32)
    k = max(1, nb // 50)
    pick = rng.choice(nb, size=min(nb, 6 * k), replace=False)
    blocks[pick[:k]] = 0.0                                   # zero blocks
    blocks[pick[k:2 * k]] = -0.0                             # negative zero blocks
    blocks[pick[2 * k:3 * k], rng.integers(0, 32)] = np.nan   # NaN somewhere
    blocks[pick[3 * k:4 * k], rng.integers(0, 32)] = np.inf
    blocks[pick[4 * k:5 * k], rng.integers(0, 32)] = -np.inf
    blocks[pick[5 * k:6 * k]] *= np.float32(2.0 ** -135)     # subnormal blocks
    if dtype == "bf16":
        return workloads.to_bf16_bits(x)
    return x


def _gpu_quantize(mx, fmt, x_host):
    x = to_dev(x_host)
    codes, scales, aux = mx.quantize(x, fmt)
    torch.cuda.synchronize()
    return to_host(codes), to_host(scales), (to_host(aux) if aux is not None else None)


SHAPES = [(1, 32), (3, 96), (67, 4096), (257, 160), (1000, 32)]


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: FMT_NAMES[f])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_quantize_parity(mx, fmt, dtype, shape):
    rng = np.random.default_rng(1000 * fmt + 100 * (dtype == "bf16") + SHAPES.index(shape))
    x = _special_input(rng, *shape, dtype)
    gc, gs, ga = _gpu_quantize(mx, fmt, x)
    oc, os_, oa = oracle.quantize(fmt, x)
    assert_bytes_equal(gs, os_, "scales")
    assert_bytes_equal(gc, oc, "codes", BPB[fmt])
    if fmt == 4:
        assert_bytes_equal(ga, oa, "aux")


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: FMT_NAMES[f])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_quantize_every_bf16_pattern(mx, fmt, dtype):
    # every finite bf16 pattern under 20 scale regimes (as the oracle's
    # exhaustive pin), through the GPU
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        vals = workloads.bf16_bits_to_f32(allb)
    fin = allb[np.isfinite(vals)]
    absv = np.abs(workloads.bf16_bits_to_f32(fin).astype(np.float64))
    blocks = []
    for E in (-133, -130, -126, -120, -60, -8, -1, 0, 1, 2, 3, 4, 5, 8, 9, 40, 100, 125, 126, 127):
        sel = fin[absv < 2.0 ** (E + 1)]
        anchor = workloads.to_bf16_bits(np.array([2.0 ** E], np.float32))[0]
        n = (len(sel) + 30) // 31
        b = np.empty((n, 32), np.uint16)
        b[:, 0] = anchor
        b[:, 1:] = np.resize(sel, n * 31).reshape(n, 31)
        blocks.append(b)
    x = np.concatenate(blocks)
    if dtype == "fp32":
        x = workloads.bf16_bits_to_f32(x)
    gc, gs, ga = _gpu_quantize(mx, fmt, x)
    oc, os_, oa = oracle.quantize(fmt, x)
    assert_bytes_equal(gs, os_, "scales")
    assert_bytes_equal(gc, oc, "codes", BPB[fmt])


def _random_packed(rng, fmt, nb):
    """Arbitrary code bytes and scale bytes (every code value, every byte,
    0xFF blocks, and for AXS-6 nonzero configs)."""
    codes = rng.integers(0, 256, (nb, BPB[fmt]), dtype=np.uint8)
    scales = rng.integers(0, 256, nb, dtype=np.uint8)
    scales[:256] = np.arange(256, dtype=np.uint8)[: min(256, nb)]
    aux = np.zeros((nb + 3) // 4, np.uint8)
    if fmt == 4:
        aux[::3] = rng.integers(0, 256, aux[::3].size, dtype=np.uint8)
    return codes, scales, aux


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: FMT_NAMES[f])
@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_dequantize_parity(mx, fmt, out):
    rng = np.random.default_rng(20 + fmt)
    rows, cols = 97, 320
    nb = rows * cols // 32
    codes, scales, aux = _random_packed(rng, fmt, nb)
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    y = mx.dequantize(to_dev(codes).reshape(rows, cols // 32, BPB[fmt]),
                      to_dev(scales).reshape(rows, cols // 32),
                      to_dev(aux) if fmt == 4 else None, fmt, odt)
    torch.cuda.synchronize()
    want = oracle.dequantize(fmt, codes, scales, aux, rows, cols,
                             oracle.BF16 if out == "bf16" else oracle.FP32)
    assert_bytes_equal(to_host(y), want, "dequantized", 64 if out == "bf16" else 128)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: FMT_NAMES[f])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_fake_quantize_parity_and_in_place(mx, fmt, dtype):
    rng = np.random.default_rng(30 + fmt)
    x = _special_input(rng, 131, 224, dtype)
    want = oracle.fake_quantize(fmt, x)
    xd = to_dev(x)
    y = mx.fake_quantize(xd, fmt)
    torch.cuda.synchronize()
    assert_bytes_equal(to_host(y), want, "fake-quantized")
    mx.fake_quantize(xd, fmt, out=xd)  # in place
    torch.cuda.synchronize()
    assert_bytes_equal(to_host(xd), want, "fake-quantized in place")


@pytest.mark.parametrize("fmt", [0, 1, 2, 3], ids=lambda f: FMT_NAMES[f])
@pytest.mark.parametrize("cols", [32, 1024, 2048 - 32, 2048, 4096, 4096 + 96, 8192, 8192 + 32])
def test_softmax_quantize_parity(mx, fmt, cols):
    # the column counts cover rows held in registers (up to 64, 128, 256 and
    # 512 half blocks per row, one block per lane pair), exactly filling the
    # lanes or not, and rows streamed twice (longer); 32 is a row of one block
    s = workloads.attn_scores(rows=37, cols=cols)
    s[3, 11] = np.nan
    s[4, 5] = np.inf
    s[5, :] = -np.inf
    s[6, :] = 0.0
    s[7] = np.linspace(-200, 0, s.shape[1], dtype=np.float32)  # underflow and subnormal P
    s[8, ::2] = -np.inf
    codes, scales = mx.softmax_quantize(to_dev(s), fmt)
    torch.cuda.synchronize()
    oc, os_ = oracle.softmax_quantize(fmt, s)
    assert_bytes_equal(to_host(scales), os_, "scales")
    assert_bytes_equal(to_host(codes), oc, "codes", BPB[fmt])


@pytest.mark.parametrize("fmt", [0, 1, 2, 3], ids=lambda f: FMT_NAMES[f])
@pytest.mark.parametrize("cols", [32 * 33, 4096 + 96, 8192 + 32])
def test_softmax_quantize_writes_only_its_bytes(mx, fmt, cols):
    # rows whose last lane pairs hold no block: codes and scales end exactly
    # at the tensor's end, and every byte in between is written
    rows = 7
    s = workloads.attn_scores(rows=rows, cols=cols)
    nb = rows * cols // 32
    guard = 4096
    cbuf = torch.full((guard + nb * BPB[fmt] + guard,), 0xA5, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((guard + nb + guard,), 0xA5, dtype=torch.uint8, device="cuda")
    st = mx.mx_softmax_quantize(fmt, 32, to_dev(s), rows, cols, cbuf[guard:guard + nb * BPB[fmt]],
                                sbuf[guard:guard + nb])
    assert st == 0
    torch.cuda.synchronize()
    c, sc = to_host(cbuf), to_host(sbuf)
    assert np.all(c[:guard] == 0xA5) and np.all(c[guard + nb * BPB[fmt]:] == 0xA5)
    assert np.all(sc[:guard] == 0xA5) and np.all(sc[guard + nb:] == 0xA5)
    oc, os_ = oracle.softmax_quantize(fmt, s)
    assert_bytes_equal(sc[guard:guard + nb], os_, "scales")
    assert_bytes_equal(c[guard:guard + nb * BPB[fmt]], oc, "codes", BPB[fmt])


def test_softmax_quantize_short_rows(mx):
    s = workloads.attn_scores(rows=300, cols=32 * 5)
    codes, scales = mx.softmax_quantize(to_dev(s), "mxfp4")
    torch.cuda.synchronize()
    oc, os_ = oracle.softmax_quantize(2, s)
    assert_bytes_equal(to_host(scales), os_, "scales")
    assert_bytes_equal(to_host(codes), oc, "codes", 16)


# ----------------------------------------------------------------------------
# write coverage, guard bands, determinism, host errors with device tensors
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: FMT_NAMES[f])
def test_every_output_byte_written_and_no_spill(mx, fmt):
    rows, cols = 45, 1056
    nb = rows * cols // 32
    x = to_dev(_special_input(np.random.default_rng(40), rows, cols, "bf16"))
    guard = 4096
    cbuf = torch.full((guard + nb * BPB[fmt] + guard,), 0xA5, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((guard + nb + guard,), 0xA5, dtype=torch.uint8, device="cuda")
    abuf = torch.full((guard + (nb + 3) // 4 + guard,), 0xA5, dtype=torch.uint8, device="cuda")
    st = mx.mx_quantize(fmt, 32, mx.MX_BF16, x, rows, cols, cbuf[guard:], sbuf[guard:],
                        abuf[guard:] if fmt == 4 else None)
    assert st == 0
    torch.cuda.synchronize()
    c, s, a = to_host(cbuf), to_host(sbuf), to_host(abuf)
    assert np.all(c[:guard] == 0xA5) and np.all(c[guard + nb * BPB[fmt]:] == 0xA5)
    assert np.all(s[:guard] == 0xA5) and np.all(s[guard + nb:] == 0xA5)
    oc, os_, oa = oracle.quantize(fmt, to_host(x))
    assert_bytes_equal(c[guard:guard + nb * BPB[fmt]], oc, "codes", BPB[fmt])
    assert_bytes_equal(s[guard:guard + nb], os_, "scales")
    if fmt == 4:
        assert_bytes_equal(a[guard:guard + (nb + 3) // 4], oa, "aux")
        assert np.all(a[guard + (nb + 3) // 4:] == 0xA5)


def test_deterministic_repeat(mx):
    x = to_dev(workloads.linear_weight(rows=512, cols=4096))
    a = mx.quantize(x, 0)
    b = mx.quantize(x, 0)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_device_argument_errors(mx):
    x = torch.zeros(4, 64, dtype=torch.bfloat16, device="cuda")
    codes, scales, _ = mx.quantize(x, 0)
    # misaligned view of x (offset 2 bytes)
    flat = torch.zeros(4 * 64 + 1, dtype=torch.bfloat16, device="cuda")
    assert mx.mx_quantize(0, 32, 0, flat[1:], 4, 64, codes, scales, None) == 3
    assert mx.mx_quantize(0, 32, 0, x, 4, 48, codes, scales, None) == 2
    assert mx.mx_quantize(4, 32, 0, x, 4, 64, codes, scales, None) == 1
    assert mx.mx_quantize(0, 64, 0, x, 4, 64, codes, scales, None) == 4
    assert mx.mx_softmax_quantize(4, 32, x, 4, 64, codes, scales) == 4
    assert mx.mx_quantize(0, 32, 0, x, 0, 64, codes, scales, None) == 0


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: FMT_NAMES[f])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("nblocks", [1, 63, 64, 65, 1000])
def test_wide_outputs_stay_in_bounds(mx, fmt, dtype, nblocks):
    # dequantize and fake-quantize write whole 64-block tiles through LDS;
    # a ragged last tile must write exactly its own bytes and nothing after
    rng = np.random.default_rng(50 + nblocks)
    rows, cols = nblocks, 32
    x = _special_input(rng, rows, cols, dtype)
    elt = 2 if dtype == "bf16" else 4
    guard = 4096
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    ybuf = torch.full((guard + rows * cols + guard,), float("nan"), dtype=tdt, device="cuda")
    ybuf.view(torch.int16 if dtype == "bf16" else torch.int32).fill_(0x5A5A)
    sentinel = to_host(ybuf[:guard]).copy()
    xd = to_dev(x)
    assert mx.mx_fake_quantize(fmt, 32, mx.MX_BF16 if dtype == "bf16" else mx.MX_FP32, xd,
                               ybuf[guard:guard + rows * cols], rows, cols) == 0
    torch.cuda.synchronize()
    yh = to_host(ybuf)
    assert np.array_equal(yh[:guard], sentinel) and np.array_equal(yh[guard + rows * cols:], sentinel)
    assert_bytes_equal(yh[guard:guard + rows * cols], oracle.fake_quantize(fmt, x).reshape(-1), "fq")
    oc, os_, oa = oracle.quantize(fmt, x)
    ybuf.view(torch.int16 if dtype == "bf16" else torch.int32).fill_(0x5A5A)
    assert mx.mx_dequantize(fmt, 32, to_dev(oc), to_dev(os_), to_dev(oa) if fmt == 4 else None,
                            rows, cols, mx.MX_BF16 if dtype == "bf16" else mx.MX_FP32,
                            ybuf[guard:guard + rows * cols]) == 0
    torch.cuda.synchronize()
    yh = to_host(ybuf)
    assert np.array_equal(yh[:guard], sentinel) and np.array_equal(yh[guard + rows * cols:], sentinel)
    want = oracle.dequantize(fmt, oc, os_, oa, rows, cols, oracle.BF16 if dtype == "bf16" else oracle.FP32)
    assert_bytes_equal(yh[guard:guard + rows * cols], want.reshape(-1), "dq", 32 * elt)
