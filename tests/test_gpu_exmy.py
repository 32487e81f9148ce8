"""Generic eXmY formats on the GPU, bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import brute
import oracle
import workloads
from gpu_util import assert_bytes_equal, to_dev, to_host

pytestmark = pytest.mark.gpu

EXMY = oracle.EXMY_FORMATS
ids = [f"e{(f >> 4) & 15}m{f & 15}" for f in EXMY]


@pytest.fixture(scope="module")
def mx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_bit_amd as m
    return m


def _special(rng, rows, cols):
    x = (rng.standard_t(3, (rows, cols)) * np.exp2(rng.integers(-60, 60, (rows, 1)))).astype(np.float32)
    flat = x.reshape(-1, 32)
    k = max(1, flat.shape[0] // 40)
    pick = rng.choice(flat.shape[0], size=min(flat.shape[0], 5 * k), replace=False)
    flat[pick[:k]] = 0.0
    flat[pick[k:2 * k], 3] = np.nan
    flat[pick[2 * k:3 * k], 7] = -np.inf
    flat[pick[3 * k:4 * k]] *= np.float32(2.0 ** -100)
    flat[pick[4 * k:5 * k], ::3] = -0.0
    return x


@pytest.mark.parametrize("fmt", EXMY, ids=ids)
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_quantize_dequantize_fake_parity(mx, fmt, dtype):
    rng = np.random.default_rng(fmt)
    x = _special(rng, 67, 320)
    if dtype == "bf16":
        x = workloads.to_bf16_bits(x)
    xd = to_dev(x)
    codes, scales, _ = mx.quantize(xd, fmt)
    odt = torch.bfloat16 if dtype == "bf16" else torch.float32
    y = mx.dequantize(codes, scales, None, fmt, odt)
    fq = mx.fake_quantize(xd, fmt)
    torch.cuda.synchronize()
    oc, os_, _ = oracle.quantize(fmt, x)
    assert_bytes_equal(to_host(scales), os_, "scales")
    assert_bytes_equal(to_host(codes), oc, "codes", oracle.BYTES_PER_BLOCK[fmt])
    want = oracle.dequantize(fmt, oc, os_, None, 67, 320, oracle.BF16 if dtype == "bf16" else oracle.FP32)
    assert_bytes_equal(to_host(y), want, "dequantized")
    assert_bytes_equal(to_host(fq), oracle.fake_quantize(fmt, x), "fake-quantized")
    mx.fake_quantize(xd, fmt, out=xd)
    torch.cuda.synchronize()
    assert_bytes_equal(to_host(xd), want, "fake-quantized in place")


@pytest.mark.parametrize("fmt", EXMY, ids=ids)
def test_every_bf16_pattern_and_every_tie(mx, fmt):
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        v = workloads.bf16_bits_to_f32(allb).astype(np.float64)
    fin = allb[np.isfinite(v)]
    absv = np.abs(workloads.bf16_bits_to_f32(fin).astype(np.float64))
    blocks = []
    for E in (-126, -70, -3, 0, 5, 60, 126):
        sel = fin[absv < 2.0 ** (E + 1)]
        anchor = workloads.to_bf16_bits(np.array([2.0 ** E], np.float32))[0]
        n = (len(sel) + 30) // 31
        b = np.empty((n, 32), np.uint16)
        b[:, 0] = anchor
        b[:, 1:] = np.resize(sel, n * 31).reshape(n, 31)
        blocks.append(b)
    x = np.concatenate(blocks)
    codes, scales, _ = mx.quantize(to_dev(x), fmt)
    torch.cuda.synchronize()
    oc, os_, _ = oracle.quantize(fmt, x)
    assert_bytes_equal(to_host(scales), os_, "scales")
    assert_bytes_equal(to_host(codes), oc, "codes", oracle.BYTES_PER_BLOCK[fmt])
    # fp32 midpoints between neighbouring grid values, and their neighbours,
    # under X = 2^-sh (e8m0's grid reaches 2^128; half of it fits fp32)
    sh = max(0, brute.emax(fmt) - 127)
    g = brute.finite_grid(fmt) * 2.0 ** -sh
    mids = ((g[:-1] + g[1:]) / 2.0).astype(np.float32)
    vals = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e30)), -mids])
    nblk = (len(vals) + 30) // 31
    t = np.empty((nblk, 32), np.float32)
    t[:, 0] = np.float32(2.0 ** (brute.emax(fmt) - sh))
    t[:, 1:] = np.resize(vals, nblk * 31).reshape(nblk, 31)
    codes, scales, _ = mx.quantize(to_dev(t), fmt)
    torch.cuda.synchronize()
    oc, os_, _ = oracle.quantize(fmt, t)
    assert_bytes_equal(to_host(scales), os_, "tie scales")
    assert_bytes_equal(to_host(codes), oc, "tie codes", oracle.BYTES_PER_BLOCK[fmt])


@pytest.mark.parametrize("fmt", EXMY, ids=ids)
@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_dequantize_arbitrary_codes(mx, fmt, out):
    rng = np.random.default_rng(1000 + fmt)
    rows, cols = 33, 160
    nb = rows * cols // 32
    bpb = oracle.BYTES_PER_BLOCK[fmt]
    codes = rng.integers(0, 256, (nb, bpb), dtype=np.uint8)
    scales = rng.integers(0, 256, nb, dtype=np.uint8)
    scales[:min(nb, 256)] = np.arange(256, dtype=np.uint8)[:min(nb, 256)]
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    y = mx.dequantize(to_dev(codes).reshape(rows, cols // 32, bpb), to_dev(scales).reshape(rows, cols // 32),
                      None, fmt, odt)
    torch.cuda.synchronize()
    want = oracle.dequantize(fmt, codes, scales, None, rows, cols, oracle.BF16 if out == "bf16" else oracle.FP32)
    assert_bytes_equal(to_host(y), want, "dequantized")


def test_axs6_equals_e0m5_on_the_gpu(mx):
    x = workloads.axs6_weight(rows=128, cols=512)
    xd = to_dev(x)
    ca, sa, _ = mx.quantize(xd, "axs6")
    ce, se, _ = mx.quantize(xd, "e0m5")
    torch.cuda.synchronize()
    assert torch.equal(ca, ce)
    assert torch.equal(sa.to(torch.int32), se.to(torch.int32) + 4)
