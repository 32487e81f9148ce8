"""Pins of the oracle's fp16 tensors (CPU only).

The "Online MXFP6" page ("Start a model") converts BF16 or FP16 weights.
The oracle reads binary16 values exactly and rounds results to binary16
once; both are pinned here to numpy's float16 (its conversions from and to
float64 are exact and correctly rounded), and quantization of every finite
fp16 pattern to the brute-force nearest-code search.
"""
import numpy as np
import pytest

import brute
import oracle

FMTS = [oracle.FP6_E2M3, oracle.FP6_E3M2, oracle.FP4_E2M1, oracle.FP8_E4M3, oracle.AXS6,
        oracle.exmy(3, 3), oracle.exmy(8, 0), oracle.exmy(0, 8)]
ids = ["e2m3", "e3m2", "e2m1", "e4m3", "axs6", "e3m3", "e8m0", "e0m8"]


def all_finite_f16():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    return h[np.isfinite(h)]


def _anchored(E, vals):
    """Blocks of 31 values and one anchor 2^E in slot 0 (fp16)."""
    n = (len(vals) + 30) // 31
    b = np.empty((n, 32), np.float16)
    b[:, 0] = np.float16(2.0 ** E)
    b[:, 1:] = np.resize(vals, n * 31).reshape(n, 31)
    return b


@pytest.mark.parametrize("fmt", FMTS, ids=ids)
def test_quantize_every_f16_pattern_vs_brute_force(fmt):
    allv = all_finite_f16()
    absv = np.abs(allv.astype(np.float64))
    for E in (-24, -14, -3, 0, 7, 15):
        blocks = _anchored(E, allv[absv < 2.0 ** (E + 1)])
        codes, scales, _ = oracle.quantize(fmt, blocks)
        vals = blocks.astype(np.float64)
        want_b = np.array([brute.scale_byte(fmt, v) for v in vals[:: max(1, len(vals) // 50)]])
        assert np.all(scales[:: max(1, len(vals) // 50), 0] == want_b), E
        assert np.all(scales == scales[0, 0]), E  # every block has the same anchor
        want = brute.encode_sorted(fmt, vals.reshape(-1), int(want_b[0])).reshape(-1, 32)
        got = np.array([brute.unpack(fmt, codes[i, 0].tobytes()) for i in range(len(blocks))])
        assert np.array_equal(got, want), E


@pytest.mark.parametrize("fmt", FMTS, ids=ids)
def test_dequantize_to_f16_is_the_rounded_exact_product(fmt):
    rng = np.random.default_rng(7 + fmt)
    rows, cols = 40, 64
    nb = rows * cols // 32
    bpb = oracle.BYTES_PER_BLOCK[fmt]
    codes = rng.integers(0, 256, (nb, bpb), dtype=np.uint8)
    scales = rng.integers(0, 255, nb, dtype=np.uint8)
    scales[:80] = np.arange(40, 200, 2, dtype=np.uint8)
    aux = np.zeros((nb + 3) // 4, np.uint8) if fmt == oracle.AXS6 else None
    y = oracle.dequantize(fmt, codes, scales, aux, rows, cols, oracle.F16).reshape(nb, 32)
    for b in range(nb):
        c = brute.unpack(fmt, codes[b].tobytes())
        exact = np.array([brute.decode(fmt, k) for k in c]) * 2.0 ** (int(scales[b]) - 127)
        with np.errstate(over="ignore", invalid="ignore"):
            want = exact.astype(np.float16)
        nan = np.isnan(want)
        assert np.array_equal(y[b][~nan].view(np.uint16), want[~nan].view(np.uint16)), b
        assert np.all(y[b][nan].view(np.uint16) == 0x7E00), b  # E4M3 NaN codes


@pytest.mark.parametrize("fmt", FMTS, ids=ids)
def test_fake_quantize_f16_equals_dequantize_of_quantize(fmt):
    rng = np.random.default_rng(30 + fmt)
    x = (rng.standard_t(3, (24, 96)) * np.exp2(rng.integers(-20, 12, (24, 1)))).astype(np.float16)
    x[0, 5] = np.nan
    x[1, :32] = 0.0
    x[2, 3] = -0.0
    x[3, 7] = np.inf
    fq = oracle.fake_quantize(fmt, x)
    codes, scales, aux = oracle.quantize(fmt, x)
    y = oracle.dequantize(fmt, codes, scales, aux, 24, 96, oracle.F16)
    assert np.array_equal(fq.view(np.uint16), y.view(np.uint16))
    assert np.all(fq[0, :32].view(np.uint16) == 0x7E00) and np.all(fq[3, :32].view(np.uint16) == 0x7E00)
    assert fq[2, 3].view(np.uint16) == 0x8000  # -0 keeps its sign


def test_f16_rounding_edges():
    # e4m3 code 0x7E (448) under scale bytes that put it at, over and far
    # over the largest fp16 (65504), and the smallest products
    f = oracle.FP8_E4M3
    codes = np.zeros((4, 32), np.uint8)
    codes[:, 0] = 0x7E
    codes[:, 1] = 0x01  # 2^-9
    scales = np.array([134, 135, 200, 112], np.uint8)
    y = oracle.dequantize(f, codes, scales, None, 4, 32, oracle.F16)
    # 448 * 2^7 = 57344; 448 * 2^8 = 114688 -> inf; 2^-9 * 2^-15 = 2^-24, the
    # smallest fp16 subnormal; 2^-9 * 2^7 = 2^-2
    assert y[0, 0] == 57344.0 and np.isinf(y[1, 0]) and np.isinf(y[2, 0])
    assert y[3, 1] == np.float16(2.0 ** -24) and y[0, 1] == 2.0 ** -2
