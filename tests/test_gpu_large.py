"""Tensors that extend past 2^31 bytes.

Every kernel addresses blocks and rows with 64-bit arithmetic; none of the
benchmark's workloads reaches a byte offset of 2^31 (the largest, 2 GiB of
fp32 scores, ends exactly there).  test_gpu_full.py's 4.8 GB tensor covers
the E2M3 quantize and dequantize; these add fake-quantize, E4M3, the batched
quantize and the exp-then-quantize rows (with the fp32 dequantization of
the probabilities): sampled rows before and after the 2^31-byte mark are
compared with the oracle bit for bit.
"""
import pytest
import torch

import oracle
from gpu_util import assert_bytes_equal, to_host

pytestmark = pytest.mark.gpu

ROWS, COLS = 1 << 19, 4096        # 2^31 bf16 values: 4 GiB in
BF16_ROWS = [0, 1, 262143, 262144, 300001, ROWS - 1]  # row 262144 starts at byte 2^31
SROWS = 140000                    # fp32 scores of 4096 keys: 2.29 GB
S_ROWS = [0, 131071, 131072, 137777, SROWS - 1]       # row 131072 starts at byte 2^31


@pytest.fixture(scope="module")
def mx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_bit_amd as m
    return m


@pytest.fixture(scope="module")
def big_bf16():
    g = torch.Generator(device="cuda").manual_seed(7)
    x = torch.empty(ROWS, COLS, dtype=torch.bfloat16, device="cuda")
    for r0 in range(0, ROWS, 1 << 16):  # drawn in slices to bound the fp32 temporary
        x[r0:r0 + (1 << 16)] = (torch.randn(1 << 16, COLS, generator=g, device="cuda")
                                * 0.02).bfloat16()
    yield x
    del x
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", [oracle.FP6_E2M3, oracle.FP8_E4M3], ids=["e2m3", "e4m3"])
def test_bf16_quantize_dequantize_fake_past_2_31_bytes(mx, big_bf16, fmt):
    x = big_bf16
    codes, scales, _ = mx.quantize(x, fmt)
    y = mx.dequantize(codes, scales, None, fmt, torch.bfloat16)
    torch.cuda.synchronize()
    for r in BF16_ROWS:
        xr = to_host(x[r:r + 1])
        oc, os_, _ = oracle.quantize(fmt, xr)
        assert_bytes_equal(to_host(scales[r]), os_, f"row {r} scales")
        assert_bytes_equal(to_host(codes[r]), oc, f"row {r} codes", oracle.BYTES_PER_BLOCK[fmt])
        oy = oracle.dequantize(fmt, oc, os_, None, 1, COLS, oracle.BF16)
        assert_bytes_equal(to_host(y[r:r + 1]), oy, f"row {r} dequantized", 64)
    del y, codes, scales
    fq = mx.fake_quantize(x, fmt)
    torch.cuda.synchronize()
    for r in BF16_ROWS:
        xr = to_host(x[r:r + 1])
        assert_bytes_equal(to_host(fq[r:r + 1]), oracle.fake_quantize(fmt, xr),
                           f"row {r} fake-quantized", 64)
    del fq
    torch.cuda.empty_cache()


def test_batched_quantize_past_2_31_bytes(mx, big_bf16):
    x = big_bf16
    small = x[:64].clone()
    (codes, scales, _), (c2, s2, _) = mx.quantize_many([x, small], oracle.FP6_E2M3)
    torch.cuda.synchronize()
    for r in BF16_ROWS:
        oc, os_, _ = oracle.quantize(oracle.FP6_E2M3, to_host(x[r:r + 1]))
        assert_bytes_equal(to_host(scales[r]), os_, f"row {r} scales")
        assert_bytes_equal(to_host(codes[r]), oc, f"row {r} codes", 24)
    oc, os_, _ = oracle.quantize(oracle.FP6_E2M3, to_host(small))
    assert_bytes_equal(to_host(c2), oc, "second tensor codes", 24)
    assert_bytes_equal(to_host(s2), os_, "second tensor scales")
    del codes, scales, c2, s2
    torch.cuda.empty_cache()


def test_scores_past_2_31_bytes(mx):
    g = torch.Generator(device="cuda").manual_seed(8)
    s = torch.randn(SROWS, 4096, generator=g, device="cuda") * 3.0
    codes, scales = mx.softmax_quantize(s, "mxfp4")
    p = mx.dequantize(codes, scales, None, oracle.FP4_E2M1, torch.float32)
    torch.cuda.synchronize()
    for r in S_ROWS:
        oc, os_ = oracle.softmax_quantize(oracle.FP4_E2M1, to_host(s[r:r + 1]))
        assert_bytes_equal(to_host(scales[r]), os_, f"row {r} scales")
        assert_bytes_equal(to_host(codes[r]), oc, f"row {r} codes", 16)
        op = oracle.dequantize(oracle.FP4_E2M1, oc, os_, None, 1, 4096, oracle.FP32)
        assert_bytes_equal(to_host(p[r:r + 1]), op, f"row {r} probabilities", 128)
    del s, codes, scales, p
    torch.cuda.empty_cache()
