"""Property-based pins of the oracle's quantizer (CPU only).

hypothesis draws whole 32-value blocks -- arbitrary bf16 or fp16 bit
patterns (NaN, inf, subnormals, signed zeros included) or fp32 values spread
over many binades -- and every block must quantize exactly as the brute-force checker
in brute.py says: the scale byte by comparison with powers of two, every
code by exhaustive nearest-grid-point search, the packing bit by bit.  The
checker shares no arithmetic with the oracle.
"""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import brute
import oracle
import workloads

MX = [oracle.FP6_E2M3, oracle.FP6_E3M2, oracle.FP4_E2M1, oracle.FP8_E4M3, oracle.AXS6]
EXMY = oracle.EXMY_FORMATS
SETTINGS = settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])

bf16_block = st.lists(st.integers(0, 0xFFFF), min_size=32, max_size=32)
# fp32 blocks: a shared binade plus per-value mantissas, signs and a few
# exact zeros, so that the rounding sees every part of the grid
fp32_block = st.tuples(
    st.integers(-140, 120),
    st.lists(st.tuples(st.floats(0.0, 2.0, allow_nan=False), st.booleans(), st.integers(-12, 0)),
             min_size=32, max_size=32))


def _bf16_vals(bits):
    with np.errstate(invalid="ignore"):
        return workloads.bf16_bits_to_f32(np.asarray(bits, np.uint16)).astype(np.float64)


def _check_block(fmt, x, vals):
    codes, scales, aux = oracle.quantize(fmt, x.reshape(1, 32))
    b, packed = brute.quantize_block(fmt, vals)
    assert scales[0, 0] == b, (vals, scales[0, 0], b)
    assert codes[0, 0].tobytes() == packed, vals
    if fmt == oracle.AXS6:
        assert not aux.any()


@pytest.mark.parametrize("fmt", MX + EXMY[::4], ids=lambda f: hex(f))
@SETTINGS
@given(bits=bf16_block)
def test_bf16_blocks_vs_brute_force(fmt, bits):
    x = np.asarray(bits, np.uint16)
    _check_block(fmt, x, _bf16_vals(x))


@pytest.mark.parametrize("fmt", MX + EXMY[2::4], ids=lambda f: hex(f))
@SETTINGS
@given(spec=fp32_block)
def test_fp32_blocks_vs_brute_force(fmt, spec):
    e, parts = spec
    x = np.array([(-1.0 if neg else 1.0) * m * 2.0 ** (e + k) for m, neg, k in parts], np.float32)
    _check_block(fmt, x, x.astype(np.float64))


@pytest.mark.parametrize("fmt", MX + EXMY[1::4], ids=lambda f: hex(f))
@SETTINGS
@given(bits=bf16_block)
def test_dequantize_of_quantize_is_fake_quantize(fmt, bits):
    x = np.asarray(bits, np.uint16).reshape(1, 32)
    codes, scales, aux = oracle.quantize(fmt, x)
    y = oracle.dequantize(fmt, codes, scales, aux, 1, 32, oracle.BF16)
    assert np.array_equal(y.view(np.uint16), oracle.fake_quantize(fmt, x).view(np.uint16))


@pytest.mark.parametrize("fmt", MX + EXMY[3::4], ids=lambda f: hex(f))
@SETTINGS
@given(bits=bf16_block)
def test_fp16_blocks_vs_brute_force(fmt, bits):
    # the same 16-bit patterns read as binary16 (numpy widens them exactly)
    x = np.asarray(bits, np.uint16).view(np.float16)
    _check_block(fmt, x, x.astype(np.float64))


@pytest.mark.parametrize("fmt", MX + EXMY[3::4], ids=lambda f: hex(f))
@SETTINGS
@given(bits=bf16_block)
def test_fp16_dequantize_of_quantize_is_fake_quantize(fmt, bits):
    x = np.asarray(bits, np.uint16).view(np.float16).reshape(1, 32)
    codes, scales, aux = oracle.quantize(fmt, x)
    y = oracle.dequantize(fmt, codes, scales, aux, 1, 32, oracle.F16)
    assert np.array_equal(y.view(np.uint16), oracle.fake_quantize(fmt, x).view(np.uint16))
