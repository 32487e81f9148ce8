"""Pins of the CPU oracle to things other than itself (CPU only).

Each test fixes a part of the oracle with a library dtype, a closed form, an
invariant or an exhaustive brute-force search (tests/brute.py), so that a
dropped term, a wrong sign, a wrong index or a transposed operand anywhere in
oracle/mxref.c fails at least one of them.
"""
import json
import os
import re

import numpy as np
import pytest
import torch

import brute
import oracle
import workloads

FMTS = [oracle.FP6_E2M3, oracle.FP6_E3M2, oracle.FP4_E2M1, oracle.FP8_E4M3, oracle.AXS6]
MX_FMTS = FMTS[:4]
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32_from_bits(u):
    return np.asarray(u, dtype=np.uint32).view(np.float32)


def bf16_to_f64(b):
    with np.errstate(invalid="ignore"):
        return workloads.bf16_bits_to_f32(np.asarray(b, np.uint16)).astype(np.float64)


def all_finite_bf16():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return b[np.isfinite(bf16_to_f64(b))]


# ----------------------------------------------------------------------------
# (a) format tables
# ----------------------------------------------------------------------------
def test_e4m3_decode_is_torch_float8_e4m3fn():
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    ours = np.array([oracle.decode(oracle.FP8_E4M3, c) for c in range(256)])
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])
    fin = ~np.isnan(lib)
    assert np.array_equal(ours[fin], lib[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(lib[fin]))


@pytest.mark.parametrize("fmt", FMTS)
def test_grids_match_structural_derivation(fmt):
    bits = oracle.CODE_BITS[fmt]
    half = 1 << (bits - 1)
    mags = np.array([oracle.decode(fmt, c) for c in range(half)])
    g = brute.grid(fmt)
    assert np.array_equal(np.isnan(mags), np.isnan(g))
    fin = ~np.isnan(g)
    assert np.array_equal(mags[fin], g[fin])
    neg = np.array([oracle.decode(fmt, c | half) for c in range(half)])
    assert np.array_equal(neg[fin], -mags[fin])
    assert np.all(np.signbit(neg[fin]))
    # magnitude codes are ordered by value
    assert np.all(np.diff(mags[fin]) > 0)


def test_format_ranges():
    # largest finite, smallest normal, smallest subnormal per format
    expect = {oracle.FP6_E2M3: (7.5, 1.0, 0.125), oracle.FP6_E3M2: (28.0, 0.25, 0.0625),
              oracle.FP4_E2M1: (6.0, 1.0, 0.5), oracle.FP8_E4M3: (448.0, 2.0 ** -6, 2.0 ** -9)}
    for fmt, (mx, mn, sub) in expect.items():
        g = brute.finite_grid(fmt)
        assert g.max() == mx and g[1] == sub
        assert oracle.decode(fmt, 1) == sub
        mbits = {0: 3, 1: 2, 2: 1, 3: 3}[fmt]
        assert oracle.decode(fmt, 1 << mbits) == mn
    assert brute.finite_grid(oracle.AXS6).max() == 31 / 16


def test_e8m0_scale_decode_is_torch_float8_e8m0fnu():
    # dequantize one E4M3 block holding the code for 1.0 under every scale byte
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).float().numpy()
    nb = 256
    one = 0x38  # E4M3 1.0
    codes = np.full((nb, 32), one, np.uint8)
    scales = np.arange(256, dtype=np.uint8)
    y = oracle.dequantize(oracle.FP8_E4M3, codes, scales, None, nb, 32, oracle.FP32)
    assert np.all(np.isnan(y[255]))
    assert np.array_equal(y[:255, 0], lib[:255])
    assert np.array_equal(y[255].view(np.uint32), np.full(32, 0x7FC00000, np.uint32))


# ----------------------------------------------------------------------------
# (b) exhaustive brute force: every bf16 pattern under many scale regimes
# ----------------------------------------------------------------------------
ANCHOR_EXPONENTS = [-133, -131, -128, -126, -125, -120, -60, -8, -3, -1, 0, 1, 2, 3, 5,
                    9, 40, 100, 125, 127]


def _anchored_blocks(E, values_bits):
    """Blocks of 31 test values + one anchor 2^E at slot 0 (bf16 bits)."""
    anchor = workloads.to_bf16_bits(np.array([2.0 ** E], np.float32))[0]
    assert bf16_to_f64([anchor])[0] == 2.0 ** E
    n = len(values_bits)
    nblk = (n + 30) // 31
    pad = np.resize(values_bits, nblk * 31)
    blocks = np.empty((nblk, 32), np.uint16)
    blocks[:, 0] = anchor
    blocks[:, 1:] = pad.reshape(nblk, 31)
    return blocks


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_bf16_exhaustive_vs_brute_force(fmt):
    allv = all_finite_bf16()
    absv = np.abs(bf16_to_f64(allv))
    for E in ANCHOR_EXPONENTS:
        sel = allv[absv < 2.0 ** (E + 1)]
        blocks = _anchored_blocks(E, sel)
        codes, scales, _ = oracle.quantize(fmt, blocks)
        want_b = brute.scale_byte(fmt, bf16_to_f64(blocks[0]))
        assert np.all(scales == want_b), (fmt, E)
        vals = bf16_to_f64(blocks).reshape(-1)
        want_codes = brute.encode(fmt, vals, want_b).reshape(-1, 32)
        got = [brute.unpack(fmt, codes[i, 0].tobytes()) for i in range(len(blocks))]
        assert np.array_equal(np.array(got), want_codes), (fmt, E)
        # the packed bytes themselves, for a handful of blocks
        for i in range(0, len(blocks), max(1, len(blocks) // 7)):
            assert codes[i, 0].tobytes() == brute.pack(fmt, want_codes[i]), (fmt, E, i)


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_fp32_ties_and_neighbours(fmt):
    # exact midpoints between neighbouring grid values, and one fp32 ulp
    # either side, in the block whose scale byte is 127 and around it
    g = brute.finite_grid(fmt)
    mids = (g[:-1] + g[1:]) / 2.0
    m32 = mids.astype(np.float32)
    assert np.array_equal(m32.astype(np.float64), mids)
    vals = np.concatenate([m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1e9)),
                           g.astype(np.float32)])
    vals = np.concatenate([vals, -vals])
    top = np.float32(2.0 ** brute.emax(fmt))
    for k in (0, -3, 7):
        scale = np.float32(2.0 ** k)
        blocks = _anchor_f32(vals * scale, top * scale)
        codes, scales, _ = oracle.quantize(fmt, blocks)
        assert np.all(scales == 127 + k)
        want = brute.encode(fmt, blocks.reshape(-1).astype(np.float64), 127 + k).reshape(-1, 32)
        got = np.array([brute.unpack(fmt, codes[i, 0].tobytes()) for i in range(len(blocks))])
        assert np.array_equal(got, want), (fmt, k)


def _anchor_f32(values, anchor):
    n = len(values)
    nblk = (n + 30) // 31
    blocks = np.empty((nblk, 32), np.float32)
    blocks[:, 0] = anchor
    blocks[:, 1:] = np.resize(values, nblk * 31).reshape(nblk, 31)
    return blocks


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_random_blocks_vs_brute_force(fmt, dtype):
    rng = np.random.default_rng(100 + fmt)
    x = (rng.standard_normal((64, 32)) * np.exp2(rng.integers(-20, 20, (64, 1)))).astype(np.float32)
    x[3, 5] = np.nan
    x[4, 0] = np.inf
    x[5, 31] = -np.inf
    x[6] = 0.0
    x[7] = -0.0
    x[8, ::2] = -0.0
    x[9] = np.float32(1e-40)  # fp32 subnormals
    x[10] = rng.standard_normal(32).astype(np.float32) * np.float32(2.0 ** -130)
    if dtype == "bf16":
        xb = workloads.to_bf16_bits(x)
        vals = bf16_to_f64(xb)
        codes, scales, aux = oracle.quantize(fmt, xb)
    else:
        vals = x.astype(np.float64)
        codes, scales, aux = oracle.quantize(fmt, x)
    for i in range(64):
        b, packed = brute.quantize_block(fmt, vals[i])
        assert scales[i, 0] == b, (i, vals[i])
        assert codes[i, 0].tobytes() == packed, i
    if fmt == oracle.AXS6:
        assert aux.size == 16 and not aux.any()


# ----------------------------------------------------------------------------
# (c) special values
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("fmt", FMTS)
def test_nonfinite_block_is_poisoned(fmt):
    x = np.ones((3, 32), np.float32)
    x[0, 7] = np.nan
    x[1, 0] = np.inf
    x[2, 31] = -np.inf
    codes, scales, aux = oracle.quantize(fmt, x)
    assert np.all(scales == 0xFF) and not codes.any()
    for out, nanbits in ((oracle.FP32, 0x7FC00000), (oracle.BF16, 0x7FC0)):
        y = oracle.dequantize(fmt, codes, scales, aux, 3, 32, out)
        assert np.all(y.view(np.uint32 if out == oracle.FP32 else np.uint16) == nanbits)
        fq = oracle.fake_quantize(fmt, x if out == oracle.FP32 else workloads.to_bf16_bits(x))
        assert np.array_equal(fq.view(np.uint8), y.view(np.uint8))


@pytest.mark.parametrize("fmt", FMTS)
def test_zero_blocks_keep_signs(fmt):
    x = np.zeros((1, 32), np.float32)
    x[0, 1::3] = -0.0
    codes, scales, _ = oracle.quantize(fmt, x)
    assert scales[0, 0] == 0
    c = brute.unpack(fmt, codes[0, 0].tobytes())
    sb = 1 << (oracle.CODE_BITS[fmt] - 1)
    assert [ci == sb for ci in c] == list(np.signbit(x[0]))
    y = oracle.fake_quantize(fmt, x)
    assert np.array_equal(y.view(np.uint32), x.view(np.uint32))


@pytest.mark.parametrize("fmt", FMTS)
def test_tiny_negative_rounds_to_minus_zero(fmt):
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 2.0 ** brute.emax(fmt)          # scale byte 127
    x[0, 1] = -1e-6                            # far below half the smallest step
    y = oracle.fake_quantize(fmt, x)
    assert y[0, 1] == 0.0 and np.signbit(y[0, 1])


@pytest.mark.parametrize("fmt", FMTS)
def test_saturation_at_top_of_scale_binade(fmt):
    top = brute.finite_grid(fmt).max()
    e = brute.emax(fmt)
    just_below_next = np.float32(np.nextafter(np.float32(2.0 ** (e + 1)), np.float32(0)))
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = just_below_next
    x[0, 1] = -just_below_next
    x[0, 2] = np.float32(top)
    codes, scales, _ = oracle.quantize(fmt, x)
    assert scales[0, 0] == 127
    y = oracle.fake_quantize(fmt, x)
    assert y[0, 0] == top and y[0, 1] == -top and y[0, 2] == top


def test_e4m3_saturates_where_torch_gives_nan():
    x = np.zeros((1, 32), np.float32)
    x[0, :4] = [448.0, 464.0, 470.0, 511.0]
    y = oracle.fake_quantize(oracle.FP8_E4M3, x)
    assert list(y[0, :4]) == [448.0] * 4
    t = torch.from_numpy(x[0, :4]).to(torch.float8_e4m3fn).float().numpy()
    assert t[1] == 448.0 and np.isnan(t[2])  # the library cast differs above 464


@pytest.mark.parametrize("fmt", FMTS)
def test_subnormal_inputs_exact(fmt):
    # a block made only of bf16 subnormals: scale byte clamps to 0 and the
    # element codes are still the exact nearest grid points
    sub = np.arange(1, 128, dtype=np.uint16)  # bf16 subnormal patterns
    blocks = np.resize(sub, 4 * 32).reshape(4, 32)
    blocks[1] |= 0x8000
    codes, scales, _ = oracle.quantize(fmt, blocks)
    for i in range(4):
        b, packed = brute.quantize_block(fmt, bf16_to_f64(blocks[i]))
        assert scales[i, 0] == b == 0
        assert codes[i, 0].tobytes() == packed


# ----------------------------------------------------------------------------
# (d) reductions to library rounding (round-to-nearest-even of torch casts)
# ----------------------------------------------------------------------------
def _rand_block_top_binade(rng, n, e):
    """n blocks whose max magnitude lies in [2^e, 2^(e+1)) (scale byte 127)."""
    x = rng.uniform(-1, 1, (n, 32)) * 2.0 ** (e + 1)
    x *= np.exp2(rng.integers(-12, 1, (n, 32)))  # spread over many binades
    x[:, 0] = np.sign(rng.uniform(-1, 1, n)) * rng.uniform(2.0 ** e, 2.0 ** (e + 1), n)
    return x.astype(np.float32)


def _codes_as_ints(fmt, codes):
    return np.array([brute.unpack(fmt, codes[i, j].tobytes())
                     for i in range(codes.shape[0]) for j in range(codes.shape[1])])


def test_e4m3_rounding_is_torch_cast():
    rng = np.random.default_rng(7)
    x = _rand_block_top_binade(rng, 400, 8)
    codes, scales, _ = oracle.quantize(oracle.FP8_E4M3, x)
    assert np.all(scales == 127)
    lib = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes.reshape(400, 32), lib)


def _map_fp8_to_narrow(lib_bytes, bits):
    sign = (lib_bytes >> 7) & 1
    mag = lib_bytes & 0x7F
    assert mag.max() < (1 << (bits - 1))
    return (sign << (bits - 1)) | mag


def test_e2m3_rounding_is_torch_e4m3_cast_shifted():
    rng = np.random.default_rng(8)
    x = _rand_block_top_binade(rng, 400, 2)
    codes, scales, _ = oracle.quantize(oracle.FP6_E2M3, x)
    assert np.all(scales == 127)
    t = torch.from_numpy(np.clip(x, -7.5, 7.5).astype(np.float64) * 2.0 ** -6).float()
    lib = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int64)
    assert np.array_equal(_codes_as_ints(oracle.FP6_E2M3, codes), _map_fp8_to_narrow(lib, 6))


def test_e3m2_rounding_is_torch_e5m2_cast_shifted():
    rng = np.random.default_rng(9)
    x = _rand_block_top_binade(rng, 400, 4)
    codes, scales, _ = oracle.quantize(oracle.FP6_E3M2, x)
    assert np.all(scales == 127)
    t = torch.from_numpy(np.clip(x, -28, 28).astype(np.float64) * 2.0 ** -12).float()
    lib = t.to(torch.float8_e5m2).view(torch.uint8).numpy().astype(np.int64)
    assert np.array_equal(_codes_as_ints(oracle.FP6_E3M2, codes), _map_fp8_to_narrow(lib, 6))


@pytest.mark.parametrize("fmt", MX_FMTS)
def test_dequant_rounding_is_library_cast(fmt):
    # every code under extreme and ordinary scale bytes: the fp32 output is
    # numpy's RNE cast of the exact product, the bf16 output torch's RNE cast
    # of that fp32 value (exact whenever the product is a normal or
    # subnormal fp32)
    bits = oracle.CODE_BITS[fmt]
    ncode = 1 << bits
    codes_int = np.arange(ncode)
    byts = [0, 1, 2, 20, 126, 127, 128, 200, 246, 250, 254]
    nb_per = (ncode + 31) // 32
    blocks = []
    for b in byts:
        blocks.append(np.resize(codes_int, nb_per * 32).reshape(nb_per, 32))
    blocks = np.concatenate(blocks)
    scales = np.repeat(np.array(byts, np.uint8), nb_per)
    packed = np.stack([np.frombuffer(brute.pack(fmt, blk), np.uint8) for blk in blocks])
    nbk = len(blocks)
    y32 = oracle.dequantize(fmt, packed, scales, None, nbk, 32, oracle.FP32)
    yb = oracle.dequantize(fmt, packed, scales, None, nbk, 32, oracle.BF16)
    exact = np.array([[brute.decode(fmt, int(c)) for c in row] for row in blocks]) \
        * np.exp2(scales.astype(np.float64) - 127)[:, None]
    with np.errstate(over="ignore"):
        lib32 = exact.astype(np.float32)
    assert np.array_equal(np.isnan(y32), np.isnan(lib32))
    fin = ~np.isnan(lib32)
    assert np.array_equal(y32.view(np.uint32)[fin], lib32.view(np.uint32)[fin])
    libb = torch.from_numpy(lib32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(yb[fin], libb[fin])


# ----------------------------------------------------------------------------
# (e) invariants
# ----------------------------------------------------------------------------
def _mixed_input(rng, rows, cols, dtype):
    x = (rng.standard_t(3, (rows, cols)) * np.exp2(rng.integers(-30, 30, (rows, 1)))).astype(np.float32)
    flat = x.reshape(-1)
    idx = rng.choice(flat.size, 12, replace=False)
    flat[idx[:4]] = np.nan
    flat[idx[4:8]] = np.inf
    flat[idx[8:]] = -0.0
    x[1, :32] = 0.0
    return workloads.to_bf16_bits(x) if dtype == "bf16" else x


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_fake_quant_idempotent(fmt, dtype):
    rng = np.random.default_rng(11)
    x = _mixed_input(rng, 40, 96, dtype)
    y1 = oracle.fake_quantize(fmt, x)
    y2 = oracle.fake_quantize(fmt, y1)
    assert np.array_equal(y1.view(np.uint8), y2.view(np.uint8))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_dequant_of_quant_equals_fake_quant(fmt, dtype):
    rng = np.random.default_rng(12)
    x = _mixed_input(rng, 40, 96, dtype)
    codes, scales, aux = oracle.quantize(fmt, x)
    out = oracle.BF16 if dtype == "bf16" else oracle.FP32
    y = oracle.dequantize(fmt, codes, scales, aux, 40, 96, out)
    fq = oracle.fake_quantize(fmt, x)
    assert np.array_equal(y.view(np.uint8), fq.view(np.uint8))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("k", [-9, -1, 1, 5, 30])
def test_power_of_two_equivariance(fmt, k):
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((50, 64)) * np.exp2(rng.integers(-20, 20, (50, 1)))).astype(np.float32)
    xs = (x.astype(np.float64) * 2.0 ** k).astype(np.float32)
    assert np.array_equal(xs.astype(np.float64), x.astype(np.float64) * 2.0 ** k)
    c1, s1, _ = oracle.quantize(fmt, x)
    c2, s2, _ = oracle.quantize(fmt, xs)
    ok = (s1.astype(int) >= 1) & (s1.astype(int) <= 254 - max(k, 0)) & (s1.astype(int) + k >= 1)
    assert ok.mean() > 0.9
    assert np.array_equal(s2[ok].astype(int), s1[ok].astype(int) + k)
    assert np.array_equal(c2[ok], c1[ok])
    f1 = oracle.fake_quantize(fmt, x).astype(np.float64).reshape(50, 2, 32)
    f2 = oracle.fake_quantize(fmt, xs).astype(np.float64).reshape(50, 2, 32)
    assert np.array_equal(f2[ok], f1[ok] * 2.0 ** k)


@pytest.mark.parametrize("fmt", FMTS)
def test_every_code_is_a_fixed_point(fmt):
    bits = oracle.CODE_BITS[fmt]
    half = 1 << (bits - 1)
    g = brute.grid(fmt)
    valid = [c for c in range(1 << bits) if not np.isnan(g[c & (half - 1)])]
    top = int(np.nanargmax(np.where(np.isnan(g), -1, g)))  # largest finite magnitude code
    rows = []
    for i in range(0, len(valid), 31):
        chunk = valid[i:i + 31]
        rows.append([top] + list(np.resize(chunk, 31)))
    rows = np.array(rows)
    for b in (3, 127, 140, 240):
        packed = np.stack([np.frombuffer(brute.pack(fmt, r), np.uint8) for r in rows])
        scales = np.full(len(rows), b, np.uint8)
        aux = np.zeros((len(rows) + 3) // 4, np.uint8)
        y = oracle.dequantize(fmt, packed, scales, aux, len(rows), 32, oracle.FP32)
        c2, s2, _ = oracle.quantize(fmt, y)
        assert np.all(s2 == b)
        assert np.array_equal(c2.reshape(len(rows), -1), packed)


@pytest.mark.parametrize("fmt", FMTS)
def test_error_bound_closed_form(fmt):
    # |x - fq(x)| <= half the grid step at |x| for unsaturated elements,
    # and <= |x| - maxnorm*X + 0 for saturated ones (clamp then exact)
    rng = np.random.default_rng(14)
    x = (rng.standard_normal((200, 32)) * np.exp2(rng.integers(-10, 10, (200, 1)))).astype(np.float32)
    y = oracle.fake_quantize(fmt, x).astype(np.float64)
    _, scales, _ = oracle.quantize(fmt, x)
    X = np.exp2(np.repeat(scales.reshape(-1), 32).astype(np.float64) - 127).reshape(200, 32)
    a = np.abs(x.astype(np.float64)) / X
    g = brute.finite_grid(fmt)
    if fmt == oracle.AXS6:
        step = np.full_like(a, 1 / 16)
    else:
        mbits = {0: 3, 1: 2, 2: 1, 3: 3}[fmt]
        emin = {0: 0, 1: -2, 2: 0, 3: -6}[fmt]
        ea = np.floor(np.log2(np.where(a > 0, a, 1)))
        step = np.exp2(np.maximum(ea, emin) - mbits)
    err = np.abs(x - y) / X
    sat = a > g.max()
    assert np.all(err[~sat] <= step[~sat] / 2)
    assert np.allclose(err[sat], a[sat] - g.max())
    if fmt != oracle.AXS6:
        rel = err[(a >= 2.0 ** emin) & ~sat] / a[(a >= 2.0 ** emin) & ~sat]
        assert rel.max() <= 2.0 ** -(mbits + 1)


# ----------------------------------------------------------------------------
# (f) bit accounting printed on the AXS-6 page
# ----------------------------------------------------------------------------
def test_axs6_bits_per_value_golden():
    with open(os.path.join(GOLDEN, "axs6_bits.json")) as f:
        gold = json.load(f)
    rows, cols = 64, 4096
    ncode, nb, naux = oracle.buffer_sizes(oracle.AXS6, rows, cols)
    total_bits = 8 * (ncode + nb) + 2 * nb  # codes, exponent plane, 2-bit config per block
    bpv = total_bits / (rows * cols)
    assert bpv == 6.3125
    assert round(bpv, 2) == gold["bits_per_value"]
    saving = 100 * (1 - bpv / gold["fp8_bits_per_value"])
    assert round(saving) == gold["memory_saving_vs_fp8_percent"]
    assert naux * 8 >= 2 * nb
    # the MX formats for comparison: codes plus one E8M0 byte per 32 values
    for fmt, want in ((oracle.FP6_E2M3, 6.25), (oracle.FP8_E4M3, 8.25), (oracle.FP4_E2M1, 4.25)):
        ncode, nb, _ = oracle.buffer_sizes(fmt, rows, cols)
        assert 8 * (ncode + nb) / (rows * cols) == want


# ----------------------------------------------------------------------------
# (g) exp-then-quantize probabilities
# ----------------------------------------------------------------------------
def _exp_many(d):
    # softmax_probs of rows [d, 0] is exp_ref(d - 0) = exp_ref(d)
    d = np.asarray(d, np.float32)
    s = np.stack([d, np.zeros_like(d)], axis=1)
    return oracle.softmax_probs(s)[:, 0]


def test_exp_ref_positive_arguments():
    # d > 0 does not occur after subtracting the row maximum, but exp_ref is
    # defined there too (overflow to inf past the largest fp32)
    d = np.linspace(0.0, 88.72, 100001).astype(np.float32)
    p = np.array([oracle.exp_ref(v) for v in d[::50]], np.float64)
    ref = np.exp(d[::50].astype(np.float64))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    assert np.all(np.isfinite(p)) and np.max(np.abs(p - ref) / ulp) <= 2.0
    assert np.isinf(oracle.exp_ref(88.8))


def test_exp_ref_special_points():
    assert oracle.exp_ref(0.0) == 1.0
    assert oracle.exp_ref(-np.inf) == 0.0
    assert np.isnan(oracle.exp_ref(np.nan))
    assert oracle.exp_ref(-200.0) == 0.0
    assert np.isinf(oracle.exp_ref(100.0))
    assert np.array_equal(_exp_many([-1.0, -5.0, 0.0]), oracle.exp_ref([-1.0, -5.0, 0.0]))


def test_exp_ref_within_two_ulp_of_exp():
    d = np.linspace(-87.0, 0.0, 400001).astype(np.float32)
    d = np.concatenate([d, -np.abs(np.random.default_rng(3).standard_normal(200000).astype(np.float32) * 9)])
    p = _exp_many(d).astype(np.float64)
    ref = np.exp(d.astype(np.float64))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    err = np.abs(p - ref) / ulp
    assert err.max() <= 2.0, err.max()
    assert np.mean(err <= 0.5) > 0.9


def test_exp_ref_subnormal_range_and_monotone():
    d = np.linspace(-104.5, -80.0, 200001).astype(np.float32)
    p = _exp_many(d).astype(np.float64)
    ref = np.exp(d.astype(np.float64))
    # absolute error within 2 ulps of the result's binade (subnormal ulp 2^-149)
    ulp = np.maximum(np.spacing(ref.astype(np.float32)).astype(np.float64), 2.0 ** -149)
    assert np.max(np.abs(p - ref) / ulp) <= 2.0
    dd = np.sort(np.concatenate([d, np.linspace(-30, 0, 300001).astype(np.float32)]))
    pp = _exp_many(dd)
    assert np.all(np.diff(pp.astype(np.float64)) >= 0)


# ----------------------------------------------------------------------------
# (g2) the attention forward's base-2 exponential
# ----------------------------------------------------------------------------
def _exp2_literals():
    """The coefficients C1..C5 as written in mxref_exp2's source."""
    src = open(os.path.join(os.path.dirname(oracle.__file__), "mxref.c")).read()
    body = src[src.index("float mxref_exp2(float u)"):]
    body = body[:body.index("float nf")]
    return {int(j): float.fromhex(v)
            for j, v in re.findall(r"C(\d) = (0x[0-9a-f.]+p[+-]\d+)f", body)}


def test_exp2_coefficients_are_a_constrained_minimax_polynomial():
    # the stated construction, computed here: the smallest possible largest
    # relative error of 1 + f (c1 + c2 f + ... + c5 f^4) against 2^f on
    # [-1/2, 1/2] (a linear program on a grid); in exact arithmetic the
    # literals come within 1.5x of it (they were moved a few fp32 ulps from
    # the optimum towards the values whose fp32 evaluation errs least)
    from scipy.optimize import linprog
    f = np.linspace(-0.5, 0.5, 4001)
    ex = np.exp2(f)
    V = np.stack([f ** (j + 1) for j in range(5)], 1)
    A = np.vstack([np.hstack([V, -ex[:, None]]), np.hstack([-V, -ex[:, None]])])
    b = np.r_[ex - 1, 1 - ex]
    res = linprog(np.r_[np.zeros(5), 1.0], A_ub=A, b_ub=b, bounds=[(None, None)] * 6,
                  method="highs")
    assert res.success and res.x[-1] < 1e-7  # under one fp32 ulp of 1
    lit = _exp2_literals()
    assert sorted(lit) == [1, 2, 3, 4, 5]
    g = np.linspace(-0.5, 0.5, 200001)
    p = np.zeros_like(g)
    for j in (5, 4, 3, 2, 1):
        p = (p + lit[j]) * g
    err = np.max(np.abs((1.0 + p) / np.exp2(g) - 1.0))
    assert err <= 1.5 * res.x[-1], (err, res.x[-1])


def _ulps(p, ref):
    # error in units of the last place of the exact value's binade (normal
    # range); one subnormal ulp 2^-149 below 2^-126
    _, e = np.frexp(ref)
    ulp = np.maximum(np.ldexp(1.0, e - 24), 2.0 ** -149)
    return np.abs(p - ref) / ulp


def test_exp2_ref_within_its_bound():
    # within 2.1 ulp (over every fp32 f in [-1/2, 1/2], the whole reduced
    # range, the largest error is 2.093 ulp; the scaling by 2^n keeps the
    # count)
    rng = np.random.default_rng(21)
    u = np.concatenate([np.linspace(-0.5, 0.5, 400001), rng.uniform(-0.5, 0.5, 300000),
                        rng.uniform(-151.0, 0.0, 300000), -rng.exponential(4.0, 100000)])
    u = u.astype(np.float32)
    err = _ulps(oracle.exp2_ref(u).astype(np.float64), np.exp2(u.astype(np.float64)))
    assert err.max() <= 2.1, err.max()
    assert np.mean(err <= 1.0) > 0.7


def test_exp2_ref_special_values():
    k = np.arange(150, dtype=np.float32)
    # exact powers of two down to the smallest subnormal
    assert np.array_equal(oracle.exp2_ref(-k), np.exp2(-k.astype(np.float64)).astype(np.float32))
    # 2^-150 is the midpoint between 0 and 2^-149 (ties to even: 0); below
    # it everything is 0, and just above it the result is 2^-149
    zero = np.array([-150.0, -150.5, -151.0, -151.5, -1e6, -3e38, -np.inf], np.float32)
    assert np.all(oracle.exp2_ref(zero) == 0.0)
    assert oracle.exp2_ref(np.nextafter(np.float32(-150.0), np.float32(0.0)))[0] == 2.0 ** -149
    assert np.isnan(oracle.exp2_ref(np.array([np.nan], np.float32))[0])
    assert np.isinf(oracle.exp2_ref(np.array([128.5], np.float32))[0])


def test_exp2_ref_agrees_with_exp_ref_in_base_e():
    # exp_ref(d) and exp2_ref(fp32(d log2 e)) evaluate the same function;
    # they differ by the roundings of log2 e and of d log2 e (together
    # <= |u| 2^-23 in the exponent, a relative ln2 |u| 2^-23) plus the two
    # evaluations' own errors (2 and 2.1 ulp)
    rng = np.random.default_rng(22)
    d = -np.abs(rng.standard_normal(200000) * 8).astype(np.float32)
    u = (d * np.float32(1.4426950408889634)).astype(np.float32)
    a = oracle.exp2_ref(u).astype(np.float64)
    b = _exp_many(d).astype(np.float64)
    rel = np.abs(a - b) / b
    assert np.all(rel <= np.log(2) * np.abs(u) * 2.0 ** -23 + 9 * 2.0 ** -24)


def test_softmax_quantize_structure():
    s = workloads.attn_scores(rows=48, cols=4096)
    s[5, 100] = np.nan          # row 5 poisoned
    s[6, 7] = np.inf            # row 6: inf - inf = NaN there, exp(-inf) = 0 elsewhere
    s[7, :] = -np.inf           # fully masked row: -inf - -inf = NaN
    codes, scales = oracle.softmax_quantize(oracle.FP4_E2M1, s)
    p = oracle.softmax_probs(s)
    # exp-then-quantize == quantize of the materialized probabilities
    c2, s2, _ = oracle.quantize(oracle.FP4_E2M1, p)
    assert np.array_equal(codes, c2) and np.array_equal(scales, s2)
    for r in range(48):
        if r in (5, 6, 7):
            continue
        j = int(np.argmax(s[r])) // 32
        assert p[r].max() == 1.0
        assert scales[r, j] == 125          # E = 0, emax = 2
        assert np.all(scales[r] <= 125)
    # probability codes are nonnegative: every sign bit is 0
    ints = _codes_as_ints(oracle.FP4_E2M1, codes)
    assert not np.any(ints & 0x8)
    assert np.all(scales[5] == 0xFF) and np.all(scales[7] == 0xFF)
    assert scales[6, 0] == 0xFF and np.all(scales[6, 1:] == 0)


def test_axs6_nonzero_config_decodes_to_nan():
    x = np.random.default_rng(15).standard_normal((1, 256)).astype(np.float32)
    codes, scales, aux = oracle.quantize(oracle.AXS6, x)
    assert aux.size == 2 and not aux.any()
    aux2 = aux.copy()
    aux2[0] = 0b00100000  # block 2 of the first byte gets config 2
    aux2[1] = 0b00000001  # block 4 (first of the second byte) gets config 1
    y = oracle.dequantize(oracle.AXS6, codes, scales, aux2, 1, 256, oracle.FP32).reshape(8, 32)
    y0 = oracle.dequantize(oracle.AXS6, codes, scales, aux, 1, 256, oracle.FP32).reshape(8, 32)
    assert np.all(np.isnan(y[2])) and np.all(np.isnan(y[4]))
    keep = [0, 1, 3, 5, 6, 7]
    assert np.array_equal(y[keep], y0[keep]) and not np.isnan(y0).any()


@pytest.mark.parametrize("fmt", [0, 1, 2, 3, 4])
def test_bisection_encoder_equals_exhaustive_search(fmt):
    """brute.encode_sorted (used for the hardware sweeps) picks the same code
    as the all-pairs nearest-grid search on random values, every grid point,
    every midpoint and its fp32 neighbours, signed zeros and saturating
    values, under several scale bytes."""
    rng = np.random.default_rng(40 + fmt)
    g = brute.finite_grid(fmt)
    mids = (g[:-1] + g[1:]) / 2
    base = np.concatenate([rng.standard_normal(20000) * g.max() / 2, mids, -mids, g, -g,
                           np.nextafter(mids, 0), np.nextafter(mids, 1e30), [0.0, -0.0, 1e9, -1e9]])
    for b in (0, 3, 120, 126, 127, 128, 200, 254):
        v = (base * 2.0 ** (b - 127)).astype(np.float32).astype(np.float64)
        assert np.array_equal(brute.encode(fmt, v, b), brute.encode_sorted(fmt, v, b)), b
