"""Pins of the oracle's generic eXmY formats (CPU only).

The eXmY abstract defines a format for every split of a bit width into
exponent and mantissa bits (e0m6 .. e6m0 for 7 bits) and a dense, byte-
addressable packing for widths that are not powers of two.  The grids are
pinned to library dtypes where formats coincide, and to closed forms; the
rounding, scale and packing through brute force, as for the MX formats.
"""
import numpy as np
import pytest
import torch

import brute
import oracle
import workloads

EXMY = oracle.EXMY_FORMATS
ids = [f"e{(f >> 4) & 15}m{f & 15}" for f in EXMY]


def bf16_to_f64(b):
    with np.errstate(invalid="ignore"):
        return workloads.bf16_bits_to_f32(np.asarray(b, np.uint16)).astype(np.float64)


def test_every_split_of_3_to_9_bits():
    splits = {(f >> 4) & 15: [] for f in EXMY}
    widths = sorted({1 + ((f >> 4) & 15) + (f & 15) for f in EXMY})
    assert widths == list(range(3, 10))
    for w in range(3, 10):  # every split of the w-1 non-sign bits
        got = sorted(((f >> 4) & 15, f & 15) for f in EXMY if 1 + ((f >> 4) & 15) + (f & 15) == w)
        assert got == [(e, w - 1 - e) for e in range(w)], w
    assert len(EXMY) == 42 and splits


@pytest.mark.parametrize("fmt", EXMY, ids=ids)
def test_oracle_decode_equals_field_enumeration(fmt):
    e, m = brute.exmy_em(fmt)
    n = 1 << (e + m)
    ours = np.array([oracle.decode(fmt, c) for c in range(2 * n)])
    g = brute.grid(fmt)
    assert np.array_equal(ours[:n], g) and np.array_equal(ours[n:], -g)
    assert np.all(np.signbit(ours[n:]))
    assert np.all(np.diff(g) > 0)  # magnitude codes ordered by value


def test_grids_against_library_dtypes():
    # formats that coincide with the OCP MX element formats
    for (e, m), mx_fmt in (((2, 3), oracle.FP6_E2M3), ((3, 2), oracle.FP6_E3M2),
                           ((2, 1), oracle.FP4_E2M1)):
        assert np.array_equal(brute.grid(oracle.exmy(e, m)), brute.grid(mx_fmt))
    # e4m3: torch float8_e4m3fn for codes 0..126; eXmY keeps 0x7F finite (480)
    lib = torch.arange(128, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    g = brute.grid(oracle.exmy(4, 3))
    assert np.array_equal(g[:127], lib[:127]) and g[127] == 480.0
    # e5m2: torch float8_e5m2 for fields 0..30; eXmY's field 31 is finite
    lib = torch.arange(128, dtype=torch.uint8).view(torch.float8_e5m2).double().numpy()
    g = brute.grid(oracle.exmy(5, 2))
    assert np.array_equal(g[:124], lib[:124])
    assert np.array_equal(g[124:], 2.0 ** 16 * np.array([1, 1.25, 1.5, 1.75]))


def test_grids_closed_forms():
    for m in range(2, 9):  # e0mY: sign-magnitude integers
        assert np.array_equal(brute.grid(oracle.exmy(0, m)), np.arange(2 ** m))
    for m in range(1, 8):  # e1mY: the same uniform grid as e0m(Y+1), step 2^(1-Y)
        assert np.array_equal(brute.grid(oracle.exmy(1, m)),
                              np.arange(2 ** (m + 1)) * 2.0 ** (1 - m))
    for e in range(2, 9):  # eXm0: zero and powers of two (e8m0: 2^-126 .. 2^128)
        bias = 2 ** (e - 1) - 1
        want = np.concatenate([[0.0], 2.0 ** (np.arange(1, 2 ** e) - bias)])
        assert np.array_equal(brute.grid(oracle.exmy(e, 0)), want)
    assert oracle.BYTES_PER_BLOCK[oracle.exmy(3, 3)] == 28  # 32 x 7 bits, no padding
    assert oracle.BYTES_PER_BLOCK[oracle.exmy(8, 0)] == 36  # 32 x 9 bits


def test_e8m0_grid_is_torch_float8_e8m0fnu_between_its_ends():
    # fields 1..254 are 2^(f - 127), as in the E8M0 scale type; eXmY's field
    # 0 is zero (a subnormal with no mantissa bits) and 255 is finite, 2^128
    g = brute.grid(oracle.exmy(8, 0))
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    assert np.array_equal(g[1:255], lib[1:255])
    assert g[0] == 0.0 and g[255] == 2.0 ** 128 and np.isnan(lib[255])


def test_e8m0_beyond_the_fp32_range():
    f = oracle.exmy(8, 0)
    fmax = np.finfo(np.float32).max
    # the block maximum sits in the top binade [2^128, 2^129) of the scaled
    # values: byte = floor(log2 amax) - 128 + 127
    x = np.zeros((1, 32), np.float32)
    x[0, :5] = [fmax, 2.0 ** 127, 1.5 * 2.0 ** 126, 1.25 * 2.0 ** 126, 3.0 * 2.0 ** -127]
    codes, scales, _ = oracle.quantize(f, x)
    assert scales[0, 0] == 126  # X = 2^-1
    c = brute.unpack(f, codes[0, 0].tobytes())
    # fmax / X is just under 2^129: saturates to 2^128 (field 255); 2^127 / X
    # is 2^128 itself; 1.5 2^127 is a tie between fields 254 and 255 and
    # goes to the even field; 1.25 2^127 rounds down; 3 2^-126 is a tie
    # between fields 2 and 3 (2^-125, 2^-124) and goes to field 2
    assert list(c[:5]) == [255, 255, 254, 254, 2]
    y = oracle.fake_quantize(f, x)
    assert list(y[0, :5]) == [2.0 ** 127, 2.0 ** 127, 2.0 ** 126, 2.0 ** 126, 2.0 ** -126]
    # a block whose maximum is below 2 takes the clamped byte 0, X = 2^-127
    x = np.zeros((1, 32), np.float32)
    x[0, :4] = [1.0, 2.0 ** -126, 1.5 * 2.0 ** -127, 2.0 ** -149]
    codes, scales, _ = oracle.quantize(f, x)
    assert scales[0, 0] == 0
    assert list(brute.unpack(f, codes[0, 0].tobytes())[:4]) == [254, 128, 128, 105]


def test_e8m0_dequantize_overflows_and_underflows_like_the_exact_product():
    f = oracle.exmy(8, 0)
    nb = 6
    packed = b"".join(brute.pack(f, [c] + [0] * 31) for c in (255, 255, 1, 1, 2, 0x1FF))
    codes = np.frombuffer(packed, np.uint8).reshape(nb, 36)
    scales = np.array([127, 126, 104, 103, 103, 126], np.uint8)
    y = oracle.dequantize(f, codes, scales, None, nb, 32, oracle.FP32).reshape(nb, 32)[:, 0]
    # 2^128 overflows fp32; 2^127; 2^-149 is the smallest subnormal; 2^-150
    # is a tie between 0 and 2^-149 and rounds to 0; 2^-125 2^-24 = 2^-149;
    # -2^128 2^-1 = -2^127
    assert list(y) == [np.inf, 2.0 ** 127, 2.0 ** -149, 0.0, 2.0 ** -149, -(2.0 ** 127)]


def _anchored(E, values_bits):
    anchor = workloads.to_bf16_bits(np.array([2.0 ** E], np.float32))[0]
    nblk = (len(values_bits) + 30) // 31
    blocks = np.empty((nblk, 32), np.uint16)
    blocks[:, 0] = anchor
    blocks[:, 1:] = np.resize(values_bits, nblk * 31).reshape(nblk, 31)
    return blocks


@pytest.mark.parametrize("fmt", EXMY, ids=ids)
def test_quantize_bf16_vs_brute_force(fmt):
    allv = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = bf16_to_f64(allv)
    fin = allv[np.isfinite(v)]
    absv = np.abs(bf16_to_f64(fin))
    em = brute.emax(fmt)
    # the scale byte clamped at 0, a middle byte, and a byte near the top
    for E in (-130 + em if em < 3 else -126, 0, 100):
        sel = fin[absv < 2.0 ** (E + 1)]
        if sel.size > 40000:
            sel = sel[:: max(1, sel.size // 40000)]
        blocks = _anchored(E, sel)
        codes, scales, _ = oracle.quantize(fmt, blocks)
        want_b = brute.scale_byte(fmt, bf16_to_f64(blocks[0]))
        assert np.all(scales == want_b), (E,)
        want = brute.encode(fmt, bf16_to_f64(blocks).reshape(-1), want_b).reshape(-1, 32)
        got = np.array([brute.unpack(fmt, codes[i, 0].tobytes()) for i in range(len(blocks))])
        assert np.array_equal(got, want), (E,)
        for i in range(0, len(blocks), max(1, len(blocks) // 5)):
            assert codes[i, 0].tobytes() == brute.pack(fmt, want[i])


@pytest.mark.parametrize("fmt", EXMY, ids=ids)
def test_ties_and_neighbours(fmt):
    # every midpoint between neighbouring grid values: ties go to the even
    # code (for m = 0 that is the even exponent field, not the larger value)
    # the grid times X = 2^-sh, which keeps it inside fp32 (e8m0 reaches
    # 2^128; its values times 1/2 are still exact there)
    sh = max(0, brute.emax(fmt) - 127)
    g = brute.finite_grid(fmt) * 2.0 ** -sh
    mids = ((g[:-1] + g[1:]) / 2.0).astype(np.float32)
    vals = np.concatenate([mids, np.nextafter(mids, np.float32(0)),
                           np.nextafter(mids, np.float32(1e30)), g.astype(np.float32)])
    vals = np.concatenate([vals, -vals])
    top = np.float32(2.0 ** (brute.emax(fmt) - sh))
    nblk = (len(vals) + 30) // 31
    blocks = np.empty((nblk, 32), np.float32)
    blocks[:, 0] = top
    blocks[:, 1:] = np.resize(vals, nblk * 31).reshape(nblk, 31)
    codes, scales, _ = oracle.quantize(fmt, blocks)
    assert np.all(scales == 127 - sh)
    want = brute.encode(fmt, blocks.reshape(-1).astype(np.float64), 127 - sh).reshape(-1, 32)
    got = np.array([brute.unpack(fmt, codes[i, 0].tobytes()) for i in range(nblk)])
    assert np.array_equal(got, want)


def test_exponent_only_ties_alternate():
    # e3m0: grid 0, 1/4, 1/2, 1, 2, 4, 8, 16; 3 lies between 2 (field 4) and
    # 4 (field 5) and goes to field 4; 6 lies between 4 and 8 and goes to 8
    f = oracle.exmy(3, 0)
    x = np.zeros((1, 32), np.float32)
    x[0, :3] = [16.0, 3.0, 6.0]
    y = oracle.fake_quantize(f, x)
    assert list(y[0, :3]) == [16.0, 2.0, 8.0]


@pytest.mark.parametrize("fmt", EXMY[::3], ids=ids[::3])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_invariants(fmt, dtype):
    rng = np.random.default_rng(fmt)
    x = (rng.standard_t(3, (24, 96)) * np.exp2(rng.integers(-30, 30, (24, 1)))).astype(np.float32)
    x[0, 5] = np.nan
    x[1, :32] = 0.0
    x[2, 3] = -0.0
    x = workloads.to_bf16_bits(x) if dtype == "bf16" else x
    fq = oracle.fake_quantize(fmt, x)
    assert np.array_equal(oracle.fake_quantize(fmt, fq).view(np.uint8), fq.view(np.uint8))
    codes, scales, aux = oracle.quantize(fmt, x)
    y = oracle.dequantize(fmt, codes, scales, aux, 24, 96, oracle.BF16 if dtype == "bf16" else oracle.FP32)
    assert np.array_equal(y.view(np.uint8), fq.view(np.uint8))
    assert scales[0, 0] == 0xFF and not codes[0, 0].any()


def test_axs6_is_e0m5_with_the_scale_shifted_by_4():
    x = (np.random.default_rng(9).standard_normal((64, 256))
         * np.exp2(np.random.default_rng(10).integers(-40, 40, (64, 1)))).astype(np.float32)
    ca, sa, _ = oracle.quantize(oracle.AXS6, x)
    ce, se, _ = oracle.quantize(oracle.exmy(0, 5), x)
    assert np.array_equal(ca, ce)
    assert np.array_equal(sa.astype(int), se.astype(int) + 4)
