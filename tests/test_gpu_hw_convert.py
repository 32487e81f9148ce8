"""Exhaustive checks of the gfx950 scaled-conversion instructions the library
relies on, against the brute-force nearest-code search (tests/brute.py).

Each instruction runs in a test-only kernel (tests/hwprobe/cvt_probe.hip) on
every finite bf16 or fp16 pattern under every finite scale byte (0..254), on
every fp32 rounding class under every byte, or on every code under every
scale byte for the reverse direction.  The library uses an
instruction only for the cases asserted here:

  quantize   from bf16 and from fp16 (E2M3 / E3M2 32-wide, E2M1 and E4M3
             pairwise): every finite bf16 or fp16 pattern under every byte
             0..254, bit-exact, saturation included (E4M3 within the
             block domain, as below).
             from fp32 (E2M3 / E3M2 as two 16-wide operands whose values
             land at the even and odd code positions; E2M1 and E4M3
             pairwise): every rounding class under every byte 0..254.  A
             round-to-nearest-even conversion of v / X depends only on the
             exponent, the mantissa bits the target keeps, the first bit
             below them and whether any lower bit is set; the sweep takes
             every fp32 exponent field (subnormals included), every pattern
             of the top 8 mantissa bits (which hold the kept bits and the
             round bit of every target binade), the low 15 bits as none,
             the lowest, the highest or all of them set, and both signs:
             522,240 values x 255 bytes per form, bit-exact for every value
             a block can hold (|v| / X < 2^(emax + 1)).
             E4M3 (bf16, fp16 and fp32): bit-exact for |v| / X < 512 once a
             rounded magnitude of 0x7F (the instruction does not saturate)
             is replaced by 0x7E (448).
  dequantize every code under scale bytes 0..254 is the exact product
             rounded to the output type; byte 255 gives a NaN, which the
             library replaces by the canonical quiet NaN.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import brute
import workloads

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
E2M3, E3M2, E2M1, E4M3 = 0, 1, 2, 3
EMAX = {E2M3: 2, E3M2: 4, E2M1: 2, E4M3: 8}
BYTES = np.arange(255, dtype=np.uint8)


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    path = os.path.join(HERE, "hwprobe", "libcvtprobe.so")
    if not os.path.exists(path):
        from hwprobe import build as hb
        hb.build()
    lib = ctypes.CDLL(path)
    P, I = ctypes.c_void_p, ctypes.c_int
    for f in ("probe_q_fp6_bf16", "probe_q_fp6_f32", "probe_q_fp6_f16", "probe_dq_fp6_bf16",
              "probe_dq_fp6_f32"):
        getattr(lib, f).argtypes = [I, P, P, P, I]
    for f in ("probe_q_fp8_bf16", "probe_q_fp8_f32", "probe_q_fp4_bf16", "probe_q_fp4_f32",
              "probe_q_fp8_f16", "probe_q_fp4_f16",
              "probe_dq_fp8_bf16", "probe_dq_fp4_bf16", "probe_dq_fp8_f32", "probe_dq_fp4_f32"):
        getattr(lib, f).argtypes = [P, P, P, I]
    return lib


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def all_bf16():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        v = workloads.bf16_bits_to_f32(b).astype(np.float64)
    return b, v


def all_f16():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return b, b.view(np.float16).astype(np.float64)


def fp32_set():
    """Widened bf16 patterns, random fp32 over all exponents, and every grid
    midpoint (and its fp32 neighbours) of every format over many scales."""
    _, v = all_bf16()
    rng = np.random.default_rng(0)
    r = (rng.uniform(1, 2, 131072) * np.exp2(rng.integers(-149, 128, 131072))).astype(np.float32)
    r *= np.where(rng.random(r.size) < 0.5, -1, 1).astype(np.float32)
    mids = []
    for fmt in (E2M3, E3M2, E2M1, E4M3):
        g = brute.finite_grid(fmt)
        m = ((g[:-1] + g[1:]) / 2).astype(np.float32)
        for k in range(-12, 12):
            mm = (m.astype(np.float64) * 2.0 ** k).astype(np.float32)
            mids += [mm, np.nextafter(mm, np.float32(0)), np.nextafter(mm, np.float32(1e30))]
    mids = np.concatenate(mids)
    s = np.concatenate([v.astype(np.float32), r, mids, -mids])
    s = s[np.isfinite(s)]
    return s[: (s.size // 32) * 32]


def fp32_rounding_classes() -> np.ndarray:
    """Every fp32 exponent field 0..254, every top-8 mantissa pattern, the
    low 15 bits in {0, 1, 0x4000, 0x7FFF}, both signs (522,240 values)."""
    e = np.arange(255, dtype=np.uint32)
    t = np.arange(256, dtype=np.uint32)
    lo = np.array([0, 1, 0x4000, 0x7FFF], np.uint32)
    bits = ((e[:, None, None] << 23) | (t[None, :, None] << 15) | lo[None, None, :]).reshape(-1)
    return np.concatenate([bits, bits | np.uint32(0x80000000)]).view(np.float32)


def sweep_fp32(fmt, run, group):
    """Run `run(values_dev, bytes_dev, nlanes) -> codes [n]` for every byte
    0..254 over the rounding classes (`group` values per lane) and compare
    with the bisection nearest-code search; returns (mismatches inside the
    block domain, mismatches outside it, values checked)."""
    vals = fp32_rounding_classes()
    lanes = vals.size // group
    d_in = dev(vals)
    v64 = vals.astype(np.float64)
    absv, sign = np.abs(v64), np.signbit(v64).astype(np.int64) << (brute.CODE_BITS[fmt] - 1)
    g = brute.finite_grid(fmt)
    bad_in, bad_out, checked = [], 0, 0
    chunk = 8  # bytes per launch
    d_vals = torch.cat([d_in] * chunk)
    for b0 in range(0, 255, chunk):
        bs = np.arange(b0, min(b0 + chunk, 255), dtype=np.uint8)
        sb = dev(np.repeat(bs, lanes))
        got = run(d_vals[: bs.size * vals.size], sb, bs.size * lanes).reshape(bs.size, -1)
        for j, b in enumerate(bs):
            a = absv / 2.0 ** (int(b) - 127)
            # clamped to the top value: its code; at most half the smallest
            # nonzero value: code 0 (a tie there goes to the even code 0);
            # between: the nearest-code search
            want = np.where(a >= g[-1], g.size - 1, 0) | sign
            mid = (a > g[1] / 2) & (a < g[-1])
            want[mid] = brute.encode_sorted(fmt, v64[mid], int(b))
            inside = a < 2.0 ** (EMAX[fmt] + 1)
            gj = got[j]
            if fmt == E4M3:
                gj = np.where((gj & 0x7F) == 0x7F, gj - 1, gj)  # the library's saturation fix
            diff = gj != want
            if diff[inside].any():
                i = np.nonzero(diff & inside)[0][:3]
                bad_in.append((int(b), v64[i].tolist(), gj[i].tolist(), want[i].tolist()))
            bad_out += int((diff & ~inside).sum())
            checked += vals.size
    return bad_in, bad_out, checked


SCALE_SAMPLE = np.array([0, 1, 2, 5, 60, 100, 117, 120, 124, 125, 126, 127, 128, 129, 130, 135,
                         140, 200, 250, 254], np.uint8)


def expected(fmt, vals, byte_of):
    out = np.zeros(vals.size, np.int64)
    for b in np.unique(byte_of):
        sel = byte_of == b
        out[sel] = brute.encode(fmt, vals[sel], int(b))
    return out


def unpack_stream(words, w, count):
    n = words.shape[0]
    bits = np.unpackbits(words.view(np.uint8).reshape(n, -1), axis=1, bitorder="little")
    bits = bits[:, : count * w].reshape(n, count, w)
    return (bits.astype(np.int64) << np.arange(w)).sum(axis=2)


def in_range(vals, byte_of, fmt):
    return np.abs(vals) / np.exp2(byte_of.astype(np.float64) - 127) < 2.0 ** (EMAX[fmt] + 1)


# ----------------------------------------------------------------------------
# quantize direction
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("src", ["bf16", "f16"])
@pytest.mark.parametrize("kind,fmt", [(0, E2M3), (1, E3M2)], ids=["e2m3", "e3m2"])
def test_pk32_fp6_from_16bit_all_patterns_all_scales(lib, kind, fmt, src):
    b, v = all_bf16() if src == "bf16" else all_f16()
    fin = np.isfinite(v)
    lanes = 65536 // 32
    inp = np.tile(b.reshape(lanes, 32).view(np.uint32).reshape(lanes, 16), (255, 1))
    sb = np.repeat(BYTES, lanes)
    d_in, d_sb = dev(inp), dev(sb)
    out = torch.zeros(inp.shape[0] * 6, dtype=torch.int32, device="cuda")
    fn = lib.probe_q_fp6_bf16 if src == "bf16" else lib.probe_q_fp6_f16
    assert fn(kind, d_in.data_ptr(), d_sb.data_ptr(), out.data_ptr(), inp.shape[0]) == 0
    got = unpack_stream(out.cpu().numpy().view(np.uint32).reshape(-1, 6), 6, 32).reshape(-1)
    vals = np.tile(v, 255)
    byte_of = np.repeat(BYTES, 65536)
    m = np.tile(fin, 255)
    want = expected(fmt, vals[m], byte_of[m])
    bad = np.nonzero(got[m] != want)[0]
    assert bad.size == 0, (bad.size, vals[m][bad[:5]], byte_of[m][bad[:5]], got[m][bad[:5]], want[bad[:5]])


@pytest.mark.parametrize("kind,fmt", [(0, E2M3), (1, E3M2)], ids=["e2m3", "e3m2"])
def test_2xpk16_fp6_from_fp32_every_rounding_class_every_scale(lib, kind, fmt):
    def run(d_vals, sb, nl):
        out = torch.zeros(nl * 6, dtype=torch.int32, device="cuda")
        assert lib.probe_q_fp6_f32(kind, d_vals.data_ptr(), sb.data_ptr(), out.data_ptr(), nl) == 0
        return unpack_stream(out.cpu().numpy().view(np.uint32).reshape(-1, 6), 6, 32).reshape(-1)

    bad_in, bad_out, n = sweep_fp32(fmt, run, 32)
    assert n == 522240 * 255
    assert not bad_in, bad_in[:4]
    print(f"fp6 f32 sweep: {n} values, {bad_out} differ only where |v|/X >= 2^(emax+1)")


@pytest.mark.parametrize("fmt", [E2M1, E4M3], ids=["e2m1", "e4m3"])
def test_pk_fp4_fp8_from_fp32_every_rounding_class_every_scale(lib, fmt):
    w = 4 if fmt == E2M1 else 8
    fn = lib.probe_q_fp4_f32 if fmt == E2M1 else lib.probe_q_fp8_f32

    def run(d_vals, sb, nl):
        out = torch.zeros(nl, dtype=torch.int32, device="cuda")
        assert fn(d_vals.data_ptr(), sb.data_ptr(), out.data_ptr(), nl) == 0
        o = out.cpu().numpy().view(np.uint32)
        return np.stack([o & ((1 << w) - 1), (o >> w) & ((1 << w) - 1)], axis=1).reshape(-1).astype(np.int64)

    bad_in, bad_out, n = sweep_fp32(fmt, run, 2)
    assert n == 522240 * 255
    assert not bad_in, bad_in[:4]
    print(f"pk f32 sweep: {n} values, {bad_out} differ only where |v|/X >= 2^(emax+1)")


@pytest.mark.parametrize("kind,fmt", [(0, E2M3), (1, E3M2)], ids=["e2m3", "e3m2"])
def test_2xpk16_fp6_from_fp32(lib, kind, fmt):
    s = fp32_set()
    lanes = s.size // 32
    inp = np.tile(s.reshape(lanes, 32), (SCALE_SAMPLE.size, 1))
    sb = np.repeat(SCALE_SAMPLE, lanes)
    d_in, d_sb = dev(inp), dev(sb)
    out = torch.zeros(inp.shape[0] * 6, dtype=torch.int32, device="cuda")
    assert lib.probe_q_fp6_f32(kind, d_in.data_ptr(), d_sb.data_ptr(), out.data_ptr(), inp.shape[0]) == 0
    got = unpack_stream(out.cpu().numpy().view(np.uint32).reshape(-1, 6), 6, 32).reshape(-1)
    vals = inp.reshape(-1).astype(np.float64)
    byte_of = np.repeat(SCALE_SAMPLE, s.size)
    want = expected(fmt, vals, byte_of)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (bad.size, vals[bad[:5]], byte_of[bad[:5]], got[bad[:5]], want[bad[:5]])


@pytest.mark.parametrize("src", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("fmt", [E2M1, E4M3], ids=["e2m1", "e4m3"])
def test_pk_fp4_fp8_pairs(lib, src, fmt):
    if src in ("bf16", "f16"):
        b, v = all_bf16() if src == "bf16" else all_f16()
        fin = np.isfinite(v)
        words = b.reshape(-1, 2).view(np.uint32).reshape(-1)
        inp = np.tile(words, 255)
        sb = np.repeat(BYTES, words.size)
        vals = np.tile(v, 255)
        byte_of = np.repeat(BYTES, 65536)
        fn = {("bf16", E2M1): lib.probe_q_fp4_bf16, ("bf16", E4M3): lib.probe_q_fp8_bf16,
              ("f16", E2M1): lib.probe_q_fp4_f16, ("f16", E4M3): lib.probe_q_fp8_f16}[src, fmt]
        n = inp.size
    else:
        s = fp32_set()
        inp = np.tile(s, SCALE_SAMPLE.size)
        sb = np.repeat(SCALE_SAMPLE, s.size // 2)
        vals = inp.astype(np.float64)
        byte_of = np.repeat(SCALE_SAMPLE, s.size)
        fn = lib.probe_q_fp4_f32 if fmt == E2M1 else lib.probe_q_fp8_f32
        n = sb.size
        fin = np.ones(s.size, bool)
    d_in, d_sb = dev(inp), dev(sb)
    out = torch.zeros(n, dtype=torch.int32, device="cuda")
    assert fn(d_in.data_ptr(), d_sb.data_ptr(), out.data_ptr(), n) == 0
    o = out.cpu().numpy().view(np.uint32)
    w = 4 if fmt == E2M1 else 8
    got = np.stack([o & ((1 << w) - 1), (o >> w) & ((1 << w) - 1)], axis=1).reshape(-1).astype(np.int64)
    m = np.tile(fin, vals.size // fin.size)
    if fmt == E4M3:
        m &= in_range(vals, byte_of, fmt)
        got = np.where((got & 0x7F) == 0x7F, got - 1, got)  # the library's saturation fix
    want = expected(fmt, vals[m], byte_of[m])
    bad = np.nonzero(got[m] != want)[0]
    assert bad.size == 0, (bad.size, vals[m][bad[:5]], byte_of[m][bad[:5]], got[m][bad[:5]], want[bad[:5]])


# ----------------------------------------------------------------------------
# dequantize direction: every code under every scale byte
# ----------------------------------------------------------------------------
def _expected_dequant(fmt, codes, byte_of, out):
    w = brute.CODE_BITS[fmt]
    table = np.array([brute.decode(fmt, c) for c in range(1 << w)])
    with np.errstate(over="ignore", invalid="ignore"):
        f = (table[codes] * np.exp2(byte_of.astype(np.float64) - 127)).astype(np.float32)
    f[byte_of == 255] = np.nan
    if out == "f32":
        return f.view(np.uint32).astype(np.int64), np.isnan(f)
    t = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return t.astype(np.int64), np.isnan(f)


def _check_dequant(fmt, codes, byte_of, got, out):
    want, nan = _expected_dequant(fmt, codes, byte_of, out)
    mag = got & (0x7FFFFFFF if out == "f32" else 0x7FFF)
    got_nan = mag > (0x7F800000 if out == "f32" else 0x7F80)
    assert np.array_equal(got_nan, nan)
    bad = np.nonzero(~nan & (got != want))[0]
    assert bad.size == 0, (bad.size, codes[bad[:5]], byte_of[bad[:5]], got[bad[:5]], want[bad[:5]])


ALLB = np.arange(256, dtype=np.uint8)


@pytest.mark.parametrize("kind,fmt", [(0, E2M3), (1, E3M2)], ids=["e2m3", "e3m2"])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_pk32_fp6_decode_every_code_every_scale(lib, kind, fmt, out):
    codes = np.tile(np.arange(64), 256)
    byte_of = np.repeat(ALLB, 64)
    c2 = codes.reshape(-1, 32)
    words = np.zeros((c2.shape[0], 6), np.uint32)
    for k in range(32):
        bit = 6 * k
        j, s = bit // 32, bit % 32
        words[:, j] |= (c2[:, k].astype(np.uint32) << s) & 0xFFFFFFFF
        if s + 6 > 32:
            words[:, j + 1] |= c2[:, k].astype(np.uint32) >> (32 - s)
    sb = byte_of.reshape(-1, 32)[:, 0].copy()
    d_w, d_sb = dev(words), dev(sb)
    n = c2.shape[0]
    if out == "bf16":
        res = torch.zeros(n * 16, dtype=torch.int32, device="cuda")
        assert lib.probe_dq_fp6_bf16(kind, d_w.data_ptr(), d_sb.data_ptr(), res.data_ptr(), n) == 0
        got = res.cpu().numpy().view(np.uint16).astype(np.int64)
    else:
        res = torch.zeros(n * 32, dtype=torch.float32, device="cuda")
        assert lib.probe_dq_fp6_f32(kind, d_w.data_ptr(), d_sb.data_ptr(), res.data_ptr(), n) == 0
        got = res.cpu().numpy().view(np.uint32).astype(np.int64)
    _check_dequant(fmt, codes, byte_of, got, out)


@pytest.mark.parametrize("fmt", [E2M1, E4M3], ids=["e2m1", "e4m3"])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_pk_fp4_fp8_decode_every_code_every_scale(lib, fmt, out):
    w = 4 if fmt == E2M1 else 8
    ncode = 1 << w
    pairs = np.array([(a, b) for a in range(ncode) for b in range(ncode)], np.int64)
    words = (pairs[:, 0] | (pairs[:, 1] << w)).astype(np.uint32)
    win = np.tile(words, 256)
    sb = np.repeat(ALLB, words.size)
    d_w, d_sb = dev(win), dev(sb)
    if out == "bf16":
        fn = lib.probe_dq_fp4_bf16 if fmt == E2M1 else lib.probe_dq_fp8_bf16
        res = torch.zeros(win.size, dtype=torch.int32, device="cuda")
        assert fn(d_w.data_ptr(), d_sb.data_ptr(), res.data_ptr(), win.size) == 0
        o = res.cpu().numpy().view(np.uint32)
        got = np.stack([o & 0xFFFF, o >> 16], axis=1).reshape(-1).astype(np.int64)
    else:
        fn = lib.probe_dq_fp4_f32 if fmt == E2M1 else lib.probe_dq_fp8_f32
        res = torch.zeros(win.size * 2, dtype=torch.float32, device="cuda")
        assert fn(d_w.data_ptr(), d_sb.data_ptr(), res.data_ptr(), win.size) == 0
        got = res.cpu().numpy().view(np.uint32).astype(np.int64)
    codes = np.tile(pairs.reshape(-1), 256)
    byte_of = np.repeat(ALLB, pairs.size)
    _check_dequant(fmt, codes, byte_of, got, out)
