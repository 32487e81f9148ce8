"""Brute-force checker for the CPU oracle (independent of its arithmetic).

Nothing here calls the oracle.  Element grids come from library dtypes plus
structural facts about the formats, and encoding is an exhaustive
nearest-grid-point search instead of the oracle's rounding formula:

* E4M3 grid: torch.float8_e4m3fn decoded for every byte (a library routine).
* E2M3 grid: E4M3 and E2M3 share 3 mantissa bits; with E2M3's bias 1 and
  E4M3's bias 7 the magnitude codes 0..31 of the two formats name the same
  numbers up to a factor 2^6 (E2M3 code c == E4M3 code c times 2^6).
* E3M2 grid: likewise from torch.float8_e5m2 (2 mantissa bits; biases 3 and
  15, factor 2^12).
* E2M1 grid: E2M1 keeps E2M3's exponent field and bias with 1 mantissa bit,
  so E2M1 magnitude (e, m) equals E2M3 magnitude (e, m << 2).
* AXS-6 grid: m/16, m = 0..31 (the reading of the AXS-6 page's sign+5-bit
  mantissa block; there is no library dtype for it).
"""
from __future__ import annotations

import math

import numpy as np
import torch

E2M3, E3M2, E2M1, E4M3, AXS6 = 0, 1, 2, 3, 4


def is_exmy(fmt):
    return (fmt & ~0xFF) == 0x100


def exmy_em(fmt):
    return (fmt >> 4) & 0xF, fmt & 0xF


class _Table(dict):
    def __init__(self, base, generic):
        super().__init__(base)
        self._generic = generic

    def __missing__(self, fmt):
        if is_exmy(fmt):
            return self._generic(*exmy_em(fmt))
        raise KeyError(fmt)


CODE_BITS = _Table({E2M3: 6, E3M2: 6, E2M1: 4, E4M3: 8, AXS6: 6}, lambda e, m: 1 + e + m)
BPB = _Table({E2M3: 24, E3M2: 24, E2M1: 16, E4M3: 32, AXS6: 24}, lambda e, m: 4 * (1 + e + m))


def exmy_grid(e: int, m: int) -> np.ndarray:
    """Magnitudes of a generic eXmY format by enumeration of its fields:
    e = 0: the integers 0 .. 2^m - 1; e >= 1: field f = 0 gives mant/2^m *
    2^(1 - bias), f >= 1 gives (1 + mant/2^m) * 2^(f - bias), bias =
    2^(e-1) - 1, every field finite.  (Pinned against library dtypes and
    closed forms in tests/test_oracle_exmy.py.)"""
    if e == 0:
        return np.arange(2 ** m, dtype=np.float64)
    bias = 2 ** (e - 1) - 1
    vals = []
    for f in range(2 ** e):
        for mant in range(2 ** m):
            if f == 0:
                vals.append(math.ldexp(mant / 2 ** m, 1 - bias))
            else:
                vals.append(math.ldexp(1 + mant / 2 ** m, f - bias))
    return np.array(vals, dtype=np.float64)


def _torch_decode(dtype) -> np.ndarray:
    return torch.arange(256, dtype=torch.uint8).view(dtype).to(torch.float64).numpy()


def grid(fmt: int) -> np.ndarray:
    """Magnitudes indexed by magnitude code (NaN where the code is NaN)."""
    if is_exmy(fmt):
        return exmy_grid(*exmy_em(fmt))
    if fmt == E4M3:
        return _torch_decode(torch.float8_e4m3fn)[:128].copy()
    if fmt == E2M3:
        return _torch_decode(torch.float8_e4m3fn)[:32] * 2.0 ** 6
    if fmt == E3M2:
        return _torch_decode(torch.float8_e5m2)[:32] * 2.0 ** 12
    if fmt == E2M1:
        g = grid(E2M3)
        return np.array([g[((c >> 1) << 3) | ((c & 1) << 2)] for c in range(8)])
    if fmt == AXS6:
        return np.arange(32, dtype=np.float64) / 16.0
    raise ValueError(fmt)


def finite_grid(fmt: int) -> np.ndarray:
    g = grid(fmt)
    return g[np.isfinite(g)]


def emax(fmt: int) -> int:
    """floor(log2) of the largest finite magnitude, found by comparison."""
    top = finite_grid(fmt).max()
    e = 0
    while 2.0 ** (e + 1) <= top:
        e += 1
    while 2.0 ** e > top:
        e -= 1
    return e


def floor_log2(a: float) -> int:
    """floor(log2 a) for finite a > 0 by comparison with powers of two."""
    e = 0
    while 2.0 ** e > a:
        e -= 1
    while 2.0 ** (e + 1) <= a:
        e += 1
    return e


def scale_byte(fmt: int, block: np.ndarray) -> int:
    v = np.asarray(block, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        return 0xFF
    amax = float(np.max(np.abs(v)))
    if amax == 0.0:
        return 0
    return int(min(max(floor_log2(amax) - emax(fmt) + 127, 0), 254))


def encode(fmt: int, v: np.ndarray, byte: int) -> np.ndarray:
    """Nearest grid point to |v|/2^(byte-127) after clamping to the largest
    finite magnitude; an exact tie goes to the even code; sign bit copied."""
    v = np.asarray(v, dtype=np.float64)
    g = finite_grid(fmt)
    a = np.minimum(np.abs(v) / 2.0 ** (byte - 127), g.max())
    d = np.abs(a[:, None] - g[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    codes_idx = np.arange(g.size)[None, :]
    # among the nearest (one, or two on an exact tie) prefer an even code
    score = np.where(cand, np.where(codes_idx % 2 == 0, 0, 1), 9)
    mag = score.argmin(axis=1)
    sign = np.signbit(v).astype(np.int64)
    return (sign << (CODE_BITS[fmt] - 1)) | mag


def encode_sorted(fmt: int, v: np.ndarray, byte: int) -> np.ndarray:
    """The same nearest-grid-point choice as encode(), found by bisection on
    the sorted grid instead of an all-pairs distance table (for sweeps of
    millions of values): the two grid points around |v|/X are the only
    candidates; the nearer wins, an exact tie goes to the even code."""
    v = np.asarray(v, dtype=np.float64)
    g = finite_grid(fmt)
    assert np.all(np.diff(g) > 0)
    a = np.minimum(np.abs(v) / 2.0 ** (byte - 127), g[-1])
    hi = np.minimum(np.searchsorted(g, a, side="left"), g.size - 1)
    lo = np.maximum(hi - 1, 0)
    dl, dh = a - g[lo], g[hi] - a
    mag = np.where(dh < dl, hi, np.where(dl < dh, lo, np.where(lo % 2 == 0, lo, hi)))
    sign = np.signbit(v).astype(np.int64)
    return (sign << (CODE_BITS[fmt] - 1)) | mag


def pack(fmt: int, codes) -> bytes:
    """Little-endian bit stream: code k occupies bits [k*w, k*w + w)."""
    w = CODE_BITS[fmt]
    acc = 0
    for k, c in enumerate(codes):
        acc |= int(c) << (w * k)
    return acc.to_bytes(BPB[fmt], "little")


def unpack(fmt: int, data: bytes):
    w = CODE_BITS[fmt]
    acc = int.from_bytes(bytes(data), "little")
    return [(acc >> (w * k)) & ((1 << w) - 1) for k in range(32)]


def decode(fmt: int, code: int) -> float:
    w = CODE_BITS[fmt]
    mag = code & ((1 << (w - 1)) - 1)
    val = grid(fmt)[mag]
    return -val if (code >> (w - 1)) & 1 else val


def quantize_block(fmt: int, block: np.ndarray):
    """(scale byte, packed bytes) of one 32-value block."""
    b = scale_byte(fmt, block)
    if b == 0xFF:
        return b, bytes(BPB[fmt])
    return b, pack(fmt, encode(fmt, block, b))


def ulp_rel_bound(fmt: int) -> float:
    """Half a grid step relative to the value, for normal magnitudes."""
    mbits = {E2M3: 3, E3M2: 2, E2M1: 1, E4M3: 3}[fmt]
    return 2.0 ** -(mbits + 1)


def log2_exact(x: float) -> int:
    m, e = math.frexp(x)
    assert m == 0.5
    return e - 1
