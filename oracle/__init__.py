"""CPU oracle for block-shared-exponent quantization -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product (``block_scaled_bit_amd``)
never touches it, and it never touches the product: the two share no code.

The arithmetic lives in ``mxref.c`` (plain C, exact double precision, one
block at a time); this module only marshals numpy arrays through ctypes.
bf16 tensors are carried as ``numpy.uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

FP6_E2M3, FP6_E3M2, FP4_E2M1, FP8_E4M3, AXS6 = 0, 1, 2, 3, 4
BF16, FP32, F16 = 0, 1, 2
BLOCK = 32
NAMES = {"mxfp6_e2m3": FP6_E2M3, "mxfp6_e3m2": FP6_E3M2, "mxfp4": FP4_E2M1,
         "mxfp8": FP8_E4M3, "axs6": AXS6}


def exmy(e: int, m: int) -> int:
    """Identifier of the generic eXmY format with e exponent and m mantissa
    bits (width 1 + e + m, 3..9 bits, so e <= 8)."""
    return 0x100 | (e << 4) | m


EXMY_FORMATS = [exmy(e, w - 1 - e) for w in range(3, 10) for e in range(0, w)]


class _Table(dict):
    """Per-format constant that also answers for generic eXmY identifiers."""

    def __init__(self, base, generic):
        super().__init__(base)
        self._generic = generic

    def __missing__(self, fmt):
        if (fmt & ~0xFF) == 0x100:
            return self._generic((fmt >> 4) & 0xF, fmt & 0xF)
        raise KeyError(fmt)


CODE_BITS = _Table({FP6_E2M3: 6, FP6_E3M2: 6, FP4_E2M1: 4, FP8_E4M3: 8, AXS6: 6},
                   lambda e, m: 1 + e + m)
BYTES_PER_BLOCK = _Table({FP6_E2M3: 24, FP6_E3M2: 24, FP4_E2M1: 16, FP8_E4M3: 32, AXS6: 24},
                         lambda e, m: 4 * (1 + e + m))


def _load():
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    lib.mxref_decode.argtypes = [I, I]
    lib.mxref_decode.restype = ctypes.c_double
    lib.mxref_encode.argtypes = [I, ctypes.c_double, I]
    lib.mxref_encode.restype = I
    lib.mxref_scale_byte.argtypes = [I, P, I]
    lib.mxref_scale_byte.restype = I
    lib.mxref_bytes_per_block.argtypes = [I]
    lib.mxref_quantize.argtypes = [I, I, I, P, I64, I64, P, P, P]
    lib.mxref_dequantize.argtypes = [I, I, P, P, P, I64, I64, I, P]
    lib.mxref_fake_quantize.argtypes = [I, I, I, P, P, I64, I64]
    lib.mxref_exp.argtypes = [ctypes.c_float]
    lib.mxref_exp.restype = ctypes.c_float
    lib.mxref_exp2.argtypes = [ctypes.c_float]
    lib.mxref_exp2.restype = ctypes.c_float
    lib.mxref_exp2_n.argtypes = [P, I64, P]
    lib.mxref_exp2_n.restype = I
    lib.mxref_softmax_probs.argtypes = [P, I64, I64, P]
    lib.mxref_softmax_quantize.argtypes = [I, I, P, I64, I64, P, P]
    lib.mxref_attention_fwd.argtypes = [I, I, P, P, P, P, I64, I64, I64, I64, ctypes.c_float, I,
                                        I, P, P, P, P, P]
    lib.mxref_attention_fwd_efq.argtypes = lib.mxref_attention_fwd.argtypes
    lib.mxref_efq_block.argtypes = [P, P]
    lib.mxref_efq_quantize_block.argtypes = [P, P]
    lib.mxref_efq_block_log2.argtypes = [P, P]
    lib.mxref_efq_quantize_block_log2.argtypes = [P, P]
    lib.mxref_efq_attention_block.argtypes = [P, ctypes.c_float, ctypes.c_float, P]
    for f in ("mxref_quantize", "mxref_dequantize", "mxref_fake_quantize",
              "mxref_softmax_probs", "mxref_softmax_quantize", "mxref_attention_fwd",
              "mxref_attention_fwd_efq", "mxref_efq_block", "mxref_efq_quantize_block",
              "mxref_efq_block_log2", "mxref_efq_quantize_block_log2",
              "mxref_efq_attention_block"):
        getattr(lib, f).restype = I
    return lib


_lib = _load()


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype_of(x: np.ndarray) -> int:
    if x.dtype == np.uint16:
        return BF16
    if x.dtype == np.float32:
        return FP32
    if x.dtype == np.float16:
        return F16
    raise TypeError(f"oracle input must be uint16 (bf16 bits), float32 or float16, got {x.dtype}")


_OUT_NP = {BF16: np.uint16, FP32: np.float32, F16: np.float16}


def _rows_cols(x: np.ndarray):
    if x.ndim == 0:
        raise ValueError("need at least one dimension")
    cols = x.shape[-1]
    rows = int(np.prod(x.shape[:-1])) if x.ndim > 1 else 1
    return rows, cols


def buffer_sizes(fmt: int, rows: int, cols: int):
    nb = rows * (cols // BLOCK)
    aux = (nb + 3) // 4 if fmt == AXS6 else 0
    return nb * BYTES_PER_BLOCK[fmt], nb, aux


def decode(fmt: int, code: int) -> float:
    """Unscaled value of one element code (sign included)."""
    return _lib.mxref_decode(fmt, int(code))


def encode(fmt: int, v: float, byte: int) -> int:
    """Element code of value v in a block with scale byte `byte`."""
    return _lib.mxref_encode(fmt, float(v), int(byte))


def scale_byte(fmt: int, values) -> int:
    v = np.ascontiguousarray(np.asarray(values, dtype=np.float64))
    return _lib.mxref_scale_byte(fmt, _ptr(v), v.size)


def quantize(fmt: int, x: np.ndarray):
    """Returns (codes[rows, cols/32, bpb], scales[rows, cols/32], aux[ceil(nb/4)])."""
    x = np.ascontiguousarray(x)
    rows, cols = _rows_cols(x)
    ncode, nb, naux = buffer_sizes(fmt, rows, cols)
    codes = np.zeros(ncode, np.uint8)
    scales = np.zeros(nb, np.uint8)
    aux = np.zeros(max(naux, 1), np.uint8)
    rc = _lib.mxref_quantize(fmt, BLOCK, _dtype_of(x), _ptr(x), rows, cols,
                             _ptr(codes), _ptr(scales), _ptr(aux))
    if rc:
        raise ValueError("oracle quantize: bad arguments")
    nbr = cols // BLOCK
    return (codes.reshape(rows, nbr, BYTES_PER_BLOCK[fmt]), scales.reshape(rows, nbr),
            aux[:naux])


def dequantize(fmt: int, codes: np.ndarray, scales: np.ndarray, aux, rows: int, cols: int,
               out_dtype: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    auxa = np.ascontiguousarray(aux if aux is not None and len(aux) else np.zeros(1, np.uint8),
                                dtype=np.uint8)
    y = np.empty((rows, cols), _OUT_NP[out_dtype])
    rc = _lib.mxref_dequantize(fmt, BLOCK, _ptr(codes), _ptr(scales), _ptr(auxa), rows, cols,
                               out_dtype, _ptr(y))
    if rc:
        raise ValueError("oracle dequantize: bad arguments")
    return y


def fake_quantize(fmt: int, x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x)
    rows, cols = _rows_cols(x)
    y = np.empty_like(x)
    rc = _lib.mxref_fake_quantize(fmt, BLOCK, _dtype_of(x), _ptr(x), _ptr(y), rows, cols)
    if rc:
        raise ValueError("oracle fake_quantize: bad arguments")
    return y


def exp_ref(d) -> np.ndarray:
    d = np.asarray(d, dtype=np.float32)
    out = np.empty_like(d)
    flat_in, flat_out = d.reshape(-1), out.reshape(-1)
    for i in range(flat_in.size):
        flat_out[i] = _lib.mxref_exp(float(flat_in[i]))
    return out


def exp2_ref(u) -> np.ndarray:
    """The attention forward's fixed base-2 exponential, elementwise (fp32)."""
    u = np.ascontiguousarray(u, dtype=np.float32)
    out = np.empty_like(u)
    _lib.mxref_exp2_n(_ptr(u), u.size, _ptr(out))
    return out


def softmax_probs(s: np.ndarray) -> np.ndarray:
    s = np.ascontiguousarray(s, dtype=np.float32)
    rows, cols = _rows_cols(s)
    p = np.empty_like(s)
    _lib.mxref_softmax_probs(_ptr(s), rows, cols, _ptr(p))
    return p


def softmax_quantize(fmt: int, s: np.ndarray):
    """Row max, exp_ref(s - rowmax), block quantize: (codes, scales)."""
    s = np.ascontiguousarray(s, dtype=np.float32)
    rows, cols = _rows_cols(s)
    ncode, nb, _ = buffer_sizes(fmt, rows, cols)
    codes = np.zeros(ncode, np.uint8)
    scales = np.zeros(nb, np.uint8)
    rc = _lib.mxref_softmax_quantize(fmt, BLOCK, _ptr(s), rows, cols, _ptr(codes), _ptr(scales))
    if rc:
        raise ValueError("oracle softmax_quantize: bad arguments")
    nbr = cols // BLOCK
    return codes.reshape(rows, nbr, BYTES_PER_BLOCK[fmt]), scales.reshape(rows, nbr)


def efq_block(d) -> tuple:
    """EFQ reading on 32 shifted scores (fp32): (scale byte, codes[32])."""
    d = np.ascontiguousarray(np.asarray(d, np.float32).reshape(BLOCK))
    codes = np.zeros(BLOCK, np.int32)
    byte = _lib.mxref_efq_block(_ptr(d), _ptr(codes))
    return byte, codes


def efq_quantize_block(d) -> tuple:
    """EFQ reading on 32 shifted scores: (scale byte, 16 packed bytes)."""
    d = np.ascontiguousarray(np.asarray(d, np.float32).reshape(BLOCK))
    packed = np.zeros(16, np.uint8)
    byte = _lib.mxref_efq_quantize_block(_ptr(d), _ptr(packed))
    return byte, packed


def efq_block_log2(u) -> tuple:
    """EFQ reading on 32 shifted scores already in powers of two (the
    attention forward's t - m): (scale byte, codes[32])."""
    u = np.ascontiguousarray(np.asarray(u, np.float32).reshape(BLOCK))
    codes = np.zeros(BLOCK, np.int32)
    byte = _lib.mxref_efq_block_log2(_ptr(u), _ptr(codes))
    return byte, codes


def efq_quantize_block_log2(u) -> tuple:
    """The same, packed: (scale byte, 16 packed bytes)."""
    u = np.ascontiguousarray(np.asarray(u, np.float32).reshape(BLOCK))
    packed = np.zeros(16, np.uint8)
    byte = _lib.mxref_efq_quantize_block_log2(_ptr(u), _ptr(packed))
    return byte, packed


def efq_attention_block(s, c: float, m: float) -> tuple:
    """EFQ in the attention forward's form on 32 raw fp32 scores s, with
    c = fp32(scale * log2 e) and the running maximum m of fp32(s * c):
    (scale byte, codes[32])."""
    s = np.ascontiguousarray(np.asarray(s, np.float32).reshape(BLOCK))
    codes = np.zeros(BLOCK, np.int32)
    byte = _lib.mxref_efq_attention_block(_ptr(s), float(c), float(m), _ptr(codes))
    return byte, codes


def attention_fwd(v_fmt: int, q: np.ndarray, k: np.ndarray, v_codes: np.ndarray,
                  v_scales: np.ndarray, scale: float, kv_tile: int = 64, out_dtype: int = FP32,
                  efq: bool = False):
    """Attention forward with E2M1 probabilities (online softmax over
    `kv_tile` keys at a time); efq=True uses the exp-free EFQ reading for the
    probability blocks instead of exp-then-quantize.  Probabilities are
    evaluated in base 2: t = fp32(s * fp32(scale * log2 e)), p =
    exp2_ref(t - m) with m the running maximum of t.  q [heads, lq, d] and
    k [heads, lk, d] are bf16 bit patterns; v_codes/v_scales are V^T
    ([heads, d, lk]) quantized with ``quantize(v_fmt, .)``.  Returns
    (o [heads, lq, d], row_max (the largest fp32(s * scale) of the row),
    row_sum [heads, lq], p_codes [heads, lq, lk/32, 16], p_scales
    [heads, lq, lk/32])."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    heads, lq, d = q.shape
    lk = k.shape[1]
    if k.shape != (heads, lk, d):
        raise ValueError("q and k must be [heads, lq, d] and [heads, lk, d]")
    v_codes = np.ascontiguousarray(v_codes, dtype=np.uint8)
    v_scales = np.ascontiguousarray(v_scales, dtype=np.uint8)
    nbk = lk // BLOCK
    if v_codes.size != heads * d * nbk * BYTES_PER_BLOCK[v_fmt] or v_scales.size != heads * d * nbk:
        raise ValueError("v_codes / v_scales do not match V^T [heads, d, lk]")
    o = np.empty((heads, lq, d), np.uint16 if out_dtype == BF16 else np.float32)
    row_max = np.empty((heads, lq), np.float32)
    row_sum = np.empty((heads, lq), np.float32)
    p_codes = np.empty((heads, lq, nbk, 16), np.uint8)
    p_scales = np.empty((heads, lq, nbk), np.uint8)
    fn = _lib.mxref_attention_fwd_efq if efq else _lib.mxref_attention_fwd
    rc = fn(v_fmt, BLOCK, _ptr(q), _ptr(k), _ptr(v_codes), _ptr(v_scales), heads, lq, lk, d,
            float(scale), kv_tile, out_dtype, _ptr(o), _ptr(row_max), _ptr(row_sum),
            _ptr(p_codes), _ptr(p_scales))
    if rc:
        raise ValueError("oracle attention_fwd: bad arguments")
    return o, row_max, row_sum, p_codes, p_scales


def worker_threads() -> int:
    """Threads for a row-split oracle pass: the CPUs this process may run on,
    at most 16 (a one-GPU host's CPU share)."""
    return max(1, min(len(os.sched_getaffinity(0)), 16))


def by_rows(fn, rows: int, threads: int | None = None):
    """Run fn(r0, r1) on `threads` contiguous row ranges at once and join the
    parts: fn returns a tuple of arrays whose leading axis is the rows r0..r1
    (1-D arrays, such as an AXS-6 config plane, are joined end to end; for
    that plane every range must start at a multiple of 4 blocks).  The
    oracle's functions work one block at a time and blocks never cross rows,
    so the joined result equals one call over all rows.  The C library
    releases the interpreter lock, so the ranges run in parallel."""
    import concurrent.futures as cf
    threads = threads or worker_threads()
    threads = max(1, min(threads, rows)) if rows else 1
    bounds = [(rows * i) // threads for i in range(threads + 1)]
    with cf.ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda i: fn(bounds[i], bounds[i + 1]), range(threads)))
    if not isinstance(parts[0], tuple):
        return np.concatenate(parts)
    return tuple(np.concatenate([p[j] for p in parts]) for j in range(len(parts[0])))
