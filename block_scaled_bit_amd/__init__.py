"""Python binding of libmx.so: block-shared-exponent quantization on gfx950.

The functions named ``mx_*`` mirror the C ABI of ``include/mx.h`` one for one
(argument marshalling only: torch tensors become device pointers, the
current torch stream becomes the HIP stream).  ``quantize``,
``quantize_many``, ``dequantize``, ``fake_quantize``, ``softmax_quantize``,
``quantize_v`` and ``attention_fwd`` additionally allocate their outputs
with torch.  All arithmetic runs in the HIP kernels; if the library
is not built this module raises at import time instead of falling back.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime that libmx.so binds to)

__all__ = [
    "MX_FP6_E2M3", "MX_FP6_E3M2", "MX_FP4_E2M1", "MX_FP8_E4M3", "MX_AXS6", "MX_BF16", "MX_FP32",
    "MX_FP16",
    "FORMATS", "MX_EXMY", "MxError", "mx_abi_version", "mx_status_str", "mx_buffer_sizes", "mx_quantize",
    "mx_quantize_batch", "quantize_many", "mx_dequantize", "mx_fake_quantize", "mx_softmax_quantize", "mx_attention_fwd",
    "mx_attention_fwd_efq", "quantize",
    "dequantize", "fake_quantize", "softmax_quantize", "quantize_v", "attention_fwd",
    "library_path",
]

MX_FP6_E2M3, MX_FP6_E3M2, MX_FP4_E2M1, MX_FP8_E4M3, MX_AXS6 = 0, 1, 2, 3, 4
MX_BF16, MX_FP32, MX_FP16 = 0, 1, 2
BLOCK = 32


def MX_EXMY(e: int, m: int) -> int:
    """Generic eXmY format id (width 1 + e + m in 3..9, so e <= 8), as mx.h."""
    return 0x100 | (e << 4) | m


class _BytesPerBlock(dict):
    def __missing__(self, fmt):
        if (fmt & ~0xFF) == 0x100:
            return 4 * (1 + ((fmt >> 4) & 0xF) + (fmt & 0xF))
        raise KeyError(fmt)


BYTES_PER_BLOCK = _BytesPerBlock({0: 24, 1: 24, 2: 16, 3: 32, 4: 24})
# format names used by the pages' configuration strings; "eXmY" strings
# (e.g. "e3m3") name the generic formats
FORMATS = {"mxfp6": MX_FP6_E2M3, "mxfp6_e2m3": MX_FP6_E2M3, "mxfp6_e3m2": MX_FP6_E3M2,
           "mxfp4": MX_FP4_E2M1, "mxfp8": MX_FP8_E4M3, "axs6": MX_AXS6}

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libmx.so")


class MxError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {mx_status_str(status)} (status {status})")
        self.status = status


class _TensorDesc(ctypes.Structure):
    """mx_tensor_desc of include/mx.h."""
    _fields_ = [("x", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("aux", ctypes.c_void_p)]


def _load():
    if not os.path.exists(library_path):
        raise ImportError(
            f"{library_path} is missing: build the HIP library first "
            "(python -m block_scaled_bit_amd.build)")
    lib = ctypes.CDLL(library_path)
    P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.mx_abi_version.restype = I
    lib.mx_status_str.argtypes = [I]
    lib.mx_status_str.restype = ctypes.c_char_p
    lib.mx_buffer_sizes.argtypes = [I, I, I64, I64, P, P, P]
    lib.mx_quantize.argtypes = [I, I, I, P, I64, I64, P, P, P, P]
    lib.mx_quantize_batch.argtypes = [I, I, I, ctypes.POINTER(_TensorDesc), I, P]
    lib.mx_dequantize.argtypes = [I, I, P, P, P, I64, I64, I, P, P]
    lib.mx_fake_quantize.argtypes = [I, I, I, P, P, I64, I64, P]
    lib.mx_softmax_quantize.argtypes = [I, I, P, I64, I64, P, P, P]
    lib.mx_attention_fwd.argtypes = [I, I, P, P, P, P, I64, I64, I64, I64, ctypes.c_float, I, P,
                                     P, P, P, P, P]
    lib.mx_attention_fwd_efq.argtypes = lib.mx_attention_fwd.argtypes
    for f in ("mx_buffer_sizes", "mx_quantize", "mx_quantize_batch", "mx_dequantize", "mx_fake_quantize",
              "mx_softmax_quantize", "mx_attention_fwd", "mx_attention_fwd_efq"):
        getattr(lib, f).restype = I
    return lib


_lib = _load()


def _fmt(f) -> int:
    if isinstance(f, str):
        if f in FORMATS:
            return FORMATS[f]
        import re
        m = re.fullmatch(r"e(\d)m(\d)", f)
        if m:
            return MX_EXMY(int(m.group(1)), int(m.group(2)))
        raise KeyError(f"unknown format name {f!r}")
    return int(f)


def _ptr(t) -> int | None:
    """Device address of a tensor, an int address, or None (NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != 0:
        raise MxError(status, where)


# ---------------------------------------------------------------------------
# one-for-one C ABI
# ---------------------------------------------------------------------------
def mx_abi_version() -> int:
    return _lib.mx_abi_version()


def mx_status_str(status: int) -> str:
    return _lib.mx_status_str(int(status)).decode()


def mx_buffer_sizes(fmt, block: int, rows: int, cols: int):
    c, s, a = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(_lib.mx_buffer_sizes(_fmt(fmt), block, rows, cols, ctypes.byref(c), ctypes.byref(s),
                                ctypes.byref(a)), "mx_buffer_sizes")
    return c.value, s.value, a.value


def mx_quantize(fmt, block, in_dtype, x, rows, cols, codes, scales, aux, stream=None) -> int:
    return _lib.mx_quantize(_fmt(fmt), block, in_dtype, _ptr(x), rows, cols, _ptr(codes),
                            _ptr(scales), _ptr(aux), _stream(stream))


def mx_quantize_batch(fmt, block, in_dtype, tensors, stream=None) -> int:
    """tensors: a sequence of (x, rows, cols, codes, scales, aux) with
    tensors, int addresses or None, as mx_quantize takes them."""
    tensors = list(tensors)
    arr = (_TensorDesc * max(1, len(tensors)))()
    for i, (x, rows, cols, codes, scales, aux) in enumerate(tensors):
        arr[i] = _TensorDesc(_ptr(x), rows, cols, _ptr(codes), _ptr(scales), _ptr(aux))
    return _lib.mx_quantize_batch(_fmt(fmt), block, in_dtype, arr, len(tensors), _stream(stream))


def mx_dequantize(fmt, block, codes, scales, aux, rows, cols, out_dtype, y, stream=None) -> int:
    return _lib.mx_dequantize(_fmt(fmt), block, _ptr(codes), _ptr(scales), _ptr(aux), rows, cols,
                              out_dtype, _ptr(y), _stream(stream))


def mx_fake_quantize(fmt, block, dtype, x, y, rows, cols, stream=None) -> int:
    return _lib.mx_fake_quantize(_fmt(fmt), block, dtype, _ptr(x), _ptr(y), rows, cols,
                                 _stream(stream))


def mx_softmax_quantize(fmt, block, s, rows, cols, codes, scales, stream=None) -> int:
    return _lib.mx_softmax_quantize(_fmt(fmt), block, _ptr(s), rows, cols, _ptr(codes),
                                    _ptr(scales), _stream(stream))


def mx_attention_fwd(v_fmt, block, q, k, v_codes, v_scales, heads, lq, lk, d, scale, out_dtype,
                     o, row_max, row_sum, p_codes, p_scales, stream=None) -> int:
    return _lib.mx_attention_fwd(_fmt(v_fmt), block, _ptr(q), _ptr(k), _ptr(v_codes),
                                 _ptr(v_scales), heads, lq, lk, d, float(scale), out_dtype, _ptr(o),
                                 _ptr(row_max), _ptr(row_sum), _ptr(p_codes), _ptr(p_scales),
                                 _stream(stream))


def mx_attention_fwd_efq(v_fmt, block, q, k, v_codes, v_scales, heads, lq, lk, d, scale,
                         out_dtype, o, row_max, row_sum, p_codes, p_scales, stream=None) -> int:
    return _lib.mx_attention_fwd_efq(_fmt(v_fmt), block, _ptr(q), _ptr(k), _ptr(v_codes),
                                     _ptr(v_scales), heads, lq, lk, d, float(scale), out_dtype,
                                     _ptr(o), _ptr(row_max), _ptr(row_sum), _ptr(p_codes),
                                     _ptr(p_scales), _stream(stream))


# ---------------------------------------------------------------------------
# tensor-level helpers (allocate outputs with torch)
#
# The C ABI takes bare pointers and cannot see buffer sizes, so every tensor
# a helper passes down is checked here first: contiguous, of the expected
# dtype and byte size, and on the same GPU as the first input.  The checks
# run in that order (shape and size before the device), so a wrong buffer is
# reported as such even for host tensors.  Any failure raises ValueError
# before anything is launched.
# ---------------------------------------------------------------------------
def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MX_BF16
    if t.dtype == torch.float32:
        return MX_FP32
    if t.dtype == torch.float16:
        return MX_FP16
    raise MxError(4, f"dtype {t.dtype}")


def _on_gpu(t: torch.Tensor, name: str, like: torch.Tensor | None = None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be in GPU memory (the kernels read device pointers)")
    if like is not None and t.device != like.device:
        raise ValueError(f"{name} is on {t.device}, the inputs on {like.device}")


def _need(t, name: str, dtype: torch.dtype, nbytes: int):
    """t must be a contiguous tensor of `dtype` holding exactly `nbytes`
    bytes (where it lives is checked separately, after every size)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    got = t.numel() * t.element_size()
    if got != nbytes:
        raise ValueError(f"{name} holds {got} bytes, {nbytes} expected")


def _rows_cols(t: torch.Tensor, name: str = "tensor"):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dim() == 0:
        raise ValueError(f"{name} needs at least one dimension")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    _dtype_code(t)
    cols = t.shape[-1]
    if cols % BLOCK:
        raise ValueError(f"{name}: the last dimension ({cols}) must be a multiple of {BLOCK}")
    return (t.numel() // cols if cols else 0), cols


def _block(block: int):
    if block != BLOCK:
        raise MxError(4, f"block {block}")


def _alloc_outputs(f: int, x: torch.Tensor, rows: int, cols: int):
    nbr = cols // BLOCK
    lead = tuple(x.shape[:-1])
    codes = torch.empty(lead + (nbr, BYTES_PER_BLOCK[f]), dtype=torch.uint8, device=x.device)
    scales = torch.empty(lead + (nbr,), dtype=torch.uint8, device=x.device)
    aux = (torch.empty(((rows * nbr) + 3) // 4, dtype=torch.uint8, device=x.device)
           if f == MX_AXS6 else None)
    return codes, scales, aux


def quantize(x: torch.Tensor, fmt="mxfp6_e2m3", block: int = BLOCK):
    """Returns (codes uint8 [.., cols/32, bpb], scales uint8 [.., cols/32],
    aux uint8 [ceil(nblocks/4)] (AXS-6) or None)."""
    f = _fmt(fmt)
    _block(block)
    rows, cols = _rows_cols(x, "x")
    _on_gpu(x, "x")
    codes, scales, aux = _alloc_outputs(f, x, rows, cols)
    _check(mx_quantize(f, block, _dtype_code(x), x, rows, cols, codes, scales, aux), "mx_quantize")
    return codes, scales, aux


def quantize_many(xs, fmt="mxfp6_e2m3", block: int = BLOCK):
    """quantize() of every tensor in xs (one format and input dtype) through
    mx_quantize_batch: a list of (codes, scales, aux)."""
    f = _fmt(fmt)
    _block(block)
    xs = list(xs)
    if not xs:
        return []
    dt = _dtype_code(xs[0])
    shapes = []
    for i, x in enumerate(xs):
        shapes.append(_rows_cols(x, f"xs[{i}]"))
        if _dtype_code(x) != dt:
            raise ValueError("quantize_many takes tensors of one dtype")
    outs, descs = [], []
    for i, (x, (rows, cols)) in enumerate(zip(xs, shapes)):
        _on_gpu(x, f"xs[{i}]", xs[0])
        codes, scales, aux = _alloc_outputs(f, x, rows, cols)
        outs.append((codes, scales, aux))
        descs.append((x, rows, cols, codes, scales, aux))
    _check(mx_quantize_batch(f, block, dt, descs), "mx_quantize_batch")
    return outs


def dequantize(codes: torch.Tensor, scales: torch.Tensor, aux=None, fmt="mxfp6_e2m3",
               out_dtype=torch.bfloat16, block: int = BLOCK):
    """Inverse of quantize(): the [.., cols] tensor of out_dtype that codes,
    scales (and, for AXS-6, aux) describe; the shape comes from scales."""
    f = _fmt(fmt)
    _block(block)
    if not isinstance(scales, torch.Tensor) or scales.dim() == 0:
        raise ValueError("scales must be a tensor [.., cols/32]")
    nbr = scales.shape[-1]
    rows = scales.numel() // nbr if nbr else 0
    nb = rows * nbr
    if f not in (MX_FP6_E2M3, MX_FP6_E3M2, MX_FP4_E2M1, MX_FP8_E4M3, MX_AXS6) and \
            (f & ~0xFF) != 0x100:
        raise MxError(4, f"format {fmt}")
    _need(scales, "scales", torch.uint8, nb)
    _need(codes, "codes", torch.uint8, nb * BYTES_PER_BLOCK[f])
    if f == MX_AXS6:
        _need(aux, "aux", torch.uint8, (nb + 3) // 4)
    if out_dtype not in (torch.bfloat16, torch.float32, torch.float16):
        raise MxError(4, f"dtype {out_dtype}")
    _on_gpu(scales, "scales")
    _on_gpu(codes, "codes", scales)
    if f == MX_AXS6:
        _on_gpu(aux, "aux", scales)
    y = torch.empty(tuple(scales.shape[:-1]) + (nbr * BLOCK,), dtype=out_dtype,
                    device=codes.device)
    _check(mx_dequantize(f, block, codes, scales, aux if f == MX_AXS6 else None, rows,
                         nbr * BLOCK, _dtype_code(y), y), "mx_dequantize")
    return y


def fake_quantize(x: torch.Tensor, fmt="mxfp6_e2m3", block: int = BLOCK, out=None):
    """Fused quantize->dequantize in x's dtype (out=x works in place; any
    other out must be a separate tensor of x's shape and dtype)."""
    f = _fmt(fmt)
    _block(block)
    rows, cols = _rows_cols(x, "x")
    if out is None:
        _on_gpu(x, "x")
        y = torch.empty_like(x)
    else:
        if not isinstance(out, torch.Tensor) or out.shape != x.shape:
            raise ValueError("out must be a tensor of x's shape")
        _need(out, "out", x.dtype, x.numel() * x.element_size())
        _on_gpu(x, "x")
        _on_gpu(out, "out", x)
        if out.data_ptr() != x.data_ptr():
            lo, hi = x.data_ptr(), x.data_ptr() + x.numel() * x.element_size()
            olo, ohi = out.data_ptr(), out.data_ptr() + out.numel() * out.element_size()
            if olo < hi and lo < ohi:
                raise ValueError("out overlaps x without being x (only in-place use is allowed)")
        y = out
    _check(mx_fake_quantize(f, block, _dtype_code(x), x, y, rows, cols), "mx_fake_quantize")
    return y


def softmax_quantize(s: torch.Tensor, fmt="mxfp4", block: int = BLOCK):
    """P = exp(s - rowmax) per row, then block quantization of P."""
    f = _fmt(fmt)
    _block(block)
    if not isinstance(s, torch.Tensor) or s.dtype != torch.float32:
        raise MxError(4, "softmax_quantize needs fp32 scores")
    rows, cols = _rows_cols(s, "s")
    _on_gpu(s, "s")
    codes, scales, _ = _alloc_outputs(f, s, rows, cols)
    _check(mx_softmax_quantize(f, block, s, rows, cols, codes, scales), "mx_softmax_quantize")
    return codes, scales


def quantize_v(v: torch.Tensor, fmt="mxfp8"):
    """V [heads, lk, d] -> (codes, scales) of V^T [heads, d, lk] in blocks of
    32 keys, the layout attention_fwd reads.  The transpose is a torch copy
    (memory plumbing); the quantization runs in the library."""
    if v.dim() != 3:
        raise ValueError("v must be [heads, lk, d]")
    codes, scales, _ = quantize(v.transpose(1, 2).contiguous(), fmt)
    return codes, scales


_V_FORMATS = (MX_FP6_E2M3, MX_FP6_E3M2, MX_FP4_E2M1, MX_FP8_E4M3)


def attention_fwd(q: torch.Tensor, k: torch.Tensor, v_codes: torch.Tensor,
                  v_scales: torch.Tensor, v_fmt="mxfp8", scale=None, out_dtype=torch.bfloat16,
                  stats: bool = False, probs: bool = False, efq: bool = False):
    """Attention forward with E2M1 probabilities.  q [heads, lq, 128] and k
    [heads, lk, 128] bf16; V given as ``quantize_v`` returns it; scale
    defaults to 1/sqrt(128) and must be positive.  The probabilities are
    2^(t - m) of the scores in powers of two, t = s * scale * log2(e).
    Returns o [heads, lq, 128]; with stats=True also (row_max in natural
    units, row_sum); with probs=True also the E2M1 probability blocks
    (p_codes, p_scales).  efq=True: the exp-free EFQ probability rule
    (mx_attention_fwd_efq)."""
    f = _fmt(v_fmt)
    if f not in _V_FORMATS:
        raise MxError(4, f"V format {v_fmt}")
    for t, nm in ((q, "q"), (k, "k")):
        if not isinstance(t, torch.Tensor) or t.dim() != 3:
            raise ValueError(f"{nm} must be a [heads, len, d] tensor")
        if t.dtype != torch.bfloat16:
            raise MxError(4, "attention_fwd needs bf16 q and k")
    heads, lq, d = q.shape
    lk = k.shape[1]
    if k.shape != (heads, lk, d):
        raise ValueError("k must be [heads, lk, d] with q's heads and d")
    if lk % BLOCK:
        raise ValueError(f"lk ({lk}) must be a multiple of {BLOCK}")
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise MxError(4, f"dtype {out_dtype}")
    _need(q, "q", torch.bfloat16, heads * lq * d * 2)
    _need(k, "k", torch.bfloat16, heads * lk * d * 2)
    nbv = heads * d * (lk // BLOCK)
    _need(v_codes, "v_codes", torch.uint8, nbv * BYTES_PER_BLOCK[f])
    _need(v_scales, "v_scales", torch.uint8, nbv)
    _on_gpu(q, "q")
    for t, nm in ((k, "k"), (v_codes, "v_codes"), (v_scales, "v_scales")):
        _on_gpu(t, nm, q)
    if scale is None:
        scale = d ** -0.5
    o = torch.empty((heads, lq, d), dtype=out_dtype, device=q.device)
    rm = rs = pc = ps = None
    if stats:
        rm = torch.empty((heads, lq), dtype=torch.float32, device=q.device)
        rs = torch.empty((heads, lq), dtype=torch.float32, device=q.device)
    if probs:
        pc = torch.empty((heads, lq, lk // BLOCK, 16), dtype=torch.uint8, device=q.device)
        ps = torch.empty((heads, lq, lk // BLOCK), dtype=torch.uint8, device=q.device)
    fn, name = (mx_attention_fwd_efq, "mx_attention_fwd_efq") if efq else \
        (mx_attention_fwd, "mx_attention_fwd")
    _check(fn(f, BLOCK, q, k, v_codes, v_scales, heads, lq, lk, d, scale, _dtype_code(o), o, rm,
              rs, pc, ps), name)
    out = (o,)
    if stats:
        out += (rm, rs)
    if probs:
        out += (pc, ps)
    return out[0] if len(out) == 1 else out
