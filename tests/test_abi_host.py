"""The C-ABI library on the host: it loads, exports every symbol include/mx.h
declares, and rejects bad arguments before anything reaches a GPU (these
calls pass fake pointers and the NULL stream; none of them launches)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mx.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mx_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def mx():
    import block_scaled_bit_amd as m
    return m


def test_header_declares_the_boundary():
    names = declared_functions()
    for f in ("mx_quantize", "mx_dequantize", "mx_fake_quantize", "mx_softmax_quantize",
              "mx_buffer_sizes", "mx_status_str", "mx_abi_version", "mx_attention_fwd",
              "mx_attention_fwd_efq", "mx_quantize_batch"):
        assert f in names


def test_library_exports_every_declared_symbol(mx):
    out = subprocess.run(["nm", "-D", "--defined-only", mx.library_path], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (mx_\w+)", out))
    missing = [f for f in declared_functions() if f not in exported]
    assert not missing, missing
    lib = ctypes.CDLL(mx.library_path)
    for f in declared_functions():
        assert getattr(lib, f) is not None


def test_library_is_gfx950_only(mx):
    # the offload targets named in the embedded code objects (our own build)
    data = open(mx.library_path, "rb").read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa--(gfx[0-9a-z]+)", data))
    assert targets == {b"gfx950"}, targets


def test_version_and_status_strings(mx):
    assert mx.mx_abi_version() == 7
    for s in range(0, 8):
        assert isinstance(mx.mx_status_str(s), str) and mx.mx_status_str(s)


@pytest.mark.parametrize("fmt,code,scale,aux", [(0, 24, 1, 0), (1, 24, 1, 0), (2, 16, 1, 0),
                                                (3, 32, 1, 0), (4, 24, 1, 1)])
def test_buffer_sizes(mx, fmt, code, scale, aux):
    rows, cols = 14336, 4096
    nb = rows * cols // 32
    c, s, a = mx.mx_buffer_sizes(fmt, 32, rows, cols)
    assert (c, s) == (nb * code, nb * scale)
    assert a == ((nb + 3) // 4 if aux else 0)
    assert mx.mx_buffer_sizes(fmt, 32, 0, 4096) == (0, 0, 0)


S, OK, NULL, SHAPE, ALIGN, UNSUP = None, 0, 1, 2, 3, 4
A = 0x10000  # a 16-byte aligned fake device address (never dereferenced)


@pytest.mark.parametrize("args,want", [
    ((0, 32, 0, A, 4, 33, A, A, None), SHAPE),        # cols not a multiple of 32
    ((0, 32, 0, A, -1, 32, A, A, None), SHAPE),       # negative rows
    ((0, 16, 0, A, 4, 32, A, A, None), UNSUP),        # block size
    ((5, 32, 0, A, 4, 32, A, A, None), UNSUP),        # format
    ((0, 32, 3, A, 4, 32, A, A, None), UNSUP),        # dtype
    ((0, 32, 2, None, 4, 32, A, A, None), NULL),      # fp16 is accepted
    ((0, 32, 0, None, 4, 32, A, A, None), NULL),      # x
    ((0, 32, 0, A, 4, 32, None, A, None), NULL),      # codes
    ((0, 32, 0, A, 4, 32, A, None, None), NULL),      # scales
    ((4, 32, 0, A, 4, 32, A, A, None), NULL),         # AXS-6 needs aux
    ((0, 32, 0, A + 8, 4, 32, A, A, None), ALIGN),    # x misaligned
    ((0, 32, 0, A, 4, 32, A + 4, A, None), ALIGN),    # codes misaligned
    ((0, 32, 0, None, 0, 32, None, None, None), OK),  # empty: no-op
    ((0, 32, 0, None, 5, 0, None, None, None), OK),   # empty: no-op
])
def test_quantize_argument_errors(mx, args, want):
    assert mx.mx_quantize(*args, stream=0) == want


def test_other_entry_points_argument_errors(mx):
    assert mx.mx_dequantize(0, 32, A, A, None, 4, 31, 0, A, stream=0) == SHAPE
    assert mx.mx_dequantize(0, 32, A, A, None, 4, 32, 7, A, stream=0) == UNSUP
    assert mx.mx_dequantize(0, 32, A, A, None, 4, 32, 0, None, stream=0) == NULL
    assert mx.mx_dequantize(4, 32, A, A, None, 4, 32, 0, A, stream=0) == NULL
    assert mx.mx_dequantize(0, 32, A + 1, A, None, 4, 32, 0, A, stream=0) == ALIGN
    assert mx.mx_fake_quantize(0, 32, 0, A, None, 4, 32, stream=0) == NULL
    assert mx.mx_fake_quantize(0, 32, 0, A, A + 2, 4, 32, stream=0) == ALIGN
    assert mx.mx_fake_quantize(0, 8, 0, A, A, 4, 32, stream=0) == UNSUP
    assert mx.mx_softmax_quantize(4, 32, A, 4, 32, A, A, stream=0) == UNSUP
    assert mx.mx_softmax_quantize(2, 32, A, 4, 30, A, A, stream=0) == SHAPE
    assert mx.mx_softmax_quantize(2, 32, None, 4, 32, A, A, stream=0) == NULL
    assert mx.mx_softmax_quantize(2, 32, None, 0, 32, None, None, stream=0) == OK


def test_quantize_batch_argument_errors(mx):
    import ctypes
    good = (A, 4, 64, A, A, None)
    lib = mx._lib
    assert lib.mx_quantize_batch(0, 32, 0, None, -1, None) == SHAPE
    assert lib.mx_quantize_batch(0, 32, 0, None, 2, None) == NULL
    assert lib.mx_quantize_batch(0, 32, 0, None, 0, None) == OK
    assert mx.mx_quantize_batch(0, 32, 0, [], stream=0) == OK
    # the first failing tensor's status, wherever it is in the batch
    assert mx.mx_quantize_batch(0, 32, 0, [good, (A, 4, 48, A, A, None)], stream=0) == SHAPE
    assert mx.mx_quantize_batch(0, 32, 0, [good, good, (A, 4, 64, None, A, None)], stream=0) == NULL
    assert mx.mx_quantize_batch(0, 32, 0, [(A + 8, 4, 64, A, A, None), good], stream=0) == ALIGN
    assert mx.mx_quantize_batch(4, 32, 0, [good], stream=0) == NULL       # AXS-6 needs aux
    assert mx.mx_quantize_batch(0, 16, 0, [good], stream=0) == UNSUP
    assert mx.mx_quantize_batch(0, 32, 3, [good], stream=0) == UNSUP
    assert mx.mx_quantize_batch(0x200, 32, 0, [good], stream=0) == UNSUP
    # empty tensors only: nothing to do, even with NULL pointers
    assert mx.mx_quantize_batch(0, 32, 0, [(None, 0, 64, None, None, None)] * 3, stream=0) == OK
    assert ctypes.sizeof(mx._TensorDesc) == 48


def test_python_helpers_reject_host_tensors(mx):
    import torch
    with pytest.raises(ValueError):
        mx.quantize(torch.zeros(2, 64), "mxfp6")
    with pytest.raises(ValueError):
        mx.fake_quantize(torch.zeros(2, 64), "axs6")
    assert mx.FORMATS["mxfp6"] == mx.MX_FP6_E2M3 and mx.FORMATS["mxfp8"] == mx.MX_FP8_E4M3


def test_python_helpers_check_every_buffer_before_launching(mx):
    """Each helper refuses a buffer of the wrong dtype, byte size, layout or
    device with ValueError before anything reaches the C ABI; the size and
    layout checks come first, so host tensors exercise them here."""
    import torch
    u8 = torch.uint8
    nb = 4 * 2  # a [4, 64] tensor: 8 blocks
    good_codes, good_scales = torch.zeros(4, 2, 24, dtype=u8), torch.zeros(4, 2, dtype=u8)

    def bad(fn, *a, match, **kw):
        with pytest.raises(ValueError, match=match):
            fn(*a, **kw)

    # dequantize: codes must hold nb * bytes-per-block bytes of uint8
    bad(mx.dequantize, torch.zeros(4, 2, 16, dtype=u8), good_scales, fmt="mxfp6", match="codes holds")
    bad(mx.dequantize, torch.zeros(4, 2, 24, dtype=u8), good_scales, fmt="mxfp4", match="codes holds")
    bad(mx.dequantize, torch.zeros(4, 2, 12, dtype=torch.int16), good_scales, match="codes must be")
    bad(mx.dequantize, torch.zeros(4, 2, 48, dtype=u8)[..., ::2], good_scales, match="contiguous")
    bad(mx.dequantize, good_codes, torch.zeros(4, 2, dtype=torch.int32), match="scales must be")
    bad(mx.dequantize, good_codes, good_scales, fmt="e3m3", match="codes holds")  # 28 B per block
    # AXS-6 also needs its config plane of ceil(nb / 4) bytes
    bad(mx.dequantize, good_codes, good_scales, None, "axs6", match="aux must be a torch tensor")
    bad(mx.dequantize, good_codes, good_scales, torch.zeros(nb, dtype=u8), "axs6", match="aux holds")
    # well-formed host buffers fail only on the device check
    bad(mx.dequantize, good_codes, good_scales, match="GPU memory")
    bad(mx.dequantize, good_codes, good_scales, torch.zeros(2, dtype=u8), "axs6", match="GPU memory")
    with pytest.raises(mx.MxError):
        mx.dequantize(good_codes, good_scales, fmt="mxfp6", block=16)

    # fake_quantize: out must match x's shape and dtype exactly
    x = torch.zeros(4, 64)
    bad(mx.fake_quantize, x, out=torch.zeros(4, 64, dtype=torch.bfloat16), match="out must be")
    bad(mx.fake_quantize, x, out=torch.zeros(4, 32), match="shape")
    bad(mx.fake_quantize, x, out=torch.zeros(64, 4).t(), match="contiguous")
    bad(mx.fake_quantize, x, out=torch.zeros(4, 64), match="GPU memory")
    bad(mx.fake_quantize, torch.zeros(4, 48), match="multiple of 32")
    bad(mx.quantize, torch.zeros(8, 64)[:, :32], match="contiguous")
    bad(mx.quantize_many, [torch.zeros(4, 64), torch.zeros(4, 40)], match="multiple of 32")

    # attention_fwd: V's codes and scales must match (heads, 128, lk/32) of
    # the V format
    q = torch.zeros(2, 64, 128, dtype=torch.bfloat16)
    k = torch.zeros(2, 96, 128, dtype=torch.bfloat16)
    vc = torch.zeros(2, 128, 3, 32, dtype=u8)
    vs = torch.zeros(2, 128, 3, dtype=u8)
    bad(mx.attention_fwd, q, k, vc, vs, "mxfp6", match="v_codes holds")
    bad(mx.attention_fwd, q, k, vc[:, :, :2].contiguous(), vs, "mxfp8", match="v_codes holds")
    bad(mx.attention_fwd, q, k, vc, vs[:, :, :2].contiguous(), "mxfp8", match="v_scales holds")
    bad(mx.attention_fwd, q, k[:, :80].contiguous(), vc, vs, "mxfp8", match="multiple of 32")
    bad(mx.attention_fwd, q, torch.zeros(3, 96, 128, dtype=torch.bfloat16), vc, vs, match="k must be")
    bad(mx.attention_fwd, q, k, vc.to(torch.int16), vs, "mxfp8", match="v_codes must be")
    bad(mx.attention_fwd, q, k, vc, vs, "mxfp8", match="GPU memory")
    with pytest.raises(mx.MxError):
        mx.attention_fwd(q, k, vc, vs, "axs6")
    with pytest.raises(mx.MxError):
        mx.attention_fwd(q.float(), k, vc, vs, "mxfp8")


def test_generic_exmy_formats_host_checks(mx):
    assert mx.mx_buffer_sizes(mx.MX_EXMY(3, 3), 32, 4, 64) == (4 * 2 * 28, 8, 0)
    assert mx.mx_buffer_sizes("e0m8", 32, 1, 32) == (36, 1, 0)
    assert mx.mx_buffer_sizes(mx.MX_EXMY(8, 0), 32, 2, 64) == (2 * 2 * 36, 4, 0)
    for bad in (mx.MX_EXMY(8, 1), mx.MX_EXMY(9, 0), mx.MX_EXMY(0, 1), mx.MX_EXMY(1, 0),
                mx.MX_EXMY(4, 5), 0x200):
        assert mx.mx_quantize(bad, 32, 0, A, 4, 32, A, A, None, stream=0) == UNSUP
    assert mx.mx_softmax_quantize(mx.MX_EXMY(2, 1), 32, A, 4, 32, A, A, stream=0) == UNSUP
    assert mx.mx_quantize(mx.MX_EXMY(2, 2), 32, 0, None, 4, 32, A, A, None, stream=0) == NULL


def test_attention_argument_errors(mx):
    A = 1 << 20  # a fake 16-byte-aligned address; nothing is launched
    OK, NULL, SHAPE, ALIGN, UNSUP, VALUE = 0, 1, 2, 3, 4, 6
    E4M3, E2M3, E3M2, E2M1, AXS6 = mx.MX_FP8_E4M3, mx.MX_FP6_E2M3, mx.MX_FP6_E3M2, \
        mx.MX_FP4_E2M1, mx.MX_AXS6

    def call(v_fmt=E4M3, block=32, q=A, k=A, vc=A, vs=A, heads=2, lq=64, lk=128, d=128,
             out=mx.MX_BF16, o=A, pc=None, ps=None, scale=0.125):
        rc = mx.mx_attention_fwd(v_fmt, block, q, k, vc, vs, heads, lq, lk, d, scale, out, o,
                                 None, None, pc, ps, stream=0)
        rc_efq = mx.mx_attention_fwd_efq(v_fmt, block, q, k, vc, vs, heads, lq, lk, d, scale, out,
                                         o, None, None, pc, ps, stream=0)
        assert rc == rc_efq
        return rc

    assert call(v_fmt=AXS6) == UNSUP
    assert call(v_fmt=mx.MX_EXMY(2, 3)) == UNSUP
    assert call(block=16) == UNSUP
    assert call(d=64) == UNSUP
    assert call(out=7) == UNSUP
    assert call(out=mx.MX_FP16) == UNSUP  # bf16 or fp32 output only
    assert call(lk=0) == SHAPE
    assert call(lk=48) == SHAPE
    assert call(lk=(1 << 24) + 32) == SHAPE
    assert call(lq=-1) == SHAPE
    assert call(heads=-1) == SHAPE
    # the scale must be positive with scale * log2(e) finite (the kernel
    # orders the scores before scaling them)
    for bad in (0.0, -0.0, -0.125, float("nan"), float("inf"), 3e38):
        assert call(scale=bad) == VALUE, bad
        assert call(scale=bad, heads=0) == VALUE, bad
    assert call(scale=2e38, q=None) == NULL  # 2e38 log2(e) is still finite
    assert call(scale=1e-45, q=None) == NULL
    assert call(pc=A) == NULL           # probability codes without their scales
    assert call(q=None) == NULL
    assert call(vs=None) == NULL
    assert call(q=A + 8) == ALIGN
    assert call(o=A + 4) == ALIGN
    assert call(pc=A + 8, ps=A) == ALIGN
    # empty work is a no-op even with NULL pointers
    assert call(heads=0, q=None, k=None, vc=None, vs=None, o=None) == OK
    assert call(lq=0, q=None, k=None, vc=None, vs=None, o=None) == OK
    for f in (E4M3, E2M3, E3M2, E2M1):
        assert call(v_fmt=f, heads=0) == OK


FORCED_FAILURE_CHILD = r"""
import block_scaled_bit_amd as mx
A = 1 << 20  # fake 16-byte-aligned addresses: the hook returns before any launch
DEV, OK, SHAPE, NULL = 5, 0, 2, 1
got = {
    "quantize": mx.mx_quantize(0, 32, 0, A, 4, 32, A, A, None, stream=0),
    "quantize_exmy": mx.mx_quantize(mx.MX_EXMY(3, 3), 32, 1, A, 4, 32, A, A, None, stream=0),
    "dequantize": mx.mx_dequantize(3, 32, A, A, None, 4, 32, 1, A, stream=0),
    "fake_quantize": mx.mx_fake_quantize(4, 32, 0, A, A, 4, 32, stream=0),
    "softmax_quantize": mx.mx_softmax_quantize(2, 32, A, 4, 64, A, A, stream=0),
    "attention": mx.mx_attention_fwd(3, 32, A, A, A, A, 2, 64, 128, 128, 0.125, 0, A,
                                     None, None, None, None, stream=0),
    "quantize_batch": mx.mx_quantize_batch(2, 32, 0, [(A, 4, 64, A, A, None)] * 20, stream=0),
    "quantize_batch_exmy": mx.mx_quantize_batch(0x133, 32, 0, [(A, 4, 64, A, A, None)], stream=0),
    "attention_efq": mx.mx_attention_fwd_efq(3, 32, A, A, A, A, 2, 64, 128, 128, 0.125, 0, A,
                                             None, None, None, None, stream=0),
    # argument errors are still found first, and empty work is still a no-op
    "bad_shape": mx.mx_quantize(0, 32, 0, A, 4, 31, A, A, None, stream=0),
    "null": mx.mx_dequantize(0, 32, None, A, None, 4, 32, 0, A, stream=0),
    "empty": mx.mx_quantize(0, 32, 0, None, 0, 32, None, None, None, stream=0),
}
want = {k: DEV for k in got}
want.update(bad_shape=SHAPE, null=NULL, empty=OK)
assert got == want, got
try:
    mx._check(mx.mx_quantize(0, 32, 0, A, 4, 32, A, A, None, stream=0), "mx_quantize")
except mx.MxError as e:
    assert e.status == DEV and "launch failed" in str(e)
else:
    raise AssertionError("no MxError")
print("forced failure ok")
"""


def test_forced_launch_failure_returns_device_error():
    # MX_TEST_FAIL_LAUNCH=1 (read once per process) turns every call that
    # passes its argument checks into MX_ERR_DEVICE without a launch; run in
    # a child process so no other test sees the hook
    env = dict(os.environ, MX_TEST_FAIL_LAUNCH="1")
    r = subprocess.run(["python", "-c", FORCED_FAILURE_CHILD], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "forced failure ok" in r.stdout
