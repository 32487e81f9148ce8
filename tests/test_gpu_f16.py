"""fp16 tensors on the GPU ("Online MXFP6", "Start a model": BF16 or FP16
weights), bit-exact against the oracle: quantize over every finite fp16
pattern, dequantize to fp16 of arbitrary codes under every scale byte,
fake-quantize with specials and in place, the batched quantize and the
conversion driver."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_bytes_equal, to_host

pytestmark = pytest.mark.gpu

FMTS = [oracle.FP6_E2M3, oracle.FP6_E3M2, oracle.FP4_E2M1, oracle.FP8_E4M3, oracle.AXS6,
        oracle.exmy(3, 3), oracle.exmy(5, 2), oracle.exmy(8, 0), oracle.exmy(0, 8),
        oracle.exmy(2, 0)]
ids = ["e2m3", "e3m2", "e2m1", "e4m3", "axs6", "x-e3m3", "x-e5m2", "x-e8m0", "x-e0m8", "x-e2m0"]


@pytest.fixture(scope="module")
def mx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_bit_amd as m
    return m


def dev16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16)).cuda()


def all_finite_f16():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    return h[np.isfinite(h)]


def anchored_blocks(vals, E):
    n = (len(vals) + 30) // 31
    b = np.empty((n, 32), np.float16)
    b[:, 0] = np.float16(2.0 ** E)
    b[:, 1:] = np.resize(vals, n * 31).reshape(n, 31)
    return b


@pytest.mark.parametrize("fmt", FMTS, ids=ids)
def test_quantize_every_f16_pattern(mx, fmt):
    allv = all_finite_f16()
    absv = np.abs(allv.astype(np.float64))
    x = np.concatenate([anchored_blocks(allv[absv < 2.0 ** (E + 1)], E)
                        for E in (-24, -14, -3, 0, 7, 15)])
    codes, scales, aux = mx.quantize(dev16(x), fmt)
    torch.cuda.synchronize()
    oc, os_, oa = oracle.quantize(fmt, x)
    assert_bytes_equal(to_host(scales), os_, "scales")
    assert_bytes_equal(to_host(codes), oc, "codes", oracle.BYTES_PER_BLOCK[fmt])
    if fmt == oracle.AXS6:
        assert_bytes_equal(to_host(aux), oa, "config plane")


@pytest.mark.parametrize("fmt", FMTS, ids=ids)
def test_dequantize_to_f16_every_scale_byte(mx, fmt):
    rng = np.random.default_rng(200 + fmt)
    rows, cols = 97, 96
    nb = rows * cols // 32
    bpb = oracle.BYTES_PER_BLOCK[fmt]
    codes = rng.integers(0, 256, (nb, bpb), dtype=np.uint8)
    scales = np.resize(np.arange(256, dtype=np.uint8), nb)
    aux = np.zeros((nb + 3) // 4, np.uint8) if fmt == oracle.AXS6 else None
    y = mx.dequantize(torch.from_numpy(codes).cuda().reshape(rows, cols // 32, bpb),
                      torch.from_numpy(scales).cuda().reshape(rows, cols // 32),
                      torch.from_numpy(aux).cuda() if aux is not None else None, fmt,
                      torch.float16)
    torch.cuda.synchronize()
    want = oracle.dequantize(fmt, codes, scales, aux, rows, cols, oracle.F16)
    assert_bytes_equal(to_host(y).view(np.uint16), want.view(np.uint16), "dequantized fp16")


def special_f16(rng, rows, cols):
    x = (rng.standard_t(3, (rows, cols)) * np.exp2(rng.integers(-22, 12, (rows, 1))))
    with np.errstate(over="ignore"):
        x = x.astype(np.float16)  # the rare overflow to inf is one more special
    flat = x.reshape(-1, 32)
    k = flat.shape[0] // 30
    if k == 0:
        return x
    pick = rng.choice(flat.shape[0], size=5 * k, replace=False)
    flat[pick[:k]] = 0.0
    flat[pick[k:2 * k], 3] = np.nan
    flat[pick[2 * k:3 * k], 7] = -np.inf
    flat[pick[3 * k:4 * k], ::3] = -0.0
    flat[pick[4 * k:5 * k], 5] = np.float16(65504.0)
    return x


@pytest.mark.parametrize("fmt", FMTS, ids=ids)
def test_fake_quantize_f16_and_round_trip(mx, fmt):
    rng = np.random.default_rng(300 + fmt)
    x = special_f16(rng, 67, 320)
    xd = dev16(x)
    fq = mx.fake_quantize(xd, fmt)
    codes, scales, aux = mx.quantize(xd, fmt)
    y = mx.dequantize(codes, scales, aux, fmt, torch.float16)
    torch.cuda.synchronize()
    want = oracle.fake_quantize(fmt, x)
    assert_bytes_equal(to_host(fq).view(np.uint16), want.view(np.uint16), "fake-quantized")
    assert_bytes_equal(to_host(y).view(np.uint16), want.view(np.uint16), "dequantize(quantize)")
    mx.fake_quantize(xd, fmt, out=xd)
    torch.cuda.synchronize()
    assert_bytes_equal(to_host(xd).view(np.uint16), want.view(np.uint16), "in place")


@pytest.mark.parametrize("fmt", [oracle.FP6_E2M3, oracle.FP8_E4M3], ids=["e2m3", "e4m3"])
def test_batched_quantize_f16(mx, fmt):
    rng = np.random.default_rng(400 + fmt)
    shapes = [(33, 64), (1, 32), (300, 256), (64, 1024)]
    xs = [special_f16(rng, r, c) for r, c in shapes]
    outs = mx.quantize_many([dev16(x) for x in xs], fmt)
    torch.cuda.synchronize()
    for x, (codes, scales, _) in zip(xs, outs):
        oc, os_, _ = oracle.quantize(fmt, x)
        assert_bytes_equal(to_host(scales), os_, "scales")
        assert_bytes_equal(to_host(codes), oc, "codes", oracle.BYTES_PER_BLOCK[fmt])


def test_converter_takes_fp16_and_bf16_weights(mx):
    from block_scaled_bit_amd import convert
    g = torch.Generator(device="cuda").manual_seed(5)
    model = {
        "model.layers.0.self_attn.q_proj.weight":
            (torch.randn(256, 256, generator=g, device="cuda") * 0.02).half(),
        "model.layers.0.self_attn.k_proj.weight":
            (torch.randn(128, 256, generator=g, device="cuda") * 0.02).bfloat16(),
        "model.layers.0.mlp.up_proj.weight":
            (torch.randn(384, 256, generator=g, device="cuda") * 0.02).half(),
        "model.layers.1.mlp.down_proj.weight":
            (torch.randn(256, 384, generator=g, device="cuda") * 0.02).half().cpu(),
    }
    out, _ = convert.convert_model(model, convert.QuantConfig.from_options("mxfp6"))
    torch.cuda.synchronize()
    for name, t in model.items():
        h = t.detach().cpu()
        x = h.numpy() if h.dtype == torch.float16 else h.view(torch.int16).numpy().view(np.uint16)
        oc, os_, _ = oracle.quantize(oracle.FP6_E2M3, x)
        assert_bytes_equal(to_host(out[name].scales), os_, name + " scales")
        assert_bytes_equal(to_host(out[name].codes), oc, name + " codes", 24)


@pytest.mark.parametrize("fmt", FMTS[:5], ids=ids[:5])
@pytest.mark.parametrize("nblocks", [1, 63, 64, 65, 1000])
def test_f16_outputs_stay_in_bounds(mx, fmt, nblocks):
    # fp16 outputs leave through the same 64-block LDS tiles as bf16; a
    # ragged last tile writes its own bytes and nothing after them
    rng = np.random.default_rng(500 + nblocks)
    x = special_f16(rng, nblocks, 32)
    guard, n = 4096, nblocks * 32
    ybuf = torch.empty(guard + n + guard, dtype=torch.float16, device="cuda")
    ybuf.view(torch.int16).fill_(0x5A5A)
    sentinel = to_host(ybuf[:guard]).view(np.uint16).copy()

    def check(want, what):
        torch.cuda.synchronize()
        yh = to_host(ybuf).view(np.uint16)
        assert np.array_equal(yh[:guard], sentinel) and np.array_equal(yh[guard + n:], sentinel)
        assert_bytes_equal(yh[guard:guard + n], want.reshape(-1).view(np.uint16), what, 64)

    assert mx.mx_fake_quantize(fmt, 32, mx.MX_FP16, dev16(x), ybuf[guard:guard + n],
                               nblocks, 32) == 0
    check(oracle.fake_quantize(fmt, x), "fq")
    oc, os_, oa = oracle.quantize(fmt, x)
    ybuf.view(torch.int16).fill_(0x5A5A)
    assert mx.mx_dequantize(fmt, 32, torch.from_numpy(oc).cuda(), torch.from_numpy(os_).cuda(),
                            torch.from_numpy(oa).cuda() if fmt == oracle.AXS6 else None,
                            nblocks, 32, mx.MX_FP16, ybuf[guard:guard + n]) == 0
    check(oracle.dequantize(fmt, oc, os_, oa, nblocks, 32, oracle.F16), "dq")


@pytest.mark.parametrize("fmt", oracle.EXMY_FORMATS, ids=lambda f: f"e{(f >> 4) & 15}m{f & 15}")
def test_every_exmy_split_on_every_f16_pattern(mx, fmt):
    # quantize and fake-quantize of every finite fp16 pattern under three
    # anchors, for each of the 42 splits of 3 to 9 bits
    allv = all_finite_f16()
    absv = np.abs(allv.astype(np.float64))
    x = np.concatenate([anchored_blocks(allv[absv < 2.0 ** (E + 1)], E) for E in (-14, 0, 15)])
    xd = dev16(x)
    codes, scales, _ = mx.quantize(xd, fmt)
    fq = mx.fake_quantize(xd, fmt)
    torch.cuda.synchronize()
    oc, os_, _ = oracle.quantize(fmt, x)
    assert_bytes_equal(to_host(scales), os_, "scales")
    assert_bytes_equal(to_host(codes), oc, "codes", oracle.BYTES_PER_BLOCK[fmt])
    want = oracle.fake_quantize(fmt, x)
    assert_bytes_equal(to_host(fq).view(np.uint16), want.view(np.uint16), "fake-quantized", 64)
