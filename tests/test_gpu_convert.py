"""The layer-by-layer converter on the GPU: every converted weight equals the
oracle's quantization of that tensor; kept tensors are untouched."""
import warnings

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import assert_bytes_equal, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def conv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_scaled_bit_amd import convert
    return convert


@pytest.mark.parametrize("source", ["device", "host"])
def test_convert_synthetic_model(conv, source):
    model = workloads.synthetic_model(layers=3, moe_layers=(1,))
    host = {k: torch.from_numpy(v.view(np.int16)).view(torch.bfloat16) for k, v in model.items()}
    if source == "device":
        tensors = {k: v.cuda() for k, v in host.items()}
    else:
        tensors = {k: v.pin_memory() for k, v in host.items()}
    cfg = conv.QuantConfig.from_options("online", {
        "moe": {"activation": "mxfp6_e2m3_dynamic", "weight": "mxfp6_e3m2"},
        "overrides": [{"pattern": "model.layers.2.mlp.down_proj", "weight": "mxfp8"},
                      {"pattern": "re:model\\.layers\\.0\\.self_attn\\.(q|k)_proj$", "weight": "axs6"}]})
    n_before = len(tensors)
    with warnings.catch_warnings(record=True) as w:
        warnings.simplefilter("always")
        out, decisions = conv.convert_model(tensors, cfg, consume=True)
    torch.cuda.synchronize()
    assert len(tensors) == n_before - sum(d.weight != "bf16" for d in decisions)
    assert any("lm_head.weight stays bf16" in str(x.message) for x in w)  # 1000 rows
    by = {d.name: d for d in decisions}
    assert by["model.layers.1.mlp.gate.weight"].weight == "bf16"
    assert by["model.layers.1.mlp.shared_expert_gate.weight"].weight == "bf16"
    assert by["model.layers.1.mlp.experts.2.up_proj.weight"].weight == "mxfp6_e3m2"
    assert by["model.layers.2.mlp.down_proj.weight"].weight == "mxfp8"
    assert by["model.layers.0.self_attn.k_proj.weight"].weight == "axs6"
    assert by["model.layers.0.self_attn.v_proj.weight"].weight == "mxfp6_e2m3"
    n_conv = 0
    for name, d in by.items():
        got = out[name]
        if d.weight == "bf16":
            assert isinstance(got, torch.Tensor)
            assert np.array_equal(to_host(got).reshape(-1), model[name].reshape(-1))
            continue
        n_conv += 1
        fmt = conv.WEIGHT_FORMATS[d.weight]
        oc, os_, oa = oracle.quantize(fmt, model[name])
        assert_bytes_equal(to_host(got.scales), os_, name + " scales")
        assert_bytes_equal(to_host(got.codes), oc, name + " codes", oracle.BYTES_PER_BLOCK[fmt])
        if fmt == oracle.AXS6:
            assert_bytes_equal(to_host(got.aux), oa, name + " aux")
        rows, cols = got.shape
        y = got.dequantize(torch.bfloat16)
        assert_bytes_equal(to_host(y), oracle.dequantize(fmt, oc, os_, oa, rows, cols, oracle.BF16),
                           name + " dequantized")
    assert n_conv >= 20


def test_activation_quantization_follows_the_decision(conv):
    x = workloads.activations(rows=64, cols=256)
    codes, scales, _ = conv.quantize_activations(to_dev(x), "mxfp8")
    torch.cuda.synchronize()
    oc, os_, _ = oracle.quantize(oracle.FP8_E4M3, x)
    assert_bytes_equal(to_host(codes), oc, "codes", 32)
    assert_bytes_equal(to_host(scales), os_, "scales")
    assert conv.quantize_activations(to_dev(x), "bf16") is None


def test_peak_extra_memory_is_one_tensor(conv):
    # host-resident sources: the device holds the converted codes plus at most
    # one bf16 source copy at a time
    model = workloads.synthetic_model(layers=4, hidden=1024, intermediate=2048, kv=256, vocab=1024,
                                      moe_layers=())
    tensors = {k: torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).pin_memory()
               for k, v in model.items()}
    cfg = conv.QuantConfig.from_options("mxfp6")
    largest = max(v.numel() * 2 for v in tensors.values())
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    out, _ = conv.convert_model(tensors, cfg, consume=True)
    torch.cuda.synchronize()
    kept = sum(v.nbytes() for v in out.values() if isinstance(v, conv.QuantizedWeight))
    peak = torch.cuda.max_memory_allocated() - base
    assert peak <= kept + largest + (4 << 20), (peak, kept, largest)
