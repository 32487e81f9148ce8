"""Seeded synthetic inputs for the five workloads (no quantization arithmetic).

This module is the only code the HIP path's tests and the CPU oracle's tests
share: it draws random tensors and nothing else.  bf16 tensors are returned as
``numpy.uint16`` bit patterns (fp32 values rounded to bf16 by torch's
round-to-nearest-even cast); fp32 tensors as ``numpy.float32``.

Workloads (shapes and value distributions stand in for the pages' trained
checkpoints, activations and attention scores, which are not available):

  weights_small  fp32 [128, 256], N(0, 1)                       (seed 1)
  axs6_weight    bf16 [4096, 4096], N(0, 0.02^2), 0.1% of the
                 entries multiplied by 50 (outliers)             (seed 2)
  linear_weight  bf16 [14336, 4096], N(0, 0.02^2)                (seed 3)
                 (linear_weight_f16: the same draw rounded to fp16)
  attn_scores    fp32 [32*4096, 4096] (32 heads x 4096 queries
                 x 4096 keys), N(0, 3^2)                         (seed 4)
  activations    bf16 [16384, 8192], 0.5 * Student-t(nu=3); 1% of
                 the 32-value blocks zeroed; 0.01% of the entries
                 set to +inf, -inf, NaN (in turn)                (seed 5)

Every generator accepts a smaller (rows, cols) so tests can run the same
recipe at a size the oracle finishes in seconds.  ``synthetic_model`` draws
a small decoder's named bf16 weights (dense and MoE layers, gates, norms,
embeddings) for the conversion driver's tests.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32

FULL_SHAPES = {
    "weights_small": (128, 256),
    "axs6_weight": (4096, 4096),
    "linear_weight": (14336, 4096),
    "attn_scores": (32 * 4096, 4096),
    "activations": (16384, 8192),
}
SEEDS = {"weights_small": 1, "axs6_weight": 2, "linear_weight": 3, "attn_scores": 4,
         "activations": 5}


def to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even, via torch's cast) as uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def weights_small(rows=128, cols=256, seed=None) -> np.ndarray:
    rng = np.random.default_rng(SEEDS["weights_small"] if seed is None else seed)
    return rng.standard_normal((rows, cols), dtype=np.float32)


def axs6_weight(rows=4096, cols=4096, seed=None) -> np.ndarray:
    rng = np.random.default_rng(SEEDS["axs6_weight"] if seed is None else seed)
    x = (0.02 * rng.standard_normal((rows, cols))).astype(np.float32)
    n = x.size
    k = n // 1000  # 0.1 % outliers
    idx = rng.choice(n, size=k, replace=False)
    x.reshape(-1)[idx] *= np.float32(50.0)
    return to_bf16_bits(x)


def linear_weight(rows=14336, cols=4096, seed=None) -> np.ndarray:
    rng = np.random.default_rng(SEEDS["linear_weight"] if seed is None else seed)
    x = (0.02 * rng.standard_normal((rows, cols))).astype(np.float32)
    return to_bf16_bits(x)


def linear_weight_f16(rows=14336, cols=4096, seed=None) -> np.ndarray:
    """linear_weight's draw rounded to fp16 (numpy's nearest-even cast)
    instead of bf16: the same weight as an FP16 checkpoint would hold it."""
    rng = np.random.default_rng(SEEDS["linear_weight"] if seed is None else seed)
    return (0.02 * rng.standard_normal((rows, cols))).astype(np.float32).astype(np.float16)


def attn_scores(rows=32 * 4096, cols=4096, seed=None) -> np.ndarray:
    rng = np.random.default_rng(SEEDS["attn_scores"] if seed is None else seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    x *= np.float32(3.0)
    return x


def activations(rows=16384, cols=8192, seed=None) -> np.ndarray:
    rng = np.random.default_rng(SEEDS["activations"] if seed is None else seed)
    x = (0.5 * rng.standard_t(3, size=(rows, cols))).astype(np.float32)
    flat = x.reshape(-1)
    nblocks = flat.size // BLOCK
    nz = nblocks // 100  # 1 % all-zero blocks
    zb = rng.choice(nblocks, size=nz, replace=False)
    flat.reshape(nblocks, BLOCK)[zb, :] = 0.0
    nspecial = flat.size // 10000  # 0.01 % non-finite entries
    si = rng.choice(flat.size, size=nspecial, replace=False)
    specials = np.array([np.inf, -np.inf, np.nan], np.float32)
    flat[si] = specials[np.arange(nspecial) % 3]
    return to_bf16_bits(x)


def synthetic_model(layers=2, hidden=256, intermediate=512, kv=128, vocab=1000, experts=4,
                    moe_intermediate=128, moe_layers=(1,), seed=7) -> dict:
    """Tensor names and shapes of a small decoder (attention projections,
    dense or mixture-of-experts MLPs with a router gate, a shared expert and
    its gate, norms, embeddings, output head), every weight N(0, 0.02^2) in
    bf16 bits.  Stands in for a checkpoint being loaded."""
    rng = np.random.default_rng(seed)

    def w(*shape):
        return to_bf16_bits((0.02 * rng.standard_normal(shape)).astype(np.float32))

    t = {"model.embed_tokens.weight": w(vocab, hidden)}
    for i in range(layers):
        p = f"model.layers.{i}."
        t[p + "input_layernorm.weight"] = to_bf16_bits(np.ones(hidden, np.float32))
        t[p + "self_attn.q_proj.weight"] = w(hidden, hidden)
        t[p + "self_attn.k_proj.weight"] = w(kv, hidden)
        t[p + "self_attn.v_proj.weight"] = w(kv, hidden)
        t[p + "self_attn.o_proj.weight"] = w(hidden, hidden)
        t[p + "post_attention_layernorm.weight"] = to_bf16_bits(np.ones(hidden, np.float32))
        if i in moe_layers:
            t[p + "mlp.gate.weight"] = w(experts, hidden)
            for e in range(experts):
                q = p + f"mlp.experts.{e}."
                t[q + "gate_proj.weight"] = w(moe_intermediate, hidden)
                t[q + "up_proj.weight"] = w(moe_intermediate, hidden)
                t[q + "down_proj.weight"] = w(hidden, moe_intermediate)
            for nm in ("gate_proj", "up_proj"):
                t[p + f"mlp.shared_expert.{nm}.weight"] = w(moe_intermediate, hidden)
            t[p + "mlp.shared_expert.down_proj.weight"] = w(hidden, moe_intermediate)
            t[p + "mlp.shared_expert_gate.weight"] = w(1, hidden)
        else:
            t[p + "mlp.gate_proj.weight"] = w(intermediate, hidden)
            t[p + "mlp.up_proj.weight"] = w(intermediate, hidden)
            t[p + "mlp.down_proj.weight"] = w(hidden, intermediate)
    t["model.norm.weight"] = to_bf16_bits(np.ones(hidden, np.float32))
    t["lm_head.weight"] = w(vocab, hidden)
    return t


GENERATORS = {
    "weights_small": weights_small,
    "axs6_weight": axs6_weight,
    "linear_weight": linear_weight,
    "attn_scores": attn_scores,
    "activations": activations,
}


def make(name: str, rows=None, cols=None, seed=None) -> np.ndarray:
    r0, c0 = FULL_SHAPES[name]
    return GENERATORS[name](rows or r0, cols or c0, seed=seed)
