"""The entry points under HIP graph capture.

The library launches kernels and nothing else (no allocation, no memset, no
synchronisation), so a sequence of its calls can be captured into a graph
and replayed.  A graph over static buffers runs quantize, dequantize,
fake-quantize, the exp-then-quantize prologue and the attention forward;
it is replayed on three input sets, with eager work and synchronisations
between the replays, and every replay must equal the same calls made
eagerly on separate output buffers, byte for byte.
"""
import pytest
import torch

pytestmark = pytest.mark.gpu

ROWS, COLS = 256, 4096  # bf16 weights, E2M3
SROWS = 64              # exp-then-quantize rows of 4096 fp32 scores
HEADS, LQ, LK, D = 2, 256, 512, 128


@pytest.fixture(scope="module")
def mx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_bit_amd as m
    return m


def _outputs(mx, dev):
    nb = ROWS * COLS // 32
    nbs = SROWS * 4096 // 32
    nbp = HEADS * LQ * (LK // 32)
    u8 = dict(dtype=torch.uint8, device=dev)
    return {
        "codes": torch.empty(nb * 24, **u8), "scales": torch.empty(nb, **u8),
        "y": torch.empty(ROWS, COLS, dtype=torch.bfloat16, device=dev),
        "fq": torch.empty(ROWS, COLS, dtype=torch.bfloat16, device=dev),
        "pcodes": torch.empty(nbs * 16, **u8), "pscales": torch.empty(nbs, **u8),
        "o": torch.empty(HEADS, LQ, D, dtype=torch.bfloat16, device=dev),
        "row_max": torch.empty(HEADS, LQ, dtype=torch.float32, device=dev),
        "row_sum": torch.empty(HEADS, LQ, dtype=torch.float32, device=dev),
        "apc": torch.empty(nbp * 16, **u8), "aps": torch.empty(nbp, **u8),
    }


def _enqueue(mx, inp, out):
    """The whole sequence on the current stream (the capture stream while
    a graph is being captured)."""
    st = [
        mx.mx_quantize(mx.MX_FP6_E2M3, 32, mx.MX_BF16, inp["x"], ROWS, COLS, out["codes"],
                       out["scales"], None),
        mx.mx_dequantize(mx.MX_FP6_E2M3, 32, out["codes"], out["scales"], None, ROWS, COLS,
                         mx.MX_BF16, out["y"]),
        mx.mx_fake_quantize(mx.MX_FP6_E2M3, 32, mx.MX_BF16, inp["x"], out["fq"], ROWS, COLS),
        mx.mx_softmax_quantize(mx.MX_FP4_E2M1, 32, inp["s"], SROWS, 4096, out["pcodes"],
                               out["pscales"]),
        mx.mx_attention_fwd(mx.MX_FP8_E4M3, 32, inp["q"], inp["k"], inp["vc"], inp["vs"], HEADS,
                            LQ, LK, D, D ** -0.5, mx.MX_BF16, out["o"], out["row_max"],
                            out["row_sum"], out["apc"], out["aps"]),
    ]
    assert st == [0] * len(st), st


def _fill(mx, inp, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    inp["x"].copy_((torch.randn(ROWS, COLS, generator=g, device="cuda") * 0.02).bfloat16())
    inp["s"].copy_(torch.randn(SROWS, 4096, generator=g, device="cuda") * 3.0)
    inp["q"].copy_(torch.randn(HEADS, LQ, D, generator=g, device="cuda").bfloat16())
    inp["k"].copy_(torch.randn(HEADS, LK, D, generator=g, device="cuda").bfloat16())
    vc, vs = mx.quantize_v(torch.randn(HEADS, LK, D, generator=g, device="cuda").bfloat16(),
                           "mxfp8")
    inp["vc"].copy_(vc.reshape(-1))
    inp["vs"].copy_(vs.reshape(-1))


def test_graph_replays_equal_eager_calls(mx):
    dev = torch.device("cuda")
    nbv = HEADS * D * (LK // 32)
    inp = {
        "x": torch.empty(ROWS, COLS, dtype=torch.bfloat16, device=dev),
        "s": torch.empty(SROWS, 4096, dtype=torch.float32, device=dev),
        "q": torch.empty(HEADS, LQ, D, dtype=torch.bfloat16, device=dev),
        "k": torch.empty(HEADS, LK, D, dtype=torch.bfloat16, device=dev),
        "vc": torch.empty(nbv * 32, dtype=torch.uint8, device=dev),
        "vs": torch.empty(nbv, dtype=torch.uint8, device=dev),
    }
    ref, gout = _outputs(mx, dev), _outputs(mx, dev)
    # every kernel runs once before capture (code objects load on first use)
    _fill(mx, inp, 0)
    _enqueue(mx, inp, ref)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _enqueue(mx, inp, gout)
    torch.cuda.synchronize()

    for seed in (1, 2, 3):
        _fill(mx, inp, seed)
        for t in gout.values():
            t.view(torch.uint8).fill_(0xA5)  # stale contents must not survive a replay
        _enqueue(mx, inp, ref)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, want in ref.items():
            got = gout[name]
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), (seed, name)
        # the replay also agrees with itself when run again on the same inputs
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(gout["codes"], ref["codes"]) and torch.equal(gout["apc"], ref["apc"])
