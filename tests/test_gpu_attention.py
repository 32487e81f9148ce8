"""Fused attention forward with E2M1 probabilities (mx_attention_fwd, and
mx_attention_fwd_efq with the exp-free EFQ reading) against the CPU oracle,
through the C ABI.

Inputs the oracle and the kernel share: q and k as bf16 bits, V^T quantized
by the *oracle* (its codes are uploaded; nothing expected comes from the
GPU).  Two kinds of scores:
* exact: q and k hold multiples of 1/4 in [-3, 3], so every product and
  partial sum of q . k (d = 128) is exact in fp32 whatever the
  accumulation order; the scores in powers of two, t = fp32(s *
  fp32(scale * log2 e)), are then the same numbers on both sides, and the
  probability blocks, the scale bytes and the row maxima must agree bit
  for bit;
* natural: bf16 N(0, 1) q and k; the fp32 matrix-core sum may differ from
  the oracle's correctly rounded score in the last bits, which can move a
  probability across an E2M1 rounding boundary; such blocks are counted
  and their effect is bounded exactly from the two sets of codes.
Output bound (matching probability blocks): with A >= max over keys of |v|,
    |o - o_ref| <= (c_V + g) A + (g + 2^-24) |o_ref| (+ 2^-7 |o_ref| in bf16)
where g = (lk/8 + 2 ntiles + 2) 2^-24 covers the fp32 additions of group
sums and the rescalings, and c_V = 2^-10 for E4M3 V (the matrix core's
truncation inside groups of 8 FP8 products), 0 for FP6/FP4 V.
"""
import zlib

import numpy as np
import pytest
import torch

import brute
import oracle
import workloads
from gpu_util import to_dev, to_host

pytestmark = pytest.mark.gpu

V_FORMATS = {"e4m3": oracle.FP8_E4M3, "e2m3": oracle.FP6_E2M3, "e3m2": oracle.FP6_E3M2,
             "e2m1": oracle.FP4_E2M1}
D = 128


@pytest.fixture(scope="module")
def mx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_bit_amd as m
    return m


def bf16(x):
    return workloads.to_bf16_bits(np.asarray(x, np.float32))


def exact_qk(rng, heads, lq, lk):
    q = rng.integers(-12, 13, (heads, lq, D)).astype(np.float32) / 4
    k = rng.integers(-12, 13, (heads, lk, D)).astype(np.float32) / 4
    return bf16(q), bf16(k)


def natural_qk(rng, heads, lq, lk):
    return (bf16(rng.standard_normal((heads, lq, D))),
            bf16(rng.standard_normal((heads, lk, D))))


def v_input(rng, heads, lk, fmt):
    v = (rng.standard_normal((heads, lk, D)) * np.exp2(rng.integers(-3, 4, (1, 1, D)))).astype(
        np.float32)
    vt = np.ascontiguousarray(v.transpose(0, 2, 1))
    codes, scales, _ = oracle.quantize(fmt, vt)
    return codes, scales


def vhat_absmax(fmt, codes, scales, heads, lk):
    """Upper bound of max over keys of |decoded V| per (head, d): the
    format's largest finite magnitude times the block scale."""
    top = brute.finite_grid(fmt).max()
    s = scales.reshape(heads, D, lk // 32).astype(np.float64)
    return (top * np.exp2(s - 127)).max(-1)


def run_gpu(mx, fmt, q, k, vc, vs, scale, out_dtype, efq=False):
    heads, lq, _ = q.shape
    lk = k.shape[1]
    o, rm, rs, pc, ps = mx.attention_fwd(to_dev(q), to_dev(k), to_dev(vc), to_dev(vs), fmt,
                                         scale=scale, out_dtype=out_dtype, stats=True, probs=True,
                                         efq=efq)
    torch.cuda.synchronize()
    return (to_host(o), to_host(rm), to_host(rs), to_host(pc).reshape(heads, lq, lk // 32, 16),
            to_host(ps).reshape(heads, lq, lk // 32))


def out_bound(fmt, lk, vmax, o_ref, bf16_out):
    ntiles = -(-lk // 64)
    g = (lk / 8 + 2 * ntiles + 2) * 2.0 ** -24
    c = 2.0 ** -10 if fmt == oracle.FP8_E4M3 else 0.0
    ao = np.abs(o_ref)
    b = (c + g) * vmax[:, None, :] + (g + 2.0 ** -24) * ao
    if bf16_out:
        b = b + 2.0 ** -7 * ao
    return b


def as_f64(o, bf16_out):
    return workloads.bf16_bits_to_f32(o).astype(np.float64) if bf16_out else o.astype(np.float64)


@pytest.mark.parametrize("rule", ["exp", "efq"])
@pytest.mark.parametrize("vname", list(V_FORMATS))
@pytest.mark.parametrize("shape", [(2, 200, 416), (1, 1, 32), (3, 128, 64), (1, 33, 96)])
@pytest.mark.parametrize("out", ["fp32", "bf16"])
def test_exact_scores_parity(mx, vname, shape, out, rule):
    fmt = V_FORMATS[vname]
    heads, lq, lk = shape
    efq = rule == "efq"
    rng = np.random.default_rng(zlib.crc32(repr((vname, shape, out, rule)).encode()))
    q, k = exact_qk(rng, heads, lq, lk)
    vc, vs = v_input(rng, heads, lk, fmt)
    scale = np.float32(D ** -0.5)
    bf = out == "bf16"
    od = oracle.BF16 if bf else oracle.FP32
    o_ref, rm_ref, rs_ref, pc_ref, ps_ref = oracle.attention_fwd(fmt, q, k, vc, vs, scale, 64, od,
                                                                 efq=efq)
    o, rm, rs, pc, ps = run_gpu(mx, fmt, q, k, vc, vs, scale,
                                torch.bfloat16 if bf else torch.float32, efq=efq)
    assert np.array_equal(ps, ps_ref), "probability scale bytes"
    assert np.array_equal(pc, pc_ref), "probability codes"
    assert np.array_equal(rm, rm_ref)  # by value (a zero maximum may differ in sign)
    assert np.all(np.abs(rs.astype(np.float64) - rs_ref) <= 2.0 ** -20 * rs_ref)
    ref = as_f64(o_ref, bf)
    got = as_f64(o, bf)
    vmax = vhat_absmax(fmt, vc, vs, heads, lk)
    bound = out_bound(fmt, lk, vmax, ref, bf)
    err = np.abs(got - ref)
    assert np.all(err <= bound), float((err / bound).max())


@pytest.mark.parametrize("rule", ["exp", "efq"])
@pytest.mark.parametrize("vname", ["e4m3", "e2m3"])
def test_natural_scores(mx, vname, rule):
    fmt = V_FORMATS[vname]
    heads, lq, lk = 2, 256, 512
    efq = rule == "efq"
    rng = np.random.default_rng(7)
    q, k = natural_qk(rng, heads, lq, lk)
    vc, vs = v_input(rng, heads, lk, fmt)
    scale = np.float32(D ** -0.5)
    o_ref, rm_ref, rs_ref, pc_ref, ps_ref = oracle.attention_fwd(fmt, q, k, vc, vs, scale, 64,
                                                                 oracle.FP32, efq=efq)
    o, rm, rs, pc, ps = run_gpu(mx, fmt, q, k, vc, vs, scale, torch.float32, efq=efq)
    same_block = np.all(pc == pc_ref, axis=-1) & (ps == ps_ref)
    assert same_block.mean() > 0.999, same_block.mean()
    # decoded E2M1 probabilities of both sides
    g = brute.grid(oracle.FP4_E2M1)

    def decode(pcodes, pscales):
        nib = np.stack([pcodes & 15, pcodes >> 4], -1).reshape(pcodes.shape[:-1] + (32,))
        return g[nib & 7] * np.exp2(pscales.astype(np.float64) - 127)[..., None]

    dp = np.abs(decode(pc, ps) - decode(pc_ref, ps_ref)).reshape(heads, lq, lk)
    vmax = vhat_absmax(fmt, vc, vs, heads, lk)
    ref = o_ref.astype(np.float64)
    bound = out_bound(fmt, lk, vmax, ref, False) + 1e-5 * vmax[:, None, :]
    # a probability that moved by dp changes the numerator by at most
    # dp (|v| + |o|) and the denominator by dp (rescale factors are <= 1)
    flip = dp.sum(-1)[..., None] * (vmax[:, None, :] + np.abs(ref))
    bound = bound + flip / np.maximum(rs_ref.astype(np.float64) - dp.sum(-1), 1e-30)[..., None]
    err = np.abs(o.astype(np.float64) - ref)
    assert np.all(err <= bound), float((err / bound).max())


@pytest.mark.parametrize("efq", [False, True])
def test_equal_scores_give_the_mean_of_v(mx, efq):
    # q = 0: every probability is exp(0) = 1 (EFQ: code 6 under 2^-2, also
    # 1), o = the plain mean of decoded V
    rng = np.random.default_rng(3)
    heads, lq, lk = 2, 40, 160
    q = bf16(np.zeros((heads, lq, D)))
    k = bf16(rng.standard_normal((heads, lk, D)))
    vc, vs = v_input(rng, heads, lk, oracle.FP6_E2M3)
    o, rm, rs, pc, ps = run_gpu(mx, oracle.FP6_E2M3, q, k, vc, vs, 0.125, torch.float32, efq=efq)
    vt = oracle.dequantize(oracle.FP6_E2M3, vc, vs, None, heads * D, lk, oracle.FP32)
    want = vt.reshape(heads, D, lk).astype(np.float64).mean(-1)
    assert np.allclose(o, np.broadcast_to(want[:, None, :], o.shape), rtol=1e-6, atol=1e-7)
    assert np.all(rs == lk) and np.all(rm == 0.0)


@pytest.mark.parametrize("efq", [False, True])
def test_one_dominant_key_gives_its_v_row(mx, efq):
    rng = np.random.default_rng(4)
    heads, lq, lk = 1, 64, 256
    qf = np.zeros((heads, lq, D), np.float32)
    qf[..., 0] = 1.0
    kf = rng.uniform(-1, 1, (heads, lk, D)).astype(np.float32)
    kf[0, 200, 0] = 120.0
    vc, vs = v_input(rng, heads, lk, oracle.FP8_E4M3)
    o, rm, rs, pc, ps = run_gpu(mx, oracle.FP8_E4M3, bf16(qf), bf16(kf), vc, vs, 1.0,
                                torch.float32, efq=efq)
    vt = oracle.dequantize(oracle.FP8_E4M3, vc, vs, None, heads * D, lk, oracle.FP32)
    assert np.array_equal(o[0], np.broadcast_to(vt.reshape(D, lk)[:, 200], (lq, D)))
    assert np.all(rm == 120.0) and np.all(rs == 1.0)


@pytest.mark.parametrize("efq", [False, True])
def test_nan_score_poisons_its_row_only(mx, efq):
    rng = np.random.default_rng(5)
    heads, lq, lk = 1, 64, 128
    qf = rng.standard_normal((heads, lq, D)).astype(np.float32)
    qf[0, 9, 17] = np.nan
    q, k = bf16(qf), bf16(rng.standard_normal((heads, lk, D)))
    vc, vs = v_input(rng, heads, lk, oracle.FP8_E4M3)
    o, rm, rs, pc, ps = run_gpu(mx, oracle.FP8_E4M3, q, k, vc, vs, 0.1, torch.bfloat16, efq=efq)
    _, _, _, pc_ref, ps_ref = oracle.attention_fwd(oracle.FP8_E4M3, q, k, vc, vs, 0.1, 64,
                                                   oracle.BF16, efq=efq)
    assert np.array_equal(pc, pc_ref) and np.array_equal(ps, ps_ref)
    assert np.all(o[0, 9] == 0x7FC0)  # canonical bf16 NaN
    assert np.all(ps[0, 9] == 0xFF) and np.all(ps_ref[0, 9] == 0xFF)
    others = np.delete(np.arange(lq), 9)
    assert np.all(np.isfinite(workloads.bf16_bits_to_f32(o[0, others])))


ROWS_FULL = [(0, 0), (5, 1234), (17, 4095), (31, 2048), (12, 77), (31, 4095), (8, 3000),
             (20, 511)]


def _row_ref(fmt, q, k, vc, vs, heads, h, i, scale, efq=False):
    """The oracle on one query row (each row depends only on its own query)."""
    return oracle.attention_fwd(fmt, q[h:h + 1, i:i + 1], k[h:h + 1],
                                vc.reshape(heads, -1)[h:h + 1], vs.reshape(heads, -1)[h:h + 1],
                                scale, 64, oracle.FP32, efq=efq)


@pytest.mark.parametrize("rule", ["exp", "efq"])
def test_full_size_exact_scores_rows_bit_exact(mx, rule):
    """32 heads x 4096 queries x 4096 keys, d = 128, E4M3 V, bf16 output, in
    the launch the benchmark times, on exactly summable scores: sampled rows'
    probability blocks, scale bytes and row maxima bit-exact against the
    oracle, and the output inside the exact bound."""
    heads, lq, lk = 32, 4096, 4096
    efq = rule == "efq"
    rng = np.random.default_rng(13)
    qd = (torch.randint(-12, 13, (heads, lq, D), device="cuda").float() / 4).to(torch.bfloat16)
    kd = (torch.randint(-12, 13, (heads, lk, D), device="cuda").float() / 4).to(torch.bfloat16)
    q, k = to_host(qd), to_host(kd)
    vc, vs = v_input(rng, heads, lk, oracle.FP8_E4M3)
    scale = np.float32(D ** -0.5)
    o, rm, rs, pc, ps = mx.attention_fwd(qd, kd, to_dev(vc), to_dev(vs), "mxfp8", scale=scale,
                                         out_dtype=torch.bfloat16, stats=True, probs=True, efq=efq)
    torch.cuda.synchronize()
    vmax_all = vhat_absmax(oracle.FP8_E4M3, vc, vs, heads, lk)
    for h, i in ROWS_FULL:
        o_ref, rm_ref, _, pc_ref, ps_ref = _row_ref(oracle.FP8_E4M3, q, k, vc, vs, heads, h, i,
                                                    scale, efq)
        assert np.array_equal(to_host(pc[h, i]), pc_ref[0, 0]), (h, i)
        assert np.array_equal(to_host(ps[h, i]), ps_ref[0, 0]), (h, i)
        assert float(rm[h, i]) == float(rm_ref[0, 0]), (h, i)
        ref = o_ref[0, 0].astype(np.float64)
        got = workloads.bf16_bits_to_f32(to_host(o[h, i])).astype(np.float64)
        bound = out_bound(oracle.FP8_E4M3, lk, vmax_all[h:h + 1], ref[None, None, :], True)[0, 0]
        assert np.all(np.abs(got - ref) <= bound), (h, i, float((np.abs(got - ref) / bound).max()))


def test_full_size_natural_scores_rows(mx):
    """The benchmark's workload (bf16 N(0, 1) q and k, E4M3 V, bf16 output)
    on sampled rows: nearly every probability block equal to the oracle's,
    and the output inside the bound derived from the two sets of
    probability codes (as on the small natural-score inputs)."""
    heads, lq, lk = 32, 4096, 4096
    rng = np.random.default_rng(11)
    qd = torch.randn(heads, lq, D, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    kd = torch.randn(heads, lk, D, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    q, k = to_host(qd), to_host(kd)
    vc, vs = v_input(rng, heads, lk, oracle.FP8_E4M3)
    scale = np.float32(D ** -0.5)
    o, rm, rs, pc, ps = mx.attention_fwd(qd, kd, to_dev(vc), to_dev(vs), "mxfp8", scale=scale,
                                         out_dtype=torch.bfloat16, stats=True, probs=True)
    torch.cuda.synchronize()
    vmax_all = vhat_absmax(oracle.FP8_E4M3, vc, vs, heads, lk)
    g = brute.grid(oracle.FP4_E2M1)

    def decode(pcodes, pscales):
        nib = np.stack([pcodes & 15, pcodes >> 4], -1).reshape(pcodes.shape[:-1] + (32,))
        return g[nib & 7] * np.exp2(pscales.astype(np.float64) - 127)[..., None]

    same, total = 0, 0
    for h, i in ROWS_FULL:
        o_ref, rm_ref, rs_ref, pc_ref, ps_ref = _row_ref(oracle.FP8_E4M3, q, k, vc, vs, heads, h,
                                                         i, scale)
        gpc, gps = to_host(pc[h, i]), to_host(ps[h, i])
        same += int((np.all(gpc == pc_ref[0, 0], axis=-1) & (gps == ps_ref[0, 0])).sum())
        total += gps.size
        dp = np.abs(decode(gpc, gps) - decode(pc_ref[0, 0], ps_ref[0, 0])).sum()
        ref = o_ref[0, 0].astype(np.float64)
        vmax = vmax_all[h]
        bound = out_bound(oracle.FP8_E4M3, lk, vmax_all[h:h + 1], ref[None, None, :], True)[0, 0]
        bound = bound + 1e-5 * vmax
        # a probability that moved by dp changes the numerator by at most
        # dp (|v| + |o|) and the denominator by dp
        bound = bound + dp * (vmax + np.abs(ref)) / max(float(rs_ref[0, 0]) - dp, 1e-30)
        got = workloads.bf16_bits_to_f32(to_host(o[h, i])).astype(np.float64)
        assert np.all(np.abs(got - ref) <= bound), (h, i, float((np.abs(got - ref) / bound).max()))
        assert abs(float(rm[h, i]) - rm_ref[0, 0]) <= 1e-5 * max(1.0, abs(rm_ref[0, 0]))
    assert same / total > 0.999, same / total


@pytest.mark.parametrize("rule", ["exp", "efq"])
def test_scores_far_below_the_maximum(mx, rule):
    """Scores 100 to 10^6 below the running maximum and -inf scores (fp32
    overflow of q . k) with a finite maximum: the fast path's unclamped exp
    leaves its range there and must fall back to the clamped one; the
    probability blocks equal the oracle's bit for bit."""
    efq = rule == "efq"
    rng = np.random.default_rng(17)
    heads, lq, lk = 1, 64, 192
    qf = rng.integers(-12, 13, (heads, lq, D)).astype(np.float32) / 4
    kf = rng.integers(-12, 13, (heads, lk, D)).astype(np.float32) / 4
    # dims 0 and 1 are zero in every query and key but the ones named: query 5's
    # score with key 70 overflows to -inf; query 9's scores with keys 33
    # and 150 are -2^60 and -2^10 (the other scores are a few units)
    qf[:, :, :2] = 0.0
    kf[:, :, :2] = 0.0
    qf[0, 5, 0] = 2.0 ** 100
    kf[0, 70, 0] = -(2.0 ** 100)
    qf[0, 9, 1] = 2.0 ** 30
    kf[0, 33, 1] = -(2.0 ** 30)
    kf[0, 150, 1] = -(2.0 ** -20)
    q, k = bf16(qf), bf16(kf)
    vc, vs = v_input(rng, heads, lk, oracle.FP6_E2M3)
    for scale in (np.float32(0.125), np.float32(40.0), np.float32(3000.0)):
        _, rm_ref, _, pc_ref, ps_ref = oracle.attention_fwd(oracle.FP6_E2M3, q, k, vc, vs, scale,
                                                            64, oracle.FP32, efq=efq)
        o, rm, rs, pc, ps = run_gpu(mx, oracle.FP6_E2M3, q, k, vc, vs, scale, torch.float32,
                                    efq=efq)
        assert np.array_equal(ps, ps_ref), scale
        assert np.array_equal(pc, pc_ref), scale
        assert np.array_equal(rm, rm_ref), scale
        assert np.all(np.isfinite(o)), scale
