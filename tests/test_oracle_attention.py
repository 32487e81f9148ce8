"""Pins of the oracle's attention forward with E2M1 probabilities (CPU only).

What is pinned, independently of the oracle's own arithmetic:
* closed forms: equal scores give the plain mean of V; one key far above
  the others gives that key's V row; scores built so that every
  probability lands on an E2M1 grid point give a weighted mean with known
  weights, including a rise of the running maximum between two key tiles
  (the rescale factor is then exp of the rise, taken from math.exp);
* the probability blocks handed to the PV product: the scores in powers of
  two (t = fp32(s * fp32(scale * log2 e))), their running maximum per
  64-key tile, exp2_ref, and a brute-force nearest-grid-point E2M1
  quantization reproduce the oracle's codes and scales bit for bit; with
  the whole row in one tile the blocks agree with the stand-alone
  exp-then-quantize prologue, which evaluates exp in base e;
* random inputs: the output lies within a bound derived from the E2M1 grid
  of the exact fp64 softmax attention;
* invariants: V scaled by 2^k gives O scaled by 2^k; permuting V's columns
  permutes O's.
V is always decoded here by brute force from library-derived grids.
"""
import math

import numpy as np
import pytest

import brute
import oracle
import workloads

E2M1, E4M3 = oracle.FP4_E2M1, oracle.FP8_E4M3
LOG2E = np.float32(1.4426950408889634)
V_FORMATS = [oracle.FP8_E4M3, oracle.FP6_E2M3, oracle.FP6_E3M2, oracle.FP4_E2M1]


def bf16(x):
    return workloads.to_bf16_bits(np.asarray(x, np.float32))


def bf16_f64(b):
    return workloads.bf16_bits_to_f32(b).astype(np.float64)


def quantize_v(fmt, v):
    """v [heads, lk, d] fp32 -> (codes, scales) of V^T [heads, d, lk]."""
    vt = np.ascontiguousarray(np.asarray(v, np.float32).transpose(0, 2, 1))
    codes, scales, _ = oracle.quantize(fmt, vt)
    return codes, scales


def brute_vhat(fmt, codes, scales, heads, lk, d):
    """Decoded V [heads, lk, d] from V^T blocks, by grid lookup."""
    g = brute.grid(fmt)
    w = brute.CODE_BITS[fmt]
    codes = codes.reshape(heads * d * (lk // 32), -1)
    scales = scales.reshape(-1)
    out = np.empty(heads * d * lk)
    for b in range(codes.shape[0]):
        c = np.array(brute.unpack(fmt, codes[b].tobytes()))
        mag, sign = c & ((1 << (w - 1)) - 1), c >> (w - 1)
        vals = np.where(sign == 1, -g[mag], g[mag]) * 2.0 ** (int(scales[b]) - 127)
        out[b * 32:(b + 1) * 32] = np.nan if scales[b] == 0xFF else vals
    return out.reshape(heads, d, lk).transpose(0, 2, 1)


def run(q, k, v, fmt=E4M3, scale=1.0, kv_tile=64, out_dtype=oracle.FP32):
    heads, lk, d = k.shape
    vc, vs = quantize_v(fmt, v)
    res = oracle.attention_fwd(fmt, q, k, vc, vs, scale, kv_tile, out_dtype)
    return res + (brute_vhat(fmt, vc, vs, heads, lk, d),)


def test_equal_scores_give_the_mean_of_v():
    rng = np.random.default_rng(1)
    heads, lq, lk, d = 2, 8, 160, 32
    q = bf16(np.zeros((heads, lq, d)))
    k = bf16(rng.standard_normal((heads, lk, d)))
    v = rng.standard_normal((heads, lk, d)).astype(np.float32)
    for fmt in V_FORMATS:
        o, m, l, pc, ps, vhat = run(q, k, v, fmt, scale=0.125)
        want = vhat.mean(axis=1)  # every probability is exp(0) = 1
        assert np.allclose(o, np.broadcast_to(want[:, None, :], o.shape), rtol=1e-6, atol=1e-7)
        assert np.all(m == 0.0) and np.all(l == lk)
        assert np.all(ps == 127 - 2)  # amax 1 -> floor(log2 1) - emax(E2M1) + 127
        # 1.0 / 2^-2 = 4.0 = 1.0 x 2^2: exponent field 3, mantissa 0 -> code 0b0110
        assert np.all(pc == 0x66)


@pytest.mark.parametrize("where", [0, 70, 159])
def test_one_dominant_key_gives_its_v_row(where):
    rng = np.random.default_rng(2)
    heads, lq, lk, d = 1, 4, 160, 32
    q = np.zeros((heads, lq, d), np.float32)
    q[..., 0] = 1.0
    kf = rng.uniform(-1, 1, (heads, lk, d)).astype(np.float32)
    kf[0, where, 0] = 120.0  # every other score is at least 104 below
    v = rng.standard_normal((heads, lk, d)).astype(np.float32)
    o, m, l, pc, ps, vhat = run(bf16(q), bf16(kf), v)
    assert np.array_equal(o[0], np.broadcast_to(vhat[0, where], (lq, d)).astype(np.float32))
    assert np.all(m == 120.0) and np.all(l == 1.0)


def _snapped_row(rng, weights_per_block, m0):
    """Scores (in bf16 bits of q.k with q = e0) whose exp(t - m0) land on
    the given E2M1 weights after block quantization."""
    t = []
    for ws in weights_per_block:
        for w in ws:
            t.append(m0 - 200.0 if w == 0 else m0 + math.log(w))
    return np.array(t, np.float64)


def test_snapped_weights_and_a_rising_maximum():
    # two 64-key tiles; the maximum rises by 11/16 in the second, so the
    # first tile's sums are rescaled by exp(-11/16)
    rng = np.random.default_rng(3)
    d, lk = 16, 128
    # grid points of E2M1 under the block scale: 2^-2 when the block holds
    # a 1 (grid 0, 1/8, 1/4, 3/8, 1/2, 3/4, 1, 3/2), 2^-3 when its largest
    # weight is 3/4 (grid 0, 1/16, 1/8, 3/16, 1/4, 3/8, 1/2, 3/4)
    pool_1 = [1.0, 0.75, 0.5, 0.375, 0.25, 0.125, 0.0]
    pool_34 = [0.75, 0.5, 0.375, 0.25, 0.1875, 0.125, 0.0625, 0.0]
    blocks = []
    for b in range(4):
        ws = [1.0] + list(rng.choice(pool_1, 31)) if b != 1 else [0.75] + list(rng.choice(pool_34, 31))
        blocks.append(ws)
    m0, rise = 0.0, 0.6875
    t = np.concatenate([_snapped_row(rng, blocks[:2], m0), _snapped_row(rng, blocks[2:], m0 + rise)])
    q = np.zeros((1, 1, d), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((1, lk, d), np.float32)
    k[0, :, 0] = t
    kb = bf16(k)
    v = rng.integers(-8, 9, (1, lk, d)).astype(np.float32)
    o, m, l, pc, ps, vhat = run(bf16(q), kb, v)
    w = np.array(sum(blocks, []), np.float64)
    alpha = math.exp(-rise)
    wt = np.where(np.arange(lk) < 64, alpha * w, w)
    want = (wt[:, None] * vhat[0]).sum(0) / wt.sum()
    assert m[0, 0] == np.float32(rise)
    assert abs(l[0, 0] - wt.sum()) <= 1e-6 * wt.sum()
    assert np.allclose(o[0, 0], want, rtol=1e-6, atol=1e-6)
    # and with the maximum in the first tile nothing is rescaled
    t2 = np.concatenate([_snapped_row(rng, blocks[2:], m0 + rise), _snapped_row(rng, blocks[:2], m0)])
    k[0, :, 0] = t2
    o2, m2, l2, *_ = run(bf16(q), bf16(k), v)
    w2 = np.array(blocks[2] + blocks[3] + blocks[0] + blocks[1], np.float64)
    # second tile quantized against the first tile's maximum: the weights
    # exp(t - rise) no longer sit on the grid, so only the maximum and the
    # first tile's share are closed-form here
    assert m2[0, 0] == np.float32(rise)
    assert l2[0, 0] >= w2[:64].sum() * (1 - 1e-6)


def test_probability_blocks_match_brute_force():
    rng = np.random.default_rng(4)
    heads, lq, lk, d = 2, 6, 224, 64
    q = bf16(rng.standard_normal((heads, lq, d)))
    k = bf16(rng.standard_normal((heads, lk, d)) * np.linspace(0.2, 2.0, lk)[None, :, None])
    v = rng.standard_normal((heads, lk, d)).astype(np.float32)
    scale = np.float32(d ** -0.5)
    for tile in (32, 64, 96):
        o, m, l, pc, ps, vhat = run(q, k, v, scale=scale, kv_tile=tile)
        s = np.einsum("hqd,hkd->hqk", bf16_f64(q), bf16_f64(k)).astype(np.float32)
        t = (s * np.float32(scale * LOG2E)).astype(np.float32)
        for h in range(heads):
            for i in range(lq):
                run_max = np.float32(-np.inf)
                for j in range(0, lk, tile):
                    run_max = max(run_max, t[h, i, j:j + tile].max())
                    for b in range(j, min(j + tile, lk), 32):
                        p = oracle.exp2_ref((t[h, i, b:b + 32] - run_max).astype(np.float32))
                        byte, packed = brute.quantize_block(E2M1, p.astype(np.float64))
                        assert ps[h, i, b // 32] == byte
                        assert pc[h, i, b // 32].tobytes() == packed
                # the reported maximum is in natural units
                assert m[h, i] == (s[h, i] * scale).astype(np.float32).max()


@pytest.mark.parametrize("fmt", V_FORMATS)
def test_within_the_e2m1_bound_of_exact_attention(fmt):
    rng = np.random.default_rng(5 + fmt)
    heads, lq, lk, d = 2, 16, 256, 32
    qf = rng.standard_normal((heads, lq, d)) * 1.5
    kf = rng.standard_normal((heads, lk, d))
    v = rng.standard_normal((heads, lk, d)).astype(np.float32)
    q, k = bf16(qf), bf16(kf)
    scale = d ** -0.5
    o, m, l, pc, ps, vhat = run(q, k, v, fmt, scale=np.float32(scale))
    s = np.einsum("hqd,hkd->hqk", bf16_f64(q), bf16_f64(k)) * scale
    P = np.exp(s - s.max(-1, keepdims=True))
    o_exact = np.einsum("hqk,hkd->hqd", P, v.astype(np.float64)) / P.sum(-1)[..., None]
    o_bar = np.einsum("hqk,hkd->hqd", P, vhat) / P.sum(-1)[..., None]
    # Per element, in units of the final maximum: with the MX rule the
    # block scale X is at most (block max)/4, E2M1's half steps are X/4 on
    # [0, 2X), X/2 on [2X, 4X), X on [4X, 6X] and saturation loses less
    # than p/4, so |p_hat - p| <= max(p/4, (block max)/16); zero is a grid
    # point, so it is also <= p.  1e-4 covers fp32 scores, exp_ref and the
    # rescale factors.
    mb = np.broadcast_to(P.reshape(heads, lq, lk // 32, 32).max(-1, keepdims=True),
                         (heads, lq, lk // 32, 32)).reshape(P.shape)
    E = np.minimum(P, np.maximum(0.25 * P, mb / 16)) * 1.0001 + 1e-4 * P
    num = np.einsum("hqk,hqkd->hqd", E, np.abs(vhat[:, None, :, :] - o_bar[:, :, None, :]))
    bound = num / (P.sum(-1) - E.sum(-1))[..., None]
    bound += np.abs(o_bar - o_exact) + 1e-6
    err = np.abs(o.astype(np.float64) - o_exact)
    assert np.all(err <= bound)
    # a loose bound (it adds every element's worst case), but one that
    # still says something: it is below the spread of V
    assert np.median(bound) < np.std(v)


def test_output_is_the_normalized_pv_of_its_blocks():
    # O = sum_k W_k vhat_k / sum_k W_k with W_k = p_hat_k (brute-decoded
    # from the probability blocks) times exp(m_tile - m_final), the
    # rescaling a block's sums receive from later tiles
    rng = np.random.default_rng(10)
    heads, lq, lk, d = 2, 8, 320, 32
    q = bf16(rng.standard_normal((heads, lq, d)) * 2.0)
    k = bf16(rng.standard_normal((heads, lk, d)) * np.linspace(0.3, 1.5, lk)[None, :, None])
    v = rng.standard_normal((heads, lk, d)).astype(np.float32)
    scale = np.float32(d ** -0.5)
    o, m, l, pc, ps, vhat = run(q, k, v, oracle.FP6_E3M2, scale=scale)
    s = np.einsum("hqd,hkd->hqk", bf16_f64(q), bf16_f64(k)).astype(np.float32)
    t = (s * scale).astype(np.float32)
    g = brute.grid(E2M1)
    for h in range(heads):
        for i in range(lq):
            run_max, tile_max = -np.inf, np.empty(lk)
            for j in range(0, lk, 64):
                run_max = max(run_max, float(t[h, i, j:j + 64].max()))
                tile_max[j:j + 64] = run_max
            phat = np.empty(lk)
            for b in range(lk // 32):
                c = np.array(brute.unpack(E2M1, pc[h, i, b].tobytes()))
                phat[32 * b:32 * b + 32] = g[c & 7] * 2.0 ** (int(ps[h, i, b]) - 127)
            w = phat * np.exp(tile_max - run_max)
            assert abs(l[h, i] - w.sum()) <= 1e-5 * w.sum()
            want = (w[:, None] * vhat[h]).sum(0) / w.sum()
            assert np.allclose(o[h, i], want, rtol=1e-5, atol=1e-6 * np.abs(vhat[h]).max())


def test_invariants():
    rng = np.random.default_rng(6)
    heads, lq, lk, d = 1, 8, 128, 32
    q = bf16(rng.standard_normal((heads, lq, d)))
    k = bf16(rng.standard_normal((heads, lk, d)))
    v = rng.standard_normal((heads, lk, d)).astype(np.float32)
    o, *_ = run(q, k, v)
    o2, *_ = run(q, k, v * np.float32(8.0))
    assert np.array_equal(o2, o * np.float32(8.0))
    perm = rng.permutation(d)
    o3, *_ = run(q, k, np.ascontiguousarray(v[..., perm]))
    assert np.array_equal(o3, o[..., perm])


def test_nan_score_poisons_its_row_only():
    rng = np.random.default_rng(7)
    heads, lq, lk, d = 1, 4, 128, 32
    qf = rng.standard_normal((heads, lq, d)).astype(np.float32)
    qf[0, 2, 5] = np.nan
    q, k = bf16(qf), bf16(rng.standard_normal((heads, lk, d)))
    v = rng.standard_normal((heads, lk, d)).astype(np.float32)
    o, m, l, pc, ps, vhat = run(q, k, v)
    assert np.all(np.isnan(o[0, 2])) and np.all(ps[0, 2] == 0xFF)
    assert np.all(np.isfinite(o[0, [0, 1, 3]]))


def test_bf16_output_is_the_rounded_fp32_output():
    rng = np.random.default_rng(8)
    q = bf16(rng.standard_normal((1, 8, 32)))
    k = bf16(rng.standard_normal((1, 96, 32)))
    v = rng.standard_normal((1, 96, 32)).astype(np.float32)
    o32, *_ = run(q, k, v, out_dtype=oracle.FP32)
    o16, *_ = run(q, k, v, out_dtype=oracle.BF16)
    # fp32 output rounded once to bf16 equals the bf16 output unless the
    # fp64 value sits within an fp32 ulp of a bf16 midpoint (none here)
    assert np.array_equal(o16, bf16(o32))


def test_one_tile_agrees_with_the_softmax_prologue():
    # with the whole row in one tile the running maximum is the row maximum,
    # so the blocks are those of the stand-alone exp-then-quantize prologue
    # up to the two evaluations of exp (base 2 here, base e there): the same
    # scale bytes, and codes that differ only where the two roundings
    # straddle an E2M1 rounding boundary (never by more than one step)
    rng = np.random.default_rng(9)
    heads, lq, lk, d = 1, 64, 192, 32
    q = bf16(rng.standard_normal((heads, lq, d)) * 2)
    k = bf16(rng.standard_normal((heads, lk, d)))
    v = rng.standard_normal((heads, lk, d)).astype(np.float32)
    o, m, l, pc, ps, vhat = run(q, k, v, kv_tile=lk, scale=np.float32(0.25))
    s = np.einsum("hqd,hkd->hqk", bf16_f64(q), bf16_f64(k)).astype(np.float32)
    t = (s * np.float32(0.25)).astype(np.float32)
    c, sc = oracle.softmax_quantize(E2M1, t.reshape(lq, lk))
    assert np.array_equal(ps.reshape(sc.shape), sc)
    nib = lambda x: np.stack([x & 15, x >> 4], -1).astype(np.int64)
    diff = np.abs(nib(pc.reshape(c.shape)) - nib(c))
    assert diff.max() <= 1 and diff.mean() < 1e-3


def test_argument_errors():
    q = bf16(np.zeros((1, 4, 32)))
    k = bf16(np.zeros((1, 48, 32)))  # lk not a multiple of 32
    with pytest.raises(ValueError):
        oracle.attention_fwd(E4M3, q, k, np.zeros(1 * 32 * 1 * 32, np.uint8), np.zeros(32, np.uint8), 1.0)
    # the scale must be positive with scale * log2 e finite
    q = bf16(np.zeros((1, 4, 32)))
    k = bf16(np.zeros((1, 64, 32)))
    vc, vs = quantize_v(E4M3, np.zeros((1, 64, 32), np.float32))
    oracle.attention_fwd(E4M3, q, k, vc, vs, 1.0)
    for bad in (0.0, -1.0, np.nan, np.inf, 3e38):
        with pytest.raises(ValueError):
            oracle.attention_fwd(E4M3, q, k, vc, vs, bad)
