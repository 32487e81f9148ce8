"""EFQ's exp-free probability blocks in the oracle (CPU only).

The EFQ explainer says what the rule does (an exponent-only block scale
taken from the largest value in the block, then one affine map from shifted scores to
nonnegative E2M1 codes, no exp) but prints no constants, so the oracle
implements a stated reading: u = fp32(d log2 e), byte = the MX rule on 2^U
(U = max u), w = u - (byte - 127), code = trunc(clamp(2w + 2.5, 0, 7.5)); the
attention forward, whose scores are already in powers of two, applies the
rule to u = t - m and evaluates the affine map from the raw score in one
fused multiply-add (efq_attention_block).
PARITY UNPINNED by the pages: these tests pin the reading's own properties
(exact powers of two land on the even codes, monotonicity, the block
maximum's code, the log-domain rounding bound, agreement with
exp-then-quantize up to one code) and the attention forward built on it.
"""
import math

import numpy as np
import pytest

import brute
import oracle
import workloads

E2M1 = oracle.FP4_E2M1
G = brute.grid(E2M1)            # magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6
L2 = np.log2(np.where(G > 0, G, 1.0))
LOG2E = np.float32(1.4426950408889634)


def block(rng, spread):
    d = -np.abs(rng.standard_normal(32) * spread).astype(np.float32)
    d[rng.integers(32)] = 0.0 if rng.random() < 0.5 else d.max()
    return d


def u_of(d):
    return (np.asarray(d, np.float32) * LOG2E).astype(np.float32)


def test_powers_of_two_land_on_the_even_codes():
    # d = n ln2 rounded so that fp32(d log2 e) is exactly n: exp(d) is then
    # 2^n and the code's value must be exactly 2^n
    for n in range(0, -40, -1):
        d = np.float32(n * math.log(2))
        for cand in (d, np.nextafter(d, np.float32(0)), np.nextafter(d, np.float32(-1e9))):
            if np.float32(cand * LOG2E) == n:
                d = cand
                break
        else:
            continue
        blk = np.full(32, d, np.float32)
        blk[0] = 0.0 if n > -3 else d  # the block maximum decides the scale
        byte, codes = oracle.efq_block(blk)
        for k in range(1, 32):
            assert G[codes[k]] * 2.0 ** (byte - 127) == 2.0 ** n or (codes[k] == 0 and n < -3), n


def test_block_maximum_code_and_monotone():
    rng = np.random.default_rng(1)
    for spread in (0.1, 1.0, 4.0, 30.0):
        for _ in range(200):
            d = block(rng, spread)
            byte, codes = oracle.efq_block(d)
            u = u_of(d)
            top = int(np.argmax(u))
            assert codes[top] in (6, 7)          # 2^U / X is in [4, 8)
            assert byte == math.floor(float(u.max())) - 2 + 127
            order = np.argsort(d, kind="stable")
            assert np.all(np.diff(codes[order]) >= 0)  # larger score, never a smaller code


def test_log_domain_rounding_bound():
    # codes 2..6 sit within 0.34 of w in log2 units; code 7 (6 X) takes
    # w up to 3 (the block maximum's 2^U / X < 8); code 1 covers
    # w in [-0.75, -0.25); code 0 means w < -0.75
    rng = np.random.default_rng(2)
    for _ in range(500):
        d = block(rng, 3.0)
        byte, codes = oracle.efq_block(d)
        w = u_of(d).astype(np.float64) - (byte - 127)
        for c, wk in zip(codes, w):
            if c == 7:
                assert -0.34 <= wk - L2[c] and wk < 3.0
            elif c >= 2:
                assert abs(wk - L2[c]) <= 0.34
            elif c == 1:
                assert -0.75 <= wk < -0.25
            else:
                assert wk < -0.75


def test_close_to_exp_then_quantize():
    # the exp-free codes differ from exp-then-quantize's by at most one code
    # and the scale byte agrees unless exp rounds across a power of two
    rng = np.random.default_rng(3)
    same_byte, n = 0, 0
    for _ in range(400):
        d = block(rng, 2.0)
        byte, codes = oracle.efq_block(d)
        p = oracle.exp_ref(d).astype(np.float64)
        b2, packed = brute.quantize_block(E2M1, p)
        c2 = np.array(brute.unpack(E2M1, packed))
        assert np.all(np.abs(codes - c2) <= 1)
        assert abs(byte - b2) <= 1
        same_byte += byte == b2
        n += 1
    assert same_byte / n > 0.99


def test_specials():
    d = np.zeros(32, np.float32)
    d[3] = np.nan
    assert oracle.efq_block(d) == (0xFF, pytest.approx(np.zeros(32)))
    byte, codes = oracle.efq_block(np.full(32, -np.inf, np.float32))
    assert byte == 0 and not codes.any()
    d = np.full(32, -np.inf, np.float32)
    d[5] = -1.0
    byte, codes = oracle.efq_block(d)
    assert codes[5] in (6, 7) and codes.sum() == codes[5]
    # packing matches the MX E2M1 layout (even element in the low nibble)
    byte, packed = oracle.efq_quantize_block(-np.arange(32, dtype=np.float32) / 8)
    _, codes = oracle.efq_block(-np.arange(32, dtype=np.float32) / 8)
    assert packed.tobytes() == brute.pack(E2M1, codes)


def _bf16(x):
    return workloads.to_bf16_bits(np.asarray(x, np.float32))


def _vt(fmt, v):
    c, s, _ = oracle.quantize(fmt, np.ascontiguousarray(v.transpose(0, 2, 1)))
    return c, s


def test_attention_closed_forms():
    rng = np.random.default_rng(4)
    heads, lq, lk, d = 1, 6, 128, 32
    v = rng.standard_normal((heads, lk, d)).astype(np.float32)
    vc, vs = _vt(oracle.FP6_E2M3, v)
    vhat = oracle.dequantize(oracle.FP6_E2M3, vc, vs, None, d, lk, oracle.FP32).reshape(d, lk)
    # equal scores: every code is 6 (value 4 X = 1), o = mean of V
    q = _bf16(np.zeros((heads, lq, d)))
    k = _bf16(rng.standard_normal((heads, lk, d)))
    o, m, l, pc, ps = oracle.attention_fwd(oracle.FP6_E2M3, q, k, vc, vs, 0.5, efq=True)
    assert np.allclose(o[0], vhat.mean(1)[None, :], rtol=1e-6, atol=1e-7)
    assert np.all(pc == 0x66) and np.all(l == lk)
    # one dominant key: o is its V row
    qf = np.zeros((heads, lq, d), np.float32)
    qf[..., 0] = 1.0
    kf = rng.uniform(-1, 1, (heads, lk, d)).astype(np.float32)
    kf[0, 77, 0] = 200.0
    o, m, l, pc, ps = oracle.attention_fwd(oracle.FP6_E2M3, _bf16(qf), _bf16(kf), vc, vs, 1.0,
                                           efq=True)
    assert np.array_equal(o[0], np.broadcast_to(vhat[:, 77], (lq, d)))


def test_attention_blocks_follow_the_block_rule():
    rng = np.random.default_rng(5)
    heads, lq, lk, d = 2, 5, 224, 64
    q = _bf16(rng.standard_normal((heads, lq, d)))
    k = _bf16(rng.standard_normal((heads, lk, d)))
    v = rng.standard_normal((heads, lk, d)).astype(np.float32)
    vc, vs = _vt(oracle.FP8_E4M3, v)
    scale = np.float32(d ** -0.5)
    o, m, l, pc, ps = oracle.attention_fwd(oracle.FP8_E4M3, q, k, vc, vs, scale, efq=True)
    s = np.einsum("hqd,hkd->hqk", workloads.bf16_bits_to_f32(q).astype(np.float64),
                  workloads.bf16_bits_to_f32(k).astype(np.float64)).astype(np.float32)
    # the forward's scores in powers of two: t = fp32(s * c), c = fp32(scale * log2 e);
    # its blocks are the attention form of the rule (the affine map as one
    # fused multiply-add from the raw score), which must agree with the
    # stand-alone rule on u = t - m: the same scale bytes, and codes that
    # differ only where the two roundings straddle a code boundary
    c = np.float32(scale * LOG2E)
    t = (s * c).astype(np.float32)
    nib = lambda x: np.stack([x & 15, x >> 4], -1).reshape(-1).astype(np.int64)
    moved, total = 0, 0
    for h in range(heads):
        for i in range(lq):
            run_max = np.float32(-np.inf)
            for j in range(0, lk, 64):
                run_max = max(run_max, t[h, i, j:j + 64].max())
                for b in range(j, min(j + 64, lk), 32):
                    byte, codes = oracle.efq_attention_block(s[h, i, b:b + 32], c, run_max)
                    assert ps[h, i, b // 32] == byte
                    assert np.array_equal(nib(pc[h, i, b // 32]), codes)
                    byte2, codes2 = oracle.efq_block_log2((t[h, i, b:b + 32] - run_max)
                                                          .astype(np.float32))
                    assert byte2 == byte and np.abs(codes - codes2).max() <= 1
                    moved += int((codes != codes2).sum())
                    total += 32
    assert moved / total < 1e-3


def test_attention_form_special_blocks():
    c = np.float32(0.125 * LOG2E)
    zero = np.zeros(32, np.float32)
    # the block holding the running maximum: u = 0 there, code 6 (value 4 X = 1)
    s = -np.abs(np.random.default_rng(7).standard_normal(32)).astype(np.float32)
    s[5] = 0.0
    byte, codes = oracle.efq_attention_block(s, c, np.float32(0.0))
    assert byte == 125 and codes[5] == 6 and codes.max() == 6
    # a NaN score poisons its block
    s2 = zero.copy()
    s2[3] = np.nan
    assert oracle.efq_attention_block(s2, c, 0.0)[0] == 0xFF
    # -inf scores under a finite maximum: byte 0 and no codes
    byte, codes = oracle.efq_attention_block(np.full(32, -np.inf, np.float32), c, 1.0)
    assert byte == 0 and not codes.any()
    # an infinite maximum: finite scores give u = -inf (byte 0, no codes);
    # an infinite score gives inf - inf and poisons the block
    byte, codes = oracle.efq_attention_block(zero, c, np.inf)
    assert byte == 0 and not codes.any()
    s3 = zero.copy()
    s3[0] = np.inf
    assert oracle.efq_attention_block(s3, c, np.inf)[0] == 0xFF
    # scores far below the maximum: byte 0 and no codes (no overflow on the way)
    byte, codes = oracle.efq_attention_block(np.full(32, -1e30, np.float32), c, 5.0)
    assert byte == 0 and not codes.any()
