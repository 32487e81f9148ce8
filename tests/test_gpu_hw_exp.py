"""The library's fixed exponentials on the GPU against the CPU oracle, bit
for bit, element by element (tests/hwprobe/exp_probe.hip applies the
library's own device functions; nothing around them quantizes, so an ulp of
difference anywhere would show).

* 2^u of the attention forward (exp2_ref): every 31st fp32 bit pattern of
  the reduced range [-1/2, 1/2] (68 M values), every 31st of [-151, -1/2),
  integers, the zero/tie boundary and -inf; the clamped form, the
  NaN-preserving form (NaN in, NaN out) and the fast path's unclamped form
  (the same value for every finite u <= 0, NaN for -inf).
* exp of the stand-alone prologue (exp_ref): every 31st fp32 bit pattern of
  [-104.5, 0], and values below where it returns 0.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def probe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib = ctypes.CDLL(os.path.join(HERE, "hwprobe", "libcvtprobe.so"))
    lib.probe_exp.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
    lib.probe_exp.restype = ctypes.c_int

    def run(form, x):
        x = np.ascontiguousarray(x, np.float32)
        xin = torch.from_numpy(x).cuda()
        out = torch.empty_like(xin)
        assert lib.probe_exp(form, xin.data_ptr(), out.data_ptr(), x.size) == 0
        torch.cuda.synchronize()
        return out.cpu().numpy()
    return run


def patterns(lo_bits, hi_bits, stride):
    return np.arange(lo_bits, hi_bits + 1, stride, dtype=np.uint64).astype(np.uint32).view(np.float32)


def exp2_inputs():
    u = np.concatenate([
        patterns(0x00000000, 0x3F000000, 31),           # +0 .. +1/2
        patterns(0x80000000, 0xBF000000, 31),           # -0 .. -1/2
        patterns(0xBF000000, 0xC3170000, 31),           # -1/2 .. -151
        -np.arange(0, 160, dtype=np.float32),           # integers
        np.array([-149.5, -150.0, -150.25, -151.0, -151.5, -1e6, -3e38, -np.inf], np.float32),
        np.nextafter(np.float32(-150.0), np.float32(0.0))[None],
    ]).astype(np.float32)
    return u


def same_bits(a, b):
    return np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_exp2_clamped_and_nan_forms_equal_the_oracle(probe):
    u = exp2_inputs()  # shifted scores are <= 0; the positive half of the
    ref = oracle.exp2_ref(u)  # reduced range runs the same sequence
    for form in (1, 2):
        assert same_bits(probe(form, u), ref), form
    # NaN in, NaN out for the NaN-preserving form
    nan_in = np.full(64, np.nan, np.float32)
    assert np.all(np.isnan(probe(2, nan_in)))


def test_exp2_unclamped_equals_the_clamped_form_for_finite_u(probe):
    u = exp2_inputs()
    finite = np.isfinite(u)
    got = probe(3, u[finite])
    assert same_bits(got, oracle.exp2_ref(u[finite]))
    assert np.isnan(probe(3, np.array([-np.inf], np.float32))[0])


def test_exp_ref_equals_the_oracle(probe):
    d = np.concatenate([
        patterns(0x80000000, 0xC2D10000, 31),           # -0 .. -104.5
        np.array([-104.0, -104.5, -200.0, -1e30, -np.inf], np.float32),
    ]).astype(np.float32)
    # the oracle's exp_ref through its row softmax: rows [d, 0] give exp(d - 0)
    rows = np.stack([d, np.zeros_like(d)], axis=1)
    ref = oracle.softmax_probs(rows)[:, 0].copy()
    got = probe(0, d)
    assert same_bits(got, ref)
