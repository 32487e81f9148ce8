#!/usr/bin/env python3
"""Throughput of MX quantize+pack on one MI355X.

Headline: a bf16 linear weight [14336, 4096] (N(0, 0.02^2), seed 3) quantized
to packed MXFP6 E2M3 with one E8M0 scale per 32 values.  One step = one
mx_quantize call over the whole tensor; inputs and outputs rotate over enough
buffer sets (>= 1 GiB in total) that no set is still in the 256 MB last-level
cache when it is reused, and everything is resident in HBM before timing.

Prints ONE JSON line.  value = GB/s of bf16 input consumed (1 GB = 1e9 B);
roofline.achieved = algorithmic bytes (input + codes + scales) per launch over
the measured average launch time, against the 8 TB/s HBM peak.  The other
steps of the path (E3M2, dequantize, AXS-6 fake-quantize, exp-then-quantize
probabilities, dynamic activations) are timed the same way and reported under
"secondary".  cpu_baseline times the CPU oracle on a bounded row sample of the
same input, and the same rows are compared byte for byte with the GPU output.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E datasheet peak, GB/s
# fp32 vector issue rate without packed math: 256 CUs x 4 SIMDs x 16 lanes x
# 2.4 GHz, in 10^12 lane-operations per second
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
CACHE_BYTES = 256 << 20
ROTATE_BYTES = 1 << 30
METRIC = "MX quantize+pack GB/s and % of HBM peak, bf16 14336×4096 → MXFP6 E2M3"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# seconds of untimed launches before each secondary line (clock ramp-up)
SECONDARY_WARM_S = 0.2
CSRC = os.path.join(ROOT, "block_scaled_bit_amd", "csrc")


# the translation unit the headline kernel is compiled from
HEADLINE_SOURCES = ("mx_exp.h", "mx_formats.h", "mx_hw.h", "mx_kernels.h", "mx_kernels.hip")


def source_digest() -> str:
    """Digest of the headline kernel's sources with comments and whitespace
    removed, so that counter figures stay attached to the code they were
    taken on."""
    import re
    h = hashlib.sha256()
    for name in sorted(HEADLINE_SOURCES):
        with open(os.path.join(CSRC, name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        text = " ".join(text.split())
        h.update(name.encode() + b"\0" + text.encode())
    return h.hexdigest()[:16]


def rotation_sets(bytes_per_set: int) -> int:
    return max(2, -(-ROTATE_BYTES // bytes_per_set))


def time_launches(fn, nsets, steps, warmup, min_warm_s=0.0):
    """Average device time per launch (ms) over `steps` back-to-back launches,
    measured with HIP events on the stream the launches go to.  At least
    `warmup` untimed launches come first, and more until `min_warm_s`
    seconds have passed: after an idle gap (host-side input generation) the
    GPU takes a while under load to return to its steady clock."""
    import time
    import torch
    torch.cuda.synchronize()
    for i in range(warmup):
        fn(i % nsets)
    torch.cuda.synchronize()
    t_start, i = time.perf_counter(), warmup
    while time.perf_counter() - t_start < min_warm_s:
        for _ in range(8):
            fn(i % nsets)
            i += 1
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(steps):
        fn(i % nsets)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def bf16_dev(bits_np, copies):
    import numpy as np
    import torch
    base = torch.from_numpy(np.ascontiguousarray(bits_np).view(np.int16)).view(torch.bfloat16).cuda()
    return [base] + [base.clone() for _ in range(copies - 1)]


def headline(mx, x_np, steps, warmup):
    import torch
    rows, cols = x_np.shape
    nb = rows * cols // 32
    in_bytes = rows * cols * 2
    out_bytes = nb * 24 + nb
    nsets = rotation_sets(in_bytes + out_bytes)
    xs = bf16_dev(x_np, nsets)
    codes = [torch.empty(nb * 24, dtype=torch.uint8, device="cuda") for _ in range(nsets)]
    scales = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(nsets)]
    stream = torch.cuda.current_stream().cuda_stream

    def step(i):
        st = mx.mx_quantize(0, 32, mx.MX_BF16, xs[i], rows, cols, codes[i], scales[i], None, stream)
        if st:
            raise mx.MxError(st, "mx_quantize")

    ms = time_launches(step, nsets, steps, warmup)

    # the same HBM, same rotation: a plain device-to-device copy of the input
    # (reads and writes in_bytes each) as a measured streaming ceiling
    def copy(i):
        xs[(i + 1) % nsets].copy_(xs[i])

    ms_copy = time_launches(copy, nsets, max(50, steps // 10), 20, min_warm_s=SECONDARY_WARM_S)
    copy_gbs = 2 * in_bytes / ms_copy / 1e6

    # the ceiling of this byte mix: a copy kernel with the quantizer's grid,
    # loads and stores and no arithmetic (tests/hwprobe/bw_probe.hip), timed
    # exactly like the quantizer on the same buffers
    ms_mix = None
    probe = mix_copy_probe()
    if probe is not None:
        def mix(i):
            if probe(xs[i].data_ptr(), nb, codes[i].data_ptr(), scales[i].data_ptr(), stream):
                raise RuntimeError("probe_mix_copy launch failed")

        ms_mix = time_launches(mix, nsets, steps, warmup)
        # the probe wrote its own bytes into the output buffers: set 0 gets
        # the quantizer's output back for the parity check against the oracle
        step(0)
        torch.cuda.synchronize()
    return ms, in_bytes, in_bytes + out_bytes, nsets, codes[0], scales[0], copy_gbs, ms_mix


def rows_floor_probe():
    """probe_rows_floor from the test probe library, or None if it is not built."""
    import ctypes
    path = os.path.join(ROOT, "tests", "hwprobe", "libcvtprobe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    if not hasattr(lib, "probe_rows_floor"):
        return None
    fn = lib.probe_rows_floor
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                   ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    return fn


def mix_copy_probe():
    """probe_mix_copy from the test probe library, or None if it is not built."""
    import ctypes
    path = os.path.join(ROOT, "tests", "hwprobe", "libcvtprobe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    if not hasattr(lib, "probe_mix_copy"):
        return None
    fn = lib.probe_mix_copy
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                   ctypes.c_void_p]
    fn.restype = ctypes.c_int
    return fn


def secondary(mx, steps):
    """Other steps of the path, each at its workload's full size."""
    import numpy as np
    import torch
    import workloads
    res = {}
    stream = torch.cuda.current_stream().cuda_stream
    k = max(10, steps // 4)

    def record(name, ms, in_b, out_b, note):
        res[name] = {"us": round(ms * 1e3, 2), "input_GBps": round(in_b / ms / 1e6, 1),
                     "hbm_frac": round((in_b + out_b) / ms / 1e6 / HBM_PEAK_GBS, 4),
                     "bytes": in_b + out_b, "workload": note}

    # linear weight: E3M2 quantize, E2M3 and E3M2 dequantize to bf16
    w = workloads.linear_weight()
    rows, cols = w.shape
    nb = rows * cols // 32
    n = rotation_sets(rows * cols * 2 + nb * 25)
    xs = bf16_dev(w, n)
    cs = [torch.empty(nb * 24, dtype=torch.uint8, device="cuda") for _ in range(n)]
    ss = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(n)]
    for f, nm in ((1, "e3m2"), (0, "e2m3")):
        ms = time_launches(lambda i: mx.mx_quantize(f, 32, 0, xs[i], rows, cols, cs[i], ss[i], None, stream), n, k, 3,
                           min_warm_s=SECONDARY_WARM_S)
        if f == 1:
            record("quantize_e3m2", ms, rows * cols * 2, nb * 25, "linear_weight bf16 14336x4096")
        ms = time_launches(lambda i: mx.mx_dequantize(f, 32, cs[i], ss[i], None, rows, cols, 0, xs[i], stream), n, k, 3,
                           min_warm_s=SECONDARY_WARM_S)
        record(f"dequantize_{nm}_to_bf16", ms, nb * 25, rows * cols * 2, "linear_weight bf16 14336x4096")
    # a generic eXmY format (7-bit e3m3, 28 B per block; rounding in fp32)
    g = mx.MX_EXMY(3, 3)
    cg = [torch.empty(nb * 28, dtype=torch.uint8, device="cuda") for _ in range(n)]
    ms = time_launches(lambda i: mx.mx_quantize(g, 32, 0, xs[i], rows, cols, cg[i], ss[i], None, stream), n, k, 3,
                       min_warm_s=SECONDARY_WARM_S)
    record("quantize_exmy_e3m3", ms, rows * cols * 2, nb * 29, "linear_weight bf16 14336x4096")
    ms = time_launches(lambda i: mx.mx_dequantize(g, 32, cg[i], ss[i], None, rows, cols, 0, xs[i], stream), n, k, 3,
                       min_warm_s=SECONDARY_WARM_S)
    record("dequantize_exmy_e3m3_to_bf16", ms, nb * 29, rows * cols * 2, "linear_weight bf16 14336x4096")
    del xs, cs, ss, cg

    # AXS-6 weight: fake-quantize and quantize
    a = workloads.axs6_weight()
    rows, cols = a.shape
    nb = rows * cols // 32
    n = rotation_sets(rows * cols * 4)
    xs = bf16_dev(a, n)
    ys = [torch.empty_like(xs[0]) for _ in range(n)]
    ms = time_launches(lambda i: mx.mx_fake_quantize(4, 32, 0, xs[i], ys[i], rows, cols, stream), n, k, 3,
                       min_warm_s=SECONDARY_WARM_S)
    record("fake_quantize_axs6", ms, rows * cols * 2, rows * cols * 2, "axs6_weight bf16 4096x4096")
    cs = [torch.empty(nb * 24, dtype=torch.uint8, device="cuda") for _ in range(n)]
    ss = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(n)]
    aa = [torch.empty((nb + 3) // 4, dtype=torch.uint8, device="cuda") for _ in range(n)]
    ms = time_launches(lambda i: mx.mx_quantize(4, 32, 0, xs[i], rows, cols, cs[i], ss[i], aa[i], stream), n, k, 3,
                       min_warm_s=SECONDARY_WARM_S)
    record("quantize_axs6", ms, rows * cols * 2, nb * 24 + nb + (nb + 3) // 4, "axs6_weight bf16 4096x4096")
    del xs, ys, cs, ss, aa

    # dynamic activations: E4M3 and E2M3 quantize, E4M3 dequantize
    act = workloads.activations()
    rows, cols = act.shape
    nb = rows * cols // 32
    n = rotation_sets(rows * cols * 2 + nb * 33)
    xs = bf16_dev(act, n)
    cs = [torch.empty(nb * 32, dtype=torch.uint8, device="cuda") for _ in range(n)]
    ss = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(n)]
    for f, nm, bpb in ((3, "e4m3", 32), (0, "e2m3", 24)):
        ms = time_launches(lambda i: mx.mx_quantize(f, 32, 0, xs[i], rows, cols, cs[i], ss[i], None, stream), n, k, 3,
                           min_warm_s=SECONDARY_WARM_S)
        record(f"quantize_{nm}_activations", ms, rows * cols * 2, nb * (bpb + 1), "activations bf16 16384x8192")
    ms = time_launches(lambda i: mx.mx_dequantize(3, 32, cs[i], ss[i], None, rows, cols, 0, xs[i], stream), n, k, 3,
                       min_warm_s=SECONDARY_WARM_S)
    record("dequantize_e4m3_activations", ms, nb * 33, rows * cols * 2, "activations bf16 16384x8192")
    del xs, cs, ss

    # attention probabilities: exp-then-quantize to E2M1 (2 GiB of scores)
    s = workloads.attn_scores()
    rows, cols = s.shape
    nb = rows * cols // 32
    sd = torch.from_numpy(s).cuda()
    del s
    c = torch.empty(nb * 16, dtype=torch.uint8, device="cuda")
    sc = torch.empty(nb, dtype=torch.uint8, device="cuda")
    ms = time_launches(lambda i: mx.mx_softmax_quantize(2, 32, sd, rows, cols, c, sc, stream), 1, max(5, k // 4), 2,
                       min_warm_s=SECONDARY_WARM_S)
    record("softmax_quantize_e2m1", ms, rows * cols * 4, nb * 17, "attn_scores fp32 32x4096x4096")
    # its floor: the same grid, loads and stores with the arithmetic folded
    # away (tests/hwprobe/bw_probe.hip), then the real outputs again
    floor = rows_floor_probe()
    if floor is not None:
        def fl(i):
            if floor(sd.data_ptr(), rows, cols, c.data_ptr(), sc.data_ptr(), stream):
                raise RuntimeError("probe_rows_floor launch failed")

        ms_floor = time_launches(fl, 1, max(5, k // 4), 2, min_warm_s=SECONDARY_WARM_S)
        res["softmax_quantize_e2m1"].update(
            floor_us=round(ms_floor * 1e3, 2), frac_of_floor=round(ms_floor / ms, 4),
            floor_note="same grid, loads and stores with no exp or conversion")
        mx.mx_softmax_quantize(2, 32, sd, rows, cols, c, sc, stream)
    ms = time_launches(lambda i: mx.mx_dequantize(2, 32, c, sc, None, rows, cols, 1, sd, stream), 1, max(5, k // 4), 2,
                       min_warm_s=SECONDARY_WARM_S)
    record("dequantize_e2m1_to_fp32", ms, nb * 17, rows * cols * 4, "attn_scores fp32 32x4096x4096")
    del sd, c, sc

    # the same scores inside a fused attention forward: 32 heads x 4096
    # queries x 4096 keys, d = 128, bf16 q/k, V^T in MXFP8, bf16 output
    res.update(attention_line(mx, k))

    # layer-by-layer conversion of a synthetic dense decoder (4 layers,
    # hidden 4096, MLP 14336, 1024-wide k/v): weights already on the GPU, and
    # again from pinned host memory (that rate includes the PCIe upload)
    from block_scaled_bit_amd import convert
    g = torch.Generator(device="cuda").manual_seed(11)
    shapes = {"self_attn.q_proj": (4096, 4096), "self_attn.k_proj": (1024, 4096),
              "self_attn.v_proj": (1024, 4096), "self_attn.o_proj": (4096, 4096),
              "mlp.gate_proj": (14336, 4096), "mlp.up_proj": (14336, 4096),
              "mlp.down_proj": (4096, 14336)}
    model = {f"model.layers.{i}.{k}.weight": (torch.randn(v, generator=g, device="cuda") * 0.02)
             .to(torch.bfloat16) for i in range(4) for k, v in shapes.items()}
    cfg = convert.QuantConfig.from_options("mxfp6")
    in_b = sum(t.numel() * 2 for t in model.values())
    out_b = sum(t.numel() // 32 * 25 for t in model.values())
    for src_name, src in (("device", model), ("pinned_host", None)):
        if src is None:
            src = {k: v.cpu().pin_memory() for k, v in model.items()}
        convert.convert_model(src, cfg)  # warm-up
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        reps = 5
        for _ in range(reps):
            out, _ = convert.convert_model(src, cfg)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        record(f"convert_dense_4_layers_from_{src_name}", ms, in_b, out_b,
               "synthetic decoder, 4 layers x 7 weights, hidden 4096, MLP 14336 (mxfp6 shorthand)")
        del out
    del model, src

    # small fp32 tensor: latency of the three ops
    xsm = torch.from_numpy(workloads.weights_small()).cuda()
    cc = torch.empty(1024 * 24, dtype=torch.uint8, device="cuda")
    s1 = torch.empty(1024, dtype=torch.uint8, device="cuda")
    yy = torch.empty_like(xsm)
    ms = time_launches(lambda i: mx.mx_quantize(0, 32, 1, xsm, 128, 256, cc, s1, None, stream), 1, k, 3,
                       min_warm_s=SECONDARY_WARM_S)
    record("quantize_e2m3_weights_small", ms, 131072, 25600, "weights_small fp32 128x256 (launch-bound)")
    return res


def attention_line(mx, k, heads=32, lq=4096, lk=4096, d=128):
    """Fused attention forward with E2M1 probabilities (one launch), with
    exp-then-quantize probabilities and with the exp-free EFQ reading."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(21)
    q = torch.randn(heads, lq, d, generator=g, device="cuda").to(torch.bfloat16)
    kk = torch.randn(heads, lk, d, generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn(heads, lk, d, generator=g, device="cuda")
    vc, vs = mx.quantize_v(v, "mxfp8")
    o = torch.empty(heads, lq, d, dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    scale = d ** -0.5

    out = {}
    flops = 4.0 * heads * lq * lk * d
    scores = heads * lq * lk
    # fp32 VALU operations the method fixes per score -- exp-then-quantize:
    # the scaling, the shift, exp_ref's 14 and the block maximum = 17;
    # EFQ: the scaling, the shift, log2 e, the block maximum, the affine
    # map (subtract, fma, clamp, convert) = 8.  The chip issues 256 CUs x 4
    # SIMDs x 16 lanes x 2.4 GHz of them per second.
    for name, fn, ops_per in (("attention_fwd_e2m1_p_mxfp8_v", mx.mx_attention_fwd, 17.0),
                              ("attention_fwd_efq_e2m1_p_mxfp8_v", mx.mx_attention_fwd_efq, 8.0)):
        def step(i, fn=fn):
            st = fn(mx.MX_FP8_E4M3, 32, q, kk, vc, vs, heads, lq, lk, d, scale, mx.MX_BF16, o,
                    None, None, None, None, stream)
            if st:
                raise mx.MxError(st, "attention forward")

        ms = time_launches(step, 1, max(10, k // 4), 5, min_warm_s=SECONDARY_WARM_S)
        out[name] = {
            "us": round(ms * 1e3, 2), "TFLOPs": round(flops / ms / 1e9, 1),
            "Gscores_per_s": round(scores / ms / 1e6, 1),
            "valu_frac": round(ops_per * scores / ms / 1e9 / VALU_PEAK_TOPS, 4),
            "workload": f"{heads} heads x {lq} queries x {lk} keys, d {d}, bf16 q/k, MXFP8 V^T, "
                        "bf16 out"}
    return out


def cpu_baseline(x_np, gpu_codes, gpu_scales, passes=3):
    """The CPU oracle, as it stands, on the same input: T threads, each on one
    contiguous range of rows (blocks never cross rows); the minimum of
    `passes` full passes.  The oracle's output is compared with the GPU's."""
    import numpy as np

    import oracle
    rows, cols = x_np.shape
    threads = max(1, min(len(os.sched_getaffinity(0)), 16))
    bounds = [(rows * i) // threads for i in range(threads + 1)]
    best, parts = None, None
    for _ in range(passes):
        t = time.perf_counter()
        with cf.ThreadPoolExecutor(threads) as ex:
            parts = list(ex.map(lambda i: oracle.quantize(0, x_np[bounds[i]:bounds[i + 1]]),
                                range(threads)))
        wall = time.perf_counter() - t
        best = wall if best is None else min(best, wall)
    oc = np.concatenate([p[0] for p in parts])
    os_ = np.concatenate([p[1] for p in parts])
    g_codes = gpu_codes.cpu().numpy().reshape(oc.shape)
    g_scales = gpu_scales.cpu().numpy().reshape(os_.shape)
    parity = bool(np.array_equal(g_codes, oc) and np.array_equal(g_scales, os_))
    value = rows * cols * 2 / best / 1e9
    base = {"value": round(value, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole bf16 14336x4096 input ({rows * cols} values), E2M3 "
                      f"quantize+pack, {threads} threads x ~{rows // threads} rows, best of "
                      f"{passes} passes ({best:.2f} s wall each)"}
    return base, parity, rows


def traffic_for(digest):
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_digest") != digest:
        return None
    return t.get("hbm_bytes_per_launch")


def copy_calibration(steps):
    """A plain device copy of the headline's byte count (for counter scaling)."""
    import torch
    n = 163315712
    a = torch.empty(n, dtype=torch.uint8, device="cuda").random_()
    b = torch.empty_like(a)
    ms = time_launches(lambda i: b.copy_(a), 1, steps, 3, min_warm_s=SECONDARY_WARM_S)
    print(json.dumps({"copy_bytes_each_way": n, "us": round(ms * 1e3, 2),
                      "GBps_read_plus_write": round(2 * n / ms / 1e6, 1)}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--no-secondary", action="store_true", help="time only the headline kernel")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only time a plain device copy of the headline's byte count")
    ap.add_argument("--only-attention", action="store_true",
                    help="only time the fused attention forward (for profiling it alone)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: the quantizer shards by rows with no exchange, so "
              f"--gpus {args.gpus} (WORLD_SIZE={world}) is not run here; use --gpus 1.",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import torch

    import block_scaled_bit_amd as mx
    import workloads
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(args.steps)
        return
    if args.only_attention:
        print(json.dumps(attention_line(mx, args.steps)), flush=True)
        return

    x = workloads.linear_weight()
    ms, in_b, alg_b, nsets, codes0, scales0, copy_gbs, ms_mix = headline(mx, x, args.steps,
                                                                         args.warmup)
    achieved = alg_b / ms / 1e6
    digest = source_digest()
    out = {
        "metric": METRIC,
        "value": round(in_b / ms / 1e6, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "linear_weight bf16 14336x4096 -> MXFP6 E2M3 quantize+pack",
                   "rows": 14336, "cols": 4096, "block": 32, "format": "mxfp6_e2m3",
                   "input_dtype": "bf16", "rotation_sets": nsets,
                   "algorithmic_bytes_per_pass": alg_b, "source_digest": digest},
        "hbm_frac": round(achieved / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for(digest)},
        "copy_ceiling": {"d2d_copy_GBps": round(copy_gbs, 1),
                         "frac_of_copy": round(achieved / copy_gbs, 4),
                         "note": "device-to-device copy of the bf16 input (read + write "
                                 "bytes / time), same buffers and rotation"},
    }
    if ms_mix is not None:
        out["mix_ceiling"] = {
            "us": round(ms_mix * 1e3, 3), "GBps": round(alg_b / ms_mix / 1e6, 1),
            "frac_of_peak": round(alg_b / ms_mix / 1e6 / HBM_PEAK_GBS, 4),
            "headline_frac_of_ceiling": round(ms_mix / ms, 4),
            "note": "copy kernel with the quantizer's grid, loads and stores and no arithmetic "
                    "(tests/hwprobe/bw_probe.hip), same buffers, rotation, warm-up and steps"}
    if not args.no_cpu_baseline:
        base, parity, nrows = cpu_baseline(x, codes0, scales0)
        out["cpu_baseline"] = base
        out["parity"] = {"bit_exact": parity, "rows_compared": nrows}
    if not args.no_secondary:
        del codes0, scales0
        torch.cuda.empty_cache()
        out["secondary"] = secondary(mx, args.steps)
    print(json.dumps(out), flush=True)
    if out.get("parity", {}).get("bit_exact") is False:
        print("bench.py: the GPU's codes or scales differ from the oracle's", file=sys.stderr,
              flush=True)
        sys.exit(1)


if __name__ == "__main__":
    main()
