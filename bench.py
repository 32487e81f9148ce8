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
steps of the path (E3M2, dequantize, eXmY, AXS-6, exp-then-quantize
probabilities, dynamic activations, the fused attention forward, the layer
conversion, the small fp32 tensor) are timed the same way and reported under
"secondary".  The cpu_baseline leg runs the CPU oracle on the host's cores:
it times the headline op (T threads over the whole input, one thread over a
row sample), and compares every op's full output with the GPU's byte for
byte, recording the oracle's rate beside each; any difference makes the run
exit with status 1 after printing its line.
"""
from __future__ import annotations

import argparse
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


def _smi_clock_doc(text):
    """The "clock" object of amd-smi's JSON list, found among whatever else
    the tool prints (warnings before or after it)."""
    dec = json.JSONDecoder()
    start = text.find("[")
    while start >= 0:
        try:
            doc, _ = dec.raw_decode(text[start:])
            if isinstance(doc, list) and doc and isinstance(doc[0], dict) and "clock" in doc[0]:
                return doc[0]["clock"]
        except ValueError:
            pass
        start = text.find("[", start + 1)
    raise ValueError("no clock list in the output")


def gpu_clocks_under_load(step, nsets, seconds=1.5, samples=3, lead_s=1.0):
    """The GPU's clocks as amd-smi reports them while `step` (the headline
    kernel) runs back to back: per sample the mean, lowest and highest of
    the eight XCDs' graphics clocks, the memory clock and the rated
    maximum, in MHz, and the seconds since the load started.  The first
    sample waits lead_s so the clocks have left any idle state.  None when
    the tool is missing; a sample that fails records the error.  Reported
    beside the timing, never used by it."""
    import shutil
    import subprocess
    import threading
    import time
    import torch
    exe = shutil.which("amd-smi")
    if exe is None:
        return None
    cmd = [exe]
    with open(exe, "rb") as f:
        if b"python" in f.readline():
            # a Python script: start it with this interpreter, so that no
            # `#!/usr/bin/env` launcher replaces itself with python
            cmd = [sys.executable, exe]
    readings = []

    t_start = time.perf_counter()

    def sample():
        time.sleep(lead_s)
        for _ in range(samples):
            time.sleep(seconds / (samples + 1))
            t_at = round(time.perf_counter() - t_start, 2)
            try:
                r = subprocess.run(cmd + ["metric", "-c", "--json"], capture_output=True,
                                   text=True, timeout=10)
                c = _smi_clock_doc(r.stdout)
                gfx = [v["clk"]["value"] for k, v in c.items() if k.startswith("gfx_")]
                readings.append({"gfx_mean_MHz": round(sum(gfx) / len(gfx)),
                                 "gfx_min_MHz": min(gfx), "gfx_max_MHz": max(gfx),
                                 "mem_MHz": c.get("mem_0", {}).get("clk", {}).get("value"),
                                 "gfx_rated_max_MHz": c["gfx_0"]["max_clk"]["value"],
                                 "s_under_load": t_at})
            except Exception as e:  # a reading, not a measurement: never fatal
                readings.append({"error": type(e).__name__})

    th = threading.Thread(target=sample)
    th.start()
    i = 0
    while th.is_alive():
        for _ in range(256):  # ~8 ms of work queued between host waits
            step(i % nsets)
            i += 1
        torch.cuda.synchronize()
    th.join()
    return {"samples": readings, "tool": "amd-smi metric -c --json",
            "note": "sampled while the headline kernel runs back to back after the timed region"}


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

    ms = time_launches(step, nsets, steps, warmup, min_warm_s=SECONDARY_WARM_S)
    # the same launches again as 5 batches of steps/5, each between its own
    # events: the spread of the per-launch time, and its median
    per = max(1, steps // 5)
    batches = sorted(time_launches(step, nsets, per, 0) for _ in range(5))
    clocks = gpu_clocks_under_load(step, nsets)

    # the same HBM, same rotation: torch's device-to-device copy of the input
    # (reads and writes in_bytes each), a reference rate, not a ceiling
    def copy(i):
        xs[(i + 1) % nsets].copy_(xs[i])

    ms_copy = time_launches(copy, nsets, max(50, steps // 10), 20, min_warm_s=SECONDARY_WARM_S)
    copy_gbs = 2 * in_bytes / ms_copy / 1e6

    # the ceiling of this byte mix: copy kernels with the quantizer's bytes
    # read and written and no arithmetic (tests/hwprobe/bw_probe.hip), in
    # several access schedules, timed exactly like the quantizer on the same
    # buffers; and the two halves of the mix alone (reads only, writes only)
    sched = {}
    probe = mix_variant_probe()
    if probe is not None:
        sink = torch.empty((nb + 255) // 256, dtype=torch.int32, device="cuda")
        for v, name in MIX_VARIANTS.items():
            def mix(i, v=v):
                if probe(v, xs[i].data_ptr(), nb, codes[i].data_ptr(), scales[i].data_ptr(),
                         sink.data_ptr(), stream):
                    raise RuntimeError(f"probe_mix_variant {v} launch failed")

            sched[name] = time_launches(mix, nsets, steps, warmup, min_warm_s=SECONDARY_WARM_S)
        # the probes wrote their own bytes into the output buffers: set 0
        # gets the quantizer's output back for the parity check
        step(0)
        torch.cuda.synchronize()
    clocks = {"gpu_clocks": clocks, "batches": {
        "count": 5, "launches_each": per, "median_us": round(batches[2] * 1e3, 3),
        "min_us": round(batches[0] * 1e3, 3), "max_us": round(batches[-1] * 1e3, 3)}}
    return ms, in_bytes, in_bytes + out_bytes, nsets, codes[0], scales[0], copy_gbs, sched, clocks


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


# access schedules of the byte-mix copy (tests/hwprobe/bw_probe.hip)
MIX_VARIANTS = {12: "quantizer_grid", 0: "lane_16B_loads", 1: "xcd_contiguous",
                2: "read_phase_then_write_4_blocks", 3: "read_phase_then_write_4_blocks_xcd",
                7: "nontemporal_stores", 11: "coalesced_1KB_instructions",
                4: "reads_only", 5: "writes_only", 10: "reads_only_coalesced",
                9: "writes_only_coalesced", 13: "reads_only_lds"}
MIX_COPIES = ("quantizer_grid", "lane_16B_loads", "xcd_contiguous",
              "read_phase_then_write_4_blocks", "read_phase_then_write_4_blocks_xcd",
              "nontemporal_stores", "coalesced_1KB_instructions")
MIX_READS = ("reads_only", "reads_only_coalesced", "reads_only_lds")
MIX_WRITES = ("writes_only", "writes_only_coalesced")


def mix_variant_probe():
    """probe_mix_variant from the test probe library, or None if it is not built."""
    import ctypes
    path = os.path.join(ROOT, "tests", "hwprobe", "libcvtprobe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    if not hasattr(lib, "probe_mix_variant"):
        return None
    fn = lib.probe_mix_variant
    fn.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                   ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    return fn


def bytes_copy_probe():
    """probe_bytes_copy from the test probe library, or None if it is not built."""
    import ctypes
    path = os.path.join(ROOT, "tests", "hwprobe", "libcvtprobe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    if not hasattr(lib, "probe_bytes_copy"):
        return None
    fn = lib.probe_bytes_copy
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                   ctypes.c_void_p]
    fn.restype = ctypes.c_int
    return fn


def host(t):
    """Device tensor -> numpy (bf16 as uint16 bit patterns)."""
    import numpy as np
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class Secondary:
    """The other steps of the path, each at its workload's full size: timed
    like the headline, then compared byte for byte with the oracle over the
    whole tensor (row ranges on the host's cores), with the oracle's own
    rate recorded beside the GPU's."""

    def __init__(self, mx, steps, threads):
        import torch
        self.mx, self.torch = mx, torch
        self.stream = torch.cuda.current_stream().cuda_stream
        self.k = max(10, steps // 4)
        self.threads = threads
        self.res = {}
        self.failed = []
        self.copy = bytes_copy_probe()

    def launch(self, name, fn):
        """fn(i) -> mx status; a nonzero status raises instead of being timed."""
        mx = self.mx

        def call(i):
            st = fn(i)
            if st:
                raise mx.MxError(st, name)
        return call

    def time(self, name, fn, nsets, in_b, out_b, note, steps=None, warm=3, copy_bpb=None):
        """copy_bpb = (bytes read, bytes written) per 32-value block: also
        time a plain copy of those byte counts (tests/hwprobe/bw_probe.hip,
        every instruction covering 1 KB of consecutive bytes) on buffers of
        its own, as the row's streaming floor."""
        ms = time_launches(self.launch(name, fn), nsets, steps or self.k, warm,
                           min_warm_s=SECONDARY_WARM_S)
        self.res[name] = {"us": round(ms * 1e3, 2), "input_GBps": round(in_b / ms / 1e6, 1),
                          "hbm_frac": round((in_b + out_b) / ms / 1e6 / HBM_PEAK_GBS, 4),
                          "bytes": in_b + out_b, "workload": note}
        if copy_bpb is not None and self.copy is not None:
            ib, ob = copy_bpb
            nb = (in_b + out_b) // (ib + ob)
            ms_c = self.copy_floor(nb, ib, ob, steps or self.k, warm)
            self.res[name].update(copy_us=round(ms_c * 1e3, 2), frac_of_copy=round(ms_c / ms, 4),
                                  copy_note=f"{ib} B read and {ob} B written per block, copied "
                                            "with 1 KB instructions")
        return ms

    def copy_floor(self, nb, ib, ob, steps, warm):
        torch = self.torch
        per = -(-nb * ib // 16) * 16 + -(-nb * ob // 16) * 16
        n = rotation_sets(per)
        xs = [torch.empty(-(-nb * ib // 16) * 16, dtype=torch.uint8, device="cuda")
              for _ in range(n)]
        ys = [torch.empty(-(-nb * ob // 16) * 16, dtype=torch.uint8, device="cuda")
              for _ in range(n)]
        st = self.stream

        def f(i):
            return self.copy(xs[i].data_ptr(), nb, ib, ys[i].data_ptr(), ob, st)

        ms = time_launches(self.launch("probe_bytes_copy", f), n, steps, warm,
                           min_warm_s=SECONDARY_WARM_S)
        del xs, ys
        return ms

    def oracle(self, fn, rows):
        """The oracle over all rows, split across the host threads; returns
        (result, wall seconds)."""
        import oracle
        t = time.perf_counter()
        out = oracle.by_rows(fn, rows, self.threads)
        return out, time.perf_counter() - t

    def parity(self, name, pairs, in_b, oracle_s, what):
        """pairs: (gpu array, oracle array) compared byte for byte."""
        import numpy as np
        ok = all(np.array_equal(np.ascontiguousarray(g).reshape(-1).view(np.uint8),
                                np.ascontiguousarray(o).reshape(-1).view(np.uint8))
                 for g, o in pairs)
        self.res[name]["parity"] = {"bit_exact": bool(ok), "compared": what}
        self.res[name]["oracle_GBps"] = round(in_b / oracle_s / 1e9, 3)
        self.res[name]["oracle_threads"] = self.threads
        if not ok:
            self.failed.append(name)


def secondary(mx, steps, threads, check=True):
    """Other steps of the path, each at its workload's full size, each
    compared with the oracle over the whole tensor (check=False: timing
    only, for profiling runs)."""
    import numpy as np
    import torch

    import oracle
    import workloads
    S = Secondary(mx, steps, threads)
    st = S.stream
    BF, FP = mx.MX_BF16, mx.MX_FP32

    # -- linear weight: E3M2 quantize, E2M3 / E3M2 dequantize to bf16, and
    #    the generic 7-bit e3m3 quantize and dequantize
    w = workloads.linear_weight()
    rows, cols = w.shape
    nb = rows * cols // 32
    note = "linear_weight bf16 14336x4096"
    n = rotation_sets(rows * cols * 4 + nb * 25)
    xs = bf16_dev(w, n)
    ys = [torch.empty_like(xs[0]) for _ in range(n)]
    ss = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(n)]
    for f, nm, bpb in ((1, "e3m2", 24), (0, "e2m3", 24), (mx.MX_EXMY(3, 3), "exmy_e3m3", 28)):
        cs = [torch.empty(nb * bpb, dtype=torch.uint8, device="cuda") for _ in range(n)]
        q = lambda i, f=f, cs=cs: mx.mx_quantize(f, 32, BF, xs[i], rows, cols, cs[i], ss[i], None, st)
        dq = lambda i, f=f, cs=cs: mx.mx_dequantize(f, 32, cs[i], ss[i], None, rows, cols, BF, ys[i], st)
        if f != 0:  # the E2M3 quantize is the headline
            S.time(f"quantize_{nm}", q, n, rows * cols * 2, nb * (bpb + 1), note,
                   copy_bpb=(64, bpb + 1))
        S.launch(nm, q)(0)
        S.time(f"dequantize_{nm}_to_bf16", dq, n, nb * (bpb + 1), rows * cols * 2, note,
               copy_bpb=(bpb + 1, 64))
        S.launch(nm, dq)(0)
        torch.cuda.synchronize()
        if check:
            gc, gs, gy = host(cs[0]), host(ss[0]), host(ys[0])
            (oc, os_, _), t_q = S.oracle(lambda a, b, f=f: oracle.quantize(f, w[a:b]), rows)
            oy, t_dq = S.oracle(lambda a, b, f=f: oracle.dequantize(
                f, oc[a:b], os_[a:b], None, b - a, cols, oracle.BF16), rows)
            if f != 0:
                S.parity(f"quantize_{nm}", [(gc, oc), (gs, os_)], rows * cols * 2, t_q,
                         "all 14336 rows: codes, scales")
            S.parity(f"dequantize_{nm}_to_bf16", [(gy, oy)], nb * (bpb + 1), t_dq,
                     "all 14336 rows: bf16 output")
            del oc, os_, oy, gc, gs, gy
        del cs
    del xs, ys, ss, w

    # -- the same weight as fp16 ("Online MXFP6", "Start a model": BF16 or
    #    FP16 weights): E2M3 quantize, and dequantize back to fp16
    w = workloads.linear_weight_f16()
    rows, cols = w.shape
    nb = rows * cols // 32
    note = "linear_weight_f16 fp16 14336x4096"
    n = rotation_sets(rows * cols * 4 + nb * 25)
    xs = [torch.from_numpy(w).cuda() for _ in range(n)]
    ys = [torch.empty_like(xs[0]) for _ in range(n)]
    ss = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(n)]
    cs = [torch.empty(nb * 24, dtype=torch.uint8, device="cuda") for _ in range(n)]
    F16 = mx.MX_FP16
    q = lambda i: mx.mx_quantize(0, 32, F16, xs[i], rows, cols, cs[i], ss[i], None, st)
    dq = lambda i: mx.mx_dequantize(0, 32, cs[i], ss[i], None, rows, cols, F16, ys[i], st)
    S.time("quantize_e2m3_fp16", q, n, rows * cols * 2, nb * 25, note, copy_bpb=(64, 25))
    S.launch("q16", q)(0)
    S.time("dequantize_e2m3_to_fp16", dq, n, nb * 25, rows * cols * 2, note, copy_bpb=(25, 64))
    S.launch("dq16", dq)(0)
    torch.cuda.synchronize()
    if check:
        gc, gs, gy = host(cs[0]), host(ss[0]), host(ys[0])
        (oc, os_, _), t_q = S.oracle(lambda a, b: oracle.quantize(0, w[a:b]), rows)
        oy, t_dq = S.oracle(lambda a, b: oracle.dequantize(
            0, oc[a:b], os_[a:b], None, b - a, cols, oracle.F16), rows)
        S.parity("quantize_e2m3_fp16", [(gc, oc), (gs, os_)], rows * cols * 2, t_q,
                 "all 14336 rows: codes, scales")
        S.parity("dequantize_e2m3_to_fp16", [(gy, oy)], nb * 25, t_dq,
                 "all 14336 rows: fp16 output")
        del oc, os_, oy, gc, gs, gy
    del xs, ys, ss, cs, w

    # -- AXS-6 weight: fake-quantize and quantize (+ config plane); bits per
    #    value and each block's largest error
    a = workloads.axs6_weight()
    rows, cols = a.shape
    nb = rows * cols // 32
    note = "axs6_weight bf16 4096x4096"
    n = rotation_sets(rows * cols * 4)
    xs = bf16_dev(a, n)
    ys = [torch.empty_like(xs[0]) for _ in range(n)]
    fq = lambda i: mx.mx_fake_quantize(4, 32, BF, xs[i], ys[i], rows, cols, st)
    S.time("fake_quantize_axs6", fq, n, rows * cols * 2, rows * cols * 2, note,
           copy_bpb=(64, 64))
    cs = [torch.empty(nb * 24, dtype=torch.uint8, device="cuda") for _ in range(n)]
    ss = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(n)]
    aa = [torch.empty((nb + 3) // 4, dtype=torch.uint8, device="cuda") for _ in range(n)]
    q = lambda i: mx.mx_quantize(4, 32, BF, xs[i], rows, cols, cs[i], ss[i], aa[i], st)
    S.time("quantize_axs6", q, n, rows * cols * 2, nb * 24 + nb + (nb + 3) // 4, note,
           copy_bpb=(64, 25))
    S.launch("fq", fq)(0)
    S.launch("q", q)(0)
    torch.cuda.synchronize()
    gy, gc, gs, ga = host(ys[0]), host(cs[0]), host(ss[0]), host(aa[0])
    if check:
        oy, t_fq = S.oracle(lambda r0, r1: oracle.fake_quantize(4, a[r0:r1]), rows)
        (oc, os_, oa), t_q = S.oracle(lambda r0, r1: oracle.quantize(4, a[r0:r1]), rows)
        S.parity("fake_quantize_axs6", [(gy, oy)], rows * cols * 2, t_fq,
                 "all 4096 rows: bf16 output")
        S.parity("quantize_axs6", [(gc, oc), (gs, os_), (ga, oa)], rows * cols * 2, t_q,
                 "all 4096 rows: codes, shared exponents, config plane")
    # bits per value from the buffers; per-block error against the grid's
    # bound: half a step 2^(E-5) below the top value, 2^(E-4) where the
    # block maximum saturates at 31/16 2^E (E = byte - 127)
    S.res["quantize_axs6"]["bits_per_value"] = 8 * (gc.size + gs.size + ga.size) / (rows * cols)
    xf = workloads.bf16_bits_to_f32(a).astype(np.float64).reshape(nb, 32)
    yf = workloads.bf16_bits_to_f32(gy).astype(np.float64).reshape(nb, 32)
    err = np.abs(xf - yf)
    blk = err.max(axis=1)
    E = gs.reshape(-1).astype(np.float64) - 127
    top = (31.0 / 16.0) * np.exp2(E)[:, None]
    bound = np.where(np.abs(xf) > top, np.exp2(E - 4)[:, None], np.exp2(E - 5)[:, None])
    S.res["fake_quantize_axs6"]["block_max_abs_err"] = {
        "max": float(blk.max()), "mean": float(blk.mean()),
        "max_over_half_step": float((blk / np.exp2(E - 5)).max()),
        "bound_ok": bool(np.all(err <= bound)),
        "note": "per 32-value block: max |x - fq(x)|; bound 2^(E-5), 2^(E-4) for values above "
                "31/16 2^E"}
    del xs, ys, cs, ss, aa, a, xf, yf, err, bound

    # -- dynamic activations: E4M3 and E2M3 quantize and dequantize
    act = workloads.activations()
    rows, cols = act.shape
    nb = rows * cols // 32
    note = "activations bf16 16384x8192"
    n = rotation_sets(rows * cols * 4 + nb * 33)
    xs = bf16_dev(act, n)
    ys = [torch.empty_like(xs[0]) for _ in range(n)]
    ss = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(n)]
    for f, nm, bpb in ((3, "e4m3", 32), (0, "e2m3", 24)):
        cs = [torch.empty(nb * bpb, dtype=torch.uint8, device="cuda") for _ in range(n)]
        q = lambda i, f=f, cs=cs: mx.mx_quantize(f, 32, BF, xs[i], rows, cols, cs[i], ss[i], None, st)
        dq = lambda i, f=f, cs=cs: mx.mx_dequantize(f, 32, cs[i], ss[i], None, rows, cols, BF, ys[i], st)
        S.time(f"quantize_{nm}_activations", q, n, rows * cols * 2, nb * (bpb + 1), note,
               copy_bpb=(64, bpb + 1))
        S.launch(nm, q)(0)
        S.time(f"dequantize_{nm}_activations", dq, n, nb * (bpb + 1), rows * cols * 2, note,
               copy_bpb=(bpb + 1, 64))
        S.launch(nm, dq)(0)
        torch.cuda.synchronize()
        gs = host(ss[0])
        S.res[f"quantize_{nm}_activations"]["poisoned_blocks"] = int((gs == 0xFF).sum())
        if check:
            gc, gy = host(cs[0]), host(ys[0])
            (oc, os_, _), t_q = S.oracle(lambda a, b, f=f: oracle.quantize(f, act[a:b]), rows)
            oy, t_dq = S.oracle(lambda a, b, f=f: oracle.dequantize(
                f, oc[a:b], os_[a:b], None, b - a, cols, oracle.BF16), rows)
            S.parity(f"quantize_{nm}_activations", [(gc, oc), (gs, os_)], rows * cols * 2, t_q,
                     "all 16384 rows: codes, scales")
            S.parity(f"dequantize_{nm}_activations", [(gy, oy)], nb * (bpb + 1), t_dq,
                     "all 16384 rows: bf16 output")
            del gc, gy, oc, os_, oy
        del cs, gs
    del xs, ys, ss, act

    # -- attention probabilities: exp-then-quantize to E2M1 (2 GiB of
    #    scores), then the dequantized P
    s = workloads.attn_scores()
    rows, cols = s.shape
    nb = rows * cols // 32
    note = "attn_scores fp32 32x4096x4096"
    sd = torch.from_numpy(s).cuda()
    c = torch.empty(nb * 16, dtype=torch.uint8, device="cuda")
    sc = torch.empty(nb, dtype=torch.uint8, device="cuda")
    pd = torch.empty_like(sd)
    kk = max(5, S.k // 4)
    sq = lambda i: mx.mx_softmax_quantize(2, 32, sd, rows, cols, c, sc, st)
    S.time("softmax_quantize_e2m1", sq, 1, rows * cols * 4, nb * 17, note, steps=kk, warm=2)
    # its floor: the same grid, loads and stores with the arithmetic folded
    # away (tests/hwprobe/bw_probe.hip)
    floor = rows_floor_probe()
    if floor is not None:
        def fl(i):
            return floor(sd.data_ptr(), rows, cols, c.data_ptr(), sc.data_ptr(), st)

        ms_floor = time_launches(S.launch("probe_rows_floor", fl), 1, kk, 2,
                                 min_warm_s=SECONDARY_WARM_S)
        r = S.res["softmax_quantize_e2m1"]
        r.update(floor_us=round(ms_floor * 1e3, 2), frac_of_floor=round(ms_floor * 1e3 / r["us"], 4),
                 floor_note="same grid, loads and stores with no exp or conversion")
    S.launch("sq", sq)(0)  # the real outputs again, after the floor probe
    dq = lambda i: mx.mx_dequantize(2, 32, c, sc, None, rows, cols, FP, pd, st)
    S.time("dequantize_e2m1_to_fp32", dq, 1, nb * 17, rows * cols * 4, note, steps=kk, warm=2,
           copy_bpb=(17, 128))
    torch.cuda.synchronize()
    if check:
        gc, gs, gp = host(c), host(sc), host(pd)
        del sd, pd, c, sc
        (oc, os_), t_q = S.oracle(lambda a, b: oracle.softmax_quantize(2, s[a:b]), rows)
        op, t_dq = S.oracle(lambda a, b: oracle.dequantize(2, oc[a:b], os_[a:b], None, b - a,
                                                           cols, oracle.FP32), rows)
        S.parity("softmax_quantize_e2m1", [(gc, oc), (gs, os_)], rows * cols * 4, t_q,
                 "all 131072 rows: codes, scales")
        S.parity("dequantize_e2m1_to_fp32", [(gp, op)], nb * 17, t_dq,
                 "all 131072 rows: fp32 P")
        del gc, gs, gp, oc, os_, op
    else:
        del sd, pd, c, sc
    del s

    # -- the same scores inside a fused attention forward: 32 heads x 4096
    #    queries x 4096 keys, d = 128, bf16 q/k, V^T in MXFP8, bf16 output
    S.res.update(attention_line(mx, S.k))
    if check:
        for name, ok in attention_parity(mx).items():
            S.res[name]["parity"] = ok
            if not ok["bit_exact"]:
                S.failed.append(name)

    # -- layer-by-layer conversion of a synthetic dense decoder (4 layers,
    #    hidden 4096, MLP 14336, 1024-wide k/v): weights already on the
    #    GPU, and again from pinned host memory (that rate includes the PCIe
    #    upload)
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
    note = "synthetic decoder, 4 layers x 7 weights, hidden 4096, MLP 14336 (mxfp6 shorthand)"
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
        name = f"convert_dense_4_layers_from_{src_name}"
        S.res[name] = {"us": round(ms * 1e3, 2), "input_GBps": round(in_b / ms / 1e6, 1),
                       "hbm_frac": round((in_b + out_b) / ms / 1e6 / HBM_PEAK_GBS, 4),
                       "bytes": in_b + out_b, "workload": note}
        if src_name == "device" and check:
            # every converted tensor against the oracle
            pairs, t_or = [], 0.0
            for nm_, t in model.items():
                wq = out[nm_]
                xh = host(t)
                (oc, os_, _), dt = S.oracle(lambda a, b, xh=xh: oracle.quantize(0, xh[a:b]),
                                            xh.shape[0])
                t_or += dt
                pairs += [(host(wq.codes), oc), (host(wq.scales), os_)]
            S.parity(name, pairs, in_b, t_or, "all 28 tensors: codes, scales")
        del out
    del model, src

    # -- small fp32 tensor: the three ops (launch-bound)
    x = workloads.weights_small()
    xsm = torch.from_numpy(x).cuda()
    cc = torch.empty(1024 * 24, dtype=torch.uint8, device="cuda")
    s1 = torch.empty(1024, dtype=torch.uint8, device="cuda")
    yq = torch.empty_like(xsm)
    yf = torch.empty_like(xsm)
    note = "weights_small fp32 128x256 (launch-bound)"
    q = lambda i: mx.mx_quantize(0, 32, FP, xsm, 128, 256, cc, s1, None, st)
    dq = lambda i: mx.mx_dequantize(0, 32, cc, s1, None, 128, 256, FP, yq, st)
    fq = lambda i: mx.mx_fake_quantize(0, 32, FP, xsm, yf, 128, 256, st)
    S.time("quantize_e2m3_weights_small", q, 1, 131072, 25600, note)
    S.time("dequantize_e2m3_weights_small", dq, 1, 25600, 131072, note)
    S.time("fake_quantize_e2m3_weights_small", fq, 1, 131072, 131072, note)
    for f_ in (q, dq, fq):
        S.launch("small", f_)(0)
    torch.cuda.synchronize()
    if not check:
        return S.res, S.failed
    (oc, os_, _), t_q = S.oracle(lambda a, b: oracle.quantize(0, x[a:b]), 128)
    oy, t_dq = S.oracle(lambda a, b: oracle.dequantize(0, oc[a:b], os_[a:b], None, b - a, 256,
                                                       oracle.FP32), 128)
    of, t_fq = S.oracle(lambda a, b: oracle.fake_quantize(0, x[a:b]), 128)
    S.parity("quantize_e2m3_weights_small", [(host(cc), oc), (host(s1), os_)], 131072, t_q,
             "all 128 rows: codes, scales")
    S.parity("dequantize_e2m3_weights_small", [(host(yq), oy)], 25600, t_dq,
             "all 128 rows: fp32 output")
    S.parity("fake_quantize_e2m3_weights_small", [(host(yf), of)], 131072, t_fq,
             "all 128 rows: fp32 output")
    return S.res, S.failed


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
    # the scaling by scale * log2 e, the shift, the 2^u's 9 (rint, the
    # reduction, 5 fused multiply-adds, the conversion of n, the scaling by
    # 2^n) and the block maximum = 12; EFQ: the affine map from the raw
    # score (one fused multiply-add, the clamp, the conversion) and the
    # block maximum = 4.  The chip issues 256 CUs x 4 SIMDs x 16 lanes x
    # 2.4 GHz of them per second.
    for name, fn, ops_per in (("attention_fwd_e2m1_p_mxfp8_v", mx.mx_attention_fwd, 12.0),
                              ("attention_fwd_efq_e2m1_p_mxfp8_v", mx.mx_attention_fwd_efq, 4.0)):
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


# sampled (head, query) rows of the attention parity check
ATTN_ROWS = [(0, 0), (5, 1234), (17, 4095), (31, 2048), (12, 77), (31, 4095), (8, 3000),
             (20, 511)]


def attention_parity(mx, heads=32, lq=4096, lk=4096, d=128):
    """Both attention forwards in the benchmark's launch configuration (32
    heads x 4096 x 4096, d 128, MXFP8 V^T, bf16 output) on exactly summable
    scores: q and k entries are multiples of 1/4 in [-3, 3], so every score
    is exact in fp32 whatever the order of the sums, and the sampled rows'
    probability blocks, scale bytes and row maxima must equal the oracle's
    bit for bit.  (The output o rounds differently by construction -- fp32
    matrix-core sums against the oracle's double -- and is checked against
    its derived bound in the GPU tests.)"""
    import numpy as np
    import torch

    import oracle
    g = torch.Generator(device="cuda").manual_seed(13)
    qd = (torch.randint(-12, 13, (heads, lq, d), generator=g, device="cuda").float() / 4).to(
        torch.bfloat16)
    kd = (torch.randint(-12, 13, (heads, lk, d), generator=g, device="cuda").float() / 4).to(
        torch.bfloat16)
    vc, vs = mx.quantize_v(torch.randn(heads, lk, d, generator=g, device="cuda"), "mxfp8")
    q, k = host(qd), host(kd)
    vch, vsh = host(vc).reshape(heads, -1), host(vs).reshape(heads, -1)
    scale = np.float32(d ** -0.5)
    out = {}
    for name, efq in (("attention_fwd_e2m1_p_mxfp8_v", False),
                      ("attention_fwd_efq_e2m1_p_mxfp8_v", True)):
        _, rm, _, pc, ps = mx.attention_fwd(qd, kd, vc, vs, "mxfp8", scale=scale,
                                            out_dtype=torch.bfloat16, stats=True, probs=True,
                                            efq=efq)
        torch.cuda.synchronize()
        ok = True
        for h, i in ATTN_ROWS:
            _, rm_ref, _, pc_ref, ps_ref = oracle.attention_fwd(
                oracle.FP8_E4M3, q[h:h + 1, i:i + 1], k[h:h + 1], vch[h:h + 1], vsh[h:h + 1],
                scale, 64, oracle.FP32, efq=efq)
            ok &= bool(np.array_equal(host(pc[h, i]), pc_ref[0, 0])
                       and np.array_equal(host(ps[h, i]), ps_ref[0, 0])
                       and float(rm[h, i]) == float(rm_ref[0, 0]))
        out[name] = {"bit_exact": ok,
                     "compared": f"{len(ATTN_ROWS)} sampled rows on exactly summable q and k: "
                                 "probability blocks, scale bytes, row maxima"}
        del rm, pc, ps
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(x_np, gpu_codes, gpu_scales, threads, passes=3, single_rows=2048):
    """The CPU oracle, as it stands, on the headline's input: T threads, each
    on one contiguous range of rows (blocks never cross rows), over the whole
    tensor, and one thread on its first `single_rows` rows; the minimum of
    `passes` passes each.  The T-thread output is compared with the GPU's."""
    import numpy as np

    import oracle
    rows, cols = x_np.shape
    best, out = None, None
    for _ in range(passes):
        t = time.perf_counter()
        out = oracle.by_rows(lambda a, b: oracle.quantize(0, x_np[a:b])[:2], rows, threads)
        wall = time.perf_counter() - t
        best = wall if best is None else min(best, wall)
    oc, os_ = out
    parity = bool(np.array_equal(host(gpu_codes).reshape(oc.shape), oc)
                  and np.array_equal(host(gpu_scales).reshape(os_.shape), os_))
    sample = x_np[:single_rows]
    best1 = None
    for _ in range(passes):
        t = time.perf_counter()
        oracle.quantize(0, sample)
        wall = time.perf_counter() - t
        best1 = wall if best1 is None else min(best1, wall)
    value = rows * cols * 2 / best / 1e9
    base = {"value": round(value, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole bf16 14336x4096 input ({rows * cols} values), E2M3 "
                      f"quantize+pack, {threads} threads x ~{rows // threads} rows, best of "
                      f"{passes} passes ({best:.2f} s wall each)",
            "single_thread_GBps": round(single_rows * cols * 2 / best1 / 1e9, 4),
            "single_thread_sample": f"rows 0..{single_rows - 1} ({single_rows * cols} values), "
                                    f"one thread, best of {passes} ({best1:.2f} s)",
            "cpu_model": cpu_model(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "threads_note": "T = the CPUs this process may use, at most 16 (the host CPU share "
                            "of one GPU)"}
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
    ms, in_b, alg_b, nsets, codes0, scales0, copy_gbs, sched, clocks = headline(
        mx, x, args.steps, args.warmup)
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
        "d2d_copy_reference": {"d2d_copy_GBps": round(copy_gbs, 1),
                               "headline_over_copy": round(achieved / copy_gbs, 4),
                               "note": "torch's device-to-device copy of the bf16 input (read + "
                                       "write bytes / time), same buffers and rotation; a "
                                       "reference rate, not a ceiling"},
        "batches": clocks["batches"],
        "gpu_clocks": clocks["gpu_clocks"],
    }
    if sched:
        best = min(MIX_COPIES, key=lambda k: sched[k])
        rd = min(sched[k] for k in MIX_READS)
        wr = min(sched[k] for k in MIX_WRITES)
        serial = rd + wr
        out["best_mix_ceiling"] = {
            "us": round(sched[best] * 1e3, 3), "schedule": best,
            "frac_of_peak": round(alg_b / sched[best] / 1e6 / HBM_PEAK_GBS, 4),
            "headline_frac_of_ceiling": round(sched[best] / ms, 4),
            "schedules_us": {k: round(v * 1e3, 3) for k, v in sched.items()},
            "serial_bound_us": round(serial * 1e3, 3),
            "serial_bound_frac_of_peak": round(alg_b / serial / 1e6 / HBM_PEAK_GBS, 4),
            "read_only_GBps": round(in_b / rd / 1e6, 1),
            "write_only_GBps": round((alg_b - in_b) / wr / 1e6, 1),
            "note": "copy kernels moving the quantizer's bytes with no arithmetic, in each access "
                    "schedule (tests/hwprobe/bw_probe.hip), same buffers, rotation, warm-up and "
                    "steps; serial bound = the fastest reads alone plus the fastest writes alone"}
    import oracle
    threads = oracle.worker_threads()
    failed = []
    if not args.no_cpu_baseline:
        base, parity, nrows = cpu_baseline(x, codes0, scales0, threads)
        out["cpu_baseline"] = base
        out["parity"] = {"bit_exact": parity, "rows_compared": nrows}
        if not parity:
            failed.append("headline")
    if not args.no_secondary:
        del codes0, scales0
        torch.cuda.empty_cache()
        out["secondary"], bad = secondary(mx, args.steps, threads,
                                          check=not args.no_cpu_baseline)
        failed += bad
        if not args.no_cpu_baseline:
            out["parity"] = dict(out["parity"], all_rows_bit_exact=not failed,
                                 ops_checked=1 + sum("parity" in r
                                                     for r in out["secondary"].values()))
    print(json.dumps(out), flush=True)
    if failed:
        print(f"bench.py: the GPU's output differs from the oracle's in {failed}", file=sys.stderr,
              flush=True)
        sys.exit(1)


if __name__ == "__main__":
    main()
