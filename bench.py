"""Benchmark of the MX hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one pass of the codec over the 8192x8192 MXFP4 weight workload
(N(0, 0.02), 0.1% outliers x50): mx_quantize (f32 -> E2M1 codes + E8M0
scales) followed by mx_dequantize (back to f32).  `value` is the algorithmic
HBM traffic of the step (2 x 4.53125 B/element) divided by the step time, in
GB/s.  Inputs are resident in HBM before the timed region; consecutive steps
rotate over four copies of the workload (4 x 256 MiB of f32, larger than the
256 MiB Infinity Cache) so that no step reads what the previous one left in
the caches.  After the W warm-up steps, untimed steps run for 0.5 s more so
that the K timed steps see the card's steady clocks.

The other workloads are timed in the same run and reported under "parts",
each with its roofline: the decode-shaped MXFP4 x MXFP4 16x4096x4096 block
matmul (HBM-bound), the MXFP8 8192^3 product, the prefill linear layer
(2048x8192 activations quantized on the fly to E4M3, times MXFP4 weights
28672x8192), the block matmul with an ordinary float32 B (decode-shaped
4096x4096 MXFP4 weights times 4096x16 activations, and 4096^3), the codec
with blocks along axis 0 on the 8192x8192 weight workload, and fold_scale on
its scales.  Kernel durations come from HIP events recorded on the stream the
kernels run on (for the parts, around replays of a HIP graph of back-to-back
calls).

Before the GPU is touched, the CPU oracle runs on the host's cores (one
worker process per available core, at most 16): whole passes of the step's
workload give `cpu_baseline` and the bit-exact reference of the step's
outputs (`parity`); the oracle's float64 block_matmul is timed on each matmul
workload (in full for the decode shape, on stated output samples for the
others) and its outputs are the reference of each matmul part's `parity`.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MX quantize/dequant GB/s (% HBM peak); block_matmul TFLOP/s (% MX MFMA peak)"
HBM_PEAK_GBS = 8000.0
PEAK_TFLOPS = {"fp4": 10100.0, "fp8": 5000.0, "bf16": 2500.0, "fp32": 157.3}
PROFILE_DIR = os.path.join(ROOT, "profiles")


def codec_bytes(rows: int, cols: int, elem_bytes: float) -> int:
    """Algorithmic HBM bytes of one quantize (or dequantize) of [rows, cols]:
    4 B of f32 per element plus the codes and one scale byte per 32."""
    n = rows * cols
    return int(n * 4 + n * elem_bytes + n // 32)


def matmul_bytes(M, N, K, a_bytes, b_bytes, accumulate=False) -> int:
    return int(M * K * a_bytes + M * K // 32 + N * K * b_bytes + N * K // 32 +
               M * N * 4 * (2 if accumulate else 1))


FLOOR_SRC = os.path.join(ROOT, "bench_floor.hip")
FLOOR_LIB = os.path.join(ROOT, "bench_floor.so")


def build_floor() -> str:
    """Compile bench_floor.hip (the decode product's memory-floor reference)
    into bench_floor.so beside this file."""
    import subprocess
    from bit_gemm_mx_amd.build import ARCH, hipcc
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", FLOOR_SRC,
           "-o", FLOOR_LIB + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on bench_floor.hip:\n{r.stderr}")
    os.replace(FLOOR_LIB + ".tmp", FLOOR_LIB)
    return FLOOR_LIB


def source_hash(*names: str) -> str:
    """Hash of a kernel's source: its .hip file and the headers it includes."""
    h = hashlib.sha256()
    for n in names + ("codec_common.h", "mx_internal.h"):
        with open(os.path.join(ROOT, "bit_gemm_mx_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, src: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(PROFILE_DIR, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    e = d.get(kernel)
    if not e or e.get("source_sha256_16") != source_hash(src):
        return None
    return e.get("hbm_bytes_per_launch")


class EventTimer:
    """Per-kernel durations from HIP events on the current stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def run(self, name, fn):
        s = self.torch.cuda.Event(enable_timing=True)
        e = self.torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        self.pairs.setdefault(name, []).append((s, e))

    def mean_ms(self, name):
        v = [s.elapsed_time(e) for s, e in self.pairs[name]]
        return float(np.mean(v)), float(np.min(v))


def bench_codec(mx, W, torch, steps, warmup, ref=None):
    rows = cols = 8192
    x_host = W.weight_codec_case(rows, cols, seed=1002)
    copies = 4
    xs = [torch.from_numpy(x_host).cuda() for _ in range(copies)]
    qs = [mx.empty_mx(rows, cols, mx.MX_E2M1, xs[0].device) for _ in range(copies)]
    ys = [torch.empty_like(xs[0]) for _ in range(copies)]
    torch.cuda.synchronize()

    def step(i, timer=None):
        j = i % copies
        if timer is None:
            mx.quantize(xs[j], mx.MX_E2M1, out=qs[j])
            mx.dequantize(qs[j], out=ys[j])
        else:
            timer.run("quantize", lambda: mx.quantize(xs[j], mx.MX_E2M1, out=qs[j]))
            timer.run("dequantize", lambda: mx.dequantize(qs[j], out=ys[j]))

    # W untimed warm-up steps, then more untimed steps until 0.5 s have passed:
    # from idle the card needs tens of milliseconds to settle its clocks (the
    # quantize measured 50.2 us per call within the first ~2 ms of work and
    # 48.3 us at steady state), and the steady state is what a continuously
    # loaded GPU sees.  The matmul parts warm up the same way (timed()).
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t_warm = time.perf_counter()
    i = warmup
    while time.perf_counter() - t_warm < 0.5:
        for _ in range(50):
            step(i)
            i += 1
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # Per-kernel durations: each kernel alone, `steps` back-to-back launches
    # rotating over the copies, captured in a HIP graph and replayed between
    # HIP events on the stream the kernels run on (timed(), as for the parts),
    # so that neither the event overhead nor the host's launch path is
    # charged per launch.
    n = [0]

    def rot():
        n[0] += 1
        return n[0] % copies

    q_ms, q_min = timed(torch, "quantize",
                        lambda: (lambda j: mx.quantize(xs[j], mx.MX_E2M1, out=qs[j]))(rot()), steps)
    d_ms, d_min = timed(torch, "dequantize",
                        lambda: (lambda j: mx.dequantize(qs[j], out=ys[j]))(rot()), steps)
    per_op = codec_bytes(rows, cols, 0.5)
    kernels = {
        "quantize_e2m1": dict(ms=q_ms, min_ms=q_min, bytes=per_op, src="quantize.hip",
                              kernel="quantize_kernel<1>"),
        "dequantize_e2m1": dict(ms=d_ms, min_ms=d_min, bytes=per_op, src="dequantize.hip",
                                kernel="dequantize_kernel<1>"),
    }
    parity = None
    if ref is not None:
        # every copy holds the same workload: check copy 0's step outputs
        oc, os_, oy = ref
        same = lambda g, w: bool(np.array_equal(g.view(np.uint8) if g.dtype != np.float32
                                                else g.view(np.uint32),
                                                w.view(np.uint8) if w.dtype != np.float32
                                                else w.view(np.uint32)))
        parity = {"elements": rows * cols,
                  "codes_bit_exact": same(qs[0].codes.cpu().numpy(), oc),
                  "scales_bit_exact": same(qs[0].scales.cpu().numpy(), os_),
                  "dequantized_bit_exact": same(ys[0].cpu().numpy(), oy),
                  "against": "the oracle's quantize and dequantize of the same input"}
    del xs, qs, ys
    torch.cuda.empty_cache()
    return wall, 2 * per_op, kernels, parity


def progress(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def roofline_hbm(name, k):
    gbs = k["bytes"] / (k["ms"] * 1e-3) / 1e9
    return {"bound": "hbm", "kernel": name, "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(name, k["src"]),
            "algorithmic_bytes": k["bytes"], "avg_ms": round(k["ms"], 5)}


def timed(torch, name, fn, n, warm_s=0.5):
    """Average duration of fn over n back-to-back calls (and the fastest of
    three such groups), from HIP events on the stream the kernels run on.

    The n calls are captured once into a HIP graph and the graph is replayed
    between the events, so that kernels of a few microseconds are timed back
    to back on the GPU rather than at the rate the host can launch them.
    Before the timed groups the graph replays for warm_s seconds: a matmul
    that starts from idle runs ~15% slower for its first ~50 ms while the
    card settles its clock and power state (measured: 505 us, then 465, 445,
    then a steady 434 us per 8192^3 MXFP8 product), and the steady state is
    what a continuously loaded GPU sees."""
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            fn()
    t0 = time.perf_counter()
    while True:
        g.replay()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= warm_s:
            break
    t = EventTimer(torch)
    for _ in range(3):
        t.run(name, g.replay)
    torch.cuda.synchronize()
    mean, best = t.mean_ms(name)
    del g
    return mean / n, best / n


def sustained_clock(torch, fn, seconds=2.0):
    """Median GFX clock (MHz) while fn runs back to back on the GPU for about
    `seconds`, read every 0.1 s from the driver's pp_dpm_sclk file (the line
    marked '*' is the current clock; plain file reads, no helper process).
    The first 0.3 s of samples (clock ramp) are dropped.  None when the file
    is missing or unreadable.  The published peaks assume 2400 MHz."""
    import glob
    import re
    import threading
    files = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    if len(files) != 1:
        return None
    samples, stop = [], threading.Event()

    def sample():
        while not stop.is_set():
            try:
                with open(files[0]) as f:
                    for line in f:
                        if line.rstrip().endswith("*"):
                            m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
                            if m:
                                samples.append(float(m.group(1)))
            except OSError:
                pass
            time.sleep(0.1)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(4):
            fn()
    g.replay()
    torch.cuda.synchronize()
    th = threading.Thread(target=sample, daemon=True)
    t_end = time.perf_counter() + seconds
    th.start()
    while time.perf_counter() < t_end:
        for _ in range(8):
            g.replay()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=5)
    del g
    steady = samples[3:]
    return float(np.median(steady)) if steady else None


def hbm_part(ms, mn, byts, extra=None):
    gbs = byts / (ms * 1e-3) / 1e9
    d = {"ms": round(ms, 5), "min_ms": round(mn, 5),
         "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                      "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                      "algorithmic_bytes": int(byts)}}
    if extra:
        d.update(extra)
    return d


def bench_axis0_fold(mx, W, torch, reps):
    """The codec with blocks along axis 0, and fold_scale."""
    out = {}
    rows = cols = 8192
    # two copies of every buffer, alternated, so that no call reads what the
    # previous one left in the 256 MiB Infinity Cache
    x0 = torch.from_numpy(W.weight_codec_case(rows, cols, seed=1002)).cuda()
    xs = [x0, x0.clone()]
    qs = [mx.empty_mx(rows, cols, mx.MX_E2M1, x0.device, axis=0) for _ in range(2)]
    ys = [torch.empty_like(x0) for _ in range(2)]
    byts = codec_bytes(rows, cols, 0.5)
    n = [0]

    def alt():
        n[0] += 1
        return n[0] & 1

    ms, mn = timed(torch, "qa0", lambda: (lambda i: mx.quantize(xs[i], mx.MX_E2M1, out=qs[i],
                                                               axis=0))(alt()), reps)
    out["quantize_axis0_e2m1_8192x8192"] = hbm_part(ms, mn, byts)
    ms, mn = timed(torch, "da0", lambda: (lambda i: mx.dequantize(qs[i], out=ys[i]))(alt()), reps)
    out["dequantize_axis0_e2m1_8192x8192"] = hbm_part(ms, mn, byts)
    # fold_scale by 2^1 then 2^-1, so the scales stay in range over the reps
    ms, mn = timed(torch, "fold", lambda: (mx.fold_scale(qs[0], 1), mx.fold_scale(qs[0], -1)),
                   reps)
    out["fold_scale_8192x8192_scales"] = hbm_part(ms / 2, mn / 2, 2 * qs[0].scales.numel())
    del x0, xs, qs, ys
    progress("axis-0 codec and fold_scale done")
    return out


def bench_roundtrip(mx, W, torch, reps):
    """The 256x1024 MXFP4 round trip (the correctness workload): quantize and
    dequantize timed apart; at 1.2 MB per op this measures launch latency,
    not bandwidth."""
    case = W.roundtrip_case()
    x = torch.from_numpy(case.x).cuda()
    rows, cols = x.shape
    q = mx.empty_mx(rows, cols, mx.MX_E2M1, x.device)
    y = torch.empty_like(x)
    byts = codec_bytes(rows, cols, 0.5)
    ms, mn = timed(torch, "rt_q", lambda: mx.quantize(x, mx.MX_E2M1, out=q), max(reps, 50))
    out = {"roundtrip_quantize_e2m1_256x1024": hbm_part(ms, mn, byts)}
    # decoded from a copy whose two chosen blocks carry the NaN scale 0xFF
    qd = mx.empty_mx(rows, cols, mx.MX_E2M1, x.device)
    qd.codes.copy_(q.codes)
    qd.scales.copy_(q.scales)
    qd.scales.view(-1)[torch.from_numpy(case.ff_blocks).cuda()] = 0xFF
    ms, mn = timed(torch, "rt_d", lambda: mx.dequantize(qd, out=y), max(reps, 50))
    out["roundtrip_dequantize_e2m1_256x1024"] = hbm_part(ms, mn, byts)
    del x, q, qd, y
    return out


def bench_f32b(mx, W, torch, reps):
    """block_matmul with an ordinary float32 B: decode and square workloads."""
    out = {}

    a, b = W.f32b_decode_case()
    at = mx.quantize(torch.from_numpy(a).cuda(), mx.MX_E2M1)
    bd = torch.from_numpy(b).cuda()
    c = torch.empty((4096, 16), dtype=torch.float32, device="cuda")
    ms, mn = timed(torch, "f32b_dec", lambda: mx.block_matmul_f32b(at, bd, out=c), max(reps, 20))
    flops = 2 * 4096 * 16 * 4096
    tf = flops / (ms * 1e-3) / 1e12
    byts = 4096 * 4096 // 2 + 4096 * 4096 // 32 + 4096 * 16 * 4 * 2
    out["f32b_decode_mxfp4x4096x4096_f32x16"] = hbm_part(ms, mn, byts, {
        "tflops": round(tf, 2), "mfma_fp32_frac": round(tf / PEAK_TFLOPS["fp32"], 4)})
    del at, bd, c
    a, b = W.f32b_square_case()
    at = mx.quantize(torch.from_numpy(a).cuda(), mx.MX_E2M1)
    bd = torch.from_numpy(b).cuda()
    c = torch.empty((4096, 4096), dtype=torch.float32, device="cuda")
    ms, mn = timed(torch, "f32b_sq", lambda: mx.block_matmul_f32b(at, bd, out=c), max(3, reps // 4))
    tf = 2 * 4096 ** 3 / (ms * 1e-3) / 1e12
    # The kernel multiplies on the bf16 matrix cores, three MFMAs per product
    # (B split into three exact bf16 parts): its instruction peak is a third
    # of the bf16 rate in algorithmic flops.
    peak = PEAK_TFLOPS["bf16"] / 3
    out["f32b_mxfp4_4096x4096x4096"] = {
        "ms": round(ms, 4), "min_ms": round(mn, 4), "tflops": round(tf, 1),
        "roofline": {"bound": "mfma", "kernel": "block_matmul_f32b_bf16", "achieved": round(tf, 1),
                     "peak": round(peak, 1), "unit": "TFLOP/s", "frac": round(tf / peak, 4),
                     "peak_is": "bf16 dense 2500 TFLOP/s / 3 MFMAs per product"},
        "vs_fp32_matrix_peak": round(tf / PEAK_TFLOPS["fp32"], 4)}
    del at, bd, c
    torch.cuda.empty_cache()
    progress("f32-B block matmul done")
    return out


def bench_matmuls(mx, W, torch, reps, ref=None):
    out = {}
    mref = ref["matmul"] if ref else {}

    def attach(key, c_gpu_sample):
        """Oracle timing and parity of one matmul part (c_gpu_sample: the
        GPU's outputs at the oracle's sampled positions, on the host)."""
        if key not in mref:
            return
        want, mag = mref[key]["ref"]
        out[key]["cpu_oracle"] = mref[key]["cpu_oracle"]
        out[key]["parity"] = t1_parity(c_gpu_sample, want, mag)

    # decode-shaped MXFP4 x MXFP4
    a, bt = W.decode_matmul_case()
    at = mx.quantize(torch.from_numpy(a).cuda(), mx.MX_E2M1)
    btt = mx.quantize(torch.from_numpy(bt).cuda(), mx.MX_E2M1)
    c = torch.empty((16, 4096), dtype=torch.float32, device="cuda")
    ms, mn = timed(torch, "decode", lambda: mx.block_matmul(at, btt, out=c), max(reps, 20))
    flops = 2 * 16 * 4096 * 4096
    byts = matmul_bytes(16, 4096, 4096, 0.5, 0.5)
    gbs = byts / (ms * 1e-3) / 1e9
    out["decode_mxfp4_16x4096x4096"] = {
        "ms": round(ms, 5), "min_ms": round(mn, 5), "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes": byts}}
    # Back to back, the 8.5 MB weight stays in the 256 MiB Infinity Cache.  As
    # a decode step meets it (each layer's weight read once), rotate through 40
    # copies (340 MB) so that every call reads its weight from HBM.
    copies = [mx.MXTensor(btt.codes.clone(), btt.scales.clone(), btt.rows, btt.cols, btt.elem)
              for _ in range(40)]
    k = [0]

    def cold():
        k[0] = (k[0] + 1) % len(copies)
        mx.block_matmul(at, copies[k[0]], out=c)
    cms, cmn = timed(torch, "decode_cold", cold, 40)
    cgbs = byts / (cms * 1e-3) / 1e9
    out["decode_mxfp4_16x4096x4096"]["cold_weights"] = {
        "ms": round(cms, 5), "min_ms": round(cmn, 5), "achieved": round(cgbs, 1), "unit": "GB/s",
        "frac": round(cgbs / HBM_PEAK_GBS, 4),
        "what": "each call reads one of 40 weight copies (340 MB, beyond the Infinity Cache)"}
    # The same launch shape reading the same bytes and writing C, with no
    # arithmetic (bench_floor.hip): the memory floor of this launch, warm and
    # with the weight read from HBM.
    if os.path.exists(FLOOR_LIB):
        import ctypes
        fl = ctypes.CDLL(FLOOR_LIB)
        fl.bench_read_floor.restype = ctypes.c_int
        fl.bench_read_floor.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 3 + [ctypes.c_void_p]
        def floor(w):
            # the current stream at call time: under graph capture, the capturing one
            stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            st = fl.bench_read_floor(at.codes.data_ptr(), at.scales.data_ptr(), w.codes.data_ptr(),
                                     w.scales.data_ptr(), c.data_ptr(), 16, 4096, 4096, stream)
            if st != 0:
                raise RuntimeError(f"bench_read_floor failed ({st})")

        fms, fmn = timed(torch, "floor", lambda: floor(btt), max(reps, 20))

        def floor_cold():
            k[0] = (k[0] + 1) % len(copies)
            floor(copies[k[0]])
        fcms, fcmn = timed(torch, "floor_cold", floor_cold, 40)
        out["decode_mxfp4_16x4096x4096"]["read_floor"] = {
            "ms": round(fms, 5), "cold_ms": round(fcms, 5),
            "decode_over_floor": round(ms / fms, 3), "decode_cold_over_floor_cold": round(cms / fcms, 3),
            "what": "same grid, same bytes read and C written, no decode or MFMA (bench_floor.hip)"}
    mx.block_matmul(at, btt, out=c)
    attach("decode_mxfp4_16x4096x4096", c.cpu().numpy())
    del at, btt, c, copies

    progress(f"decode-shaped matmul done: {ms:.4f} ms")
    # MXFP8 x MXFP8 8192^3
    a, bt = W.square_fp8_case()
    at = mx.quantize(torch.from_numpy(a).cuda(), mx.MX_E4M3)
    btt = mx.quantize(torch.from_numpy(bt).cuda(), mx.MX_E4M3)
    del a, bt
    c = torch.empty((8192, 8192), dtype=torch.float32, device="cuda")
    ms, mn = timed(torch, "fp8", lambda: mx.block_matmul(at, btt, out=c), reps)
    flops = 2 * 8192 ** 3
    tf = flops / (ms * 1e-3) / 1e12
    out["mxfp8_8192x8192x8192"] = {
        "ms": round(ms, 4), "min_ms": round(mn, 4), "tflops": round(tf, 1),
        "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_TFLOPS["fp8"],
                     "unit": "TFLOP/s", "frac": round(tf / PEAK_TFLOPS["fp8"], 4)}}
    # The card is power-limited on this product: report the clock it held and
    # the fraction of the peak at that clock beside the published-peak one.
    mhz = sustained_clock(torch, lambda: mx.block_matmul(at, btt, out=c))
    if mhz:
        out["mxfp8_8192x8192x8192"]["sustained_clock_mhz"] = round(mhz)
        out["mxfp8_8192x8192x8192"]["frac_at_sustained_clock"] = round(
            tf / (PEAK_TFLOPS["fp8"] * mhz / 2400.0), 4)
    # Operands from HBM: back to back, the 138 MB of operands stay in the 256
    # MiB Infinity Cache; rotating three copies (415 MB) makes every call
    # fetch them from HBM.
    ops = [(at, btt)] + [(mx.MXTensor(at.codes.clone(), at.scales.clone(), at.rows, at.cols, at.elem),
                          mx.MXTensor(btt.codes.clone(), btt.scales.clone(), btt.rows, btt.cols,
                                      btt.elem)) for _ in range(2)]
    kk = [0]

    def fp8_cold():
        kk[0] = (kk[0] + 1) % len(ops)
        mx.block_matmul(ops[kk[0]][0], ops[kk[0]][1], out=c)
    cms, cmn = timed(torch, "fp8_cold", fp8_cold, 3 * max(1, reps // 3))
    out["mxfp8_8192x8192x8192"]["cold_operands"] = {
        "ms": round(cms, 4), "tflops": round(flops / (cms * 1e-3) / 1e12, 1),
        "frac": round(flops / (cms * 1e-3) / 1e12 / PEAK_TFLOPS["fp8"], 4),
        "what": "each call reads one of 3 operand copies (415 MB, beyond the Infinity Cache)"}
    del ops
    if ref:
        r, k = ref["rows"]["mxfp8"]
        torch.cuda.synchronize()
        attach("mxfp8_8192x8192x8192", c.cpu().numpy()[np.ix_(r, k)])
    del at, btt, c
    torch.cuda.empty_cache()

    progress(f"MXFP8 8192^3 matmul done: {ms:.3f} ms")
    # prefill linear: quantize activations to E4M3, then E4M3 x E2M1
    a, bt = W.prefill_linear_case()
    ad = torch.from_numpy(a).cuda()
    btt = mx.quantize(torch.from_numpy(bt).cuda(), mx.MX_E2M1)
    del bt
    aq = mx.empty_mx(2048, 8192, mx.MX_E4M3, ad.device)
    c = torch.empty((2048, 28672), dtype=torch.float32, device="cuda")

    def prefill():
        mx.quantize(ad, mx.MX_E4M3, out=aq)
        mx.block_matmul(aq, btt, out=c)

    ms, mn = timed(torch, "prefill", prefill, reps)
    # Operands from HBM: rotate three copies of the activations and the
    # weight (3 x 189 MB) so that no call finds them in the Infinity Cache.
    pops = [(ad, btt)] + [(ad.clone(), mx.MXTensor(btt.codes.clone(), btt.scales.clone(), btt.rows,
                                                    btt.cols, btt.elem)) for _ in range(2)]
    pk = [0]

    def prefill_cold():
        pk[0] = (pk[0] + 1) % len(pops)
        mx.quantize(pops[pk[0]][0], mx.MX_E4M3, out=aq)
        mx.block_matmul(aq, pops[pk[0]][1], out=c)
    pcms, _ = timed(torch, "prefill_cold", prefill_cold, 3 * max(1, reps // 3))
    del pops
    qms, _ = timed(torch, "prefill_q", lambda: mx.quantize(ad, mx.MX_E4M3, out=aq), reps)
    mms, _ = timed(torch, "prefill_mm", lambda: mx.block_matmul(aq, btt, out=c), reps)
    progress(f"prefill linear done: {ms:.3f} ms")
    flops = 2 * 2048 * 28672 * 8192
    tf = flops / (ms * 1e-3) / 1e12
    tfm = flops / (mms * 1e-3) / 1e12
    out["prefill_e4m3xe2m1_2048x28672x8192"] = {
        "ms": round(ms, 4), "min_ms": round(mn, 4), "tflops": round(tf, 1),
        "quantize_ms": round(qms, 4), "matmul_ms": round(mms, 4),
        "cold_operands": {"ms": round(pcms, 4), "tflops": round(flops / (pcms * 1e-3) / 1e12, 1),
                          "what": "each call reads one of 3 copies of activations and weight "
                                  "(567 MB, beyond the Infinity Cache)"},
        "roofline": {"bound": "mfma", "kernel": "block_matmul", "achieved": round(tfm, 1),
                     "peak": PEAK_TFLOPS["fp8"], "unit": "TFLOP/s",
                     "frac": round(tfm / PEAK_TFLOPS["fp8"], 4)}}
    # the same product with the activation quantize inside the matmul
    # (mx_block_matmul_quantize_a): one launch, no quantized A in memory, but
    # A re-read and re-quantized for every 256-column tile of C
    fms, fmn = timed(torch, "prefill_fused",
                     lambda: mx.block_matmul_quantize_a(ad, mx.MX_E4M3, btt, out=c), reps)
    progress(f"prefill linear, fused quantize: {fms:.3f} ms")
    ftf = flops / (fms * 1e-3) / 1e12
    out["prefill_fused_quantize_e4m3xe2m1_2048x28672x8192"] = {
        "ms": round(fms, 4), "min_ms": round(fmn, 4), "tflops": round(ftf, 1),
        "vs_two_launches": round(ms / fms, 3),
        "a_reads": "A (64 MiB f32) read and quantized once per 256-column tile of C: 112 times",
        "roofline": {"bound": "mfma", "kernel": "block_matmul_quant_a", "achieved": round(ftf, 1),
                     "peak": PEAK_TFLOPS["fp8"], "unit": "TFLOP/s",
                     "frac": round(ftf / PEAK_TFLOPS["fp8"], 4)}}
    if ref:
        prefill()
        r, k = ref["rows"]["prefill"]
        torch.cuda.synchronize()
        attach("prefill_e4m3xe2m1_2048x28672x8192", c.cpu().numpy()[np.ix_(r, k)])
    del ad, btt, aq, c
    torch.cuda.empty_cache()
    return out


def bench_copy(torch, reps):
    """Achievable-HBM context: a plain device-to-device copy of 1 GiB (read
    1 GiB, write 1 GiB), two alternating buffer pairs so that no copy reads
    what the previous one left in the 256 MiB Infinity Cache."""
    n = 256 * 1024 * 1024
    src = [torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0) for _ in range(2)]
    dst = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(2)]
    k = [0]

    def one():
        k[0] += 1
        dst[k[0] & 1].copy_(src[k[0] & 1])
    ms, mn = timed(torch, "copy", one, reps)
    byts = 2 * 4 * n
    gbs = byts / (ms * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"ms": round(ms, 4), "min_ms": round(mn, 4), "bytes": byts, "achieved": round(gbs, 1),
            "unit": "GB/s", "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "what": "torch device-to-device copy of 1 GiB (read + write), the achievable-HBM "
                    "context for the codec kernels' fractions"}


# --------------------------------------------------------------------------
# CPU side: the oracle, timed on the host's cores, and the references the
# bench line's parity entries are checked against.  All of it runs before
# the GPU is first touched, so the worker pool forks a process that holds no
# GPU state.
# --------------------------------------------------------------------------
_POOL_X = {}


def _oracle_quantize_rows(job):
    """Worker: oracle quantize (and optionally dequantize) of rows [r0, r1)
    of the array registered under `name` before the pool forked."""
    from oracle import mx_oracle as O
    name, r0, r1, elem, dequant, keep = job
    x = _POOL_X[name][r0:r1]
    c, s = O.quantize(x, elem)
    y = O.dequantize(c, s, elem, x.shape[1]) if dequant else None
    return (c, s, y) if keep else None


def _row_jobs(name, rows, elem, parts, dequant=False, keep=True):
    step = max(1, -(-rows // parts))
    return [(name, r, min(rows, r + step), elem, dequant, keep) for r in range(0, rows, step)]


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((d.get("num_threads") or 0) for d in threadpool_info()
                   if d.get("user_api") == "blas") or None
    except Exception:
        return None


def _time_matmul_oracle(O, args, min_seconds):
    """The oracle's block_matmul, repeated for at least min_seconds; returns
    (seconds per call, C, sum|ab|)."""
    t0 = time.perf_counter()
    n = 0
    while True:
        c, mag = O.block_matmul(*args)
        n += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            return dt / n, c, mag


def cpu_phase(W, codec_seconds=10.0, matmul_seconds=2.0):
    """Oracle timings and parity references.

    * Codec: whole quantize + dequantize passes of the 8192x8192 weight
      workload, rows split over one worker process per available core (at
      most 16, the CPU share of one GPU on the benchmark hosts), repeated for
      at least codec_seconds.  The first pass is kept as the bit-exact
      reference of the GPU step.
    * Matmuls: the operands are quantized by the oracle (in the same pool) --
      in full for the decode product, on a stated row sample of A and of B^T
      for the MXFP8 and prefill products -- and the oracle's block_matmul
      (float64 BLAS) is timed on them; its result is the reference of the
      same outputs of the GPU product."""
    import multiprocessing
    from oracle import mx_oracle as O
    avail = len(os.sched_getaffinity(0))
    workers = max(1, min(avail, 16))
    info = {"os_cpu_count": os.cpu_count(), "affinity_cores": avail, "workers": workers,
            "cpu_model": _cpu_model()}
    ref = {"info": info}
    x = W.weight_codec_case(8192, 8192, seed=1002)
    a3, bt3 = W.decode_matmul_case()
    a4, bt4 = W.square_fp8_case()
    a5, bt5 = W.prefill_linear_case()
    rs = np.random.default_rng(7)
    r4 = np.sort(rs.choice(8192, 512, replace=False)); c4 = np.sort(rs.choice(8192, 512, replace=False))
    r5 = np.sort(rs.choice(2048, 256, replace=False)); c5 = np.sort(rs.choice(28672, 1024, replace=False))
    _POOL_X.update(codec=x, a3=a3, bt3=bt3, a4=a4[r4], bt4=bt4[c4], a5=a5[r5], bt5=bt5[c5])
    del a4, bt4, bt5
    ctx = multiprocessing.get_context("fork")
    with ctx.Pool(workers) as pool:
        progress(f"CPU oracle: codec passes on {workers} worker processes")
        jobs = _row_jobs("codec", 8192, O.E2M1, workers * 4, dequant=True)
        t0 = time.perf_counter()
        first = pool.map(_oracle_quantize_rows, jobs)
        passes = 1
        while time.perf_counter() - t0 < codec_seconds:
            pool.map(_oracle_quantize_rows, [j[:5] + (False,) for j in jobs])
            passes += 1
        dt = time.perf_counter() - t0
        ref["codec"] = tuple(np.concatenate([f[i] for f in first]) for i in range(3))
        del first
        gbs = passes * 2 * codec_bytes(8192, 8192, 0.5) / dt / 1e9
        ref["cpu_baseline"] = {
            "value": round(gbs, 4), "unit": "GB/s", "cores": workers, "kind": "oracle",
            "sample": f"{passes} whole quantize + dequantize passes over the 8192x8192 MXFP4 "
                      f"weight workload, rows split over {workers} worker processes "
                      f"(one per available core, at most 16), {dt:.1f} s",
            **info}
        progress("CPU oracle: quantizing the matmul operands")
        q = {}
        for name, rows, elem in (("a3", 16, O.E2M1), ("bt3", 4096, O.E2M1), ("a4", 512, O.E4M3),
                                 ("bt4", 512, O.E4M3), ("a5", 256, O.E4M3), ("bt5", 1024, O.E2M1)):
            res = pool.map(_oracle_quantize_rows, _row_jobs(name, rows, elem, workers))
            q[name] = (np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res]))
    _POOL_X.clear()
    blas = _blas_threads()
    mm = {}
    for key, (an, bn, ae, be, K, what) in {
            "decode_mxfp4_16x4096x4096": ("a3", "bt3", O.E2M1, O.E2M1, 4096, "every output"),
            "mxfp8_8192x8192x8192": ("a4", "bt4", O.E4M3, O.E4M3, 8192,
                                     "512 sampled rows of A x 512 sampled rows of B^T"),
            "prefill_e4m3xe2m1_2048x28672x8192": ("a5", "bt5", O.E4M3, O.E2M1, 8192,
                                                  "256 sampled rows of A x 1024 sampled rows of B^T")
    }.items():
        (ac, asc), (bc, bsc) = q[an], q[bn]
        m, n = asc.shape[0], bsc.shape[0]
        sec, c, mag = _time_matmul_oracle(O, (ac, asc, ae, bc, bsc, be, m, n, K), matmul_seconds)
        flops = 2 * m * n * K
        mm[key] = {"cpu_oracle": {"ms": round(sec * 1e3, 3), "tflops": round(flops / sec / 1e12, 4),
                                  "blas_threads": blas, "kind": "oracle (float64 BLAS)",
                                  "sample": what}, "ref": (c, mag)}
    ref["matmul"] = mm
    ref["rows"] = {"mxfp8": (r4, c4), "prefill": (r5, c5)}
    progress("CPU oracle done")
    return ref


def t1_parity(got, want, mag):
    """Worst |gpu - oracle| / (1e-5 sum|ab|) over the outputs, and whether
    every output is within the stated tolerance (NaN positions equal)."""
    got = got.astype(np.float64)
    nan_ok = bool(np.array_equal(np.isnan(got), np.isnan(want)))
    ok = ~np.isnan(want)
    err = np.abs(got[ok] - want[ok].astype(np.float64))
    bound = 1e-5 * mag[ok]
    ratio = float(np.max(err / np.where(bound > 0, bound, 1.0))) if err.size else 0.0
    within = nan_ok and bool(np.all(err <= bound))
    return {"outputs": int(got.size), "worst_err_over_tolerance": round(ratio, 5),
            "within_tolerance": within}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-matmul", action="store_true", help="time the codec step only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-codec", action="store_true",
                    help="skip the codec step (profiling the matmul workloads alone)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run plain 1 GiB device-to-device copies up front (the size of "
                         "the copy-context part), the reference that scales the FETCH_SIZE / "
                         "WRITE_SIZE counters of a --pmc run")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the MX hot path is "
              "measured on a single GPU", file=sys.stderr)
        sys.exit(2)

    from bit_gemm_mx_amd import workloads as W
    # The oracle runs first, on the host, before anything touches the GPU.
    ref = None if args.no_cpu else cpu_phase(W)

    import torch
    import bit_gemm_mx_amd as mx

    if not os.path.exists(mx.binding.LIB_PATH):
        from bit_gemm_mx_amd.build import build
        build()
    mx.lib()
    if not torch.cuda.is_available():
        raise RuntimeError("no GPU visible: bench.py measures the HIP path only")
    torch.cuda.set_device(0)

    if args.copy_calibration:
        src = torch.empty(256 * 1024 * 1024, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.no_codec:
        parts = bench_matmuls(mx, W, torch, max(3, args.steps // 2), ref)
        print(json.dumps({"metric": METRIC, "parts": parts, "note": "matmul workloads only"}))
        return
    progress("codec step: quantize + dequantize of the 8192x8192 weight workload")
    wall, step_bytes, kernels, codec_parity = bench_codec(mx, W, torch, args.steps, args.warmup,
                                                          ref["codec"] if ref else None)
    progress(f"codec step done: {wall / args.steps * 1e3:.3f} ms/step")
    ms_step = wall / args.steps * 1e3
    value = step_bytes / (wall / args.steps) / 1e9
    rooflines = {k: roofline_hbm(k, v) for k, v in kernels.items()}
    dominant = max(kernels, key=lambda k: kernels[k]["ms"])
    parts = {"codec_kernels": rooflines}
    if not args.no_matmul:
        parts.update(bench_matmuls(mx, W, torch, max(3, args.steps // 2), ref))
        parts.update(bench_f32b(mx, W, torch, max(3, args.steps // 2)))
    parts.update(bench_axis0_fold(mx, W, torch, max(3, args.steps // 2)))
    parts.update(bench_roundtrip(mx, W, torch, max(3, args.steps // 2)))
    parts["hbm_copy_context"] = bench_copy(torch, 5)
    progress("copy context done")
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "MXFP4 weight quantize + dequantize, fp32 8192x8192, "
                               "N(0,0.02) with 0.1% outliers x50, blocks of 32 along the last axis",
                   "rows": 8192, "cols": 8192, "elem": "E2M1", "block_size": 32, "seed": 1002,
                   "step": "mx_quantize then mx_dequantize"},
        "roofline": rooflines[dominant],
        "parity": codec_parity,
        "parts": parts,
    }
    if ref:
        line["cpu_baseline"] = ref["cpu_baseline"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
