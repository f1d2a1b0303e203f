"""Benchmark of the fused quantized linear layer on one MI355X.

Headline workload: W8A8 per-channel, N=10240, K=2560, M=4096 tokens (the
operator sweep's [N=10240, K=2560] shape of the Cider pages, at M=4096).
One step = the whole layer on fp16 activations already resident in HBM:
per-token quantization (cider_quantize_act) followed by the int8 matrix-core
product with fused dequantization (cider_w8a8_gemm) -- exactly what
cider_w8a8_linear runs, issued as its two calls so the product kernel can be
timed on its own with HIP events recorded on the launch stream.

`value` is INT8 TOPS of the whole step (2*M*N*K / step time, steps back to
back).  The JSON line also carries: the roofline of the product kernel
(achieved TOPS from its average launch duration -- HIP events on the launch
stream around each product launch of the timed steps -- against the
5.0 POPS dense INT8 peak, and its HBM bytes per launch from the committed
counter summary), the
oracle's CPU throughput on a bounded sample of the same workload, the
one-token path's GB/s against 8 TB/s, and a sweep over the operator
workloads.  Inputs are rotated over >= 1 GB of copies so that the 256 MB
last-level cache cannot serve them.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-sweep]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0      # MI355X dense INT8 matrix throughput, TOP/s
PEAK_HBM_GBPS = 8000.0       # MI355X HBM3E bandwidth, GB/s
ROTATE_BYTES = 1 << 30       # working-set copies cycled through per step
WARMUP_MIN_S = 0.25          # least time of sustained load before the timed steps
PAGES_M5PRO_PC_M4096_MS = 4.41  # the pages' per-channel latency at M=4096, [10240 x 2560], Apple M5 Pro


def log(msg):
    sys.stderr.write("[bench] %s\n" % msg)
    sys.stderr.flush()


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=600)
    p.add_argument("--no-sweep", action="store_true")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--no-m1", action="store_true")
    p.add_argument("--no-stack", action="store_true")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device-to-device copy 5 times (the known-size "
                        "reference for the HBM byte counters)")
    p.add_argument("--profile", metavar="WORKLOAD[:GS]:M", default=None,
                   help="only run one operator workload (e.g. w8a8_pc:4096, w8a8_pg:64:1024) for "
                        "a profiler: 30 launches of the product kernel, then 30 of the whole "
                        "layer, over rotating copies")
    return p.parse_args()


class Layer:
    """Device buffers for one (mode, N, K, M) workload, `copies` times over."""

    def __init__(self, torch, cider, bits, gs, N, K, M, x_np, w_np, copies):
        self.torch, self.cider = torch, cider
        self.bits, self.gs, self.N, self.K, self.M = bits, gs, N, K, M
        dev = "cuda"
        x = torch.from_numpy(x_np.view("int16")).to(dev).view(torch.float16)
        w = torch.from_numpy(w_np.view("int16")).to(dev).view(torch.float16)
        G = 1 if gs == 0 else K // gs
        self.sets = []
        for _ in range(copies):
            wq = torch.empty((N, K) if bits == 8 else (N, K // 2),
                             dtype=torch.int8 if bits == 8 else torch.uint8, device=dev)
            sw = torch.empty((N,) if gs == 0 else (N, G), dtype=torch.float32, device=dev)
            cider.cider_quantize_weight(w, N, K, bits, gs, wq, sw)
            self.sets.append(dict(
                x=x.clone(), wq=wq, sw=sw,
                xq=torch.empty((M, K), dtype=torch.int8, device=dev),
                st=torch.empty((M,), dtype=torch.float32, device=dev),
                y=torch.empty((M, N), dtype=torch.float16, device=dev)))
        del x, w
        # one workspace for every copy (calls are ordered on one stream), large
        # enough for the split-K product where the shape uses it
        self.ws_bytes = cider.cider_linear_workspace_bytes_ex(M, N, K, bits, gs)
        self.ws = torch.empty((max(self.ws_bytes, 16),), dtype=torch.uint8, device=dev)
        # every copy's int8 activations and scales hold the quantized tokens,
        # so the product alone is timed on real data (the linear calls
        # quantize into the workspace instead)
        for i in range(copies):
            self.quantize(i)

    def quantize(self, i):
        s = self.sets[i % len(self.sets)]
        self.cider.cider_quantize_act(s["x"], self.M, self.K, self.K, s["xq"], s["st"])

    def gemm(self, i):
        s = self.sets[i % len(self.sets)]
        f = self.cider.cider_w8a8_gemm if self.bits == 8 else self.cider.cider_w4a8_gemm
        f(s["xq"], s["st"], s["wq"], s["sw"], self.M, self.N, self.K, self.gs, s["y"])

    def linear(self, i):
        """The whole layer through the linear entry point (M = 1: quantization
        fused into the one-token kernel, no workspace; up to 128 tokens: the
        split-K product where the shape uses it)."""
        s = self.sets[i % len(self.sets)]
        f = self.cider.cider_w8a8_linear if self.bits == 8 else self.cider.cider_w4a8_linear
        if self.M == 1:
            f(s["x"], 1, self.K, self.K, s["wq"], s["sw"], self.N, self.gs, None, 0, s["y"])
        else:
            f(s["x"], self.M, self.K, self.K, s["wq"], s["sw"], self.N, self.gs, self.ws,
              self.ws_bytes, s["y"])


class LaunchEvents:
    """HIP timing events made with hipEventDisableSystemFence, recorded on a
    given stream through the HIP runtime torch already loaded.

    A default timing event (torch.cuda.Event) ends with a system-scope
    release and makes the next dispatch acquire at system scope, which opens
    a gap of a few microseconds before the kernel after it; that gap falls
    inside the bracket of the kernel being timed.  These events only order
    and time work on the device, so a bracket around one launch comes within
    about 1% of the kernel's own duration in a kernel trace."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n):
        import ctypes
        self._c = ctypes
        hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch loaded (same soname)
        hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                            ctypes.c_void_p]
        hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._hip = hip
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE)
            if rc != 0:
                self.close()
                raise RuntimeError("hipEventCreateWithFlags failed (%d)" % rc)
            self.ev.append(e)

    def record(self, i, stream):
        rc = self._hip.hipEventRecord(self.ev[i], self._c.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError("hipEventRecord failed (%d)" % rc)

    def ms(self, i, j):
        """Milliseconds from event i to event j (both complete)."""
        f = self._c.c_float()
        rc = self._hip.hipEventElapsedTime(self._c.byref(f), self.ev[i], self.ev[j])
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed (%d)" % rc)
        return f.value

    def close(self):
        for e in self.ev:
            self._hip.hipEventDestroy(e)
        self.ev = []


def alg_bytes(bits, gs, N, K, M):
    """Bytes the layer must move: X fp16 read once, weight codes, weight
    scales, token scales, Y fp16 written once."""
    G = 1 if gs == 0 else K // gs
    wbytes = N * K if bits == 8 else N * K // 2
    return 2 * M * K + wbytes + 4 * N * G + 4 * M + 2 * M * N


def copies_for(bits, gs, N, K, M):
    per = alg_bytes(bits, gs, N, K, M) + M * K
    return max(1, min(64, math.ceil(ROTATE_BYTES / per)))


def graph_time(torch, fn, n, replays):
    """Average time per call of fn(0..n-1) captured once into a HIP graph and
    replayed `replays` times back to back (events around the replays on the
    capture stream): the device-side rate of back-to-back launches, without
    the host's per-call launch cost.  Returns seconds per call."""
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for i in range(n):          # warm (and leaves every buffer touched)
            fn(i)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                fn(i)
        g.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(replays):
            g.replay()
        b.record(stream)
    b.synchronize()
    torch.cuda.current_stream().wait_stream(stream)
    return a.elapsed_time(b) / 1e3 / (n * replays)


def traffic_record(kernel_source, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(workload)
    if not rec:
        return None
    with open(kernel_source, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    if rec.get("source_sha256") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(M, N, K, x_np, w_np, budget_s):
    """The oracle (as it stands) on the first rows of the same workload:
    quantize_act + int8 product + dequant per row, timed on the host cores."""
    from oracle.oracle import get as get_oracle
    orc = get_oracle()
    wq, sw = orc.quantize_weight(w_np, 8, 0)
    t0 = time.perf_counter()
    orc.linear(x_np[:1], wq, sw)
    per_row = time.perf_counter() - t0
    threads = orc.num_threads()  # rows are split across these OpenMP threads
    rows = int(max(1, min(M, budget_s * threads / max(per_row, 1e-6))))
    t0 = time.perf_counter()
    orc.linear(x_np[:rows], wq, sw)
    dt = time.perf_counter() - t0
    return {"value": round(2.0 * rows * N * K / dt / 1e12, 6), "unit": "TOP/s",
            "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
            "host_logical_cpus": os.cpu_count(),
            "sample": "first %d of %d tokens of W8A8 per-channel N=%d K=%d: quantize_act + "
                      "int8 product + dequant, %.2f s wall" % (rows, M, N, K, dt)}


# The operator configurations: (name, weight bits, group size, N, K).
CONFIGS = [("w8a8_pc_small", 8, 0, 512, 1024), ("w8a8_pc", 8, 0, 10240, 2560),
           ("w8a8_pg64", 8, 64, 2560, 10240), ("w8a8_pg128", 8, 128, 2560, 10240),
           ("w4a8_pc", 4, 0, 10240, 2560)]


def oracle_times(si, budget_s=3.0, M_full=4096):
    """The oracle's host time per configuration, split into its steps:
    quantize_act, then the integer product and the dequant.  The small
    configuration (M=64) runs whole, also on one thread; the operator shapes
    run the first rows that fit about budget_s and are also given per token
    and scaled to M_full tokens (the oracle's rows are independent, so its
    time is linear in M)."""
    from oracle.oracle import get as get_oracle
    orc = get_oracle()
    threads = orc.num_threads()
    out = []
    for name, bits, gs, N, K in CONFIGS:
        small = name == "w8a8_pc_small"
        w = si.weights(N, K)
        wq, sw = orc.quantize_weight(w, bits, gs)
        x = si.activations(64 if small else 8, K)
        t0 = time.perf_counter()
        orc.dequant(orc.gemm_acc(orc.quantize_act(x)[0], wq, bits, gs), np.ones(len(x), np.float32), sw)
        per_row = (time.perf_counter() - t0) / len(x)
        rows = 64 if small else int(max(8, min(M_full, budget_s / max(per_row, 1e-9))))
        x = si.activations(rows, K)

        def run():
            t0 = time.perf_counter()
            xq, st = orc.quantize_act(x)
            t1 = time.perf_counter()
            acc = orc.gemm_acc(xq, wq, bits, gs)
            orc.dequant(acc, st, sw)
            t2 = time.perf_counter()
            return t1 - t0, t2 - t1

        tq, tg = run()
        rec = {"config": name, "weight_bits": bits, "group_size": gs, "N": N, "K": K,
               "tokens": rows, "threads": threads,
               "quantize_act_s": round(tq, 5), "gemm_dequant_s": round(tg, 5),
               "total_s": round(tq + tg, 5)}
        if small:
            orc.set_num_threads(1)
            try:
                tq1, tg1 = run()
            finally:
                orc.set_num_threads(threads)
            rec.update({"single_thread_quantize_act_s": round(tq1, 5),
                        "single_thread_gemm_dequant_s": round(tg1, 5),
                        "single_thread_total_s": round(tq1 + tg1, 5)})
        else:
            f = M_full / rows
            rec.update({"per_token_us": round((tq + tg) / rows * 1e6, 2),
                        "scaled_to_M%d_s" % M_full: {"quantize_act": round(tq * f, 3),
                                                     "gemm_dequant": round(tg * f, 3),
                                                     "total": round((tq + tg) * f, 3)}})
        log("oracle %s: %d tokens, quantize_act %.3f s, gemm+dequant %.3f s" % (name, rows, tq, tg))
        out.append(rec)
    return out


# Cosine of the layer's output against the fp16 product, as measured on the
# same inputs in numpy (64 tokens, seed 0) when the scheme was surveyed: what
# a correct implementation of this quantization gives on these inputs.
QUALITY_EXPECTED = {"w8a8_pc_small": 0.99914, "w8a8_pc": 0.99892, "w8a8_pg64": 0.99834,
                    "w8a8_pg128": 0.99834, "w4a8_pc": 0.98753}


def quality_report(torch, cider, si, M=64):
    """Quality of the quantized layer per configuration: the first M tokens
    through the linear call (weights quantized on the device) against the
    fp16 product x @ w^T evaluated in float64 on the host: cosine and
    relative Frobenius error.  A property of the quantization scheme on these
    inputs (the outlier columns widen the token scales), reported, not a
    pass / fail gate."""
    out = []
    for name, bits, gs, N, K in CONFIGS:
        x = si.activations(M, K)
        w = si.weights(N, K)
        xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.float16)
        wd = torch.from_numpy(w.view(np.int16)).cuda().view(torch.float16)
        wq = torch.empty((N, K) if bits == 8 else (N, K // 2),
                         dtype=torch.int8 if bits == 8 else torch.uint8, device="cuda")
        sw = torch.empty((N,) if gs == 0 else (N, K // gs), dtype=torch.float32, device="cuda")
        cider.cider_quantize_weight(wd, N, K, bits, gs, wq, sw)
        ws_bytes = cider.cider_linear_workspace_bytes_ex(M, N, K, bits, gs)
        ws = torch.empty((max(ws_bytes, 16),), dtype=torch.uint8, device="cuda")
        y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        f = cider.cider_w8a8_linear if bits == 8 else cider.cider_w4a8_linear
        f(xd, M, K, K, wq, sw, N, gs, ws, ws_bytes, y)
        yh = y.view(torch.int16).cpu().numpy().view(np.float16).astype(np.float64)
        ref = x.astype(np.float64) @ w.astype(np.float64).T
        cos = float((yh * ref).sum() / np.sqrt((yh * yh).sum() * (ref * ref).sum()))
        rel = float(np.linalg.norm(yh - ref) / np.linalg.norm(ref))
        rec = {"config": name, "tokens": M, "N": N, "K": K, "weight_bits": bits,
               "group_size": gs, "cosine": round(cos, 6), "rel_frobenius_error": round(rel, 6),
               "cosine_expected": QUALITY_EXPECTED[name]}
        log("quality %s: cosine %.5f (expected %.5f), relative error %.5f"
            % (name, cos, QUALITY_EXPECTED[name], rel))
        out.append(rec)
        del xd, wd, wq, sw, ws, y
    torch.cuda.empty_cache()
    return out


def weight_quant_bench(torch, cider, si, reps=20):
    """Offline weight quantization on the operator shapes: plain absmax and
    99.9th-percentile clipping, time per call (events around back-to-back
    calls) and the fp16 weight read rate."""
    records = []
    cases = [(10240, 2560, 8, 0), (10240, 2560, 4, 0), (2560, 10240, 8, 64),
             (2560, 10240, 8, 128), (2560, 10240, 4, 64), (2560, 10240, 4, 128)]
    stream = torch.cuda.current_stream()
    for N, K, bits, gs in cases:
        w = torch.from_numpy(si.weights(N, K).view("int16")).cuda().view(torch.float16)
        wq = torch.empty((N, K) if bits == 8 else (N, K // 2),
                         dtype=torch.int8 if bits == 8 else torch.uint8, device="cuda")
        sw = torch.empty((N,) if gs == 0 else (N, K // gs), dtype=torch.float32, device="cuda")
        rec = {"N": N, "K": K, "weight_bits": bits, "group_size": gs}
        for name, call in (("absmax", lambda: cider.cider_quantize_weight(w, N, K, bits, gs, wq, sw)),
                           ("clip_99.9", lambda: cider.cider_quantize_weight_clipped(
                               w, N, K, bits, gs, 99.9, wq, sw))):
            call()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                call()
            e1.record(stream)
            e1.synchronize()
            t = e0.elapsed_time(e1) / 1e3 / reps
            rec[name + "_us"] = round(t * 1e6, 2)
            rec[name + "_gbps"] = round(2.0 * N * K / t / 1e9, 1)
        log("weight quantize %dx%d bits=%d gs=%d: absmax %.1f us, clipped %.1f us"
            % (N, K, bits, gs, rec["absmax_us"], rec["clip_99.9_us"]))
        records.append(rec)
        del w, wq, sw
    torch.cuda.empty_cache()
    return records


def dtype_variants_bench(torch, cider, si, steps=50):
    """The headline layer (W8A8 per channel, N=10240, K=2560, M=4096) for
    each input / output type with and without SmoothQuant smoothing: time per
    cider_linear_ex call, calls back to back over rotating copies."""
    M, N, K = 4096, 10240, 2560
    x32 = si.activations(M, K).astype(np.float32)
    x16 = torch.from_numpy(x32.astype(np.float16).view(np.int16)).cuda()
    xbf = torch.from_numpy(x32).cuda().to(torch.bfloat16).view(torch.int16)
    w = torch.from_numpy(si.weights(N, K).view(np.int16)).cuda().view(torch.float16)
    wq = torch.empty((N, K), dtype=torch.int8, device="cuda")
    sw = torch.empty((N,), dtype=torch.float32, device="cuda")
    cider.cider_quantize_weight(w, N, K, 8, 0, wq, sw)
    sm = torch.from_numpy(np.random.default_rng(5).uniform(0.5, 8.0, K).astype(np.float32)).cuda()
    B = copies_for(8, 0, N, K, M)
    xs = {0: [x16.clone() for _ in range(B)], 1: [xbf.clone() for _ in range(B)]}
    ys = [torch.empty((M, N), dtype=torch.int16, device="cuda") for _ in range(B)]
    ws_bytes = cider.cider_linear_workspace_bytes(M, K)
    ws = torch.empty((ws_bytes,), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    records = []
    for x_dt, y_dt, smooth in ((0, 0, False), (1, 1, False), (0, 0, True), (1, 1, True)):
        def call(i):
            cider.cider_linear_ex(xs[x_dt][i % B], x_dt, M, K, K, sm if smooth else None, wq, sw,
                                  N, 8, 0, y_dt, ws, ws_bytes, ys[i % B])
        # the same time-based warm-up as the headline: the first variant
        # would otherwise run on clocks still ramping up
        t0 = time.perf_counter()
        i = 0
        while i < 5 or time.perf_counter() - t0 < WARMUP_MIN_S:
            call(i)
            i += 1
            if i % 32 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            call(i)
        e1.record(stream)
        e1.synchronize()
        t = e0.elapsed_time(e1) / 1e3 / steps
        rec = {"x": ("fp16", "bf16")[x_dt], "y": ("fp16", "bf16")[y_dt], "smoothing": smooth,
               "us_per_call": round(t * 1e6, 2), "tops": round(2.0 * M * N * K / t / 1e12, 1)}
        records.append(rec)
        log("linear_ex x=%s y=%s smoothing=%s: %.2f us" % (rec["x"], rec["y"], smooth, t * 1e6))
    del xs, ys, ws, wq, sw, w
    torch.cuda.empty_cache()
    return records


def decode_bench(torch, cider, si):
    """The pages' decode variant (dequantized weights, no activation
    quantization) on the one-token operator shapes: time per call (HIP graph
    of back-to-back calls over rotating copies) and the algorithmic bytes
    (x, weight codes, scales, y) per second against 8 TB/s."""
    records = []
    for name, bits, gs, N, K in (("w8a16_pc", 8, 0, 10240, 2560), ("w4a16_pc", 4, 0, 10240, 2560),
                                 ("w8a16_pg64", 8, 64, 2560, 10240), ("w8a16_pg128", 8, 128, 2560, 10240),
                                 ("w4a16_pg64", 4, 64, 2560, 10240), ("w4a16_pg128", 4, 128, 2560, 10240)):
        x = torch.from_numpy(si.activations(1, K)[0].view(np.int16)).cuda().view(torch.float16)
        w = torch.from_numpy(si.weights(N, K).view(np.int16)).cuda().view(torch.float16)
        G = 1 if gs == 0 else K // gs
        B = copies_for(bits, gs, N, K, 1)
        sets = []
        for _ in range(B):
            wq = torch.empty((N, K) if bits == 8 else (N, K // 2),
                             dtype=torch.int8 if bits == 8 else torch.uint8, device="cuda")
            sw = torch.empty((N,) if gs == 0 else (N, G), dtype=torch.float32, device="cuda")
            cider.cider_quantize_weight(w, N, K, bits, gs, wq, sw)
            sets.append((x.clone(), wq, sw, torch.empty((N,), dtype=torch.float16, device="cuda")))

        def call(i):
            xx, wq, sw, y = sets[i % B]
            cider.cider_decode_linear(xx, K, wq, sw, N, bits, gs, 0, y)
        t = graph_time(torch, call, B, max(1, 4000 // B))
        nbytes = 2 * K + (N * K if bits == 8 else N * K // 2) + 4 * N * G + 2 * N
        rec = {"workload": name, "N": N, "K": K, "us_per_call": round(t * 1e6, 3),
               "gbps": round(nbytes / t / 1e9, 1), "frac_hbm": round(nbytes / t / 1e9 / PEAK_HBM_GBPS, 4)}
        records.append(rec)
        log("decode %s N=%d K=%d: %.2f us, %.0f GB/s" % (name, N, K, t * 1e6, nbytes / t / 1e9))
        del sets, x, w
        torch.cuda.empty_cache()
    return records


def small_m_bench(torch, cider, si):
    """Few tokens (M = 2 .. 64), the pages' small-tile regime: whole-layer
    time per call on each operator shape, through the automatic path and,
    where it applies (M <= 8, M * K <= 65536), forced onto the matrix-vector
    kernel."""
    records = []
    for name, wl in si.WORKLOADS.items():
        if name == "w8a8_pc_small":
            continue
        Nw, Kw = wl["N"], wl["K"]
        xs = si.activations(64, Kw)
        ws = si.weights(Nw, Kw)
        for gs in wl["group_sizes"]:
            for Mw in (2, 4, 6, 8, 16, 32, 64):
                Bw = copies_for(wl["bits"], gs, Nw, Kw, Mw)
                Lw = Layer(torch, cider, wl["bits"], gs, Nw, Kw, Mw, xs[:Mw], ws, Bw)
                calls = max(Bw, 8)
                rec = {"workload": name, "group_size": gs, "M": Mw}
                paths = [("auto", cider.PATH_AUTO)]
                if Mw <= 8 and Mw * Kw <= 65536:
                    paths.append(("matrix_vector", cider.PATH_GEMV))
                for pname, path in paths:
                    cider.cider_set_path(path)
                    t = graph_time(torch, Lw.linear, calls, max(1, 400 // calls))
                    rec[pname + "_us"] = round(t * 1e6, 2)
                cider.cider_set_path(cider.PATH_AUTO)
                records.append(rec)
                log("small M %s gs=%d M=%d: %s" % (name, gs, Mw, ", ".join(
                    "%s %.2f us" % (k[:-3], v) for k, v in rec.items() if k.endswith("_us"))))
                del Lw
                torch.cuda.empty_cache()
    return records


class DecoderStack:
    """The layer at model scale: the four W8A8 per-channel linears of each of
    `layers` decoder layers of an 8B-class model (QKV 6144x4096, O 4096x4096,
    gate+up 24576x4096, down 4096x12288), chained at M tokens with no glue
    kernels -- O reads the first 4096 columns of the QKV output and down the
    first 12288 columns of the gate+up output, in place, through the
    activation row stride.  Weights are distinct per layer and GEMM, drawn on
    the host by the seeded generator (in parallel threads), quantized on the
    device, and only the int8 codes and fp32 scales stay resident (6.95 GB
    for 36 layers)."""

    def __init__(self, torch, cider, si, layers=None, M=None, keep_fp16=(), threads=16):
        from concurrent.futures import ThreadPoolExecutor
        self.torch, self.cider = torch, cider
        self.layers = si.DECODER_LAYERS if layers is None else layers
        self.M = si.DECODER_TOKENS if M is None else M
        self.shapes = [(N, K) for _, N, K in si.DECODER_LAYER]
        self.weights = [[None] * len(self.shapes) for _ in range(self.layers)]
        self.fp16 = {}  # (layer, j) -> host fp16 weights kept for a checker
        tasks = [(l, j) for l in range(self.layers) for j in range(len(self.shapes))]

        def draw(t):
            l, j = t
            N, K = self.shapes[j]
            return t, si.layer_weights(l, j, N, K)

        with ThreadPoolExecutor(threads) as ex:
            for c in range(0, len(tasks), threads):
                for (l, j), w in ex.map(draw, tasks[c:c + threads]):
                    N, K = self.shapes[j]
                    wd = torch.from_numpy(w.view("int16")).to("cuda").view(torch.float16)
                    wq = torch.empty((N, K), dtype=torch.int8, device="cuda")
                    sw = torch.empty((N,), dtype=torch.float32, device="cuda")
                    cider.cider_quantize_weight(wd, N, K, 8, 0, wq, sw)
                    self.weights[l][j] = (wq, sw)
                    if l in keep_fp16:
                        self.fp16[(l, j)] = w
                    del wd, w
        M = self.M
        kmax = max(K for _, K in self.shapes)
        self.ws_bytes = cider.cider_linear_workspace_bytes(M, kmax)
        self.ws = torch.empty((self.ws_bytes,), dtype=torch.uint8, device="cuda")
        dmodel = self.shapes[0][1]
        self.x = [torch.empty((M, dmodel), dtype=torch.float16, device="cuda") for _ in range(2)]
        self.y = [torch.empty((M, N), dtype=torch.float16, device="cuda") for N, _ in self.shapes[:3]]

    def _linear(self, x, ldx, K, l, j, y):
        wq, sw = self.weights[l][j]
        self.cider.cider_w8a8_linear(x, self.M, K, ldx, wq, sw, self.shapes[j][0], 0, self.ws,
                                     self.ws_bytes, y)

    def forward(self, x0, capture=()):
        """Runs every layer on x0 (fp16 [M, 4096]); returns the final
        activations and, for each layer in `capture`, host copies of its input
        and of its four GEMM outputs [input, qkv, o, gate_up, down]."""
        torch = self.torch
        (n_qkv, k_in), (n_o, k_o), (n_gu, _), (n_dn, k_dn) = self.shapes
        cur = x0
        caps = {}
        for l in range(self.layers):
            nxt = self.x[l % 2]
            y_qkv, y_o, y_gu = self.y
            self._linear(cur, k_in, k_in, l, 0, y_qkv)
            self._linear(y_qkv, n_qkv, k_o, l, 1, y_o)       # first 4096 columns of QKV
            self._linear(y_o, n_o, k_in, l, 2, y_gu)
            self._linear(y_gu, n_gu, k_dn, l, 3, nxt)        # first 12288 columns of gate+up
            if l in capture:  # cur (the layer input) is not overwritten by this layer
                caps[l] = [t.view(torch.int16).cpu().numpy().view("float16")
                           for t in (cur, y_qkv, y_o, y_gu, nxt)]
            cur = nxt
        return cur, caps

    def ops(self):
        return 2.0 * self.M * sum(N * K for N, K in self.shapes) * self.layers


def stack_bench(torch, cider, si, passes=3):
    """Time whole passes of the 36-layer stack (each GEMM = quantize_act +
    product, through cider_w8a8_linear)."""
    t0 = time.perf_counter()
    S = DecoderStack(torch, cider, si)
    setup_s = time.perf_counter() - t0
    x0 = torch.from_numpy(si.activations(S.M, S.shapes[0][1]).view("int16")).cuda().view(torch.float16)
    out, _ = S.forward(x0)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(passes):
        out, _ = S.forward(x0)
    e1.record(stream)
    e1.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / passes
    finite = bool(torch.isfinite(out).all().item())
    rec = {"workload": "8B-class decoder stack: 36 layers x (QKV 6144x4096, O 4096x4096, "
                       "gate+up 24576x4096, down 4096x12288), W8A8 per channel, M=4096",
           "ms_per_pass": round(t * 1e3, 3), "tops": round(S.ops() / t / 1e12, 1),
           "frac_mfma": round(S.ops() / t / 1e12 / PEAK_INT8_TOPS, 4),
           "passes": passes, "output_finite": finite,
           "weight_setup_s": round(setup_s, 1)}
    log("stack: %.3f ms per pass, %.0f TOPS (weights drawn and quantized in %.1f s)"
        % (t * 1e3, S.ops() / t / 1e12, setup_s))
    del S, x0, out
    torch.cuda.empty_cache()
    return rec


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this layer has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus)
        sys.exit(2)
    import torch

    import synth_inputs as si
    import w4a8_quantized_linear_amd as cider

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        log("copied 1 GiB 5 times")
        return
    cider.load(build_if_missing=True)
    assert cider.cider_is_available(), "libcider.so reports no usable gfx950 device"
    if args.profile:
        profile_workload(torch, cider, si, args.profile)
        return

    # ---------------------------------------------------------- headline ---
    M, N, K = 4096, 10240, 2560
    log("generating inputs M=%d N=%d K=%d" % (M, N, K))
    x_np = si.activations(M, K)
    w_np = si.weights(N, K)
    B = copies_for(8, 0, N, K, M)
    L = Layer(torch, cider, 8, 0, N, K, M, x_np, w_np, B)
    ops = 2.0 * M * N * K
    # warm-up: the requested steps, then more until the chip has run this
    # load for at least WARMUP_MIN_S (the clocks settle under sustained
    # matrix-core load; a few steps are not enough)
    t0 = time.perf_counter()
    i = 0
    while i < args.warmup or time.perf_counter() - t0 < WARMUP_MIN_S:
        L.quantize(i)
        L.gemm(i)
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    log("warm-up: %d steps in %.0f ms" % (i, (time.perf_counter() - t0) * 1e3))
    log("timing %d steps (%d rotating copies)" % (args.steps, B))
    stream = torch.cuda.current_stream()
    # The timed region: K whole steps back to back, host-timed between two
    # synchronizations -> value, ms_per_step.  Inside it, a HIP event on the
    # launch stream before each step's quantize launch and one between its
    # quantize and product launches: the product kernel's duration of step i
    # is the time from the second event of step i to the first of step i+1
    # (or the closing event), so both kernel averages come from the very
    # launches the step time covers and cannot exceed it.
    # Events 2i and 2i+1 precede step i's quantize and product launches;
    # event 2K closes the region.
    S = args.steps
    ev = LaunchEvents(2 * S + 1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(S):
        ev.record(2 * i, stream)
        L.quantize(i)
        ev.record(2 * i + 1, stream)
        L.gemm(i)
    ev.record(2 * S, stream)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_per_step = dt / S * 1e3
    value = ops / (dt / S) / 1e12
    gemm_ms = [ev.ms(2 * i + 1, 2 * i + 2) for i in range(S)]
    quant_ms = [ev.ms(2 * i, 2 * i + 1) for i in range(S)]
    device_ms = ev.ms(0, 2 * S)
    ev.close()
    gemm_s = sum(gemm_ms) / args.steps / 1e3
    quant_s = sum(quant_ms) / args.steps / 1e3
    assert gemm_s + quant_s <= dt / args.steps * 1.0001, (gemm_s, quant_s, dt / args.steps)
    achieved = ops / gemm_s / 1e12
    log("step %.2f us (device %.2f us), product kernel %.2f us (%.0f TOPS; median %.2f us), "
        "quantize kernel %.2f us"
        % (ms_per_step * 1e3, device_ms * 1e3 / args.steps, gemm_s * 1e6, achieved,
           sorted(gemm_ms)[args.steps // 2] * 1e3, quant_s * 1e6))
    traffic = traffic_record(os.path.join(ROOT, "w4a8_quantized_linear_amd", "csrc", "gemm.hip"),
                             "w8a8_pc_N10240_K2560_M4096")
    result = {
        "metric": "INT8 TOPS (% of MFMA peak) at M=4096; GB/s (% of HBM peak) at M=1",
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / (ops / (PAGES_M5PRO_PC_M4096_MS * 1e-3) / 1e12), 2),
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "W8A8 per-channel linear, N=10240 K=2560 M=4096 "
                               "(fp16 X ~N(0,1) with 1% outlier columns x20, W ~0.02*N(0,1), seed 0)",
                   "M": M, "N": N, "K": K, "group_size": 0, "weight_bits": 8,
                   "step": "cider_quantize_act + cider_w8a8_gemm",
                   "rotating_copies": B},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_INT8_TOPS,
                     "unit": "TOP/s", "frac": round(achieved / PEAK_INT8_TOPS, 4),
                     "traffic": traffic,
                     "kernel": "gemm_wide_kernel<320, 256, 160, 64, 8, 0> (int8 matrix-core product "
                               "+ dequant, per channel)",
                     "kernel_us": round(gemm_s * 1e6, 2),
                     "quantize_kernel_us": round(quant_s * 1e6, 2),
                     "timing": "HIP events without system-scope fences on the launch stream "
                               "around each launch of the timed steps (the same launches as "
                               "ms_per_step)"},
    }
    del L
    torch.cuda.empty_cache()

    # --------------------------------------------------------- one token ---
    if args.no_m1:
        result["m1"] = None
    else:
        one_token(torch, cider, x_np, w_np, N, K, result)

    # ------------------------------------------------------------- sweep ---
    if not args.no_sweep:
        result["sweep"] = sweep(torch, cider, si)

    # ------------------------------------------------- the decode variant ---
    if not args.no_sweep:
        result["decode"] = decode_bench(torch, cider, si)

    # ------------------------------------------------------ few tokens ---
    if not args.no_sweep:
        result["small_m"] = small_m_bench(torch, cider, si)

    # ------------------------------------ input / output types, smoothing ---
    if not args.no_sweep:
        result["dtype_variants"] = dtype_variants_bench(torch, cider, si)

    # ------------------------------------------- offline weight quantization ---
    if not args.no_sweep:
        result["weight_quantize"] = weight_quant_bench(torch, cider, si)

    # ------------------------------------------------------------- stack ---
    if not args.no_stack:
        result["stack"] = stack_bench(torch, cider, si)

    # --------------------------------------------------- quality report ---
    result["quality"] = quality_report(torch, cider, si)

    # -------------------------------------------------------- CPU oracle ---
    if not args.no_cpu:
        log("timing the oracle on the host")
        result["cpu_baseline"] = cpu_baseline(M, N, K, x_np, w_np, args.cpu_seconds)
        result["cpu_baseline"]["per_config"] = oracle_times(si)
    else:
        result["cpu_baseline"] = None

    print(json.dumps(result), flush=True)


def profile_workload(torch, cider, si, spec, launches=30):
    """One operator workload for a profiler's counters: its product kernel,
    then its whole layer (the linear call with the split workspace), each
    `launches` times back to back over rotating copies."""
    parts = spec.split(":")
    name, M = parts[0], int(parts[-1])
    wl = si.WORKLOADS[name]
    gs = int(parts[1]) if len(parts) == 3 else wl["group_sizes"][0]
    N, K, bits = wl["N"], wl["K"], wl["bits"]
    B = copies_for(bits, gs, N, K, M)
    L = Layer(torch, cider, bits, gs, N, K, M, si.activations(M, K), si.weights(N, K), B)
    torch.cuda.synchronize()
    log("profile %s gs=%d M=%d N=%d K=%d: %d product launches, %d layer launches"
        % (name, gs, M, N, K, launches, launches))
    for i in range(launches):
        L.gemm(i)
    torch.cuda.synchronize()
    for i in range(launches):
        L.linear(i)
    torch.cuda.synchronize()


def one_token(torch, cider, x_np, w_np, N, K, result):
    """The one-token path: quantization fused into the matrix-vector kernel."""
    x1 = x_np[:1]
    B1 = copies_for(8, 0, N, K, 1)
    L1 = Layer(torch, cider, 8, 0, N, K, 1, x1, w_np, B1)
    s1 = graph_time(torch, L1.linear, B1, max(1, 4000 // B1))
    b1 = alg_bytes(8, 0, N, K, 1)
    result["m1"] = {"workload": "W8A8 per-channel N=10240 K=2560 M=1, quantization fused",
                    "us_per_call": round(s1 * 1e6, 3), "bytes": b1,
                    "gbps": round(b1 / s1 / 1e9, 1),
                    "frac": round(b1 / s1 / 1e9 / PEAK_HBM_GBPS, 4),
                    "timing": "HIP graph of back-to-back calls over rotating copies; "
                              "includes the launch-to-launch gap",
                    "rotating_copies": B1}
    log("M=1: %.2f us per call, %.0f GB/s" % (s1 * 1e6, b1 / s1 / 1e9))
    del L1
    torch.cuda.empty_cache()


def sweep(torch, cider, si):
    """Every operator workload at every M: whole-layer and product-kernel
    time per call (graph replay over rotating copies)."""
    records = []
    for name, wl in si.WORKLOADS.items():
        if name == "w8a8_pc_small":
            continue
        Nw, Kw = wl["N"], wl["K"]
        xs = si.activations(max(wl["M"]), Kw)
        ws = si.weights(Nw, Kw)
        for gs in wl["group_sizes"]:
            for Mw in wl["M"]:
                Bw = copies_for(wl["bits"], gs, Nw, Kw, Mw)
                Lw = Layer(torch, cider, wl["bits"], gs, Nw, Kw, Mw, xs[:Mw], ws, Bw)
                calls = max(Bw, 8)
                replays = max(1, (200 if Mw <= 128 else 20) // calls)
                e2e = graph_time(torch, Lw.linear, calls, replays)
                gemm = graph_time(torch, Lw.gemm, calls, replays) if Mw > 1 else None
                ab = alg_bytes(wl["bits"], gs, Nw, Kw, Mw)
                opw = 2.0 * Mw * Nw * Kw
                rec = {"workload": name, "group_size": gs, "M": Mw, "N": Nw, "K": Kw,
                       "e2e_us": round(e2e * 1e6, 2),
                       "e2e_tops": round(opw / e2e / 1e12, 2),
                       "e2e_gbps": round(ab / e2e / 1e9, 1)}
                if gemm is not None:
                    rec.update({"gemm_us": round(gemm * 1e6, 2),
                                "gemm_tops": round(opw / gemm / 1e12, 2),
                                "gemm_frac_mfma": round(opw / gemm / 1e12 / PEAK_INT8_TOPS, 4)})
                rec["e2e_frac_hbm"] = round(ab / e2e / 1e9 / PEAK_HBM_GBPS, 4)
                records.append(rec)
                log("sweep %s gs=%d M=%d: e2e %.2f us (%.1f TOPS, %.0f GB/s)%s"
                    % (name, gs, Mw, e2e * 1e6, opw / e2e / 1e12, ab / e2e / 1e9,
                       "" if gemm is None else ", gemm %.2f us" % (gemm * 1e6)))
                del Lw
                torch.cuda.empty_cache()
        del xs, ws
    return records


if __name__ == "__main__":
    main()
