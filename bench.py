#!/usr/bin/env python3
"""Benchmark of the W4A16 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extra]
                    [--only decode|prefill|q4|sweep|zp|zp_prepared|w8|w4a8|w4a8_decode|w4a8_sweep]

A step is one w4a16_matmul call (dispatch by M -> GEMV or MFMA GEMM) over one batch of seeded
synthetic input, with packed weights, activations and output already resident in HBM.  The
headline workload is the decode GEMV on the Llama-3-8B up-projection shape (M=1, K=4096,
N=14336, group-128 asymmetric format); its value is effective weight bytes (codes + scales +
mins) per second over the wall time of the K timed steps.  To keep the 256 MB Infinity Cache
from serving the weights, the steps rotate over enough packed copies to exceed 512 MB.  The K
timed steps are captured once into a HIP graph (so host launch cost does not pace the GPU) and
replayed; the graph is first replayed untimed for WARM_SECONDS so that the GPU's clocks have
settled.

Kernel durations (the roofline and every secondary figure) follow vidyal.ai "Low-Precision
Kernels", "How the measurements were taken" (medians over many launches, three rounds, cold
cache): a HIP graph of at least 100 back-to-back launches rotating over the cold copies is
replayed three times, each replay bracketed by HIP events on the launch stream, and the median of
the three per-launch averages is reported with all three.  Beside each figure stand measured
roofs timed the same way: a plain streaming read of the same bytes and an empty launch
(libw4a16_roof.so), and for prefill hipBLASLt's bf16-weight GEMM of the same shape.

Prints ONE JSON line.  Secondary figures (prefill TFLOPS at M=1024 with a hipBLASLt bf16-weight
GEMM beside it, the Q4 block-32 GEMV, the decode shape in the zero-point and W8A16 formats, the batch
sweep, W4A8) go under "extra".
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
MFMA_I8_PEAK_TOPS = 5000.0     # MI355X dense int8 MFMA, TOP/s
CACHE_BYTES = 256 * 2 ** 20    # MI355X Infinity Cache (MALL)
WARM_SECONDS = 0.25            # untimed run-up of each workload before its timed replay
ROUNDS = 3                     # timed replays of a kernel's graph; the median is reported
MIN_LAUNCHES = 100             # launches per timed replay (rounded up to whole rotations)
METRIC = "W4A16 effective weight GB/s (% HBM peak) at M=1; TFLOPS (% MFMA) at M=1024"
DECODE_KERNEL = "skinny_g128_kernel<1, 4, 2, true, false, false, false>"
PREFILL_KERNEL = "gemm_g128_kernel<256, 224, 4, 1, 3, true, 1>"


def recorded_traffic(kernel: str):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled by a copy-kernel calibration) from
    the committed counter summary profiles/traffic.json -- or None if the kernel's source has
    changed since those counters were taken."""
    import hashlib
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))["kernels"][kernel]
        src = open(os.path.join(ROOT, rec["source"]), "rb").read()
    except (OSError, KeyError, ValueError):
        return None
    if hashlib.sha256(src).hexdigest() != rec["source_sha256"]:
        return None
    if rec.get("fetch_bytes") is None or rec.get("write_bytes") is None:
        return None
    return rec["fetch_bytes"] + rec["write_bytes"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1700)
    ap.add_argument("--warmup", type=int, default=170)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--only", choices=["decode", "prefill", "q4", "sweep", "zp", "zp_prepared", "w8", "w4a8",
                                       "w4a8_decode", "w4a8_sweep", "cpu", "rowfmt_sweep", "l2_patterns", "small_n"], default=None,
                    help="time one workload only (for profiler runs); prints its JSON line")
    ap.add_argument("--eager", action="store_true",
                    help="launch every step directly instead of replaying a HIP graph (counter runs)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also copy a buffer of this many MiB 5 times (a known-size reference kernel "
                         "for scaling hardware byte counters)")
    return ap.parse_args()


EAGER = False


class Setup:
    """Packed weight copies, activations and output for one workload, resident on the GPU."""

    def __init__(self, fmt, M, N, K, x_bits, W, copies):
        import torch
        import gemm_w4a16_amd as w
        self.w, self.fmt, self.M, self.N, self.K = w, fmt, M, N, K
        self.act = w.W4A16_BF16 if fmt == w.W4A16_FMT_G128_ASYM_BF16 else w.W4A16_FP16  # Q4, zero point: fp16
        Wd = torch.from_numpy(W).cuda()
        base = w.alloc_packed(fmt, N, K)
        w.w4a16_quantize_pack(fmt, Wd, N, K, *base)
        del Wd
        self.copies = [base] + [tuple(None if t is None else t.clone() for t in base) for _ in range(copies - 1)]
        self.x = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda()
        self.y = torch.empty((M, N), dtype=torch.int16, device="cuda")
        self.ws, self.ws_bytes = w.alloc_workspace(fmt, M, N, K)
        c, s, m = w.w4a16_packed_sizes(fmt, N, K)
        self.weight_bytes = c + s + m
        torch.cuda.synchronize()

    def step(self, i):
        c, s, m = self.copies[i % len(self.copies)]
        self.w.w4a16_matmul(self.fmt, self.act, self.x, self.M, c, s, m, self.N, self.K, self.y,
                            self.ws, self.ws_bytes)


def time_steps(setup: Setup, steps: int, warmup: int):
    """W eager warmup steps, then EXACTLY `steps` steps captured in one HIP graph and replayed
    once, bracketed by synchronize.  Returns (wall seconds, event seconds)."""
    import torch
    for i in range(warmup):
        setup.step(i)
    torch.cuda.synchronize()
    if EAGER:
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record()
        for i in range(steps):
            setup.step(i)
        end.record()
        torch.cuda.synchronize()
        return time.perf_counter() - t0, start.elapsed_time(end) / 1e3
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            setup.step(i)
    # untimed replays (the first uploads the graph) until the GPU has run this work for
    # WARM_SECONDS: its clocks settle over milliseconds, far longer than a short graph takes
    t_warm = time.perf_counter()
    while True:
        g.replay()
        torch.cuda.synchronize()
        if time.perf_counter() - t_warm >= WARM_SECONDS:
            break
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    g.replay()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, start.elapsed_time(end) / 1e3


def copies_for(weight_bytes: int) -> int:
    return max(1, math.ceil(2 * CACHE_BYTES / weight_bytes))


def time_rounds(step, copies: int, rounds: int = ROUNDS):
    """Per-launch duration of `step(i)` (i selects the weight copy i % copies): L >= MIN_LAUNCHES
    launches in one HIP graph, replayed untimed for WARM_SECONDS, then `rounds` replays each
    bracketed by HIP events on the launch stream.  Returns {"us": median of the rounds' per-launch
    averages, "rounds_us": [...], "launches_per_round": L}."""
    import torch
    L = copies * math.ceil(MIN_LAUNCHES / copies)
    for i in range(min(L, 2 * copies)):
        step(i)
    torch.cuda.synchronize()
    if EAGER:  # counter runs: direct launches, no graph
        per = []
        for _ in range(rounds):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(L):
                step(i)
            e1.record()
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) * 1e3 / L)
        return {"us": float(np.median(per)), "rounds_us": [round(v, 4) for v in per], "launches_per_round": L}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(L):
            step(i)
    t_warm = time.perf_counter()
    while True:
        g.replay()
        torch.cuda.synchronize()
        if time.perf_counter() - t_warm >= WARM_SECONDS:
            break
    per = []
    for _ in range(rounds):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) * 1e3 / L)
    del g
    return {"us": float(np.median(per)), "rounds_us": [round(v, 4) for v in per], "launches_per_round": L}


class Roofs:
    """The measured roofs of libw4a16_roof.so: a plain 16-byte non-temporal streaming read and an
    empty launch, timed like the kernels (graph, rotated cold copies, median of three rounds)."""

    def __init__(self):
        import ctypes
        import torch
        path = os.path.join(ROOT, "gemm_w4a16_amd", "libw4a16_roof.so")
        self.lib = ctypes.CDLL(path)
        self.lib.roof_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_void_p]
        self.lib.roof_empty.argtypes = [ctypes.c_void_p]
        self.lib.roof_shared_read.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_void_p, ctypes.c_void_p]
        self.lib.roof_copy_pipeline.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int] * 3 + [ctypes.c_void_p]
        self.sink = torch.zeros(1024, dtype=torch.int32, device="cuda")

    def _stream(self):
        import torch
        return torch.cuda.current_stream().cuda_stream

    def empty_launch_us(self):
        def step(i):
            assert self.lib.roof_empty(self._stream()) == 0
        return time_rounds(step, 1)["us"]

    def read(self, nbytes: int, copies: int):
        """Fastest of a few grid sizes for a cold read of `nbytes` per launch."""
        import torch
        bufs = [torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda") for _ in range(copies)]
        best = None
        one_pass = (nbytes // 16 + 1023) // 1024
        for blocks in (one_pass, 2048, 1024, 512):
            def step(i, blocks=blocks):
                assert self.lib.roof_read(bufs[i % copies].data_ptr(), nbytes, self.sink.data_ptr(), blocks,
                                          self._stream()) == 0
            r = time_rounds(step, copies)
            if best is None or r["us"] < best["us"]:
                best = dict(r, blocks=blocks)
        del bufs
        torch.cuda.empty_cache()
        best["gbs"] = nbytes / best["us"] / 1e3
        best["bytes"] = nbytes
        best["kernel"] = "roof_read_kernel (16-byte non-temporal loads, 4 in flight per lane)"
        return best


    def shared_read(self, M: int, K: int, blocks: int = 224):
        """Every one of `blocks` blocks reads all of one shared bf16 [M][K] (L2-resident after the
        first) in each wave-load shape: the per-CU rates behind the mid-M kernels' designs."""
        import torch
        x = torch.randint(-2 ** 15, 2 ** 15, (M, K), dtype=torch.int16, device="cuda")
        shapes = ("1 KB of one row", "16 rows x 64 B (16x16x32 A fragments)", "32 rows x 32 B (32x32x16 A fragments)",
                  "4 rows x 256 B", "1 KB of one row, direct-to-LDS copies, 4 in flight per wave",
                  "1 KB of one row, direct-to-LDS copies, 8 in flight per wave",
                  "2 rows x 512 B, direct-to-LDS copies, 4 in flight per wave",
                  "2 rows x 512 B, chunks XOR-swizzled by row, direct-to-LDS copies, 4 in flight per wave")
        out = []
        for pat, shape in enumerate(shapes):
            def step(i, pat=pat):
                assert self.lib.roof_shared_read(x.data_ptr(), M, K, pat, blocks, self.sink.data_ptr(),
                                                 self._stream()) == 0
            r = time_rounds(step, 1)
            out.append({"pattern": pat, "shape": shape, "us": r["us"], "us_rounds": r["rounds_us"],
                        "per_cu_gbs": M * K * 2 / r["us"] / 1e3})
        del x
        return out


    def copy_pipeline(self, copies, N: int, K: int, nmodes: int = 9):
        """The 64-row factored kernel's operand copies alone (roof_copy_pipeline), over the rotated
        cold weight copies: x only, the weights only, both, and both with the two streams on
        separate waves (then the cache-policy variants of the weight copies)."""
        import torch
        x = torch.randint(-2 ** 15, 2 ** 15, (64, K), dtype=torch.int16, device="cuda")
        modes = ("x only (64 rows, from L2)", "packed words and parameters only (from HBM)", "both",
                 "both, x and weights copied by separate waves", "both, the word copies non-temporal (nt)",
                 "both, the word copies at system scope (sc0 sc1)", "both, the word copies at device scope (sc1)",
                 "words and parameters only, nt", "words and parameters only, sc0 sc1")
        out = []
        for mode, what in enumerate(modes[:nmodes]):
            def step(i, mode=mode):
                c, sc, mn = copies[i % len(copies)]
                assert self.lib.roof_copy_pipeline(x.data_ptr(), c.data_ptr(), sc.data_ptr(), mn.data_ptr(), N, K, mode,
                                                   self._stream()) == 0
            r = time_rounds(step, len(copies))
            out.append({"mode": mode, "copies": what, "us": r["us"], "us_rounds": r["rounds_us"]})
        del x
        return out


def bench_small_n():
    """The decode GEMV at a small-N shape (N = 4096, K = 14336: the 8B model's down projection), 1
    and 16 rows, cold rotated copies: w4a16_matmul with its workspace (K split over blocks) and
    without (the GEMV's 32-column blocks, 128 of them)."""
    import gemm_w4a16_amd as w
    import workloads
    N, K = 4096, 14336
    W = workloads.weights(N, K, True, 0)
    c, s_, m = w.w4a16_packed_sizes(w.W4A16_FMT_G128_ASYM_BF16, N, K)
    R = copies_for(c + s_ + m)
    out, base = [], None
    for M in (1, 16):
        x = workloads.activations(M, K, "bf16", 1, rows_drawn=16)
        st = Setup(w.W4A16_FMT_G128_ASYM_BF16, M, N, K, x, W, R if base is None else 1)
        if base is None:
            base = st.copies
        else:
            st.copies = base
        split = time_rounds(st.step, R)
        ws_bytes = st.ws_bytes
        st.ws, st.ws_bytes = None, 0
        plain = time_rounds(st.step, R)
        out.append({"M": M, "N": N, "K": K, "workspace_bytes": ws_bytes, "us_k_split": split["us"],
                    "us_k_split_rounds": split["rounds_us"], "us_no_workspace": plain["us"],
                    "us_no_workspace_rounds": plain["rounds_us"],
                    "effective_weight_gbs_k_split": (c + s_ + m) / split["us"] / 1e3})
    return {"workload": "decode_gemv_k14336_n4096", "weight_bytes": c + s_ + m, "rows": out}


def bench_copy_floor(W=None):
    """What the 64-row kernel's operand copies alone take at the decode shape (x from L2, the
    weights from HBM, cold rotated copies): the floor under the sweep's M = 64 figure."""
    import gemm_w4a16_amd as w
    import workloads
    wl = workloads.DECODE
    if W is None:
        W = workloads.weights(wl.N, wl.K, wl.outliers, wl.seed_w)
    c, s_, m = w.w4a16_packed_sizes(w.W4A16_FMT_G128_ASYM_BF16, wl.N, wl.K)
    st = Setup(w.W4A16_FMT_G128_ASYM_BF16, 1, wl.N, wl.K, np.zeros((1, wl.K), np.uint16), W, copies_for(c + s_ + m))
    modes = Roofs().copy_pipeline(st.copies, wl.N, wl.K, nmodes=4)
    return {"workload": "decode-shape weights, 64 activation rows", "kernel": "roof_copy_pipeline (libw4a16_roof.so)",
            "modes": modes}


def bench_l2_patterns():
    """roof_shared_read at K = 4096 for 32, 64 and 128 rows, 224 blocks (one per 64 columns of the
    decode shape), beside the empty launch that every figure includes; and roof_copy_pipeline over
    the decode shape's weights."""
    import gemm_w4a16_amd as w
    import workloads
    roofs = Roofs()
    out = {"blocks": 224, "K": 4096, "empty_launch_us": roofs.empty_launch_us(),
           "rows": {M: roofs.shared_read(M, 4096) for M in (32, 64, 128)}}
    wl = workloads.DECODE
    W = workloads.weights(wl.N, wl.K, wl.outliers, wl.seed_w)
    c, s_, m = w.w4a16_packed_sizes(w.W4A16_FMT_G128_ASYM_BF16, wl.N, wl.K)
    st = Setup(w.W4A16_FMT_G128_ASYM_BF16, 1, wl.N, wl.K, np.zeros((1, wl.K), np.uint16), W, copies_for(c + s_ + m))
    out["copy_pipeline"] = {"N": wl.N, "K": wl.K, "rows": 64, "modes": roofs.copy_pipeline(st.copies, wl.N, wl.K)}
    return out


def time_rounds_eager(step, rounds: int = ROUNDS):
    """As time_rounds, for library calls kept out of graphs (hipBLASLt through torch.matmul):
    MIN_LAUNCHES eager launches per round, bracketed by HIP events."""
    import torch
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < WARM_SECONDS:
        for i in range(10):
            step(i)
        torch.cuda.synchronize()
    per = []
    for _ in range(rounds):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(MIN_LAUNCHES):
            step(i)
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) * 1e3 / MIN_LAUNCHES)
    return {"us": float(np.median(per)), "rounds_us": [round(v, 4) for v in per], "launches_per_round": MIN_LAUNCHES}


def bench_decode(steps, warmup):
    """The headline: K steps for the wall-clock value, then the kernel's own duration."""
    import gemm_w4a16_amd as w
    import workloads
    wl = workloads.DECODE
    W, x = workloads.inputs(wl)
    c, s, m = w.w4a16_packed_sizes(w.W4A16_FMT_G128_ASYM_BF16, wl.N, wl.K)
    R = copies_for(c + s + m)
    st = Setup(w.W4A16_FMT_G128_ASYM_BF16, wl.M, wl.N, wl.K, x, W, R)
    wall, ev = time_steps(st, steps, warmup)
    kt = time_rounds(st.step, R)
    algo_bytes = st.weight_bytes + wl.M * wl.K * 2 + wl.M * wl.N * 2
    return wl, st, R, wall, ev, kt, algo_bytes, W, x


class ClockSampler:
    """Records the GPU clocks while a timing runs: a background thread reads the driver's
    current shader (sclk) and memory (mclk) clock levels from sysfs every `period` seconds.  The
    clocks are not set here; a compute-bound kernel runs at what the power limit allows, which is
    why the figures carry them."""

    def __init__(self, period: float = 0.05):
        import glob
        self.period = period
        self.files = {k: sorted(glob.glob(f"/sys/class/drm/card*/device/pp_dpm_{k}")) for k in ("sclk", "mclk")}
        self.samples = {k: {f: [] for f in fs} for k, fs in self.files.items()}
        self._stop = None
        self._thread = None

    @staticmethod
    def _current_mhz(path: str):
        try:
            with open(path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        return int(line.split(":", 1)[1].strip().split("M")[0].split("m")[0])
        except (OSError, ValueError, IndexError):
            return None
        return None

    def _run(self):
        while not self._stop.is_set():
            for k, fs in self.files.items():
                for f in fs:
                    v = self._current_mhz(f)
                    if v is not None:
                        self.samples[k][f].append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        import threading
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join()
        return False

    def summary(self):
        out = {}
        for k, per in self.samples.items():
            for f, vals in per.items():
                if vals:
                    card = f.split("/")[4]
                    out.setdefault(k + "_mhz", {})[card] = {"min": min(vals), "median": float(np.median(vals)),
                                                           "max": max(vals), "samples": len(vals)}
        return out or {"unavailable": "no readable pp_dpm_sclk / pp_dpm_mclk under /sys/class/drm"}


def bench_prefill():
    import torch
    import gemm_w4a16_amd as w
    import workloads
    wl = workloads.PREFILL
    W, x = workloads.inputs(wl)
    st = Setup(w.W4A16_FMT_G128_ASYM_BF16, wl.M, wl.N, wl.K, x, W, 1)
    with ClockSampler() as clocks:
        kt = time_rounds(st.step, 1)
    flops = 2.0 * wl.M * wl.N * wl.K
    t = kt["us"] * 1e-6
    # the measured roof: the same product with bf16 weights (the GPU's own dequantized weights)
    # through torch.matmul (hipBLASLt)
    Wb = torch.empty((wl.N, wl.K), dtype=torch.int16, device="cuda")
    w.w4a16_dequant(w.W4A16_FMT_G128_ASYM_BF16, *st.copies[0], wl.N, wl.K, w.W4A16_BF16, Wb)
    Wt = Wb.view(torch.bfloat16).t().contiguous()   # [K][N]
    xb = st.x.view(torch.bfloat16)
    yb = torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device="cuda")
    bt = time_rounds_eager(lambda i: torch.matmul(xb, Wt, out=yb))
    del Wb, Wt, yb
    return {
        "workload": wl.name, "M": wl.M, "N": wl.N, "K": wl.K,
        "us_per_launch": kt["us"], "us_per_launch_rounds": kt["rounds_us"],
        "launches_per_round": kt["launches_per_round"],
        "clocks_during_timing": clocks.summary(),
        "tflops": flops / t / 1e12,
        "frac_mfma_bf16_peak": flops / t / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "roofline": {"bound": "mfma", "kernel": PREFILL_KERNEL, "achieved": flops / t / 1e12,
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": flops / t / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": recorded_traffic(PREFILL_KERNEL),
                     "measured_roof": {"kernel": "hipBLASLt bf16-weight GEMM (torch.matmul) of the same shape",
                                       "us": bt["us"], "us_rounds": bt["rounds_us"],
                                       "tflops": flops / (bt["us"] * 1e-6) / 1e12,
                                       "frac_of_measured_roof": bt["us"] / kt["us"]}},
    }


def bench_q4(roofs):
    import gemm_w4a16_amd as w
    import workloads
    wl = workloads.Q4
    W, x = workloads.inputs(wl)
    c, s, m = w.w4a16_packed_sizes(w.W4A16_FMT_Q4_B32_SYM_FP16, wl.N, wl.K)
    R = copies_for(c + s + m)
    st = Setup(w.W4A16_FMT_Q4_B32_SYM_FP16, wl.M, wl.N, wl.K, x, W, R)
    del W
    kt = time_rounds(st.step, R)
    t = kt["us"] * 1e-6
    out = {
        "workload": wl.name, "M": 1, "N": wl.N, "K": wl.K, "weight_copies": R,
        "weight_bytes": st.weight_bytes, "us_per_launch": kt["us"], "us_per_launch_rounds": kt["rounds_us"],
        "launches_per_round": kt["launches_per_round"],
        "effective_weight_gbs": st.weight_bytes / t / 1e9,
        "frac_hbm_peak": st.weight_bytes / t / 1e9 / HBM_PEAK_GBS,
    }
    out["fp16_weight_gemv"] = fp16_gemv_comparator(st, wl)
    del st
    import torch
    torch.cuda.empty_cache()
    rr = roofs.read(c + s + m, R)
    out["measured_roof"] = {"read_us": rr["us"], "read_gbs": rr["gbs"], "frac_of_measured_roof": rr["us"] / kt["us"]}
    return out


def fp16_gemv_comparator(st, wl):
    """Context for the Q4 GEMV (thuongvuho.com, "Why My 4-Bit CUDA Kernel Wasn't Faster", measures
    its kernels against a GEMV over fp16 weights): the same product with the GPU's own dequantized
    weights in fp16 (512 MB, larger than the Infinity Cache, so every call reads them from HBM)
    through torch.matmul."""
    import torch
    w = st.w
    Wh = torch.empty((wl.N, wl.K), dtype=torch.int16, device="cuda")
    w.w4a16_dequant(w.W4A16_FMT_Q4_B32_SYM_FP16, *st.copies[0], wl.N, wl.K, w.W4A16_FP16, Wh)
    Wt = Wh.view(torch.float16)
    xh = st.x.view(torch.float16).reshape(wl.K, 1)
    yh = torch.empty((wl.N, 1), dtype=torch.float16, device="cuda")
    r = time_rounds_eager(lambda i: torch.matmul(Wt, xh, out=yh))
    nbytes = wl.N * wl.K * 2
    del Wh, Wt, yh
    return {"us": r["us"], "us_rounds": r["rounds_us"], "weight_bytes": nbytes, "gbs": nbytes / r["us"] / 1e3}


def bench_decode_warm(W):
    """The decode GEMV with ONE weight copy, which stays resident in the 256 MB Infinity Cache:
    a warm number, reported beside (never instead of) the cold, rotated-copy headline."""
    import gemm_w4a16_amd as w
    import workloads
    wl = workloads.DECODE
    _, x = workloads.inputs(wl)
    st = Setup(w.W4A16_FMT_G128_ASYM_BF16, wl.M, wl.N, wl.K, x, W, 1)
    kt = time_rounds(st.step, 1)
    return {"workload": wl.name + "_warm", "weight_copies": 1, "us_per_launch": kt["us"],
            "us_per_launch_rounds": kt["rounds_us"],
            "effective_weight_gbs": st.weight_bytes / kt["us"] / 1e3,
            "cache": "weights resident in the 256 MB Infinity Cache"}


def bench_rowfmt(wl, fmt, W=None):
    """A decode-shape GEMV in one of the further formats (fp16 activations)."""
    import workloads
    Wn, x = workloads.inputs(wl)
    if W is None:
        W = Wn
    import gemm_w4a16_amd as w
    c, s, m = w.w4a16_packed_sizes(fmt, wl.N, wl.K)
    R = copies_for(c + s + m)
    st = Setup(fmt, wl.M, wl.N, wl.K, x, W, R)
    kt = time_rounds(st.step, R)
    t = kt["us"] * 1e-6
    return {
        "workload": wl.name, "M": 1, "N": wl.N, "K": wl.K, "weight_copies": R,
        "weight_bytes": st.weight_bytes, "us_per_launch": kt["us"], "us_per_launch_rounds": kt["rounds_us"],
        "effective_weight_gbs": st.weight_bytes / t / 1e9,
        "frac_hbm_peak": st.weight_bytes / t / 1e9 / HBM_PEAK_GBS,
    }


ROWFMT_SWEEP_MS = (1, 2, 4, 8, 16, 32, 64)


def bench_rowfmt_sweep(wl, fmt, W=None, Ms=ROWFMT_SWEEP_MS):
    """A row-major format over several fp16 activation rows (one weight pass per call up to 64
    rows), cold weights: the time per M, to show the weight stream's cost staying flat."""
    import workloads
    import gemm_w4a16_amd as w
    if W is None:
        W = workloads.inputs(wl)[0]
    c, s, m = w.w4a16_packed_sizes(fmt, wl.N, wl.K)
    R = copies_for(c + s + m)
    out, base = [], None
    for M in Ms:
        x = workloads.activations(M, wl.K, "f16", wl.seed_x, rows_drawn=max(Ms))
        st = Setup(fmt, M, wl.N, wl.K, x, W, R if base is None else 1)
        if base is None:
            base = st.copies
        else:
            st.copies = base
        kt = time_rounds(st.step, R)
        t = kt["us"] * 1e-6
        out.append({"M": M, "us": kt["us"], "us_rounds": kt["rounds_us"],
                    "effective_weight_gbs": st.weight_bytes / t / 1e9,
                    "tflops": 2.0 * M * wl.N * wl.K / t / 1e12})
    return out


def bench_zp(W=None):
    """The decode shape in the zero-point format (fp16 scale and zero point per 128, fp16 x)."""
    import gemm_w4a16_amd as w
    import workloads
    return bench_rowfmt(workloads.ZP_DECODE, w.W4A16_FMT_G128_ZP_FP16, W)


def bench_w8(W=None):
    """The decode shape as per-row int8 weights (W8A16, fp16 x)."""
    import gemm_w4a16_amd as w
    import workloads
    return bench_rowfmt(workloads.W8_DECODE, w.W4A16_FMT_W8_ROW_FP32, W)


class W4A8Setup:
    """The prefill shape as W4A8: bf16 activations quantized per row to int8, then the int8-MFMA
    product with the same packed G128 weights.  A step is both kernels, or the product alone."""

    def __init__(self, wl, W, x_bits, gemm_only: bool):
        import torch
        import gemm_w4a16_amd as w
        self.w, self.wl, self.gemm_only = w, wl, gemm_only
        fmt = w.W4A16_FMT_G128_ASYM_BF16
        Wd = torch.from_numpy(W).cuda()
        self.packed = w.alloc_packed(fmt, wl.N, wl.K)
        w.w4a16_quantize_pack(fmt, Wd, wl.N, wl.K, *self.packed)
        del Wd
        self.x = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda()
        self.q = w.alloc_act_i8(wl.M, wl.K)
        w.w4a16_quantize_act_i8(self.x, wl.M, wl.K, *self.q)
        self.y = torch.empty((wl.M, wl.N), dtype=torch.int16, device="cuda")
        torch.cuda.synchronize()

    def step(self, i):
        w, wl = self.w, self.wl
        if not self.gemm_only:
            w.w4a16_quantize_act_i8(self.x, wl.M, wl.K, *self.q)
        w.w4a16_gemm_w4a8(w.W4A16_FMT_G128_ASYM_BF16, *self.q, wl.M, *self.packed, wl.N, wl.K, self.y)


def bench_w4a8():
    """W4A8 at the prefill shape (M=1024, K=4096, N=14336): quantize + product per step, and the
    product alone against the int8 matrix-core peak."""
    import workloads
    wl = workloads.PREFILL
    W, x = workloads.inputs(wl)
    ops = 2.0 * wl.M * wl.N * wl.K
    out = {"workload": "w4a8_gemm_m1024_k4096_n14336", "M": wl.M, "N": wl.N, "K": wl.K}
    for gemm_only in (False, True):
        st = W4A8Setup(wl, W, x, gemm_only)
        kt = time_rounds(st.step, 1)
        t = kt["us"] * 1e-6
        key = "gemm_only" if gemm_only else "quantize_and_gemm"
        out[key] = {"us_per_step": kt["us"], "us_rounds": kt["rounds_us"], "tops": ops / t / 1e12}
        if gemm_only:
            out["roofline"] = {"bound": "mfma", "kernel": "w4a8_gemm_kernel", "achieved": ops / t / 1e12,
                               "peak": MFMA_I8_PEAK_TOPS, "unit": "TOP/s", "frac": ops / t / 1e12 / MFMA_I8_PEAK_TOPS,
                               "traffic": None}
        del st
    return out


class W4A8DecodeSetup(Setup):
    """The decode shape (M=1) as W4A8: the row quantized to int8, then the few-row int8-MFMA
    product against the same G128 weights, rotated over cold copies like the W4A16 decode."""

    def __init__(self, wl, W, x_bits, copies, mode: str):
        import gemm_w4a16_amd as w
        super().__init__(w.W4A16_FMT_G128_ASYM_BF16, wl.M, wl.N, wl.K, x_bits, W, copies)
        self.mode = mode  # "quantize_and_gemm", "gemm_only" or "fused" (one launch)
        self.q = w.alloc_act_i8(wl.M, wl.K)
        w.w4a16_quantize_act_i8(self.x, wl.M, wl.K, *self.q)

    def step(self, i):
        w = self.w
        c, s, m = self.copies[i % len(self.copies)]
        if self.mode == "fused":
            w.w4a16_matmul_w4a8(self.fmt, self.x, self.M, c, s, m, self.N, self.K, self.y)
            return
        if self.mode == "quantize_and_gemm":
            w.w4a16_quantize_act_i8(self.x, self.M, self.K, *self.q)
        w.w4a16_gemm_w4a8(self.fmt, *self.q, self.M, c, s, m, self.N, self.K, self.y)


def bench_w4a8_decode(W=None):
    """W4A8 at the decode shape (M=1, K=4096, N=14336), cold weights, as effective weight GB/s
    against the HBM peak: quantize + product (two launches), the product alone, and the fused
    one-launch form."""
    import workloads
    wl = workloads.DECODE
    W0, x = workloads.inputs(wl)
    W = W0 if W is None else W
    import gemm_w4a16_amd as w
    c, s, m = w.w4a16_packed_sizes(w.W4A16_FMT_G128_ASYM_BF16, wl.N, wl.K)
    R = copies_for(c + s + m)
    out = {"workload": "w4a8_gemv_m1_k4096_n14336", "M": 1, "N": wl.N, "K": wl.K, "weight_copies": R}
    for mode in ("quantize_and_gemm", "gemm_only", "fused"):
        st = W4A8DecodeSetup(wl, W, x, R, mode)
        kt = time_rounds(st.step, R)
        t = kt["us"] * 1e-6
        out[mode] = {"us_per_step": kt["us"], "us_rounds": kt["rounds_us"],
                     "effective_weight_gbs": st.weight_bytes / t / 1e9,
                     "frac_hbm_peak": st.weight_bytes / t / 1e9 / HBM_PEAK_GBS}
        del st
    return out


def bench_w4a8_sweep(W=None):
    """W4A8 product alone (activations quantized once, before the timed steps) over the batch
    sweep's M at K=4096, N=14336, cold weights: which kernel each M takes and its time."""
    import gemm_w4a16_amd as w
    import workloads
    wl1 = workloads.DECODE
    if W is None:
        W = workloads.weights(wl1.N, wl1.K, wl1.outliers, wl1.seed_w)
    c, s, m = w.w4a16_packed_sizes(w.W4A16_FMT_G128_ASYM_BF16, wl1.N, wl1.K)
    R = copies_for(c + s + m)
    out, base = [], None
    for M in workloads.SWEEP_MS:
        wl = workloads.sweep(M)
        x = workloads.activations(M, wl.K, "bf16", wl.seed_x, rows_drawn=max(workloads.SWEEP_MS))
        st = W4A8DecodeSetup(wl, W, x, R if base is None else 1, "gemm_only")
        if base is None:
            base = st.copies
        else:
            st.copies = base  # reuse the rotated weight copies
        t = time_rounds(st.step, R)["us"] * 1e-6
        out.append({"M": M, "kernel": "rows16" if M <= 64 else "gemm", "us": t * 1e6,
                    "effective_weight_gbs": st.weight_bytes / t / 1e9, "tops": 2.0 * M * wl.N * wl.K / t / 1e12})
    return out


def bench_sweep(W=None):
    """The G128 matmul over M = 1 .. 256 (cold rotated weight copies), and beside each M
    hipBLASLt's product of the same shape with bf16 weights (the GPU's own dequantized weights,
    also cold: enough rotated bf16 copies to exceed twice the Infinity Cache) -- the pages'
    speedup-over-BF16 profile ([P1] Step 3)."""
    import torch
    import gemm_w4a16_amd as w
    import workloads
    wl1 = workloads.DECODE
    if W is None:
        W = workloads.weights(wl1.N, wl1.K, wl1.outliers, wl1.seed_w)
    c, s, m = w.w4a16_packed_sizes(w.W4A16_FMT_G128_ASYM_BF16, wl1.N, wl1.K)
    R = copies_for(c + s + m)
    out = []
    base = None
    wts = None
    for M in workloads.SWEEP_MS:
        wl = workloads.sweep(M)
        x = workloads.activations(M, wl.K, "bf16", wl.seed_x, rows_drawn=max(workloads.SWEEP_MS))
        st = Setup(w.W4A16_FMT_G128_ASYM_BF16, M, wl.N, wl.K, x, W, R if base is None else 1)
        if base is None:
            base = st.copies
        else:
            st.copies = base  # reuse the rotated weight copies
        if wts is None:
            Wb = torch.empty((wl.N, wl.K), dtype=torch.int16, device="cuda")
            w.w4a16_dequant(w.W4A16_FMT_G128_ASYM_BF16, *base[0], wl.N, wl.K, w.W4A16_BF16, Wb)
            Wt = Wb.view(torch.bfloat16).t().contiguous()  # [K][N]
            del Wb
            wts = [Wt] + [Wt.clone() for _ in range(copies_for(Wt.numel() * 2) - 1)]
        kt = time_rounds(st.step, R)
        t = kt["us"] * 1e-6
        xb = st.x.view(torch.bfloat16)
        yb = torch.empty((M, wl.N), dtype=torch.bfloat16, device="cuda")
        bt = time_rounds_eager(lambda i: torch.matmul(xb, wts[i % len(wts)], out=yb))
        out.append({"M": M, "path": "gemv" if M <= w.w4a16_matmul_gemv_cutoff() else "gemm",
                    "us": kt["us"], "us_rounds": kt["rounds_us"], "effective_weight_gbs": st.weight_bytes / t / 1e9,
                    "tflops": 2.0 * M * wl.N * wl.K / t / 1e12,
                    "hipblaslt_bf16_us": bt["us"], "hipblaslt_bf16_us_rounds": bt["rounds_us"],
                    "speedup_vs_bf16": bt["us"] / kt["us"]})
        del yb
    del wts
    torch.cuda.empty_cache()
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_threads() -> int:
    """Host threads for the all-cores run: the cores this process may run on
    (sched_getaffinity), capped by OMP_NUM_THREADS where the host sets it."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    return min(n, int(cap)) if cap.isdigit() and int(cap) > 0 else n


def oracle_outputs(fn_at, args, M, N, threads):
    """Every output of an M x N product through the oracle's per-output entry point, split into
    `threads` contiguous slices run on that many threads (the foreign calls release the GIL).
    The oracle's arithmetic is unchanged: each output is its k-ordered fp64 sum."""
    from concurrent.futures import ThreadPoolExecutor
    rows = np.repeat(np.arange(M, dtype=np.int64), N)
    cols = np.tile(np.arange(N, dtype=np.int64), M)
    parts = np.array_split(np.arange(M * N), threads)
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda idx: fn_at(*args, rows[idx], cols[idx]), parts))


def timed(fn, min_runs, budget_s):
    times, t_start = [], time.perf_counter()
    while len(times) < min_runs or (time.perf_counter() - t_start < budget_s and len(times) < 50):
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    return float(np.median(times)), len(times)


def cpu_baseline(W, x):
    """The oracle as it stands (plain C, fp64 sums in k order) on the host, single-threaded and on
    all the cores this process may use, over bounded samples of the workloads: the full decode
    GEMV, the full 16384^2 Q4 GEMV, and row slices of prefill."""
    import oracle
    import workloads
    T = cpu_threads()
    legs = {}
    tpack, npack = timed(lambda: oracle.quantize_g128(W), 1, 0.0)
    codes, scales, mins = oracle.quantize_g128(W)
    wbytes = codes.nbytes + scales.nbytes + mins.nbytes
    legs["quantize_pack_g128"] = {"workload": workloads.DECODE.name, "weights": int(W.size),
                                  "single_thread": {"s": tpack, "runs": npack,
                                                    "mweights_per_s": W.size / tpack / 1e6}}
    wl = workloads.DECODE
    t1, n1 = timed(lambda: oracle.matmul_g128(x, codes, scales, mins), 3, 5.0)
    tT, nT = timed(lambda: oracle_outputs(oracle.matmul_g128_at, (x, codes, scales, mins), 1, wl.N, T), 3, 1.0)
    legs["decode_gemv"] = {"workload": wl.name, "weight_bytes": wbytes,
                           "single_thread": {"s": t1, "runs": n1, "gbs": wbytes / t1 / 1e9},
                           "all_cores": {"s": tT, "runs": nT, "threads": T, "gbs": wbytes / tT / 1e9}}
    # prefill (M=1024): the first 4 rows on one thread, the first 64 on all cores
    pw = workloads.PREFILL
    _, xp = workloads.inputs(pw)
    rows1, rowsT = 4, 64
    t1p, _ = timed(lambda: oracle.matmul_g128(np.ascontiguousarray(xp[:rows1]), codes, scales, mins), 1, 0.0)
    tTp, _ = timed(lambda: oracle_outputs(oracle.matmul_g128_at, (np.ascontiguousarray(xp[:rowsT]), codes, scales, mins),
                                          rowsT, pw.N, T), 1, 0.0)
    legs["prefill_gemm_row_slice"] = {
        "workload": pw.name, "sample": f"rows 0..{rows1 - 1} on one thread, rows 0..{rowsT - 1} on all cores",
        "single_thread": {"s": t1p, "rows": rows1, "gflops": 2.0 * rows1 * pw.N * pw.K / t1p / 1e9},
        "all_cores": {"s": tTp, "rows": rowsT, "threads": T, "gflops": 2.0 * rowsT * pw.N * pw.K / tTp / 1e9},
        "full_m1024_all_cores_s_extrapolated": tTp * pw.M / rowsT}
    del xp
    # Q4 block-32 GEMV, 16384 x 16384 (the oracle quantizes the weights first, untimed)
    qw = workloads.Q4
    Wq, xq = workloads.inputs(qw)
    tpq, npq = timed(lambda: oracle.quantize_q4b32(Wq), 1, 0.0)
    qc, qs = oracle.quantize_q4b32(Wq)
    legs["quantize_pack_q4b32"] = {"workload": qw.name, "weights": int(Wq.size),
                                   "single_thread": {"s": tpq, "runs": npq, "mweights_per_s": Wq.size / tpq / 1e6}}
    del Wq
    qbytes = qc.nbytes + qs.nbytes
    t1q, n1q = timed(lambda: oracle.matmul_q4b32(xq, qc, qs), 1, 0.0)
    tTq, nTq = timed(lambda: oracle_outputs(oracle.matmul_q4b32_at, (xq, qc, qs), 1, qw.N, T), 3, 0.0)
    legs["q4b32_gemv"] = {"workload": qw.name, "weight_bytes": qbytes,
                          "single_thread": {"s": t1q, "runs": n1q, "gbs": qbytes / t1q / 1e9},
                          "all_cores": {"s": tTq, "runs": nTq, "threads": T, "gbs": qbytes / tTq / 1e9}}
    dec = legs["decode_gemv"]["all_cores"]
    return {"value": dec["gbs"], "unit": "GB/s", "cores": T, "kind": "oracle",
            "sample": (f"the full decode GEMV (M=1, K=4096, N=14336) in fp64 on {T} threads, median of "
                       f"{dec['runs']} runs ({dec['s'] * 1e3:.1f} ms); single-threaded, the Q4 GEMV, "
                       f"prefill row slices and the quantize/pack under 'legs'"),
            "cpu_model": cpu_model(), "cores_available": len(os.sched_getaffinity(0)), "legs": legs}


def gpu_over_oracle(line):
    """The GPU kernel's rate over the oracle's, per workload timed on both (the kernel's own
    per-launch time against the oracle on one thread and on all cores)."""
    legs = line["cpu_baseline"]["legs"]
    out = {}

    def ratio(gpu_rate, leg, key):
        return {"single_thread": gpu_rate / leg["single_thread"][key], "all_cores": gpu_rate / leg["all_cores"][key]}

    out["decode_gemv"] = ratio(line["roofline"]["achieved"], legs["decode_gemv"], "gbs")
    extra = line.get("extra", {})
    if "q4b32_m1" in extra:
        out["q4b32_gemv"] = ratio(extra["q4b32_m1"]["effective_weight_gbs"], legs["q4b32_gemv"], "gbs")
    if "prefill_m1024" in extra:
        out["prefill_gemm"] = ratio(extra["prefill_m1024"]["tflops"] * 1e3, legs["prefill_gemm_row_slice"], "gflops")
    return out


def cpu_baseline_only():
    import workloads
    return cpu_baseline(*workloads.inputs(workloads.DECODE))


def copy_calibration(mib: int):
    """Copy a buffer of known size: FETCH_SIZE / WRITE_SIZE of this kernel calibrate the counters."""
    import torch
    src = torch.empty(mib * 2 ** 20, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: 5 x {mib} MiB device-to-device")


def bench_zp_prepared(W=None, Ms=(1, 4, 16, 32, 64)):
    """The zero-point format from its prepared copy (w4a16_prepare once, then w4a16_gemv_prepared)
    at the decode shape, cold copies, fp16 activations; rates over the prepared copy's bytes and,
    for comparison with the canonical GEMV, over the format's own bytes."""
    import torch
    import gemm_w4a16_amd as w
    import workloads
    wl, fmt = workloads.ZP_DECODE, w.W4A16_FMT_G128_ZP_FP16
    if W is None:
        W = workloads.inputs(wl)[0]
    c, s, m = w.w4a16_packed_sizes(fmt, wl.N, wl.K)
    nb = w.w4a16_prepared_bytes(fmt, wl.N, wl.K)
    R = copies_for(nb)
    st = Setup(fmt, 1, wl.N, wl.K, workloads.activations(1, wl.K, "f16", wl.seed_x), W, 1)
    preps = []
    for _ in range(R):
        p = torch.empty(nb, dtype=torch.uint8, device="cuda")
        w.w4a16_prepare(fmt, *st.copies[0], wl.N, wl.K, p, nb)
        preps.append(p)
    del st
    out = []
    for M in Ms:
        x = torch.from_numpy(workloads.activations(M, wl.K, "f16", wl.seed_x, rows_drawn=max(Ms)).view(np.int16)).cuda()
        y = torch.empty((M, wl.N), dtype=torch.int16, device="cuda")
        torch.cuda.synchronize()

        def step(i, x=x, y=y, M=M):
            w.w4a16_gemv_prepared(fmt, w.W4A16_FP16, x, M, preps[i % R], wl.N, wl.K, y)

        kt = time_rounds(step, R)
        t = kt["us"] * 1e-6
        out.append({"M": M, "us": kt["us"], "us_rounds": kt["rounds_us"], "prepared_bytes": nb,
                    "prepared_gbs": nb / t / 1e9, "format_bytes": c + s + m,
                    "effective_weight_gbs": (c + s + m) / t / 1e9, "frac_hbm_peak_prepared": nb / t / 1e9 / HBM_PEAK_GBS})
    return {"workload": wl.name + "_prepared", "weight_copies": R, "rows": out}


def main():
    global EAGER
    args = parse()
    EAGER = args.eager
    if args.gpus != 1:
        msg = (f"bench.py runs on one GPU only: --gpus {args.gpus} was asked for, but the library has no "
               "multi-GPU path (sharding the weight matrix by columns or by K groups is not implemented).")
        print(msg, file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    import gemm_w4a16_amd as w  # fails loudly if libw4a16.so is missing
    props = torch.cuda.get_device_properties(0)

    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
    if args.only and args.only != "decode":
        import workloads
        fn = {"prefill": bench_prefill, "q4": lambda: bench_q4(Roofs()), "sweep": bench_sweep, "zp": bench_zp,
              "rowfmt_sweep": lambda: {
                  "zp": bench_rowfmt_sweep(workloads.ZP_DECODE, w.W4A16_FMT_G128_ZP_FP16),
                  "w8": bench_rowfmt_sweep(workloads.W8_DECODE, w.W4A16_FMT_W8_ROW_FP32),
                  "q4": bench_rowfmt_sweep(workloads.Q4, w.W4A16_FMT_Q4_B32_SYM_FP16, None, (1, 2, 4, 8, 16))},
              "w8": bench_w8, "zp_prepared": bench_zp_prepared, "w4a8": bench_w4a8, "w4a8_decode": bench_w4a8_decode,
              "w4a8_sweep": bench_w4a8_sweep, "cpu": cpu_baseline_only, "l2_patterns": bench_l2_patterns,
              "small_n": bench_small_n}[args.only]
        print(json.dumps({"only": args.only, "result": fn()}), flush=True)
        return

    log(f"decode: {args.warmup} warmup + {args.steps} timed steps")
    wl, st, R, wall, ev, kt, algo_bytes, W, x = bench_decode(args.steps, args.warmup)
    per_launch = kt["us"] * 1e-6
    value = st.weight_bytes * args.steps / wall / 1e9
    achieved = algo_bytes / per_launch / 1e9
    weight_bytes = st.weight_bytes
    del st
    torch.cuda.empty_cache()
    log("measured roofs: empty launch, streaming read of the decode weight bytes")
    roofs = Roofs()
    empty_us = roofs.empty_launch_us()
    rr = roofs.read(weight_bytes, R)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "M": wl.M, "N": wl.N, "K": wl.K,
                   "format": "int4 codes, group 128 along K, bf16 scale + bf16 min",
                   "weights": "N(0,0.02) fp32 with 0.1% x20 outliers, seed 0", "activations": "bf16 N(0,1)",
                   "weight_copies_rotated": R, "weight_bytes": weight_bytes,
                   "timing": "K eager launches" if EAGER else "K steps in one HIP graph replay",
                   "device": props.name,
                   "compute_units": props.multi_processor_count,
                   "frac_hbm_peak_effective_weight": value / HBM_PEAK_GBS},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(DECODE_KERNEL),
                     "kernel": DECODE_KERNEL, "us_per_launch": kt["us"], "us_per_launch_rounds": kt["rounds_us"],
                     "launches_per_round": kt["launches_per_round"],
                     "timing": "median of 3 rounds; a round is one HIP-graph replay of back-to-back launches "
                               "over the rotated cold copies, bracketed by HIP events",
                     "algorithmic_bytes_per_launch": algo_bytes,
                     "measured_roof": {"read_us": rr["us"], "read_gbs": rr["gbs"], "read_blocks": rr["blocks"],
                                       "read_us_rounds": rr["rounds_us"], "kernel": rr["kernel"],
                                       "empty_launch_us": empty_us,
                                       "frac_of_measured_roof": rr["us"] / kt["us"]}},
    }
    if not args.no_extra and args.only is None:
        extra = {}
        log("decode, warm (one weight copy)")
        extra["decode_warm_m1"] = bench_decode_warm(W)
        torch.cuda.empty_cache()
        log("prefill M=1024")
        extra["prefill_m1024"] = bench_prefill()
        torch.cuda.empty_cache()
        log("q4 block-32 GEMV")
        extra["q4b32_m1"] = bench_q4(roofs)
        torch.cuda.empty_cache()
        log("zero-point format GEMV (decode shape)")
        extra["zp_decode_m1"] = bench_zp(W)
        torch.cuda.empty_cache()
        log("zero-point format from its prepared copy (decode shape)")
        extra["zp_prepared"] = bench_zp_prepared(W)
        torch.cuda.empty_cache()
        log("W8A16 per-row int8 GEMV (decode shape)")
        extra["w8_decode_m1"] = bench_w8(W)
        torch.cuda.empty_cache()
        log("batch sweep")
        extra["sweep"] = bench_sweep(W)
        torch.cuda.empty_cache()
        log("small-N decode shape (K split over blocks)")
        extra["decode_small_n"] = bench_small_n()
        torch.cuda.empty_cache()
        log("copy floor of the 64-row kernel (roof_copy_pipeline)")
        extra["copy_floor_m64"] = bench_copy_floor(W)
        torch.cuda.empty_cache()
        import workloads
        log("row-major formats over M (zero point and W8 at the decode shape, Q4 at 16384^2)")
        extra["zp_sweep"] = bench_rowfmt_sweep(workloads.ZP_DECODE, w.W4A16_FMT_G128_ZP_FP16, W)
        torch.cuda.empty_cache()
        extra["w8_sweep"] = bench_rowfmt_sweep(workloads.W8_DECODE, w.W4A16_FMT_W8_ROW_FP32, W)
        torch.cuda.empty_cache()
        extra["q4_sweep"] = bench_rowfmt_sweep(workloads.Q4, w.W4A16_FMT_Q4_B32_SYM_FP16, None, (1, 2, 4, 8, 16))
        torch.cuda.empty_cache()
        log("W4A8 at the prefill shape")
        extra["w4a8_m1024"] = bench_w4a8()
        torch.cuda.empty_cache()
        log("W4A8 at the decode shape")
        extra["w4a8_decode_m1"] = bench_w4a8_decode(W)
        torch.cuda.empty_cache()
        log("W4A8 batch sweep")
        extra["w4a8_sweep"] = bench_w4a8_sweep(W)
        torch.cuda.empty_cache()
        line["extra"] = extra
    if not args.no_cpu_baseline and args.only is None:
        log("cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline(W, x)
        line["cpu_baseline"]["gpu_over_oracle"] = gpu_over_oracle(line)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
