#!/usr/bin/env python3
"""Benchmark of the int4 group-128 GEMV on one MI355X.

One step = one q4g128_gemv call on the fused 25,088 x 3,072 projection at
batch 1 (packed weights + fp16 scales + fp16 mins + fp16 activations in,
fp32 out).  Weight copies totalling >= 512 MB are rotated so that the 256 MB
Infinity Cache cannot serve repeated calls.  The timed launches go back to
back on the benchmark's stream, bracketed by HIP events on that stream; the
same launches replayed from a HIP graph are timed as a cross-check that must
reproduce the eager output.

Prints ONE JSON line.  Extra forms (the GEMV's ceilings from the diagnostics
library: its read-only twin, a plain streaming read and an empty launch;
other shapes, small batch, prompt processing, the int8 output head, the
export quantiser, and the pages' and the 36-layer decode steps as 108
launches and as grouped calls) are reported under "forms".  The CPU oracle is
timed first, before the GPU is initialised, on one thread and on all the
host's cores (cpu_baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "int4-g128 GEMV GB/s at B=1 (25088x3072) and % of MI355X HBM peak"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense fp16 matrix-core peak of the MI355X
MALL_DEFEAT_BYTES = 512 << 20
GRAPH_LAUNCHES = 100
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemv_fused_25088x3072.json")
KERNEL_SOURCES = ["int4_group_quantized_amd/csrc/gemv.hip", "int4_group_quantized_amd/csrc/gemv_pass.hpp",
                  "int4_group_quantized_amd/csrc/q4_device.hpp"]


def algorithmic_bytes(n: int, k: int, b: int = 1) -> int:
    """Packed codes + fp16 scales + fp16 mins + fp16 activations read."""
    g = k // 128
    return n * k // 2 + 2 * n * g * 2 + b * k * 2


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class Rotation:
    """R device copies of one packed weight set (R * bytes >= 512 MB)."""

    def __init__(self, torch, q4, w, dev, min_copies=1):
        codes = torch.from_numpy(w.codes).to(dev)
        packed = q4.q4g128_pack(codes)
        del codes
        scales = torch.from_numpy(w.scales).to(dev)
        mins = torch.from_numpy(w.mins).to(dev)
        self.n, self.k = w.n, w.k
        per = algorithmic_bytes(w.n, w.k, 0)
        self.copies = max(min_copies, -(-MALL_DEFEAT_BYTES // per))
        self.sets = [(packed, scales, mins)]
        for _ in range(self.copies - 1):
            self.sets.append((packed.clone(), scales.clone(), mins.clone()))
        torch.cuda.synchronize()


def time_graph(torch, stream, launch, n_launch_per_graph, steps, warmup, out=None):
    """Capture n_launch_per_graph calls into one graph; return ms per call.

    The graph is replayed on `stream` (CUDAGraph.replay launches on the
    current stream), bracketed by HIP events recorded on the same stream.
    If `out` is given, the graph must rewrite it: it is cleared, the graph is
    replayed once and the result must equal the eager result.
    """
    with torch.cuda.stream(stream):
        for i in range(max(warmup, 1)):
            launch(i, stream.cuda_stream)
        eager = out.clone() if out is not None else None
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n_launch_per_graph):
                launch(i, stream.cuda_stream)
        if out is not None:
            out.zero_()
        g.replay()
    stream.synchronize()
    if out is not None and not torch.equal(out, eager):
        raise RuntimeError("graph replay did not reproduce the eager result")
    reps = max(1, -(-steps // n_launch_per_graph))
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        # the same settle phase as the eager timing: replays for SETTLE_S first
        t0 = time.perf_counter()
        i = 0
        while time.perf_counter() - t0 < SETTLE_S:
            g.replay()
            i += 1
            if i % 16 == 0:
                stream.synchronize()
        stream.synchronize()
        start.record(stream)
        for _ in range(reps):
            g.replay()
        stop.record(stream)
    stop.synchronize()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop)
    return ms / (reps * n_launch_per_graph), reps * n_launch_per_graph, g


SETTLE_S = 0.1  # continuous load before any timed region (clocks ramp up over ~20 ms)


def time_eager(torch, stream, launch, steps, warmup, settle_s=SETTLE_S):
    """ms per call over `steps` back-to-back launches, after `warmup` untimed
    launches and at least `settle_s` seconds of continuous launching."""
    with torch.cuda.stream(stream):
        t0 = time.perf_counter()
        i = 0
        while i < warmup or time.perf_counter() - t0 < settle_s:
            launch(i, stream.cuda_stream)
            i += 1
            if i % 256 == 0:
                stream.synchronize()  # keep the queue short so the clock measures GPU time
        stream.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for i in range(steps):
            launch(i, stream.cuda_stream)
        stop.record(stream)
    stop.synchronize()
    return start.elapsed_time(stop) / steps


def time_checked(torch, stream, launch, out, steps, warmup, n_graph):
    """(eager, graph) ms per call: a HIP graph of n_graph launches, checked to
    rewrite `out` identically, replayed for `steps` launches, then `steps`
    eager launches.  For kernels shorter than the host's per-call cost of a
    ctypes launch (a few microseconds) the eager figure is the host's rate and
    the graph figure the kernel's."""
    g_ms = time_graph(torch, stream, launch, n_graph, steps, warmup, out=out)[0]
    return time_eager(torch, stream, launch, steps, warmup), g_ms


def gemv_launcher(q4, rot, x, y):
    lib = q4.library()
    ptrs = [(p.data_ptr(), s.data_ptr(), m.data_ptr()) for p, s, m in rot.sets]
    xp, yp, n, k = x.data_ptr(), y.data_ptr(), rot.n, rot.k
    R = len(ptrs)

    def launch(i, st):
        p, s, m = ptrs[i % R]
        rc = lib.q4g128_gemv(p, s, m, xp, yp, n, k, st)
        if rc != 0:
            raise RuntimeError(f"q4g128_gemv failed: {q4.q4g128_status_string(rc)}")
    return launch


def batch_launcher(q4, rot, X, Y, b):
    lib = q4.library()
    ptrs = [(p.data_ptr(), s.data_ptr(), m.data_ptr()) for p, s, m in rot.sets]
    xp, yp, n, k = X.data_ptr(), Y.data_ptr(), rot.n, rot.k
    R = len(ptrs)

    def launch(i, st):
        p, s, m = ptrs[i % R]
        rc = lib.q4g128_gemm_small_batch(p, s, m, xp, yp, n, k, b, st)
        if rc != 0:
            raise RuntimeError(f"q4g128_gemm_small_batch failed: {q4.q4g128_status_string(rc)}")
    return launch


def prefill_launcher(q4, rot, X, Y, mtok):
    lib = q4.library()
    ptrs = [(p.data_ptr(), s.data_ptr(), m.data_ptr()) for p, s, m in rot.sets]
    xp, yp, n, k = X.data_ptr(), Y.data_ptr(), rot.n, rot.k
    R = len(ptrs)

    def launch(i, st):
        p, s, m = ptrs[i % R]
        rc = lib.q4g128_gemm_prefill(p, s, m, xp, yp, n, k, mtok, st)
        if rc != 0:
            raise RuntimeError(f"q4g128_gemm_prefill failed: {q4.q4g128_status_string(rc)}")
    return launch


def quantize_bytes(n: int, k: int) -> int:
    """float32 weights read + packed codes, fp16 scales and fp16 mins written."""
    return n * k * 4 + n * k // 2 + 2 * n * (k // 128) * 2


def quantize_launcher(q4, Ws, packed, scales, mins, n, k):
    lib = q4.library()
    ptrs = [W.data_ptr() for W in Ws]
    pp, sp, mp = packed.data_ptr(), scales.data_ptr(), mins.data_ptr()
    R = len(ptrs)

    def launch(i, st):
        rc = lib.q4g128_quantize(ptrs[i % R], pp, sp, mp, n, k, st)
        if rc != 0:
            raise RuntimeError(q4.q4g128_status_string(rc))
    return launch


def head_bytes(n: int, k: int) -> int:
    """int8 codes + fp16 row scales + fp16 activations read."""
    return n * k + 2 * n + 2 * k


def head_launcher(q4, sets, x, y, n, k):
    lib = q4.library()
    ptrs = [(qq.data_ptr(), ss.data_ptr()) for qq, ss in sets]
    xp, yp = x.data_ptr(), y.data_ptr()
    R = len(ptrs)

    def launch(i, st):
        qq, ss = ptrs[i % R]
        rc = lib.q4g128_gemv_int8(qq, ss, xp, yp, n, k, st)
        if rc != 0:
            raise RuntimeError(q4.q4g128_status_string(rc))
    return launch


def prefill_epilogue_launcher(q4, rot, X, Y, mtok):
    lib = q4.library()
    ptrs = [(p.data_ptr(), s.data_ptr(), m.data_ptr()) for p, s, m in rot.sets]
    xp, yp, n, k = X.data_ptr(), Y.data_ptr(), rot.n, rot.k
    R = len(ptrs)

    def launch(i, st):
        p, s, m = ptrs[i % R]
        rc = lib.q4g128_gemm_prefill_epilogue(p, s, m, xp, yp, n, k, mtok, st)
        if rc != 0:
            raise RuntimeError(q4.q4g128_status_string(rc))
    return launch


def cpu_model() -> str:
    """CPU model name as lscpu reports it (falls back to /proc/cpuinfo)."""
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.machine()


CPU_BLOCK = 1024  # rows per oracle call
_CPU_CASE = None  # (packed, scales, mins, x) shared with forked workers


def _one_blas_thread():
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)  # for the rest of this worker process


def _oracle_rows(r0: int) -> int:
    import oracle
    packed, scales, mins, x = _CPU_CASE
    r1 = min(packed.shape[0], r0 + CPU_BLOCK)
    oracle.gemv(packed[r0:r1], scales[r0:r1], mins[r0:r1], x)
    return r1 - r0


def _time_blocks(fn, n_rows: int, budget_s: float):
    """Call fn(r0) on CPU_BLOCK-row blocks in order, wrapping, until budget_s; (rows, seconds)."""
    rows, t_total, r0 = 0, 0.0, 0
    while t_total < budget_s:
        t = time.perf_counter()
        rows += fn(r0)
        t_total += time.perf_counter() - t
        r0 = 0 if r0 + CPU_BLOCK >= n_rows else r0 + CPU_BLOCK
    return rows, t_total


def cpu_baseline(budget_s: float):
    """The fp64 NumPy oracle as it stands, on the host of the measured GPU, before any GPU work.

    Legs (the oracle is a reported baseline, not a target):
      * all cores: 1,024-row blocks of the fused 25,088 x 3,072 matrix at B = 1,
        spread over a pool of forked worker processes (one BLAS thread each),
        one pass over the matrix per ~budget/3 s; this is `value`;
      * one thread: the same blocks, in order, for ~budget/3 s;
      * one thread, the small batch at B = 16 and the prompt at M = 34 tokens
        on 1,024-row blocks of the same matrix (~budget/6 s each), scaled to
        the whole matrix.
    """
    global _CPU_CASE
    import multiprocessing as mp

    import oracle
    from threadpoolctl import threadpool_limits
    w, x = synth.workload("fused_25088x3072")
    packed = oracle.pack(w.codes)
    _CPU_CASE = (packed, w.scales, w.mins, x[0])
    n, k = w.n, w.k

    # one thread, B = 1
    with threadpool_limits(1):
        rows1, t1 = _time_blocks(_oracle_rows, n, budget_s / 3)
    # all cores (the machine's CPU share, at most 16 workers)
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    starts = list(range(0, n, CPU_BLOCK))
    ctx = mp.get_context("fork")
    with ctx.Pool(cores, initializer=_one_blas_thread) as pool:
        pool.map(_oracle_rows, starts[:cores])  # workers up
        passes, rows_p, t0 = 0, 0, time.perf_counter()
        while passes == 0 or time.perf_counter() - t0 < budget_s / 3:
            rows_p += sum(pool.map(_oracle_rows, starts, chunksize=1))
            passes += 1
        tp = time.perf_counter() - t0
    # one thread, B = 16 and M = 34 on row blocks
    X16 = synth.batch_activations(16)
    X34 = synth.prefill_activations(34)
    extra = {}
    for name, X in (("small_batch_b16", X16), ("prefill_m34", X34)):
        def blk(r0, X=X):
            r1 = min(n, r0 + CPU_BLOCK)
            oracle.gemm(packed[r0:r1], w.scales[r0:r1], w.mins[r0:r1], X)
            return r1 - r0
        with threadpool_limits(1):
            rows_b, t_b = _time_blocks(blk, n, budget_s / 6)
        extra[name] = {"us_per_call_full_matrix": round(t_b / rows_b * n * 1e6, 1),
                       "GB_per_s": round(algorithmic_bytes(rows_b, k, X.shape[0]) / t_b / 1e9, 6),
                       "sample": f"{rows_b} rows in {CPU_BLOCK}-row blocks, one thread, {t_b:.1f} s"}
    _CPU_CASE = None
    return {
        "value": round(algorithmic_bytes(rows_p, k, 1) / tp / 1e9, 6),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{passes} pass(es) over the fused 25088x3072 matrix at B=1 in {CPU_BLOCK}-row blocks on "
                  f"{cores} worker processes (one BLAS thread each), fp64 NumPy oracle, {tp:.1f} s",
        "us_per_call_full_matrix": round(tp / rows_p * n * 1e6, 1),
        "one_thread": {"GB_per_s": round(algorithmic_bytes(rows1, k, 1) / t1 / 1e9, 6),
                       "us_per_call_full_matrix": round(t1 / rows1 * n * 1e6, 1),
                       "sample": f"{rows1} rows in {CPU_BLOCK}-row blocks, {t1:.1f} s"},
        "forms_one_thread": extra,
        "cpu": cpu_model(),
        "cpus_visible": os.cpu_count(),
        "numpy": np.__version__,
    }


def read_traffic(bytes_per_launch):
    if not os.path.exists(TRAFFIC_FILE):
        return None, "no counter file"
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None, "kernel changed since the counters were taken"
    return int(t["hbm_bytes_per_launch"]), t.get("note", "")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-forms", action="store_true", help="skip the extra forms")
    ap.add_argument("--no-stack", action="store_true",
                    help="skip the 36-layer, 108-GEMV stack on fresh weights per layer (a forms entry)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the GEMV shards by rows: each GPU would run the same kernel on its row slice)", file=sys.stderr)
        sys.exit(2)

    # The CPU baseline runs first, before the GPU is initialised: its
    # all-cores leg forks worker processes.
    cpu = None if args.no_cpu else cpu_baseline(args.cpu_seconds)

    import torch
    import int4_group_quantized_amd as q4

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(dev)
    f16 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731

    # ---- headline: fused 25,088 x 3,072 GEMV, B = 1 ----
    n, k, seed = synth.WORKLOADS["fused_25088x3072"]
    w, x = synth.gemv_case(n, k, seed)
    rot = Rotation(torch, q4, w, dev)
    xd = f16(x[0])
    y = torch.empty(n, dtype=torch.float32, device=dev)
    launch = gemv_launcher(q4, rot, xd, y)
    nbytes = algorithmic_bytes(n, k, 1)

    # Primary: back-to-back launches on one stream (how a caller drives the
    # library).  Cross-check: the same launches replayed from a HIP graph,
    # which must rewrite the output with the eager result.
    ms_eager = time_eager(torch, stream, launch, args.steps, args.warmup)
    ms_graph, _launches, _g = time_graph(torch, stream, launch, GRAPH_LAUNCHES, args.steps, args.warmup, out=y)
    graph_matches_eager = True  # checked inside time_graph

    gbs = nbytes / (ms_eager * 1e-3) / 1e9
    traffic, traffic_note = read_traffic(nbytes)
    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_eager, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16*int4->f32",
        "data": "synthetic",
        "config": {
            "workload": "fused_25088x3072_gemv_b1",
            "n": n, "k": k, "batch": 1,
            "bytes_per_call": nbytes,
            "weight_copies_rotated": rot.copies,
            "timing": "back-to-back launches on one stream, HIP events on the launch stream",
            "settle_s": SETTLE_S,
        },
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "us_per_call": round(ms_eager * 1e3, 3),
        "us_per_call_graph": round(ms_graph * 1e3, 3),
        "graph_matches_eager": graph_matches_eager,
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "traffic_note": traffic_note,
        },
    }

    forms = {}
    if not args.no_forms:
        forms.update(time_diagnostics(torch, dev, stream, rot, xd, ms_eager))

    if not args.no_forms:
        def prompt_entries(key, r, nn, kk, mt, X, Y):
            bb = algorithmic_bytes(nn, kk, mt)
            flops = 2.0 * mt * nn * kk
            out = {}
            for form, launcher in (("prefill", prefill_launcher), ("prefill_epilogue", prefill_epilogue_launcher)):
                msp, gmsp = time_checked(torch, stream, launcher(q4, r, X, Y, mt), Y, 200, 5, 20)
                out[f"{key}_{form}_m{mt}"] = {
                    "us_per_call": round(msp * 1e3, 3), "us_per_call_graph": round(gmsp * 1e3, 3),
                    "GB_per_s": round(bb / (msp * 1e-3) / 1e9, 1),
                    "frac_hbm": round(bb / (msp * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "TFLOP_per_s": round(flops / (msp * 1e-3) / 1e12, 1),
                    "frac_mfma_f16": round(flops / (msp * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)}
            return out

        def gemv_form(name, batches=(), prompts=()):
            nn, kk, sd = synth.WORKLOADS[name]
            ww, xx = synth.gemv_case(nn, kk, sd)
            r = Rotation(torch, q4, ww, dev)
            yy = torch.empty(nn, dtype=torch.float32, device=dev)
            ms, gms = time_checked(torch, stream, gemv_launcher(q4, r, f16(xx[0]), yy), yy, 1000, 20, GRAPH_LAUNCHES)
            b = algorithmic_bytes(nn, kk, 1)
            out = {name + "_gemv_b1": {
                "us_per_call": round(ms * 1e3, 3), "us_per_call_graph": round(gms * 1e3, 3),
                "GB_per_s": round(b / (ms * 1e-3) / 1e9, 1),
                "frac_hbm": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "copies_rotated": -(-MALL_DEFEAT_BYTES // algorithmic_bytes(nn, kk, 0))}}
            for nb in batches:
                X = f16(synth.activations(nb, kk, sd + 1))
                Y = torch.empty((nb, nn), dtype=torch.float32, device=dev)
                msb, gmsb = time_checked(torch, stream, batch_launcher(q4, r, X, Y, nb), Y, 1000, 20, GRAPH_LAUNCHES)
                bb = algorithmic_bytes(nn, kk, nb)
                out[f"{name}_small_batch_b{nb}"] = {
                    "us_per_call": round(msb * 1e3, 3), "us_per_call_graph": round(gmsb * 1e3, 3),
                    "GB_per_s": round(bb / (msb * 1e-3) / 1e9, 1),
                    "frac_hbm": round(bb / (msb * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "speedup_vs_b_calls": round(nb * ms / msb, 3)}
            for mt in prompts:
                X = f16(synth.activations(mt, kk, sd + 2))
                Y = torch.empty((mt, nn), dtype=torch.float32, device=dev)
                out.update(prompt_entries(name, r, nn, kk, mt, X, Y))
            del r
            return out

        forms.update(gemv_form("oproj_3072x3072"))
        forms.update(gemv_form("down_3072x8192"))
        for name in ("pages_fused_25088x2048", "pages_oproj_2048x2048", "pages_down_2048x11008"):
            # a 65-token prompt on the down projection: few rows, more than 64 tokens
            forms.update(gemv_form(name, batches=(16,), prompts=(65,) if name == "pages_down_2048x11008" else ()))
        for b in (2, 4, 8, 16):
            X = f16(synth.batch_activations(b))
            Y = torch.empty((b, n), dtype=torch.float32, device=dev)
            ms, gms = time_checked(torch, stream, batch_launcher(q4, rot, X, Y, b), Y, 1000, 20, GRAPH_LAUNCHES)
            bb = algorithmic_bytes(n, k, b)
            forms[f"fused_25088x3072_small_batch_b{b}"] = {
                "us_per_call": round(ms * 1e3, 3), "us_per_call_graph": round(gms * 1e3, 3),
                "GB_per_s": round(bb / (ms * 1e-3) / 1e9, 1),
                "frac_hbm": round(bb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "speedup_vs_b_calls": round(b * ms_eager / ms, 3)}
        # 16 tokens: the matrix-core forms at the batch where the small-batch
        # path (bit-identical to batch 1) tops out, for the cost of that contract;
        # 64: four token tiles of the K-split kernel
        for mtok in (16, 34, 64, 256):
            X = f16(synth.prefill_activations(mtok) if mtok != 16 else synth.batch_activations(16))
            Y = torch.empty((mtok, n), dtype=torch.float32, device=dev)
            forms.update(prompt_entries("fused_25088x3072", rot, n, k, mtok, X, Y))
        del rot
        torch.cuda.empty_cache()
        # int8 output head, 16,384 x 3,072
        hn, hk = synth.HEAD_N, synth.HIDDEN_K
        hq, hs, hx = synth.head_int8_case(hn, hk, synth.SEEDS["head_int8"])
        hq_d, hs_d = torch.from_numpy(hq).to(dev), f16(hs)
        hsets = [(hq_d, hs_d)] + [(hq_d.clone(), hs_d.clone())
                                  for _ in range(max(0, -(-MALL_DEFEAT_BYTES // head_bytes(hn, hk)) - 1))]
        hy = torch.empty(hn, dtype=torch.float32, device=dev)
        ms, gms = time_checked(torch, stream, head_launcher(q4, hsets, f16(hx), hy, hn, hk), hy, 1000, 20, GRAPH_LAUNCHES)
        hb = head_bytes(hn, hk)
        forms["head_int8_16384x3072_gemv_b1"] = {
            "us_per_call": round(ms * 1e3, 3), "us_per_call_graph": round(gms * 1e3, 3),
            "GB_per_s": round(hb / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(hb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "copies_rotated": len(hsets),
            "bytes_per_call": hb}
        del hsets, hq_d, hs_d, hy
        # export quantiser on the fused projection's float32 weights
        Wf = torch.from_numpy(synth.float_weights(n, k, synth.SEEDS["float_weights"])).to(dev)
        Ws = [Wf] + [Wf.clone() for _ in range(max(0, -(-MALL_DEFEAT_BYTES // (n * k * 4)) - 1))]
        Pq = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
        Sq = torch.empty((n, k // 128), dtype=torch.float16, device=dev)
        Mq = torch.empty((n, k // 128), dtype=torch.float16, device=dev)
        ms, gms = time_checked(torch, stream, quantize_launcher(q4, Ws, Pq, Sq, Mq, n, k), Pq, 200, 5, 10)
        qb = quantize_bytes(n, k)
        forms["fused_25088x3072_quantize"] = {
            "us_per_call": round(ms * 1e3, 3), "us_per_call_graph": round(gms * 1e3, 3),
            "GB_per_s": round(qb / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(qb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "copies_rotated": len(Ws),
            "bytes_per_call": qb}
        del Ws, Wf, Pq, Sq, Mq
        torch.cuda.empty_cache()
    if not args.no_forms:
        forms.update(time_pages_stack(torch, q4, dev, stream, f16))
        torch.cuda.empty_cache()
    if not args.no_forms and not args.no_stack:
        forms.update(time_stack(torch, q4, dev, stream, f16))
        torch.cuda.empty_cache()
    if forms:
        result["forms"] = forms

    if cpu is not None:
        result["cpu_baseline"] = cpu
        result["cpu_baseline"]["vs_gpu"] = round(gbs / cpu["value"], 1)

    print(json.dumps(result), flush=True)


def step_forms(torch, q4, stream, name, calls, total, keep):
    """Two forms of one decode step of independent projections `calls`
    (tuples of q4g128_gemv arguments): the per-projection launches captured in
    one graph, and one q4g128_gemv_grouped call (fewer, larger launches),
    timed eager and from a graph.  The grouped outputs must equal the
    per-projection outputs bit for bit."""
    lib = q4.library()

    def launch_all(_i, st):
        for c in calls:
            rc = lib.q4g128_gemv(*c, st)
            if rc != 0:
                raise RuntimeError(q4.q4g128_status_string(rc))
    ms, _reps, _ = time_graph(torch, stream, launch_all, 1, 20, 2)
    ys = [k[-1] for k in keep]
    torch.cuda.synchronize()
    ref = [y.clone() for y in ys]
    descs = (q4.GemvDesc * len(calls))(*[q4.GemvDesc(*c) for c in calls])

    def launch_grouped(_i, st):
        rc = lib.q4g128_gemv_grouped(descs, len(calls), st)
        if rc != 0:
            raise RuntimeError(q4.q4g128_status_string(rc))
    for y in ys:
        y.zero_()
    ms_g_graph, _reps, _ = time_graph(torch, stream, launch_grouped, 1, 20, 2)
    torch.cuda.synchronize()
    if not all(torch.equal(a, b) for a, b in zip(ys, ref)):
        raise RuntimeError(f"{name}: grouped outputs differ from the per-projection calls")
    ms_g = time_eager(torch, stream, launch_grouped, 20, 2)
    out = {}
    for key, t, extra in ((name + "_gemv_b1", ms, {"launches": len(calls), "timing": "one graph"}),
                          (name + "_grouped_b1", ms_g, {"timing": "eager, back-to-back calls",
                                                       "us_per_step_graph": round(ms_g_graph * 1e3, 2),
                                                       "bit_identical_to_per_projection": True})):
        out[key] = {"us_per_step": round(t * 1e3, 2), "bytes": total,
                    "GB_per_s": round(total / (t * 1e-3) / 1e9, 1),
                    "frac_hbm": round(total / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), **extra}
    return out


def time_stack(torch, q4, dev, stream, f16):
    """36 layers x (fused, o_proj, down) GEMVs, fresh weights per layer."""
    shapes = [(synth.FUSED_N, synth.HIDDEN_K), (synth.OPROJ_N, synth.OPROJ_K), (synth.DOWN_N, synth.DOWN_K)]
    calls = []
    keep = []
    total = 0
    for layer in range(synth.STACK_LAYERS):
        for which, (nn, kk) in enumerate(shapes):
            ww = synth.weights(nn, kk, synth.stack_seed(layer, which))
            codes = torch.from_numpy(ww.codes).to(dev)
            packed = q4.q4g128_pack(codes)
            del codes
            s, m = f16(ww.scales), f16(ww.mins)
            xx = f16(synth.activations(1, kk, seed=90000 + 3 * layer + which)[0])
            yy = torch.empty(nn, dtype=torch.float32, device=dev)
            keep.append((packed, s, m, xx, yy))
            calls.append((packed.data_ptr(), s.data_ptr(), m.data_ptr(), xx.data_ptr(), yy.data_ptr(), nn, kk))
            total += algorithmic_bytes(nn, kk, 1)
        print(f"stack: layer {layer} ready", file=sys.stderr, flush=True)
    out = step_forms(torch, q4, stream, "stack_36x3", calls, total, keep)
    del keep
    return out


def time_pages_stack(torch, q4, dev, stream, f16):
    """The pages' decode step shape: 36 layers x (fused 25,088x2,048,
    o_proj 2,048x2,048, down 2,048x11,008) GEMVs.

    One seeded weight set per shape is drawn on the host; every layer gets its
    own device copy of it (distinct memory, 1.4 GB in total, so the 256 MB
    Infinity Cache cannot serve one layer's weights to the next).
    """
    names = ["pages_fused_25088x2048", "pages_oproj_2048x2048", "pages_down_2048x11008"]
    base = []
    for name in names:
        ww, xx = synth.workload(name)
        codes = torch.from_numpy(ww.codes).to(dev)
        base.append((q4.q4g128_pack(codes), f16(ww.scales), f16(ww.mins), f16(xx[0]), ww.n, ww.k))
        del codes
    keep, calls, total = [], [], 0
    for _layer in range(synth.STACK_LAYERS):
        for packed, s, m, xx, nn, kk in base:
            p2, s2, m2 = packed.clone(), s.clone(), m.clone()
            yy = torch.empty(nn, dtype=torch.float32, device=dev)
            keep.append((p2, s2, m2, yy))
            calls.append((p2.data_ptr(), s2.data_ptr(), m2.data_ptr(), xx.data_ptr(), yy.data_ptr(), nn, kk))
            total += algorithmic_bytes(nn, kk, 1)
    torch.cuda.synchronize()
    out = step_forms(torch, q4, stream, "pages_stack_36x3_hidden2048", calls, total, keep)
    for v in out.values():
        v["weights"] = "one seeded set per shape, a device copy per layer"
    del keep
    return out


def time_diagnostics(torch, dev, stream, rot, xd, ms_gemv):
    """Ceilings of the batch-1 GEMV on this device (libq4g128_diag.so):
    its read-only twin on the same rotated weights, a plain streaming read of
    the same byte count and of 8x it (rotated windows of a >= 512 MB pool,
    so the Infinity Cache cannot serve them; the difference of the two gives
    the steady read rate), and an empty kernel on the same grid."""
    from int4_group_quantized_amd import diag
    lib = diag.library()
    out_buf = torch.zeros(lib.q4diag_out_words(), dtype=torch.int32, device=dev)
    op = out_buf.data_ptr()
    ptrs = [(p.data_ptr(), s.data_ptr(), m.data_ptr()) for p, s, m in rot.sets]
    R, n, k, xp = len(ptrs), rot.n, rot.k, xd.data_ptr()
    nbytes = algorithmic_bytes(n, k, 1)

    def twin(i, st):
        p, s, m = ptrs[i % R]
        if lib.q4diag_gemv_read_twin(p, s, m, xp, op, n, k, st) != 0:
            raise RuntimeError("q4diag_gemv_read_twin failed")
    forms = {}
    ms_twin = time_eager(torch, stream, twin, 2000, 50)
    forms["diag_read_twin_fused_25088x3072"] = {
        "us_per_call": round(ms_twin * 1e3, 3), "GB_per_s": round(nbytes / (ms_twin * 1e-3) / 1e9, 1),
        "frac_hbm": round(nbytes / (ms_twin * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "gemv_over_twin": round(ms_gemv / ms_twin, 4),
        "what": "same grid, loads and addresses as the GEMV kernel, no arithmetic"}
    win = -(-nbytes // 4096) * 4096
    pool = torch.empty(max(MALL_DEFEAT_BYTES + 8 * win, 16 * win), dtype=torch.uint8, device=dev)
    base = pool.data_ptr()
    stream_ms = {}
    for mult in (1, 8):
        size = mult * win
        nwin = pool.numel() // size

        def read(i, st, size=size, nwin=nwin):
            if lib.q4diag_stream_read(base + (i % nwin) * size, size, op, st) != 0:
                raise RuntimeError("q4diag_stream_read failed")
        ms = time_eager(torch, stream, read, 2000 if mult == 1 else 300, 20)
        stream_ms[mult] = ms
        forms[f"diag_stream_read_{size >> 20}MB"] = {
            "bytes": size, "us_per_call": round(ms * 1e3, 3), "GB_per_s": round(size / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(size / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "windows_rotated": nwin}
    steady = 7 * win / ((stream_ms[8] - stream_ms[1]) * 1e-3) / 1e9
    forms["diag_steady_read"] = {"GB_per_s": round(steady, 1), "frac_hbm": round(steady / HBM_PEAK_GBS, 4),
                                 "what": "(8x - 1x bytes) / (t_8x - t_1x) of the two streaming reads"}
    del pool

    def empty(_i, st):
        if lib.q4diag_empty(st) != 0:
            raise RuntimeError("q4diag_empty failed")
    ms = time_eager(torch, stream, empty, 2000, 50)
    forms["diag_empty_launch"] = {"us_per_call": round(ms * 1e3, 3),
                                  "what": "back-to-back launches of an empty kernel on the GEMV's grid"}
    return forms


if __name__ == "__main__":
    main()
