#!/usr/bin/env python3
"""Benchmark of the int4 group-128 GEMV on one MI355X.

One step = one q4g128_gemv call on the fused 25,088 x 3,072 projection at
batch 1 (packed weights + fp16 scales + fp16 mins + fp16 activations in,
fp32 out).  Weight copies totalling >= 512 MB are rotated so that the 256 MB
Infinity Cache cannot serve repeated calls.  The timed launches go back to
back on the benchmark's stream, bracketed by HIP events on that stream; the
same launches replayed from a HIP graph are timed as a cross-check that must
reproduce the eager output.

Prints ONE JSON line.  Extra forms (other shapes, small batch, prompt
processing, the int8 output head, the export quantiser, the pages' 108-launch
step and the 36-layer stack) are reported under "forms".
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
KERNEL_SOURCES = ["int4_group_quantized_amd/csrc/gemv.hip", "int4_group_quantized_amd/csrc/q4_device.hpp"]


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
    """Eager ms per call, after checking that a HIP graph of the same launches rewrites `out` identically."""
    time_graph(torch, stream, launch, n_graph, n_graph, warmup, out=out)
    return time_eager(torch, stream, launch, steps, warmup)


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
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.machine()


def cpu_baseline(budget_s: float):
    """The fp64 oracle, single-threaded, on row blocks of the fused workload.

    Blocks of 4,096 rows are processed in order, wrapping around, until the
    time budget is used; the packed bytes are prepared outside the timing.
    """
    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    w, x = synth.workload("fused_25088x3072")
    packed = oracle.pack(w.codes)
    block = 4096
    rows_done = 0
    t_total = 0.0
    ctx = threadpool_limits(1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        r0 = 0
        while t_total < budget_s:
            r1 = min(w.n, r0 + block)
            t = time.perf_counter()
            oracle.gemv(packed[r0:r1], w.scales[r0:r1], w.mins[r0:r1], x[0])
            t_total += time.perf_counter() - t
            rows_done += r1 - r0
            r0 = 0 if r1 == w.n else r1
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    nbytes = algorithmic_bytes(rows_done, w.k, 1)
    return {
        "value": round(nbytes / t_total / 1e9, 6),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{rows_done} rows ({rows_done / w.n:.2f} passes) of the fused 25088x3072 matrix in "
                  f"4096-row blocks, B=1, fp64 NumPy oracle, one thread, {t_total:.1f} s",
        "us_per_call_full_matrix": round(t_total / rows_done * w.n * 1e6, 1),
        "cpu": cpu_model(),
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
        def gemv_form(name, batches=()):
            nn, kk, sd = synth.WORKLOADS[name]
            ww, xx = synth.gemv_case(nn, kk, sd)
            r = Rotation(torch, q4, ww, dev)
            yy = torch.empty(nn, dtype=torch.float32, device=dev)
            ms = time_checked(torch, stream, gemv_launcher(q4, r, f16(xx[0]), yy), yy, 1000, 20, GRAPH_LAUNCHES)
            b = algorithmic_bytes(nn, kk, 1)
            out = {name + "_gemv_b1": {
                "us_per_call": round(ms * 1e3, 3), "GB_per_s": round(b / (ms * 1e-3) / 1e9, 1),
                "frac_hbm": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "copies_rotated": -(-MALL_DEFEAT_BYTES // algorithmic_bytes(nn, kk, 0))}}
            for nb in batches:
                X = f16(synth.activations(nb, kk, sd + 1))
                Y = torch.empty((nb, nn), dtype=torch.float32, device=dev)
                msb = time_checked(torch, stream, batch_launcher(q4, r, X, Y, nb), Y, 1000, 20, GRAPH_LAUNCHES)
                bb = algorithmic_bytes(nn, kk, nb)
                out[f"{name}_small_batch_b{nb}"] = {
                    "us_per_call": round(msb * 1e3, 3), "GB_per_s": round(bb / (msb * 1e-3) / 1e9, 1),
                    "frac_hbm": round(bb / (msb * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "speedup_vs_b_calls": round(nb * ms / msb, 3)}
            del r
            return out

        forms.update(gemv_form("oproj_3072x3072"))
        forms.update(gemv_form("down_3072x8192"))
        for name in ("pages_fused_25088x2048", "pages_oproj_2048x2048", "pages_down_2048x11008"):
            forms.update(gemv_form(name, batches=(16,)))
        for b in (2, 4, 8, 16):
            X = f16(synth.batch_activations(b))
            Y = torch.empty((b, n), dtype=torch.float32, device=dev)
            ms = time_checked(torch, stream, batch_launcher(q4, rot, X, Y, b), Y, 1000, 20, GRAPH_LAUNCHES)
            bb = algorithmic_bytes(n, k, b)
            forms[f"fused_25088x3072_small_batch_b{b}"] = {
                "us_per_call": round(ms * 1e3, 3), "GB_per_s": round(bb / (ms * 1e-3) / 1e9, 1),
                "frac_hbm": round(bb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "speedup_vs_b_calls": round(b * ms_eager / ms, 3)}
        for mtok in (34, 256):
            X = f16(synth.prefill_activations(mtok))
            Y = torch.empty((mtok, n), dtype=torch.float32, device=dev)
            ms = time_checked(torch, stream, prefill_launcher(q4, rot, X, Y, mtok), Y, 200, 5, 20)
            bb = algorithmic_bytes(n, k, mtok)
            flops = 2.0 * mtok * n * k
            forms[f"fused_25088x3072_prefill_m{mtok}"] = {
                "us_per_call": round(ms * 1e3, 3), "GB_per_s": round(bb / (ms * 1e-3) / 1e9, 1),
                "frac_hbm": round(bb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "TFLOP_per_s": round(flops / (ms * 1e-3) / 1e12, 1),
                "frac_mfma_f16": round(flops / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)}
            ms = time_checked(torch, stream, prefill_epilogue_launcher(q4, rot, X, Y, mtok), Y, 200, 5, 20)
            forms[f"fused_25088x3072_prefill_epilogue_m{mtok}"] = {
                "us_per_call": round(ms * 1e3, 3), "GB_per_s": round(bb / (ms * 1e-3) / 1e9, 1),
                "frac_hbm": round(bb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "TFLOP_per_s": round(flops / (ms * 1e-3) / 1e12, 1),
                "frac_mfma_f16": round(flops / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)}
        del rot
        torch.cuda.empty_cache()
        # int8 output head, 16,384 x 3,072
        hn, hk = synth.HEAD_N, synth.HIDDEN_K
        hq, hs, hx = synth.head_int8_case(hn, hk, synth.SEEDS["head_int8"])
        hq_d, hs_d = torch.from_numpy(hq).to(dev), f16(hs)
        hsets = [(hq_d, hs_d)] + [(hq_d.clone(), hs_d.clone())
                                  for _ in range(max(0, -(-MALL_DEFEAT_BYTES // head_bytes(hn, hk)) - 1))]
        hy = torch.empty(hn, dtype=torch.float32, device=dev)
        ms = time_checked(torch, stream, head_launcher(q4, hsets, f16(hx), hy, hn, hk), hy, 1000, 20, GRAPH_LAUNCHES)
        hb = head_bytes(hn, hk)
        forms["head_int8_16384x3072_gemv_b1"] = {
            "us_per_call": round(ms * 1e3, 3), "GB_per_s": round(hb / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(hb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "copies_rotated": len(hsets),
            "bytes_per_call": hb}
        del hsets, hq_d, hs_d, hy
        # export quantiser on the fused projection's float32 weights
        Wf = torch.from_numpy(synth.float_weights(n, k, synth.SEEDS["float_weights"])).to(dev)
        Ws = [Wf] + [Wf.clone() for _ in range(max(0, -(-MALL_DEFEAT_BYTES // (n * k * 4)) - 1))]
        Pq = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
        Sq = torch.empty((n, k // 128), dtype=torch.float16, device=dev)
        Mq = torch.empty((n, k // 128), dtype=torch.float16, device=dev)
        ms = time_checked(torch, stream, quantize_launcher(q4, Ws, Pq, Sq, Mq, n, k), Pq, 200, 5, 10)
        qb = quantize_bytes(n, k)
        forms["fused_25088x3072_quantize"] = {
            "us_per_call": round(ms * 1e3, 3), "GB_per_s": round(qb / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(qb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "copies_rotated": len(Ws),
            "bytes_per_call": qb}
        del Ws, Wf, Pq, Sq, Mq
        torch.cuda.empty_cache()
    if not args.no_forms:
        forms["pages_stack_36x3_hidden2048_gemv_b1"] = time_pages_stack(torch, q4, dev, stream, f16)
        torch.cuda.empty_cache()
    if not args.no_forms and not args.no_stack:
        forms["stack_36x3_gemv_b1"] = time_stack(torch, q4, dev, stream, f16)
        torch.cuda.empty_cache()
    if forms:
        result["forms"] = forms

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
        result["cpu_baseline"]["vs_gpu"] = round(gbs / result["cpu_baseline"]["value"], 1)

    print(json.dumps(result), flush=True)


def time_stack(torch, q4, dev, stream, f16):
    """36 layers x (fused, o_proj, down) GEMVs, fresh weights per layer, one graph."""
    shapes = [(synth.FUSED_N, synth.HIDDEN_K), (synth.OPROJ_N, synth.OPROJ_K), (synth.DOWN_N, synth.DOWN_K)]
    lib = q4.library()
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

    def launch_all(_i, st):
        for c in calls:
            rc = lib.q4g128_gemv(*c, st)
            if rc != 0:
                raise RuntimeError(q4.q4g128_status_string(rc))
    ms, reps, _ = time_graph(torch, stream, launch_all, 1, 20, 2)
    return {"us_per_step": round(ms * 1e3, 2), "launches": len(calls), "bytes": total,
            "GB_per_s": round(total / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(total / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def time_pages_stack(torch, q4, dev, stream, f16):
    """The pages' decode step shape: 36 layers x (fused 25,088x2,048,
    o_proj 2,048x2,048, down 2,048x11,008) GEMVs in one graph of 108 launches.

    One seeded weight set per shape is drawn on the host; every layer gets its
    own device copy of it (distinct memory, 1.4 GB in total, so the 256 MB
    Infinity Cache cannot serve one layer's weights to the next).
    """
    names = ["pages_fused_25088x2048", "pages_oproj_2048x2048", "pages_down_2048x11008"]
    lib = q4.library()
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

    def launch_all(_i, st):
        for c in calls:
            rc = lib.q4g128_gemv(*c, st)
            if rc != 0:
                raise RuntimeError(q4.q4g128_status_string(rc))
    ms, _reps, _ = time_graph(torch, stream, launch_all, 1, 20, 2)
    out = {"us_per_step": round(ms * 1e3, 2), "launches": len(calls), "bytes": total,
           "GB_per_s": round(total / (ms * 1e-3) / 1e9, 1),
           "frac_hbm": round(total / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "weights": "one seeded set per shape, a device copy per layer"}
    del keep
    return out


if __name__ == "__main__":
    main()
