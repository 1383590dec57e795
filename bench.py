#!/usr/bin/env python3
"""Benchmark of the block-quantized decode GEMV library on one MI355X.

Headline: effective weight GB/s of the M=1 decode GEMVs at dense-layer shapes
-- Q8_0 and Q4_K weights, K = 4096, N = 4096, 12288 and 24576 (six GEMVs per
step; each is the activation quantizer plus the format's GEMV kernel) --
and its fraction of the 8 TB/s HBM3E peak. One step = those six calls once,
each on its own fp32 N(0, 1) activation vector. Weights rotate through
enough copies (> 2 GiB) that every step reads them from HBM, not from the
256 MB Infinity Cache or the L2s.

Also reported (same run, after the timed region): microseconds per fused
FFN sublayer (hidden 4096, intermediate 12288, Q4_K gate|up + Q6_K down),
the IQ4_NL lm_head (4096 -> 248320), the Q4_0 2048 x 2048 GEMV, the Q5_K and
IQ4_XS GEMVs (4096 -> 12288), the Q4_K GEMV with 16-bit activations
(4096 -> 12288), the MoE layer (also with 16-bit activations) (256 experts, top-8 + shared,
hidden 2048, intermediate 512) at M=1 and M=16, and the two-stage decode
attention (16 query heads, 2 key/value heads, dimension 256) at 4K and 32K
cached tokens.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12           # B/s, MI355X HBM3E
ROTATE_BYTES = 2 * 2 ** 30  # weights touched per rotation cycle
METRIC = "effective weight GB/s (% of HBM peak) for M=1 quant GEMV; µs per fused FFN"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def copies_for(nbytes, cap=4096):
    return int(min(cap, max(2, -(-ROTATE_BYTES // max(1, nbytes)))))


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def rotated(w_np, r):
    import torch
    base = dev(w_np)
    return [base] + [base.clone() for _ in range(r - 1)]


def time_calls(fn, calls, warm=5):
    """Mean microseconds per call of fn(i), back to back, with HIP events."""
    import torch
    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(calls):
        fn(warm + i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / calls


def graph_of(fn, n):
    """Capture fn(0..n-1) (launches on torch's current stream) in one HIP graph."""
    import torch
    for i in range(n):          # eager warm-up: one-time host set-up happens outside capture
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    torch.cuda.synchronize()
    return g


def time_graph(g, n_inner, reps, warm=2, trials=3):
    """Microseconds per inner call: the median over `trials` windows of
    `reps` replays of graph g each (a single short window is at the mercy
    of the clocks the previous work left behind)."""
    import torch
    for _ in range(warm):
        g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(trials):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) * 1e3 / (reps * n_inner))
    return float(np.median(out))


# The dominant kernel of the step: the Q8_0 GEMV with the activation
# quantizer fused into its prologue (one launch per call at K = 4096).
GEMV_SOURCES = ("gemv.hip", "formats.cuh", "common.cuh", "internal.h")
MFMA_SOURCES = ("mfma.hip", "quant.hip", "common.cuh", "internal.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemv_q8_0_k4096.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_counters_m32.json")
INT8_MFMA_PEAK = 5.0e15    # dense int8 ops/s, MI355X
SIMDS = 256 * 4            # 256 CUs x 4 SIMDs
XCDS = 8


def source_digest(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "block_quant_gemv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def kernel_source_digest():
    return source_digest(GEMV_SOURCES)


def recorded_traffic():
    """HBM bytes per launch of the dominant kernel from recorded counter runs
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's counts), or None when
    none is recorded or the kernel source changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_digest") != kernel_source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


def recorded_mfma():
    """Per-dispatch matrix-core counters of the M=32 GEMM kernels, or None
    when none are recorded or the kernel sources changed since."""
    try:
        with open(MFMA_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_digest") != source_digest(MFMA_SOURCES):
        return None
    return rec


COPY_BYTES = 256 * 2 ** 20    # one --calibrate-copy launch reads and writes this many bytes


def _pmc_rows(path, counter):
    """(kernel name, value) per dispatch from a rocprofv3 --pmc output: its
    SQLite database (*_results.db, view counters_collection) or its
    counter_collection CSV."""
    if path.endswith(".db"):
        import sqlite3
        con = sqlite3.connect(path)
        try:
            rows = con.execute("SELECT kernel_name, value FROM counters_collection WHERE counter_name = ?",
                               (counter,)).fetchall()
        finally:
            con.close()
        return [(n, float(v)) for n, v in rows]
    import csv
    out = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") == counter:
                out.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return out


def record_traffic(fetch_out, write_out, copy_fetch_out, copy_write_out):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the dominant GEMV
    kernel, each scaled by what the same counter reads for a plain device copy
    of COPY_BYTES (its largest dispatch), summed into HBM bytes per launch."""
    def scale(rows):
        kib = max(v for _, v in rows)
        return COPY_BYTES / (kib * 1024.0)

    def gemv_mean(rows):
        # --only-dominant runs no GEMV kernel other than the Q8_0 one
        vals = [v for name, v in rows if "gemv_kernel" in name]
        return sum(vals) / len(vals), len(vals)

    fs = scale(_pmc_rows(copy_fetch_out, "FETCH_SIZE"))
    ws_ = scale(_pmc_rows(copy_write_out, "WRITE_SIZE"))
    fk, nf = gemv_mean(_pmc_rows(fetch_out, "FETCH_SIZE"))
    wk, nw = gemv_mean(_pmc_rows(write_out, "WRITE_SIZE"))
    rec = {"kernel_source_digest": kernel_source_digest(),
           "fetch_kib_per_launch": round(fk, 1), "write_kib_per_launch": round(wk, 1),
           "fetch_scale": round(fs, 4), "write_scale": round(ws_, 4), "dispatches": [nf, nw],
           "hbm_bytes_per_launch": round(fk * 1024 * fs + wk * 1024 * ws_)}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))
    return 0


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_I8", "SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES",
                 "SQ_BUSY_CYCLES", "SQ_INSTS_VALU", "GRBM_GUI_ACTIVE")


def record_mfma(path):
    """Matrix-core counters of the M=32 GEMM kernels from one rocprofv3 --pmc
    run of `bench.py --leg m32` (counters MFMA_COUNTERS): per-dispatch means
    per kernel instance, with the derived int8 operations (MOPS_I8 counts
    operations / 512) and the matrix-core busy fraction (busy cycles summed
    over the 1024 SIMDs / (SIMDs x GUI-active cycles per XCD))."""
    per = {}
    for c in MFMA_COUNTERS:
        for name, v in _pmc_rows(path, c):
            if "gemm32_kernel" not in name:
                continue
            key = "q4_k" if "gemm32_kernel<3," in name else "q6_k" if "gemm32_kernel<4," in name else name
            per.setdefault(key, {}).setdefault(c, []).append(v)
    rec = {"kernel_source_digest": source_digest(MFMA_SOURCES), "counters": list(MFMA_COUNTERS), "kernels": {}}
    for key, d in per.items():
        mean = {c: sum(v) / len(v) for c, v in d.items()}
        ops = mean["SQ_INSTS_VALU_MFMA_MOPS_I8"] * 512
        gui = mean["GRBM_GUI_ACTIVE"] / XCDS
        rec["kernels"][key] = {
            "dispatches": len(d["SQ_INSTS_MFMA"]),
            "mean_per_dispatch": {c: round(v, 1) for c, v in mean.items()},
            "int8_ops_per_dispatch": round(ops),
            "mfma_busy_frac": round(mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * gui), 4) if gui else None,
            "valu_insts_per_mfma": round(mean["SQ_INSTS_VALU"] / max(1.0, mean["SQ_INSTS_MFMA"]), 2),
        }
    with open(MFMA_FILE, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))
    return 0


class Clocks:
    """Samples the GPU's clocks with amd-smi (about every 0.2 s, in a thread)
    and files each sample under the measurement leg running at the time."""

    def __init__(self, enabled=True):
        import threading
        self.leg = None
        self.samples = []
        self.reason = None
        self._stop = threading.Event()
        self._thread = None
        if enabled and self._sample() is None:
            self.reason = self.reason or "amd-smi gave no clock reading"
        elif not enabled:
            self.reason = "disabled"

    def _sample(self):
        import subprocess
        try:
            r = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "--json"], capture_output=True,
                               text=True, timeout=5)
            d = json.loads(r.stdout)
            c = d["gpu_data"][0]["clock"] if isinstance(d, dict) else d[0]["clock"]
            gfx = [v["clk"]["value"] for k, v in c.items()
                   if k.startswith("gfx_") and isinstance(v.get("clk"), dict)]
            mem = c.get("mem_0", {}).get("clk")
            return (sum(gfx) / len(gfx), min(gfx), mem["value"] if isinstance(mem, dict) else None)
        except Exception as e:  # no amd-smi, no JSON, another layout: no clock record
            self.reason = f"amd-smi: {type(e).__name__}"
            return None

    def _run(self):
        while not self._stop.is_set():
            leg = self.leg
            v = self._sample()
            if v is not None and leg is not None:
                self.samples.append((leg,) + v)
            self._stop.wait(0.2)

    def start(self):
        import threading
        if self.reason is None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def stop(self):
        self._stop.set()
        if self._thread:
            self._thread.join(timeout=10)

    def summary(self):
        if self.reason is not None and not self.samples:
            return {"available": False, "reason": self.reason}
        out = {"available": True, "tool": "amd-smi metric -g 0 -c --json", "legs": {}}
        for leg in dict.fromkeys(s[0] for s in self.samples):
            mean = sorted(s[1] for s in self.samples if s[0] == leg)
            low = [s[2] for s in self.samples if s[0] == leg]
            mem = [s[3] for s in self.samples if s[0] == leg and s[3] is not None]
            out["legs"][leg] = {"samples": len(mean), "gfx_mhz_median": round(mean[len(mean) // 2], 1),
                                "gfx_mhz_min": round(min(low), 1), "gfx_mhz_max": round(max(mean), 1),
                                "mem_mhz": round(sum(mem) / len(mem), 1) if mem else None}
        return out


SUSTAIN_S = 2.0  # seconds of each sustained run (--sustain-seconds)


def set_sustain(seconds):
    global SUSTAIN_S
    SUSTAIN_S = float(seconds)


def sustained(graph, n_inner, seconds, clocks, leg):
    """Replay graph back to back for about `seconds` while clocks are
    sampled under `leg`; microseconds per inner call over that window."""
    import torch
    seconds = SUSTAIN_S if seconds is None else seconds
    clocks.leg = leg
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    once = max(1e-6, time.perf_counter() - t0)
    reps = max(2, int(seconds / once))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    clocks.leg = None
    log(f"{leg}: sustained run of {reps} replays done")
    return e0.elapsed_time(e1) * 1e3 / (reps * n_inner), reps * n_inner


def ceiling_us(qg, bufs, reps=4):
    """Microseconds to stream-read one of bufs (all the same size) with the
    library's streaming-read kernel, over a graph of all of them."""
    import torch
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    g = graph_of(lambda i: qg.debug_stream_read(bufs[i], out), len(bufs))
    return time_graph(g, len(bufs), reps=reps)


def cpu_baseline(mats, k, budget_s=12.0):
    """The oracle (dequantize to fp64, fp64 matvec) timed on this host's cores
    over a bounded sample: the first rows of each headline matrix."""
    import synth
    from oracle import gemv as og
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        blas = 1
    rows = 1024
    done_bytes, t_used, reps = 0, 0.0, 0
    samples = []
    for fmt, n in mats:
        w = synth.weights(fmt, rows, k, seed=7)
        x = synth.activations(8, 1, k)
        samples.append((fmt, w, x))
    og.gemv_ref(samples[0][0], samples[0][1], rows, k, samples[0][2])  # warm-up
    while t_used < budget_s:
        for fmt, w, x in samples:
            t0 = time.perf_counter()
            og.gemv_ref(fmt, w, rows, k, x)
            t_used += time.perf_counter() - t0
            done_bytes += rows * synth.row_bytes(fmt, k)
        reps += 1
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {
        "value": done_bytes / t_used / 1e9, "unit": "GB/s", "cores": int(max(1, blas)),
        "kind": "oracle",
        "sample": (f"first {rows} rows of each of the six headline matrices ({reps} passes, "
                   f"{t_used:.1f} s), fp64 dequantize + fp64 matvec; numpy BLAS threads={blas}, "
                   f"host cores available={cores}"),
    }


LEGS = ("ffn", "lm_head", "q4_0_2048", "q5_k_iq4_xs", "s16", "f32act", "m32", "moe", "attn")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 400 steps are about 27 ms of timed work: long enough that the clocks'
    # response to the burst and the replays' start-up are a small part of it
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-clocks", action="store_true")
    ap.add_argument("--sustain-seconds", type=float, default=SUSTAIN_S,
                    help="length of each sustained run (shorter for counter passes, which serialize dispatches)")
    ap.add_argument("--leg", choices=LEGS,
                    help="run one extra measurement alone and print its results (for profiler runs)")
    ap.add_argument("--only-dominant", action="store_true",
                    help="run only the dominant GEMV kernel back to back (for counter runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a plain 256 MiB device copy a few times (counter calibration)")
    ap.add_argument("--record-traffic", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="turn rocprofv3 --pmc counter files into the recorded HBM traffic (no GPU use)")
    ap.add_argument("--record-mfma", metavar="PMC",
                    help="turn a rocprofv3 --pmc run of --leg m32 into the recorded matrix-core counters")
    args = ap.parse_args()
    set_sustain(args.sustain_seconds)
    if args.record_traffic:
        return record_traffic(*args.record_traffic)
    if args.record_mfma:
        return record_mfma(args.record_mfma)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this library has no multi-GPU path).", file=sys.stderr)
        return 2

    import torch
    import block_quant_gemv_amd as qg
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        src = torch.empty(256 * 2 ** 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(8):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copied 8 x 256 MiB")
        return 0
    if args.leg:
        clocks = Clocks(enabled=False)
        print(json.dumps({args.leg: LEG_FNS[args.leg](qg, synth, torch, clocks)}), flush=True)
        return 0

    K = 4096
    mats = [(f, n) for f in ("q8_0", "q4_k") for n in (4096, 12288, 24576)]
    step_bytes = sum(n * synth.row_bytes(f, K) for f, n in mats)
    R = copies_for(step_bytes)
    log(f"setup: 6 matrices, {step_bytes / 1e6:.1f} MB per step, {R} rotating copies")
    plans, ws, xs, ys, W = [], [], [], [], []
    for j, (f, n) in enumerate(mats):
        g = qg.GEMV(f, n, K)
        plans.append(g)
        ws.append(g.workspace(1))
        xs.append(dev(synth.activations(200 + j, 1, K)))
        ys.append(torch.empty((1, n), dtype=torch.float32, device="cuda"))
        skip = args.only_dominant and f != "q8_0"
        W.append(None if skip else rotated(synth.weights(f, n, K, seed=100 + j), R))
    # The dominant kernel is the Q8_0 GEMV with the quantizer fused into its
    # prologue: each Q8_0 call of the step is one launch of it. It runs at the
    # step's three Q8_0 shapes in equal numbers, so its average launch carries
    # the mean of their algorithmic bytes: packed weights + fp32 x + the int8
    # codes, fp32 scales and int32 block sums it writes back + fp32 y.
    dom = [j for j, (f, _) in enumerate(mats) if f == "q8_0"]
    dom_alg = sum(mats[j][1] * synth.row_bytes("q8_0", K) + 4 * K + K + 8 * (K // 32) + 4 * mats[j][1]
                  for j in dom) / len(dom)

    def step(i):
        r = i % R
        for j, g in enumerate(plans):
            g.run(W[j][r], xs[j], y=ys[j], ws=ws[j])

    def dom_launches(i):
        # the dominant kernel's launches of one step
        for j in dom:
            plans[j].run(W[j][i % R], xs[j], y=ys[j], ws=ws[j])

    if args.only_dominant:
        for i in range(args.steps):
            dom_launches(i)
        torch.cuda.synchronize()
        log(f"ran the Q8_0 GEMV launches of {args.steps} steps")
        return 0

    clocks = Clocks(enabled=not args.no_clocks).start()
    # HIP graphs hold the steps (step i on weight copy i mod R); replaying
    # them removes the Python/launch overhead between the kernels, not any of
    # their work. Exactly args.steps steps are timed: full replays of an
    # R-step graph, then one graph of the remaining steps.
    for i in range(args.warmup):
        step(i)
    graph = graph_of(step, R)
    full, rest = divmod(args.steps, R)
    tail = graph_of(step, rest) if rest else None
    steps = full * R + rest
    # One untimed replay of each graph first: a graph's first launch uploads
    # it to the device, a one-time cost that is not part of a step.
    graph.replay()
    if tail is not None:
        tail.replay()
    log(f"timing {steps} steps ({full} replays of a {R}-step graph + {rest})")
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(full):
        graph.replay()
    if tail is not None:
        tail.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / steps
    value = step_bytes / (ms_step * 1e-3) / 1e9
    # The same step graph replayed for about 2 s, with clocks sampled.
    sus_us, sus_steps = sustained(graph, R, None, clocks, "headline_step")
    # Eager (no graph) step time, for reference.
    eager_us = time_calls(lambda i: step(i), 3 * R, warm=R) if not args.no_extras else None

    # Dominant kernel alone: its launches back to back, HIP events on the
    # library's stream (torch's current stream) around a graph of R steps'
    # worth of them.
    gd = graph_of(dom_launches, R)
    dom_us = time_graph(gd, R * len(dom), reps=max(4, 64 // R))
    achieved = dom_alg / (dom_us * 1e-6) / 1e9
    log(f"step {ms_step * 1e3:.1f} us ({wall / steps * 1e3:.3f} ms wall), {value:.0f} GB/s; "
        f"Q8_0 GEMV kernel {dom_us:.2f} us per launch -> {achieved:.0f} GB/s")

    # Per-matrix call times (one qgemv_run each), graph-replayed, beside the
    # streaming-read ceiling: the library's plain read kernel over the same
    # weight copies.
    per = {}
    ceil_step_us = 0.0
    for j, (f, n) in enumerate(mats):
        gj = graph_of(lambda i, j=j: plans[j].run(W[j][i % R], xs[j], y=ys[j], ws=ws[j]), R)
        us = time_graph(gj, R, reps=max(4, 64 // R))
        cus = ceiling_us(qg, W[j])
        ceil_step_us += cus
        b = n * synth.row_bytes(f, K)
        per[f"{f}_{n}x{K}"] = {"us": round(us, 3), "gbps": round(b / (us * 1e-6) / 1e9, 1),
                               "ceiling_us": round(cus, 3), "ceiling_gbps": round(b / (cus * 1e-6) / 1e9, 1),
                               "pct_of_ceiling": round(100 * cus / us, 1)}
        log(f"{f} {n}x{K}: {us:.2f} us; streaming read of the same bytes {cus:.2f} us")
    del gj

    traffic = recorded_traffic()
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "M=1 decode GEMVs, K=4096, Q8_0 and Q4_K weights, N=4096/12288/24576 "
                               "(one qgemv_run per matrix: activation quantizer + GEMV)",
                   "m": 1, "k": K, "n": [4096, 12288, 24576], "formats": ["q8_0", "q4_k"],
                   "weight_bytes_per_step": step_bytes, "rotating_copies": R,
                   "timing": "HIP graphs of exactly `steps` steps, replayed; HIP events"},
        "pct_hbm_peak": round(100 * value * 1e9 / HBM_PEAK, 2),
        "roofline": {"bound": "hbm",
                     "kernel": "gemv_kernel<Q8_0> with the activation quantizer fused "
                               "(M=1, K=4096, N=4096/12288/24576 in equal numbers)",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": round(achieved * 1e9 / HBM_PEAK, 4), "traffic": traffic,
                     "bytes_per_launch": round(dom_alg), "avg_kernel_us": round(dom_us, 3)},
        "streaming_ceiling": {"kernel": "qgemv_debug_stream_read over the same weight copies",
                              "step_us": round(ceil_step_us, 3),
                              "gbps": round(step_bytes / (ceil_step_us * 1e-6) / 1e9, 1),
                              "value_pct_of_ceiling": round(100 * ceil_step_us / (ms_step * 1e3), 1)},
        "sustained": {"steps": sus_steps, "us_per_step": round(sus_us, 3),
                      "gbps": round(step_bytes / (sus_us * 1e-6) / 1e9, 1)},
    }

    out["per_matrix"] = per
    if eager_us is not None:
        out["eager_step_us"] = round(eager_us, 2)
    del graph, tail, gd, W
    if not args.no_extras:
        out["extras"] = extras(qg, synth, torch, clocks)
    clocks.stop()
    out["clocks"] = clocks.summary()
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(mats, K)
    print(json.dumps(out), flush=True)
    return 0


def leg_ffn(qg, synth, torch, clocks):
    """Fused FFN sublayer (hidden 4096, inter 12288; Q4_K gate|up, Q6_K down)."""
    res = {}
    H, I = 4096, 12288
    f = qg.FFN(H, I, "q4_k", "q6_k")
    b_gu = 2 * I * synth.row_bytes("q4_k", H)
    b_dn = H * synth.row_bytes("q6_k", I)
    R = copies_for(b_gu + b_dn)
    gus = rotated(synth.weights("q4_k", 2 * I, H, seed=300), R)
    dns = rotated(synth.weights("q6_k", H, I, seed=301), R)
    x = dev(synth.activations(302, 1, H))
    y = torch.empty((1, H), dtype=torch.float32, device="cuda")
    ws = f.workspace(1)
    g = graph_of(lambda i: f.run(gus[i % R], dns[i % R], x, y=y, ws=ws), R)
    us = time_graph(g, R, reps=max(4, 128 // R))
    res["ffn_us"] = round(us, 3)
    res["ffn_us_eager"] = round(time_calls(lambda i: f.run(gus[i % R], dns[i % R], x, y=y, ws=ws), 50), 3)
    res["ffn_weight_gbps"] = round((b_gu + b_dn) / (us * 1e-6) / 1e9, 1)
    res["ffn_ceiling_us"] = round(ceiling_us(qg, gus) + ceiling_us(qg, dns), 3)
    log(f"ffn: {us:.2f} us per fused FFN, {res['ffn_weight_gbps']} GB/s; streaming read {res['ffn_ceiling_us']} us")
    return res


def leg_lm_head(qg, synth, torch, clocks):
    """IQ4_NL lm_head 4096 -> 248320, short burst and about 2 s sustained."""
    res = {}
    N = 248320
    cb = synth.codebook(1)
    g = qg.GEMV("iq4_nl", N, 4096, codebook=cb)
    b = N * synth.row_bytes("iq4_nl", 4096)
    R = copies_for(b)
    Ws = rotated(synth.weights("iq4_nl", N, 4096, seed=310), R)
    x = dev(synth.activations(311, 1, 4096))
    y = torch.empty((1, N), dtype=torch.float32, device="cuda")
    gg = graph_of(lambda i: g.run(Ws[i % R], x, y=y), R)
    # sustained first (about 2 s, clocks sampled): the short burst after it
    # then starts from the clocks the chip holds under this load, not from
    # an idle GPU's
    sus, calls = sustained(gg, R, None, clocks, "lm_head")
    us = time_graph(gg, R, reps=8)
    res["lm_head_us"] = round(us, 2)
    res["lm_head_gbps"] = round(b / (us * 1e-6) / 1e9, 1)
    res["lm_head_sustained_us"] = round(sus, 2)
    res["lm_head_sustained_calls"] = calls
    cus = ceiling_us(qg, Ws)
    res["lm_head_ceiling_us"] = round(cus, 2)
    res["lm_head_pct_of_ceiling"] = round(100 * cus / us, 1)
    log(f"lm_head: {us:.1f} us ({sus:.1f} us sustained), {res['lm_head_gbps']} GB/s; streaming read {cus:.1f} us")
    return res


def leg_q4_0_2048(qg, synth, torch, clocks):
    """Q4_0 2048 x 2048, a graph over copies totalling at least 2 GiB."""
    res = {}
    g = qg.GEMV("q4_0", 2048, 2048)
    b = 2048 * synth.row_bytes("q4_0", 2048)
    R = copies_for(b)
    base = dev(synth.weights("q4_0", 2048, 2048, seed=320))
    Ws = [base] + [base.clone() for _ in range(R - 1)]
    x = dev(synth.activations(321, 1, 2048))
    y = torch.empty((1, 2048), dtype=torch.float32, device="cuda")
    gg = graph_of(lambda i: g.run(Ws[i], x, y=y), R)
    us = time_graph(gg, R, reps=2)
    cus = ceiling_us(qg, Ws, reps=2)
    res["q4_0_2048_us"] = round(us, 3)
    res["q4_0_2048_gbps"] = round(b / (us * 1e-6) / 1e9, 1)
    res["q4_0_2048_copies"] = R
    res["q4_0_2048_ceiling_us"] = round(cus, 3)
    log(f"q4_0 2048x2048: {us:.2f} us over {R} copies, {res['q4_0_2048_gbps']} GB/s; streaming read {cus:.2f} us")
    return res


def leg_q5_k_iq4_xs(qg, synth, torch, clocks):
    """Q5_K and IQ4_XS (the formats of the pages' single-matrix bandwidth
    figures) at K = 4096, N = 12288, full qgemv_run calls."""
    res = {}
    for fmt in ("q5_k", "iq4_xs"):
        n, k = 12288, 4096
        g = qg.GEMV(fmt, n, k, codebook=synth.codebook(1) if fmt == "iq4_xs" else None)
        b = n * synth.row_bytes(fmt, k)
        R = copies_for(b)
        Ws = rotated(synth.weights(fmt, n, k, seed=330), R)
        x = dev(synth.activations(331, 1, k))
        y = torch.empty((1, n), dtype=torch.float32, device="cuda")
        gg = graph_of(lambda i: g.run(Ws[i % R], x, y=y), R)
        us = time_graph(gg, R, reps=4)
        cus = ceiling_us(qg, Ws)
        res[f"{fmt}_{k}x{n}_us"] = round(us, 3)
        res[f"{fmt}_{k}x{n}_gbps"] = round(b / (us * 1e-6) / 1e9, 1)
        res[f"{fmt}_{k}x{n}_pct_of_ceiling"] = round(100 * cus / us, 1)
        log(f"{fmt} {k}x{n}: {us:.2f} us, {res[f'{fmt}_{k}x{n}_gbps']} GB/s; streaming read {cus:.2f} us")
        del Ws, gg
    return res


def leg_s16(qg, synth, torch, clocks):
    """16-bit activations (Q4_K, K = 4096, N = 12288), qgemv_run_s16 calls."""
    res = {}
    n, k = 12288, 4096
    g = qg.GEMV("q4_k", n, k)
    b = n * synth.row_bytes("q4_k", k)
    R = copies_for(b)
    Ws = rotated(synth.weights("q4_k", n, k, seed=335), R)
    x = dev(synth.activations(336, 1, k))
    y = torch.empty((1, n), dtype=torch.float32, device="cuda")
    ws16 = g.workspace_s16()
    gg = graph_of(lambda i: g.run_s16(Ws[i % R], x, y=y, ws=ws16), R)
    us = time_graph(gg, R, reps=4)
    res[f"s16_q4_k_{k}x{n}_us"] = round(us, 3)
    res[f"s16_q4_k_{k}x{n}_gbps"] = round(b / (us * 1e-6) / 1e9, 1)
    log(f"s16 q4_k {k}x{n}: {us:.2f} us, {res[f's16_q4_k_{k}x{n}_gbps']} GB/s")
    return res


def leg_f32act(qg, synth, torch, clocks):
    """Float activations (qgemv_run_f32act, fp32 matrix cores): Q8_0 and
    Q4_0, 4096 -> 12288, one token and 32 tokens (2 m n k flops per call)."""
    res = {}
    n, k = 12288, 4096
    for fmt in ("q8_0", "q4_0"):
        g = qg.GEMV(fmt, n, k, max_m=32)
        b = n * synth.row_bytes(fmt, k)
        R = copies_for(b, cap=64)
        Ws = rotated(synth.weights(fmt, n, k, seed=337), R)
        for m in (1, 32):
            x = dev(synth.activations(338, m, k))
            y = torch.empty((m, n), dtype=torch.float32, device="cuda")
            gg = graph_of(lambda i: g.run_f32act(Ws[i % R], x, y=y), R)
            us = time_graph(gg, R, reps=4)
            key = f"f32act_{fmt}_{k}x{n}_m{m}"
            res[key + "_us"] = round(us, 3)
            res[key + "_gbps"] = round(b / (us * 1e-6) / 1e9, 1)
            res[key + "_tflops"] = round(2 * m * n * k / (us * 1e-6) / 1e12, 2)
            log(f"f32act {fmt} {k}x{n} m={m}: {us:.2f} us, {res[key + '_gbps']} GB/s, {res[key + '_tflops']} TFLOP/s")
        del Ws
    return res


def leg_m32(qg, synth, torch, clocks):
    """M=32 batched GEMMs on int8 matrix cores (Q4_K 4096 -> 12288, Q6_K
    12288 -> 4096): whole calls (quantizer + GEMM) and the GEMM kernel alone
    on already-quantized activations; matrix-core utilisation from recorded
    counters (int8 operations per dispatch) over the live kernel time."""
    res = {}
    rec = recorded_mfma()
    for fmt, n, k in (("q4_k", 12288, 4096), ("q6_k", 4096, 12288)):
        g = qg.GEMV(fmt, n, k, max_m=32)
        b = n * synth.row_bytes(fmt, k)
        R = copies_for(b)
        Ws = rotated(synth.weights(fmt, n, k, seed=340), R)
        x = dev(synth.activations(341, 32, k))
        y = torch.empty((32, n), dtype=torch.float32, device="cuda")
        ws = g.workspace(32)
        gg = graph_of(lambda i: g.run(Ws[i % R], x, y=y, ws=ws), R)
        us = time_graph(gg, R, reps=max(2, 64 // R))
        g.quantize(x, ws)
        gk = graph_of(lambda i: g.run_quantized(Ws[i % R], ws, 32, y), R)
        kus = time_graph(gk, R, reps=max(2, 64 // R))
        key = f"m32_{fmt}_{n}x{k}"
        res[key + "_us"] = round(us, 2)
        res[key + "_gbps"] = round(b / (us * 1e-6) / 1e9, 1)
        res[key + "_kernel_us"] = round(kus, 2)
        res[key + "_useful_tops"] = round(2.0 * 32 * n * k / (kus * 1e-6) / 1e12, 1)
        kr = (rec or {}).get("kernels", {}).get(fmt)
        if kr:
            res[key + "_mfma_util"] = round(kr["int8_ops_per_dispatch"] / (kus * 1e-6) / INT8_MFMA_PEAK, 4)
            res[key + "_mfma_busy_frac"] = kr["mfma_busy_frac"]
            res[key + "_mfma_util_source"] = "SQ_INSTS_VALU_MFMA_MOPS_I8 x 512 per dispatch / live kernel time"
        log(f"m=32 {fmt} {n}x{k}: {us:.2f} us per call, GEMM kernel {kus:.2f} us")
        del Ws, gg, gk
    return res


def leg_moe(qg, synth, torch, clocks):
    """MoE layer (256 experts of hidden 2048 / inter 512, top-8 + shared,
    Q4_0) at M=1 and M=16: expert copies totalling at least 2 GiB and 16
    different activation vectors (so the routing, and with it the experts
    read, changes from call to call)."""
    res = {}
    E, Hm, Im, Kt = 256, 2048, 512, 8
    gu_all, dn_all = synth.moe_experts(330, E, Hm, Im)
    gu_sh, dn_sh = synth.moe_experts(331, 1, Hm, Im)
    wr = dev(synth.router_weights(332, E, Hm))
    R = copies_for(gu_all.nbytes + dn_all.nbytes, cap=16)
    GU = rotated(gu_all, R)
    DN = rotated(dn_all, R)
    gsh, dsh = dev(gu_sh), dev(dn_sh)
    NX = 16
    L = NX * R  # every (copy, x) pair once
    res["moe_expert_copies"] = R
    res["moe_x_vectors"] = NX
    for m in (1, 16):
        mo = qg.MoE(Hm, Im, E, Kt, "q4_0", max_m=m)
        xs = [dev(synth.activations(3330 + 100 * m + i, m, Hm)) for i in range(NX)]
        y = torch.empty((m, Hm), dtype=torch.float32, device="cuda")
        ws = mo.workspace(m)
        gm = graph_of(lambda i: mo.run(wr, GU[i % R], DN[i % R], gsh, dsh, xs[(i // R) % NX], y=y, ws=ws), L)
        us = time_graph(gm, L, reps=2)
        res[f"moe_m{m}_us"] = round(us, 3)
        log(f"moe m={m}: {us:.2f} us")
        gm = graph_of(lambda i: mo.run(wr, GU[i % R], DN[i % R], gsh, dsh, xs[(i // R) % NX], y=y, ws=ws,
                                       s16=True), L)
        us = time_graph(gm, L, reps=2)
        res[f"moe_s16_m{m}_us"] = round(us, 3)
        log(f"moe s16 m={m}: {us:.2f} us")
        del gm
    return res


def leg_attn(qg, synth, torch, clocks):
    """Two-stage decode attention, 16 query heads over 2 key/value heads of
    dimension 256, fp16 KV cache, at 4K and 32K cached tokens."""
    res = {}
    hq, hkv, d = 16, 2, 256
    at = qg.Attention(hq, hkv, d)
    for t in (4096, 32768):
        q, k, v = synth.attention_inputs(350, hq, hkv, d, t)
        b = 2 * k.nbytes
        R = copies_for(b, cap=64)
        Ks, Vs = rotated(k, R), rotated(v, R)
        qd = dev(q)
        o = torch.empty((hq, d), dtype=torch.float32, device="cuda")
        ws = at.workspace(t)
        ga = graph_of(lambda i: at.run(qd, Ks[i % R], Vs[i % R], out=o, ws=ws), R)
        us = time_graph(ga, R, reps=max(2, 64 // R))
        res[f"attn_{t}_us"] = round(us, 3)
        res[f"attn_{t}_kv_gbps"] = round(b / (us * 1e-6) / 1e9, 1)
        log(f"attention {hq}/{hkv}x{d} ctx {t}: {us:.2f} us, {res[f'attn_{t}_kv_gbps']} GB/s of KV cache")
        del Ks, Vs, ga
    return res


LEG_FNS = {"ffn": leg_ffn, "lm_head": leg_lm_head, "q4_0_2048": leg_q4_0_2048, "q5_k_iq4_xs": leg_q5_k_iq4_xs,
           "s16": leg_s16, "f32act": leg_f32act, "m32": leg_m32, "moe": leg_moe, "attn": leg_attn}


def extras(qg, synth, torch, clocks):
    res = {}
    for name in LEGS:
        res.update(LEG_FNS[name](qg, synth, torch, clocks))
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    sys.exit(main())
