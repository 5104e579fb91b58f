#!/usr/bin/env python3
"""Benchmark of the W3G128 fused GEMV on one MI355X.

Default workload: the gate_proj shape of a Llama-3.1-70B decoder layer,
W [28672, 8192] stored as int32 [28672, 768] + bf16 scales [28672, 64], one bf16
activation row (batch 1), fp32 output.  One step = one qgemv_w3g128 call, the
whole batch-1 hot path (weight stream, scale fetch, activation staging,
decode, multiply-accumulate, reduction, store) in a single kernel.

Inputs are seeded synthetic tensors (`synth`), resident in device memory
before timing starts.  Weight/scale copies are rotated so the bytes of all
copies exceed twice the 256 MB Infinity Cache; each step reads a copy that
is not cache resident.  The K timed steps are captured in one HIP graph and
replayed once between two HIP events recorded on the stream the kernels run
on (a decode loop replays its launches the same way); the time of K
back-to-back stream launches is reported beside it.

Prints ONE JSON line on stdout.  Unless --no-summary, the other workloads
follow on stderr, one JSON line each: the full 70B decoder layer at batch 1
(per-layer us and aggregate GB/s, 7 launches and with q/k/v and gate/up fused),
batched decode M = 4..32 and prefill M = 512 on gate_proj and down_proj --
each as device time per call from a replayed HIP graph (a host launch costs
more than the smaller projections take to run) with back-to-back stream
launches beside it.  `--extra` adds the dense branch at M = 512 and the
oracle's host rates; `--case NAME:M` times one workload alone.
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
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 matrix peak, published
MALL_BYTES = 256 * 2 ** 20
METRIC = "W3G128 GEMV effective HBM GB/s and % of peak (70B layer shapes, B=1)"
KERNEL_SRC_DIR = os.path.join(ROOT, "dequant_gemv_qgemv_amd", "csrc")
KERNEL_BUILD = os.path.join(ROOT, "dequant_gemv_qgemv_amd", "_build.py")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "qgemv_gate_proj_traffic.json")


def gemv_bytes(n: int, k: int, m: int = 1) -> int:
    """Algorithmic bytes: packed words + scales + activations + fp32 outputs."""
    return n * (3 * k // 32) * 4 + n * (k // 128) * 2 + m * k * 2 + m * n * 4


def kernel_source_hash() -> str:
    """Hash of the library's sources and its build flags (the recorded counters
    describe the code these produce)."""
    h = hashlib.sha256()
    paths = sorted(os.path.join(KERNEL_SRC_DIR, f) for f in os.listdir(KERNEL_SRC_DIR)
                   if f.endswith((".hip", ".h")))
    for path in paths + [KERNEL_BUILD]:
        h.update(os.path.basename(path).encode() + b"\0")
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    when the kernel source changed since those counters were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


class Rotation:
    """Copies of one weight tensor pair, enough to exceed 2x the MALL."""

    def __init__(self, torch, packed, scales, min_copies=2):
        per = packed.numel() * 4 + scales.numel() * 2
        copies = max(min_copies, -(-2 * MALL_BYTES // per) + 1)
        self.items = [(packed.clone(), scales.clone()) for _ in range(copies)]
        self.copies = copies

    def __getitem__(self, i):
        return self.items[i % self.copies]


def time_steps(torch, fn, steps: int, warmup: int):
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        fn(i)
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps  # ms per step


def make_weight(torch, q, name):
    import synth
    c, s = synth.layer_weights(name)
    codes = torch.from_numpy(c).cuda()
    packed = q.qpack_uint3(codes)
    del codes
    scales = torch.from_numpy(s.view(np.int16)).cuda()
    return c, s, packed, scales


def cpu_baseline(c, s, x, k, budget_s=2.5):
    """The oracle as it stands, on the host cores, over a bounded row sample."""
    import oracle
    rows = np.arange(0, c.shape[0], 4, dtype=np.int64)
    words = oracle.pack(c[rows])
    sc = np.ascontiguousarray(s[rows])
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.gemm(x, words, sc, k)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s:
            break
    nbytes = gemv_bytes(rows.size, k, x.shape[0]) * reps
    return {
        "value": round(nbytes / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": "oracle fp64 GEMV over every 4th row of gate_proj (%d of %d rows, K=%d), "
                  "%d repetitions in %.2f s" % (rows.size, c.shape[0], k, reps, dt),
    }


def cpu_rate(c, s, k, m, step):
    """The oracle's rate (algorithmic GB/s) over every `step`-th row, M rows of x."""
    import oracle
    import synth
    rows = np.arange(0, c.shape[0], step, dtype=np.int64)
    words = oracle.pack(c[rows])
    sc = np.ascontiguousarray(s[rows])
    x = synth.layer_x(m, k)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.gemm(x, words, sc, k)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 0.3:
            break
    return {"GB/s": round(gemv_bytes(rows.size, k, m) * reps / dt / 1e9, 4), "cores": oracle.num_threads()}


def cpu_one_thread():
    """The oracle's gate_proj rate on one host thread (a child process with
    OMP_NUM_THREADS=1, every 64th row)."""
    import subprocess
    code = ("import sys; sys.path.insert(0, %r); import bench, synth, json; "
            "c, s = synth.layer_weights('gate_proj'); "
            "print(json.dumps(bench.cpu_rate(c, s, c.shape[1], 1, step=64)))" % ROOT)
    env = dict(os.environ, OMP_NUM_THREADS="1")
    res = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=300)
    if res.returncode != 0:
        return None
    return json.loads(res.stdout.strip().splitlines()[-1])["GB/s"]


def graph_time(torch, fn, reps: int, replays: int, warmup: int):
    """Per-call device time of fn(i), i = 0..reps-1, captured once in a HIP graph
    and replayed: host launch overhead (which exceeds the run time of the small
    projections) stays out of the figure."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        fn(0)  # sizes the library's workspace for this stream before capture
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        for i in range(reps):
            fn(i)
    torch.cuda.synchronize()
    return time_steps(torch, lambda i: graph.replay(), replays, warmup) / reps


def graph_steps(torch, fn, steps: int, warmup: int):
    """ms per step of fn(0) .. fn(steps - 1) captured in one HIP graph and
    replayed once between two events on the launch stream: exactly `steps`
    steps are timed, with no host launch between them.  Untimed before it:
    `warmup` stream launches and one replay of the same graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        fn(0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        for i in range(steps):
            fn(i)
    torch.cuda.synchronize()
    for i in range(warmup):
        fn(i)
    graph.replay()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    graph.replay()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


LAYER_ORDER = ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj")


def layer_calls(torch, q, kept):
    """The 70B decoder layer at batch 1 over rotated weights kept[name] =
    (Rotation, N, K): one_by_one(i) makes the 7 qgemv_w3g128 calls, fused(i)
    the same work in 4 launches (q/k/v and gate/up through qgemv_w3g128_multi)."""
    import synth
    x1 = torch.from_numpy(synth.layer_x(1, 8192).reshape(-1).view(np.int16)).cuda()
    x2 = torch.from_numpy(synth.layer_x(1, 28672).reshape(-1).view(np.int16)).cuda()
    ys = {nm: torch.empty(kept[nm][1], dtype=torch.float32, device="cuda") for nm in kept}

    def one_by_one(i):
        for nm in LAYER_ORDER:
            r = kept[nm][0][i]
            q.qgemv_w3g128(x2 if nm == "down_proj" else x1, r[0], r[1], out=ys[nm])

    def fused(i):
        r = {nm: kept[nm][0][i] for nm in kept}
        q.qgemv_w3g128_multi(x1, [r["q_proj"], r["k_proj"], r["v_proj"]],
                             outs=[ys["q_proj"], ys["k_proj"], ys["v_proj"]])
        q.qgemv_w3g128(x1, r["o_proj"][0], r["o_proj"][1], out=ys["o_proj"])
        q.qgemv_w3g128_multi(x1, [r["gate_proj"], r["up_proj"]], outs=[ys["gate_proj"], ys["up_proj"]])
        q.qgemv_w3g128(x2, r["down_proj"][0], r["down_proj"][1], out=ys["down_proj"])

    return one_by_one, fused, ys


def workload_summary(torch, q, steps):
    """The other workloads of the benchmark on stderr, one JSON line each:
    the 70B decoder layer at batch 1 (7 projections, and the same layer with
    q/k/v and gate/up each fused into one launch), batched decode M = 4..32
    and prefill M = 512 on gate_proj and down_proj.  Device time per call
    from a replayed HIP graph (host launch cost excluded), and the time of
    back-to-back stream launches beside it.  Returns the same figures in
    compact form for the main JSON line (compact_summary)."""
    import synth
    kept = {}
    layer = {}
    total_bytes, total_ms = 0, 0.0
    lines = []
    for name in LAYER_ORDER:
        _, _, packed, scales = make_weight(torch, q, name)
        n, k = synth.LAYER_70B[name][:2]
        rot = Rotation(torch, packed, scales)
        del packed, scales
        kept[name] = (rot, n, k)
        xd = torch.from_numpy(synth.layer_x(1, k).reshape(-1).view(np.int16)).cuda()
        y = torch.empty(n, dtype=torch.float32, device="cuda")
        fn = lambda i: q.qgemv_w3g128(xd, rot[i][0], rot[i][1], out=y)  # noqa: E731
        ms_launch = time_steps(torch, fn, steps, max(10, steps // 10))
        ms = graph_time(torch, fn, 20, max(10, steps // 20), 3)
        b = gemv_bytes(n, k)
        layer[name] = {"us": round(ms * 1e3, 3), "GB/s": round(b / ms / 1e6, 1), "bytes": b,
                       "us_stream_launches": round(ms_launch * 1e3, 3)}
        total_bytes += b
        total_ms += ms
        if name in ("gate_proj", "down_proj"):
            for m in (4, 8, 16, 32, 512):
                xm = torch.from_numpy(synth.layer_x(m, k).view(np.int16)).cuda()
                ym = torch.empty((m, n), dtype=torch.float32, device="cuda")
                fm = lambda i: q.qgemm_w3g128_smallM(xm, rot[i][0], rot[i][1], out=ym)  # noqa: E731
                st = max(20, steps // (8 if m == 512 else 2))
                ms_l = time_steps(torch, fm, st, 5)
                ms_g = graph_time(torch, fm, 4 if m == 512 else 20, max(5, st // 20), 2)
                bm = gemv_bytes(n, k, m)
                tf = 2.0 * m * n * k / ms_g / 1e9
                lines.append({"workload": "%s [%d, %d] M=%d" % (name, n, k, m), "us": round(ms_g * 1e3, 3),
                              "GB/s": round(bm / ms_g / 1e6, 1), "HBM_frac": round(bm / ms_g / 1e6 / HBM_PEAK_GBS, 4),
                              "TFLOP/s": round(tf, 2), "MFMA_frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                              "us_stream_launches": round(ms_l * 1e3, 3), "algorithmic_bytes": bm})
    one_by_one, fused, ys = layer_calls(torch, q, kept)
    layer_ms = graph_time(torch, one_by_one, 8, max(10, steps // 20), 3)
    fused_ms = graph_time(torch, fused, 8, max(10, steps // 20), 3)
    lines.insert(0, {"workload": "Llama-3.1-70B decoder layer at B=1: q/o [8192, 8192], k/v [1024, 8192], "
                                 "gate/up [28672, 8192], down [8192, 28672] (device time, graph replay)",
                     "layer_bytes": total_bytes,
                     "layer_us": round(layer_ms * 1e3, 3), "layer_GB/s": round(total_bytes / layer_ms / 1e6, 1),
                     "layer_HBM_frac": round(total_bytes / layer_ms / 1e6 / HBM_PEAK_GBS, 4),
                     "fused_layer_us": round(fused_ms * 1e3, 3),
                     "fused_layer_GB/s": round(total_bytes / fused_ms / 1e6, 1),
                     "fused_layer_HBM_frac": round(total_bytes / fused_ms / 1e6 / HBM_PEAK_GBS, 4),
                     "fused_layer_launches": "q/k/v in one qgemv_w3g128_multi, o, gate/up in one, down",
                     "per_projection": layer, "per_projection_us_sum": round(total_ms * 1e3, 3)})
    del kept, ys
    torch.cuda.empty_cache()
    for rec in lines:
        print(json.dumps(rec), file=sys.stderr, flush=True)
    return compact_summary(layer, layer_ms, fused_ms, total_bytes, lines)


def compact_summary(layer, layer_ms, fused_ms, layer_bytes, lines):
    """The summary's figures as one small object: per workload, µs per call
    (graph replay) and the fraction of the roofline that bounds it -- of
    8 TB/s for the batch-1 and batched-decode calls (algorithmic bytes), of
    the 2.5 PFLOP/s fp16 matrix peak for prefill (M = 512)."""
    out = {"unit": "us per call, graph replay; frac of 8 TB/s HBM (M < 512) or of 2.5 PFLOP/s fp16 "
                   "MFMA (M = 512)"}
    for name, rec in layer.items():
        out["%s_M1" % name] = {"us": rec["us"], "frac": round(rec["GB/s"] / HBM_PEAK_GBS, 4)}
    out["layer_70b_M1"] = {"us": round(layer_ms * 1e3, 3),
                           "frac": round(layer_bytes / layer_ms / 1e6 / HBM_PEAK_GBS, 4)}
    out["layer_70b_M1_fused"] = {"us": round(fused_ms * 1e3, 3),
                                 "frac": round(layer_bytes / fused_ms / 1e6 / HBM_PEAK_GBS, 4)}
    for rec in lines:
        if "layer_us" in rec:  # the layer's own line, already above
            continue
        name, m = rec["workload"].split(" ")[0], int(rec["workload"].rsplit("M=", 1)[1])
        frac = rec["MFMA_frac"] if m == 512 else rec["HBM_frac"]
        out["%s_M%d" % (name, m)] = {"us": rec["us"], "frac": frac}
    return out


def bench_extra(torch, q, steps, warmup):
    """Full layer at B=1, batched decode, prefill: JSON lines on stderr."""
    import synth
    out = []
    layer = {}
    total_bytes, total_ms = 0, 0.0
    kept = {}
    cpu_layer, cpu_m32 = {}, None
    for name in ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj"):
        c, s, packed, scales = make_weight(torch, q, name)
        n, k = c.shape
        cpu_layer[name] = cpu_rate(c, s, k, 1, step=16)
        if name == "gate_proj":
            cpu_m32 = cpu_rate(c, s, k, 32, step=64)
        del c
        rot = Rotation(torch, packed, scales)
        kept[name] = (rot, n, k)
        xd = torch.from_numpy(synth.layer_x(1, k).reshape(-1).view(np.int16)).cuda()
        y = torch.empty(n, dtype=torch.float32, device="cuda")
        ms_launch = time_steps(torch, lambda i: q.qgemv_w3g128(xd, rot[i][0], rot[i][1], out=y), steps, warmup)
        ms = graph_time(torch, lambda i: q.qgemv_w3g128(xd, rot[i][0], rot[i][1], out=y), 20,
                        max(10, steps // 20), 3)
        b = gemv_bytes(n, k)
        layer[name] = {"us": round(ms * 1e3, 3), "GB/s": round(b / ms / 1e6, 1), "bytes": b,
                       "us_stream_launches": round(ms_launch * 1e3, 3)}
        total_bytes += b
        total_ms += ms
        if name in ("gate_proj", "down_proj"):
            fused_512 = None
            for m in (4, 8, 16, 32, 512):
                xm = torch.from_numpy(synth.layer_x(m, k).view(np.int16)).cuda()
                ym = torch.empty((m, n), dtype=torch.float32, device="cuda")
                st = max(10, steps // (8 if m == 512 else 2))
                ms_m = time_steps(torch, lambda i: q.qgemm_w3g128_smallM(xm, rot[i][0], rot[i][1], out=ym),
                                  st, max(2, warmup // 4))
                bm = gemv_bytes(n, k, m)
                rec = {"workload": "%s M=%d" % (name, m), "us": round(ms_m * 1e3, 3),
                       "GB/s": round(bm / ms_m / 1e6, 1), "HBM_frac": round(bm / ms_m / 1e6 / HBM_PEAK_GBS, 4),
                       "TFLOP/s": round(2.0 * m * n * k / ms_m / 1e9, 2)}
                rec["MFMA_frac"] = round(rec["TFLOP/s"] / BF16_MFMA_PEAK_TFLOPS, 4)
                out.append(rec)
                if m == 512:
                    fused_512 = ms_m
            out.append(dense_branch(torch, q, name, n, k, rot, fused_512))
        del packed, scales
    # The same layer with the projections that share an input fused into one
    # launch each: q/k/v, o, gate/up, down (4 launches instead of 7).
    x1 = torch.from_numpy(synth.layer_x(1, 8192).reshape(-1).view(np.int16)).cuda()
    x2 = torch.from_numpy(synth.layer_x(1, 28672).reshape(-1).view(np.int16)).cuda()
    ys = {nm: torch.empty(kept[nm][1], dtype=torch.float32, device="cuda") for nm in kept}

    def fused_layer(i):
        r = {nm: kept[nm][0][i] for nm in kept}
        q.qgemv_w3g128_multi(x1, [r["q_proj"], r["k_proj"], r["v_proj"]],
                             outs=[ys["q_proj"], ys["k_proj"], ys["v_proj"]])
        q.qgemv_w3g128(x1, r["o_proj"][0], r["o_proj"][1], out=ys["o_proj"])
        q.qgemv_w3g128_multi(x1, [r["gate_proj"], r["up_proj"]], outs=[ys["gate_proj"], ys["up_proj"]])
        q.qgemv_w3g128(x2, r["down_proj"][0], r["down_proj"][1], out=ys["down_proj"])

    fused_ms = graph_time(torch, fused_layer, 8, max(10, steps // 20), 3)
    del kept
    torch.cuda.empty_cache()
    out.insert(0, {"workload": "70B decoder layer, 7 projections back to back, B=1 (device time per call, "
                               "graph replay of 20 calls)",
                   "per_projection": layer, "layer_us_sum": round(total_ms * 1e3, 3),
                   "layer_GB/s": round(total_bytes / total_ms / 1e6, 1),
                   "layer_HBM_frac": round(total_bytes / total_ms / 1e6 / HBM_PEAK_GBS, 4),
                   "fused_layer_us": round(fused_ms * 1e3, 3),
                   "fused_layer_GB/s": round(total_bytes / fused_ms / 1e6, 1),
                   "fused_layer_note": "q/k/v and gate/up each in one qgemv_w3g128_multi launch; "
                                       "graph replay of 8 layers"})
    cpu_ms = sum(gemv_bytes(*synth.LAYER_70B[nm][:2]) / (r["GB/s"] * 1e6) for nm, r in cpu_layer.items())
    out.append({"workload": "oracle on the host (fp64, OpenMP over rows): one decoder layer at B=1, "
                            "every 16th row of each projection timed, the layer time scaled from those rates",
                "per_projection_GB/s": {nm: r["GB/s"] for nm, r in cpu_layer.items()},
                "layer_ms": round(cpu_ms, 2), "cores": cpu_layer["gate_proj"]["cores"],
                "gate_proj_M32_GB/s": cpu_m32["GB/s"],
                "gate_proj_1_thread_GB/s": cpu_one_thread()})
    for rec in out:
        print(json.dumps(rec), file=sys.stderr, flush=True)


def dense_branch(torch, q, name, n, k, rot, fused_ms):
    """Prefill the unfused way, for comparison with the fused tile kernel:
    qdequant_bf16 writes the dense bf16 weight, then a library bf16 GEMM
    (torch linear, hipBLASLt) multiplies the M = 512 activations by it."""
    import synth
    m = 512
    wd = torch.empty((n, k), dtype=torch.bfloat16, device="cuda")
    x = torch.from_numpy(synth.layer_x(m, k).view(np.int16)).cuda().view(torch.bfloat16)
    ms_deq = time_steps(torch, lambda i: q.qdequant_bf16(rot[i][0], rot[i][1], out=wd), 20, 3)
    ms_mm = time_steps(torch, lambda i: torch.nn.functional.linear(x, wd), 20, 3)
    del wd, x
    torch.cuda.empty_cache()
    tot = ms_deq + ms_mm
    return {"workload": "%s M=512 dense branch: qdequant_bf16, then bf16 GEMM (torch linear)" % name,
            "dequant_us": round(ms_deq * 1e3, 3), "gemm_us": round(ms_mm * 1e3, 3),
            "dense_total_us": round(tot * 1e3, 3), "fused_us": round(fused_ms * 1e3, 3),
            "fused_speedup": round(tot / fused_ms, 3),
            "gemm_TFLOP/s": round(2.0 * m * n * k / ms_mm / 1e9, 2)}


CEILING_SRC = os.path.join(ROOT, "bench_ceiling.hip")
CEILING_LIB = os.path.join(ROOT, "bench_ceiling.so")


def build_ceiling() -> str:
    """Compile the streaming-read probe (bench_ceiling.hip, a measurement tool
    beside this script; the product library does not contain it) with the
    library's own hipcc flags."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "qw3_build_step", os.path.join(ROOT, "dequant_gemv_qgemv_amd", "_build.py"))
    step = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(step)
    step.compile_hip(CEILING_SRC, CEILING_LIB)
    return CEILING_LIB


def read_sweep_ceiling(torch):
    """A plain streaming-read kernel (bench_ceiling.so) over slices of a 1 GiB
    buffer the size of the gate_proj weights + scales, rotated so no slice is
    cache resident: the read rate HBM gives a kernel on this part."""
    import ctypes
    if not os.path.exists(CEILING_LIB):
        raise SystemExit("bench_ceiling.so is not built: run __graft_entry__.build() first")
    lib = ctypes.CDLL(CEILING_LIB)
    lib.qw3_read_sweep.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                   ctypes.c_void_p]
    lib.qw3_read_sweep.restype = ctypes.c_int
    buf = torch.ones(256 * 2 ** 20, dtype=torch.int32, device="cuda")
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    n, k = 28672, 8192
    nbytes = (n * (3 * k // 32) * 4 + n * (k // 128) * 2) // 16 * 16
    slices = buf.numel() * 4 // nbytes
    base = buf.data_ptr()
    stream = torch.cuda.current_stream().cuda_stream
    best = None
    for blocks in (512, 1024, 2048):
        def step(i, blocks=blocks):
            rc = lib.qw3_read_sweep(base + (i % slices) * nbytes, nbytes, blocks, sink.data_ptr(), stream)
            if rc != 0:
                raise RuntimeError("qw3_read_sweep failed: %d" % rc)
        ms = time_steps(torch, step, 400, 40)
        if best is None or ms < best[0]:
            best = (ms, blocks)
    rec = {"workload": "ceiling: streaming read of %d-byte slices of a 1 GiB buffer (%d slices rotated)"
                       % (nbytes, slices),
           "read_GB/s": round(nbytes / best[0] / 1e6, 1), "us_per_slice": round(best[0] * 1e3, 3),
           "workgroups": best[1]}
    print(json.dumps(rec), file=sys.stderr, flush=True)
    del buf, sink
    return rec


def read_copy_ceiling(torch):
    """A plain 1 GiB device copy (torch copy_): what HBM gives a streaming kernel here."""
    src = torch.ones(256 * 2 ** 20, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    nbytes = src.numel() * 4
    ms_copy = time_steps(torch, lambda i: dst.copy_(src), 20, 3)
    rec = {"workload": "ceiling: 1 GiB device copy (read + write)",
           "copy_GB/s(read+write)": round(2 * nbytes / ms_copy / 1e6, 1)}
    print(json.dumps(rec), file=sys.stderr, flush=True)
    del src, dst


def run_layer_case(torch, q, fused: bool, steps: int):
    """The whole 70B decoder layer at batch 1 (7 launches, or 4 with q/k/v and
    gate/up fused), device time per layer from a replayed HIP graph."""
    import synth
    kept = {}
    total = 0
    for name in LAYER_ORDER:
        _, _, packed, scales = make_weight(torch, q, name)
        n, k = synth.LAYER_70B[name][:2]
        kept[name] = (Rotation(torch, packed, scales), n, k)
        total += gemv_bytes(n, k)
        del packed, scales
    one_by_one, fused_fn, _ = layer_calls(torch, q, kept)
    fn = fused_fn if fused else one_by_one
    ms = graph_time(torch, fn, 8, max(10, steps // 8), 3)
    print(json.dumps({"workload": "Llama-3.1-70B decoder layer at B=1, %s (device time, graph replay)"
                      % ("4 launches: q/k/v and gate/up fused" if fused else "7 launches"),
                      "layer_bytes": total, "layer_us": round(ms * 1e3, 3),
                      "layer_GB/s": round(total / ms / 1e6, 1),
                      "layer_HBM_frac": round(total / ms / 1e6 / HBM_PEAK_GBS, 4)}), flush=True)


def run_case(torch, q, case: str, steps: int, warmup: int):
    """One projection of the 70B layer at M rows of activations, stream launches
    (layer:1 and layer_fused:1: the whole layer at batch 1)."""
    import synth
    name, m = case.split(":")
    m = int(m)
    if name in ("layer", "layer_fused") and m == 1:
        return run_layer_case(torch, q, name == "layer_fused", steps)
    if name.endswith("_dense") and name[:-6] in synth.LAYER_70B and m == 512:
        # the unfused prefill (qdequant_bf16, then a library bf16 GEMM) beside the fused kernel
        base = name[:-6]
        _, _, packed, scales = make_weight(torch, q, base)
        n, k = synth.LAYER_70B[base][:2]
        rot = Rotation(torch, packed, scales)
        del packed, scales
        xm = torch.from_numpy(synth.layer_x(m, k).view(np.int16)).cuda()
        ym = torch.empty((m, n), dtype=torch.float32, device="cuda")
        fused = time_steps(torch, lambda i: q.qgemm_w3g128_smallM(xm, rot[i][0], rot[i][1], out=ym),
                           max(10, steps // 8), max(2, warmup // 4))
        print(json.dumps(dense_branch(torch, q, base, n, k, rot, fused)), flush=True)
        return
    invariant = name.endswith("_bi") and name[:-3] in synth.LAYER_70B
    if invariant:
        name = name[:-3]
    if name not in synth.LAYER_70B or m < 1:
        raise SystemExit("--case wants NAME:M with NAME one of %s, or layer:1 / layer_fused:1, "
                         "NAME_dense:512 or NAME_bi:M" % ", ".join(synth.LAYER_70B))
    c, s, packed, scales = make_weight(torch, q, name)
    n, k = c.shape
    del c, s
    rot = Rotation(torch, packed, scales)
    x = torch.from_numpy(synth.layer_x(m, k).view(np.int16)).cuda()
    if invariant:  # rows bit-identical to the batch-1 product, the weights read once per row
        y = torch.empty((m, n), dtype=torch.float32, device="cuda")
        fn = lambda i: q.qgemm_w3g128_batch_invariant(x, rot[i][0], rot[i][1], out=y)  # noqa: E731
    elif m == 1:
        x = x.reshape(-1)
        y = torch.empty(n, dtype=torch.float32, device="cuda")
        fn = lambda i: q.qgemv_w3g128(x, rot[i][0], rot[i][1], out=y)  # noqa: E731
    else:
        y = torch.empty((m, n), dtype=torch.float32, device="cuda")
        fn = lambda i: q.qgemm_w3g128_smallM(x, rot[i][0], rot[i][1], out=y)  # noqa: E731
    ms = time_steps(torch, fn, steps, warmup)
    ms_g = graph_time(torch, fn, 4 if m >= 128 else 20, max(5, steps // 20), 2)
    b = gemv_bytes(n, k, m)
    tf = 2.0 * m * n * k / ms / 1e9
    what = "%s [%d, %d] M=%d%s" % (name, n, k, m, ", batch-invariant (batch-1 kernel per row)" if invariant else "")
    print(json.dumps({"workload": what, "steps": steps, "us": round(ms * 1e3, 3),
                      "GB/s": round(b / ms / 1e6, 1), "HBM_frac": round(b / ms / 1e6 / HBM_PEAK_GBS, 4),
                      "TFLOP/s": round(tf, 2), "MFMA_frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                      "us_graph_replay": round(ms_g * 1e3, 3),
                      "HBM_frac_graph_replay": round(b / ms_g / 1e6 / HBM_PEAK_GBS, 4),
                      "algorithmic_bytes": b}), flush=True)


def traffic_from_counters(fetch_csv: str, write_csv: str, out_path: str = TRAFFIC_FILE) -> dict:
    """Summarise two rocprofv3 counter runs of `bench.py --calibrate` (one with
    --pmc FETCH_SIZE, one with --pmc WRITE_SIZE) into HBM bytes per launch of
    the default workload's kernel.  Both counters report KiB per dispatch; the
    calibration copies (5 x 256 MiB read and written, the largest copy
    dispatches of the run) give the factor from counter to bytes.  Writes the
    record, keyed by the kernel source hash, to out_path."""
    import csv
    kernel = "qgemv_mfma_kernel<16, 4, false>"
    copy_bytes, copies = 256 * 2 ** 20, 5

    def per_kernel(path, counter):
        vals, cps = [], []
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                v = float(r["Counter_Value"])
                if kernel in r["Kernel_Name"]:
                    vals.append(v)
                elif "copyBuffer" in r["Kernel_Name"] or "copy" in r["Kernel_Name"].lower():
                    cps.append(v)
        if not vals or len(cps) < copies:
            raise SystemExit("%s: %d dispatches of %s, %d copy dispatches" % (path, len(vals), kernel, len(cps)))
        cal = sorted(cps)[-copies:]
        return sum(vals) / len(vals), sum(cal) / len(cal), len(vals)

    f_k, f_cal, nd = per_kernel(fetch_csv, "FETCH_SIZE")
    w_k, w_cal, _ = per_kernel(write_csv, "WRITE_SIZE")
    fs, ws = copy_bytes / (f_cal * 1024), copy_bytes / (w_cal * 1024)
    rd, wr = int(round(f_k * 1024 * fs)), int(round(w_k * 1024 * ws))
    alg = gemv_bytes(28672, 8192)
    rec = {"kernel": kernel, "workload": "gate_proj W3G128 GEMV [28672, 8192], batch 1",
           "kernel_source_sha256_16": kernel_source_hash(), "fetch_size_kib_raw": round(f_k, 2),
           "write_size_kib_raw": round(w_k, 2), "calibration_copy_bytes": copy_bytes,
           "calibration_copies": copies, "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
           "hbm_read_bytes_per_launch": rd, "hbm_write_bytes_per_launch": wr, "hbm_bytes_per_launch": rd + wr,
           "algorithmic_bytes_per_launch": alg, "traffic_over_algorithmic": round((rd + wr) / alg, 4),
           "dispatches_averaged": nd,
           "commands": ["cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc %s --output-format csv -d %s -o run -- "
                        "python3 /root/repo/bench.py --steps 10 --warmup 2 --no-cpu-baseline --no-summary --calibrate"
                        % (counter, os.path.dirname(path)) for counter, path in
                        (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv))]
                       + ["python3 bench.py --traffic-from %s %s" % (fetch_csv, write_csv)]}
    with open(out_path, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    return rec


# Kernels of the library, as the tracer names them (the per-call traffic of a
# --case run is the sum over these, each dispatched once per call).
LIB_KERNELS = ("qgemv_", "qgemm_", "prep_x", "prep_tile_x")


def case_traffic_from_counters(case: str, fetch_csv: str, write_csv: str) -> dict:
    """HBM bytes per call of `bench.py --case NAME:M --calibrate` from its two
    counter runs (FETCH_SIZE, WRITE_SIZE): each library kernel's average per
    dispatch, scaled by what the counters read for the run's five 256 MiB
    calibration copies, summed over the kernels of one call."""
    import csv
    import synth
    name, m = case.split(":")
    m = int(m)
    n, k = synth.LAYER_70B[name][:2]
    copy_bytes, copies = 256 * 2 ** 20, 5

    def per_kernel(path, counter):
        vals, cps = {}, []
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                kn = r["Kernel_Name"]
                v = float(r["Counter_Value"])
                if any(t in kn for t in LIB_KERNELS) and "qpack" not in kn:
                    short = kn.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]
                    vals.setdefault(short, []).append(v)
                elif "copyBuffer" in kn or "copy" in kn.lower():
                    cps.append(v)
        if not vals or len(cps) < copies:
            raise SystemExit("%s: no library kernels or fewer than %d copy dispatches" % (path, copies))
        cal = sorted(cps)[-copies:]
        return {kk: (sum(v) / len(v), len(v)) for kk, v in vals.items()}, sum(cal) / len(cal)

    f, f_cal = per_kernel(fetch_csv, "FETCH_SIZE")
    w, w_cal = per_kernel(write_csv, "WRITE_SIZE")
    fs, ws = copy_bytes / (f_cal * 1024), copy_bytes / (w_cal * 1024)
    kernels = {}
    total = 0
    for kk in sorted(f):
        rd = int(round(f[kk][0] * 1024 * fs))
        wr = int(round(w.get(kk, (0.0, 0))[0] * 1024 * ws))
        kernels[kk] = {"fetch_bytes": rd, "write_bytes": wr, "dispatches": f[kk][1]}
        total += rd + wr
    alg = gemv_bytes(n, k, m)
    return {"case": case, "workload": "%s [%d, %d] M=%d, one qgemm_w3g128_smallM call" % (name, n, k, m),
            "per_kernel": kernels, "hbm_bytes_per_call": total, "algorithmic_bytes_per_call": alg,
            "traffic_over_algorithmic": round(total / alg, 4), "fetch_scale": round(fs, 4),
            "write_scale": round(ws, 4)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--extra", action="store_true", help="also time layer / batched / prefill workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-summary", action="store_true",
                    help="skip the other workloads' lines (layer, batched decode, prefill) on stderr")
    ap.add_argument("--calibrate", action="store_true",
                    help="first run 5 plain 256 MiB device copies (torch copy_), the known-size "
                         "reference for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE counters")
    ap.add_argument("--ceiling", action="store_true",
                    help="also time a plain 1 GiB device copy and a streaming-read kernel and print "
                         "their GB/s on stderr")
    ap.add_argument("--case-traffic-from", nargs=3, metavar=("CASE", "FETCH_CSV", "WRITE_CSV"),
                    help="summarise two counter runs (FETCH_SIZE, WRITE_SIZE) of --case CASE --calibrate into "
                         "HBM bytes per call, per library kernel; prints JSON (no GPU needed)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 counter runs (FETCH_SIZE, WRITE_SIZE) of --calibrate into "
                         "the committed traffic record and exit (no GPU needed)")
    ap.add_argument("--case", metavar="NAME:M",
                    help="time one other workload instead of the default line, e.g. gate_proj:16, "
                         "down_proj:512, layer:1 / layer_fused:1, gate_proj_dense:512 (the dequantize-then-GEMM "
                         "prefill beside the fused one) or gate_proj_bi:8 (the batch-invariant product) (for "
                         "profiling); prints its JSON line on stdout")
    args = ap.parse_args()
    if args.traffic_from:
        print(json.dumps(traffic_from_counters(*args.traffic_from)))
        return
    if args.case_traffic_from:
        print(json.dumps(case_traffic_from_counters(*args.case_traffic_from)))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import dequant_gemv_qgemv_amd as q
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.calibrate:
        src = torch.ones(64 * 2 ** 20, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    ceiling = None
    if args.ceiling:
        read_copy_ceiling(torch)
        ceiling = read_sweep_ceiling(torch)

    if args.case:
        run_case(torch, q, args.case, args.steps, args.warmup)
        return

    n, k = synth.LAYER_70B["gate_proj"][:2]
    c, s, packed, scales = make_weight(torch, q, "gate_proj")
    x = synth.layer_x(1, k)
    xd = torch.from_numpy(x.reshape(-1).view(np.int16)).cuda()
    rot = Rotation(torch, packed, scales)
    y = torch.empty(n, dtype=torch.float32, device="cuda")

    step = lambda i: q.qgemv_w3g128(xd, rot[i][0], rot[i][1], out=y)  # noqa: E731
    ms_launch = time_steps(torch, step, args.steps, args.warmup)
    ms = graph_steps(torch, step, args.steps, args.warmup)
    nbytes = gemv_bytes(n, k)
    gbs = nbytes / ms / 1e6
    if ceiling is not None:
        print(json.dumps({"workload": "gate_proj GEMV against the streaming-read ceiling",
                          "gemv_GB/s": round(gbs, 1), "read_ceiling_GB/s": ceiling["read_GB/s"],
                          "frac_of_read_ceiling": round(gbs / ceiling["read_GB/s"], 4)}),
              file=sys.stderr, flush=True)
    line = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16xf16->f32",
        "data": "synthetic",
        "config": {"workload": "gate_proj W3G128 GEMV, W [28672, 8192] -> int32 [28672, 768] + bf16 "
                               "[28672, 64], x bf16 [1, 8192], y fp32 [28672]",
                   "N": n, "K": k, "M": 1, "bytes_per_step": nbytes,
                   "weight_copies_rotated": rot.copies, "us_per_step": round(ms * 1e3, 3),
                   "timing": "the K steps captured in one HIP graph, replayed once between events",
                   "us_per_step_stream_launches": round(ms_launch * 1e3, 3)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic()},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(c, s, x, k)
    rot = packed = scales = None  # free the rotated copies before the other workloads
    torch.cuda.empty_cache()
    if not args.no_summary:
        line["other_configs"] = workload_summary(torch, q, max(200, args.steps))
    if args.extra:
        bench_extra(torch, q, max(50, args.steps // 4), max(10, args.warmup // 4))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
