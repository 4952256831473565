#!/usr/bin/env python3
"""Benchmark of the quantized linear layer on one MI355X.

A step is one pass of the W4A16 decode hot path over the LLaMA-7B MLP
workload at the batch sizes the headline metric covers: for each M in
{1, 4, 8, 16}, the fused gate/up projection (K=4096, N=22016) and the down
projection (K=11008, N=4096), int4 weights in groups of 128 (asymmetric
uint4 zero points, fp16 scales), fp16 activations.  The same workload at
M=32 is timed launch by launch in `detail` but is not part of the step.
Weights are streamed cold: every launch reads one of several weight copies
that together exceed the 256 MB Infinity Cache.

Launches are captured in HIP graphs (one graph per step, rotating the weight
copies), so the timed region measures the GPU rather than Python's launch
overhead.  `value` is the step's algorithmic bytes (packed weights + scales +
zero points + x + y) divided by the step time, in GB/s.

`roofline` covers the kernel that takes the most time in a step: the average
algorithmic bytes per launch over that kernel's launches divided by their
average duration, measured with HIP events around graphs of back-to-back
launches on the launch stream.  `traffic` is filled from the committed
rocprofv3 counter summary when it was taken on the current kernel source.
`detail` gives every launch of the step its graph-averaged duration and the
p10 / median / p90 of 100 single launches (event pairs, cold weights).
`extra` reports the LLaMA-7B q_proj GEMV (M=1), the LLaMA-13B MLP sweep
(M in {1, 8, 64, 256, 1024}, both projections, groups 32 and 128), the W4A16
prefill GEMM (M=512 fused QKV) and the W8A8 layer (QRMSNorm + int8 GEMM,
M=2048) against their rooflines, and the steps beside it (residual-fused
QRMSNorm, per-token quantisation, the GEMM with bias and residual), the
layer with FP8 E4M3 codes, and KV-cache INT8 group quantisation and
dequantisation.  Every weight-streaming extra rotates weight copies that
together exceed the Infinity Cache.  `reference` is a
plain device copy's rate, the achievable HBM bandwidth on the device.
`cpu_baseline` times the CPU oracle on a bounded sample of the same step.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
FP16_MFMA_PEAK_TFLOPS = 2500.0  # dense
INT8_MFMA_PEAK_TOPS = 5000.0    # dense
FP8_MFMA_PEAK_TFLOPS = 5000.0   # dense
DECODE_M = (1, 4, 8, 16)        # the step: the batch sizes of the headline metric (M <= 16)
DETAIL_M = (1, 4, 8, 16, 32)    # timed launch by launch
GROUP = 128
CACHE_BYTES = 256 << 20         # MI355X Infinity Cache
METRIC = "W4A16/W8A8 GEMM: HBM GB/s (M<=16), TFLOP/s (M>=512), % of MI355X peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
COPY_BYTES = 256 << 20          # calibration copy: reads and writes this many bytes


def w4a16_bytes(m, n, k, g):
    """Algorithmic bytes: packed codes, fp16 scales, uint4 zeros, fp16 x and y."""
    return n * k // 2 + n * (k // g) * 2 + n * (k // g) // 2 + m * k * 2 + m * n * 2


def kernel_source_hash():
    """Hash of the W4A16 kernel sources with comments and blank space removed,
    so that a traffic record stays valid across edits that change no code."""
    h = hashlib.sha256()
    for f in ("w4a16.hip", "dequant.hpp", "lds_dma.hpp"):
        with open(os.path.join(ROOT, "weight_quantized_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)     # block comments
        text = re.sub(r"//[^\n]*", " ", text)                   # line comments
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_records():
    """Counter-measured HBM bytes per launch, by workload ("gate_up_m16", ...)."""
    if not os.path.exists(TRAFFIC_FILE):
        return {}
    with open(TRAFFIC_FILE) as f:
        return json.load(f).get("records", {})


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500,
                    help="untimed steps before the timed ones (the default, ~55 ms of GPU work, lets the clocks "
                         "come up after the host-side phases, as WARM_MS does for the per-launch graphs)")
    ap.add_argument("--copies", type=int, default=12, help="cold-cache weight copies per shape")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--cpu-sample-rows", type=int, default=0,
                    help="output channels per launch for the oracle sample (0 = all of them)")
    ap.add_argument("--profile-launch", metavar="SHAPE,M",
                    help="run one workload for counter collection and exit: gate_up,M or down,M or q_proj,1 "
                         "(decode, cold weights), qkv,512 (prefill GEMM), w8a8,2048 (QRMSNorm + int8 GEMM), "
                         "fp8,2048 (FP8 QRMSNorm + FP8 GEMM), kv,4096 (KV cache INT8 quantise + dequantise); "
                         "then a plain "
                         f"{COPY_BYTES >> 20} MiB device copy of known size that calibrates the byte counters")
    ap.add_argument("--profile-reps", type=int, default=12)
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter files of a --profile-launch run "
                         "into the traffic record bench.py reads, and print a summary")
    ap.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV",
                    help="print a markdown table of a rocprofv3 --kernel-trace CSV: calls, average, minimum and "
                         "maximum duration per kernel and grid")
    return ap.parse_args()


def capture(torch, fns):
    """One HIP graph holding the given launches, in order."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    return g


WARM_MS = 50.0                  # replays before any timed graph: clocks ramp up under sustained load


def time_graph(torch, g, reps):
    """Average milliseconds per replay, HIP events on the launch stream, after
    at least WARM_MS of untimed replays: after an idle host-side phase (weight
    packing, copies) the GPU's clocks take tens of milliseconds of sustained
    work to come back up, and a single warm-up replay left the prefill GEMM's
    first timed replays ~20% slow."""
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < WARM_MS:
        g.replay()
        torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def launch_percentiles(torch, fns, blocker):
    """p10 / median / p90 of single-launch durations (us): each launch is
    bracketed by its own HIP events on the launch stream.  All launches are
    enqueued while `blocker` keeps the GPU busy, so they run back to back and
    no event pair includes host enqueue time."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in fns]
    torch.cuda.synchronize()
    blocker()
    for (a, b), f in zip(ev, fns):
        a.record()
        f()
        b.record()
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    return [float(v) for v in np.percentile(us, [10, 50, 90])]


def copy_rate(torch, dev, nbytes=1 << 30, reps=8):
    """Plain device-to-device copy (torch copy_), read + write bytes per second
    in GB/s: the achievable-bandwidth reference on this device."""
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    g = capture(torch, [lambda: b.copy_(a)])
    ms = time_graph(torch, g, reps)
    del g, a, b
    return 2.0 * nbytes / (ms * 1e-3) / 1e9


def main():
    args = parse()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.profile_launch:
        profile_launch(args)
        return

    import torch

    import weight_quantized_amd as ql
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def log(*a):
        print(*a, file=sys.stderr, flush=True)

    # ---------------- inputs: pack once on the host, replicate on the device
    shapes = {"gate_up": workloads.C2_GATEUP, "down": workloads.C2_DOWN}
    host = {}
    sets = {}
    for name, (n, k, g) in shapes.items():
        w = workloads.config_weight(name)
        qw, sc, qz = ql.awq_pack(w, g)
        host[name] = (qw, sc, qz)
        base = [torch.from_numpy(a).to(dev) for a in (qw, sc, qz)]
        sets[name] = [base] + [[t.clone() for t in base] for _ in range(args.copies - 1)]
        del w
    xs = {(name, m): torch.from_numpy(workloads.config_activations(name, m, shapes[name][1])).to(dev)
          for name in shapes for m in DETAIL_M}
    ys = {(name, m): torch.empty((m, shapes[name][0]), dtype=torch.float16, device=dev)
          for name in shapes for m in DETAIL_M}
    need = max(ql.w4a16_workspace_bytes(m, n, k, g) for (n, k, g) in shapes.values() for m in DETAIL_M)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
    launches = [(name, m) for m in DECODE_M for name in ("gate_up", "down")]
    detail_launches = [(name, m) for m in DETAIL_M for name in ("gate_up", "down")]
    step_bytes = sum(w4a16_bytes(m, *shapes[name]) for name, m in launches)

    def launch(name, m, copy):
        d = sets[name][copy % args.copies]
        n, k, g = shapes[name]
        return lambda: ql.w4a16_gemm(xs[(name, m)], d[0], d[1], d[2], g, out=ys[(name, m)], workspace=ws)

    # eager warm-up of every launch (first-call costs stay out of the graphs)
    for name, m in detail_launches:
        launch(name, m, 0)()
    torch.cuda.synchronize()

    # ---------------- per-launch durations: graphs of back-to-back launches
    reps = 8
    per = {}
    for name, m in detail_launches:
        g = capture(torch, [launch(name, m, c) for c in range(args.copies)])
        per[(name, m)] = time_graph(torch, g, reps) * 1e3 / args.copies      # us per launch
        del g

    # ---------------- single-launch percentiles: 100 eager launches per shape, cold copies
    pct = {}
    big = [torch.empty(1 << 30, dtype=torch.uint8, device=dev) for _ in range(2)]

    def blocker():
        for _ in range(12):
            big[1].copy_(big[0])

    for name, m in detail_launches:
        pct[(name, m)] = launch_percentiles(torch, [launch(name, m, c) for c in range(100)], blocker)
    del big
    copy_gbs = copy_rate(torch, dev)

    # ---------------- the step: graphs rotating the weight copies
    nphase = args.copies // np.gcd(len(launches), args.copies)
    step_graphs = [capture(torch, [launch(name, m, p * len(launches) + i) for i, (name, m) in enumerate(launches)])
                   for p in range(nphase)]
    log(f"[bench] warmup {args.warmup} steps")
    for s in range(args.warmup):
        step_graphs[s % nphase].replay()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step_graphs[s % nphase].replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    detail = []
    for (name, m) in detail_launches:
        n, k, g = shapes[name]
        b = w4a16_bytes(m, n, k, g)
        us = per[(name, m)]
        p10, p50, p90 = pct[(name, m)]
        detail.append({"shape": name, "m": m, "n": n, "k": k, "in_step": m in DECODE_M, "us": round(us, 2),
                       "GB/s": round(b / (us * 1e-6) / 1e9, 1),
                       "frac_hbm": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                       "single_launch_us": {"p10": round(p10, 2), "median": round(p50, 2), "p90": round(p90, 2),
                                            "launches": 100}})
    m32 = [(name, 32) for name in ("gate_up", "down")]
    m32_bytes = sum(w4a16_bytes(32, *shapes[name]) for name, _ in m32)
    m32_us = sum(per[key] for key in m32)
    dom = max(launches, key=lambda key: per[key])
    n, k, g = shapes[dom[0]]
    dom_bytes = w4a16_bytes(dom[1], n, k, g)
    achieved = dom_bytes / (per[dom] * 1e-6) / 1e9
    src_hash = kernel_source_hash()
    rec = traffic_records().get(f"{dom[0]}_m{dom[1]}", {})
    traffic = rec.get("bytes_per_launch") if rec.get("source_hash") == src_hash else None
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": f"W4A16 decode launch ({dom[0]}, M={dom[1]}, N={n}, K={k}, group {g})",
                "avg_us": round(per[dom], 3), "bytes_per_launch": dom_bytes, "source_hash": src_hash}

    extra = []
    if not args.no_extra:
        extra = measure_extra(torch, ql, workloads, dev, log)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(host, shapes, launches, args.cpu_sample_rows, log)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": "W4A16 decode, LLaMA-7B MLP: gate/up K=4096 N=22016 + down K=11008 N=4096, "
                               "M in {1,4,8,16}, group 128, asymmetric uint4, fp16 activations",
                   "group": GROUP, "m": list(DECODE_M), "cold_weight_copies": args.copies,
                   "bytes_per_step": step_bytes, "launch": "hip graph per step"},
        "roofline": roofline, "cpu_baseline": cpu, "detail": detail,
        "m32": {"note": "the same MLP workload at M=32, outside the M<=16 metric: gate/up + down, per-launch graphs",
                "us": round(m32_us, 2), "GB/s": round(m32_bytes / (m32_us * 1e-6) / 1e9, 1),
                "frac_hbm": round(m32_bytes / (m32_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        "extra": extra,
        "reference": {"d2d_copy_GBps": round(copy_gbs, 1),
                      "note": "torch copy_ of 1 GiB on the device, read + write bytes; "
                              "achievable HBM rate on this device (fractions stay against 8 TB/s)"},
    }
    print(json.dumps(line), flush=True)


def cold_copies(nbytes, least=4):
    """Weight copies whose total exceeds twice the Infinity Cache."""
    return max(least, -(-2 * CACHE_BYTES // nbytes))


def w4a16_entry(torch, ql, x, ds, g, y, ws, reps, name, m, n, k):
    """Graph-averaged time of launches rotating the weight copies `ds`; GB/s
    against HBM for M <= 64, TFLOP/s against fp16 MFMA above."""
    ql.w4a16_gemm(x, *ds[0], g, out=y, workspace=ws)
    gph = capture(torch, [(lambda d=d: ql.w4a16_gemm(x, *d, g, out=y, workspace=ws)) for d in ds])
    us = time_graph(torch, gph, reps) * 1e3 / len(ds)
    del gph
    b = w4a16_bytes(m, n, k, g)
    e = {"name": name, "m": m, "n": n, "k": k, "group": g, "us": round(us, 2), "copies": len(ds),
         "GB/s": round(b / (us * 1e-6) / 1e9, 1)}
    if m <= 64:
        e.update({"bound": "hbm", "frac_hbm": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)})
    else:
        tf = 2.0 * m * n * k / (us * 1e-6) / 1e12
        e.update({"bound": "mfma_fp16", "TFLOP/s": round(tf, 1), "frac_mfma_fp16": round(tf / FP16_MFMA_PEAK_TFLOPS, 4)})
    return e


def measure_extra(torch, ql, workloads, dev, log):
    out = []
    reps = 6
    # LLaMA-7B q_proj GEMV, M=1, group 128
    log("[bench] extra: W4A16 q_proj M=1")
    n, k, g = workloads.C1
    qw, sc, qz = ql.awq_pack(workloads.config_weight("q_proj"), g)
    copies = cold_copies(qw.nbytes)
    ds = [[torch.from_numpy(a).to(dev) for a in (qw, sc, qz)] for _ in range(copies)]
    x = torch.from_numpy(workloads.config_activations("q_proj", 1, k)).to(dev)
    y = torch.empty((1, n), dtype=torch.float16, device=dev)
    ws = torch.zeros(max(ql.w4a16_workspace_bytes(1, n, k, g), 1), dtype=torch.uint8, device=dev)
    out.append(w4a16_entry(torch, ql, x, ds, g, y, ws, reps, "w4a16_q_proj", 1, n, k))
    del ds
    # LLaMA-13B MLP sweep: both projections, groups 128 and 32, M in {1, 8, 64, 256, 1024}
    for name in ("13b_up", "13b_down"):
        w = workloads.config_weight(name)
        n, k = w.shape
        for g in (128, 32):
            log(f"[bench] extra: W4A16 LLaMA-13B {name} group {g}")
            qw, sc, qz = ql.awq_pack(w, g)
            copies = cold_copies(qw.nbytes)
            ds = [[torch.from_numpy(a).to(dev) for a in (qw, sc, qz)] for _ in range(copies)]
            need = max(ql.w4a16_workspace_bytes(m, n, k, g) for m in workloads.C5_M)
            ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
            for m in workloads.C5_M:
                x = torch.from_numpy(workloads.config_activations(name, m, k)).to(dev)
                y = torch.empty((m, n), dtype=torch.float16, device=dev)
                out.append(w4a16_entry(torch, ql, x, ds, g, y, ws, reps, "w4a16_" + name, m, n, k))
            del ds, ws
        del w
    # W4A16 prefill, fused QKV M=512, group 64
    n, k, g = workloads.C3
    w = workloads.config_weight("qkv")
    qw, sc, qz = ql.awq_pack(w, g)
    del w
    copies = cold_copies(qw.nbytes)
    ds = [[torch.from_numpy(a).to(dev) for a in (qw, sc, qz)] for _ in range(copies)]
    x = torch.from_numpy(workloads.config_activations("qkv", 512, k)).to(dev)
    y = torch.empty((512, n), dtype=torch.float16, device=dev)
    log("[bench] extra: W4A16 prefill M=512")
    ql.w4a16_gemm(x, *ds[0], g, out=y)
    gph = capture(torch, [(lambda d=d: ql.w4a16_gemm(x, *d, g, out=y)) for d in ds])
    us = time_graph(torch, gph, reps) * 1e3 / copies
    flops = 2.0 * 512 * n * k
    out.append({"name": "w4a16_prefill_qkv", "m": 512, "n": n, "k": k, "group": g, "us": round(us, 2),
                "TFLOP/s": round(flops / (us * 1e-6) / 1e12, 1),
                "frac_mfma_fp16": round(flops / (us * 1e-6) / 1e12 / FP16_MFMA_PEAK_TFLOPS, 4)})
    del gph, ds
    # context, not part of the path: the vendor library's plain fp16 GEMM
    # (torch.mm on hipBLASLt) at the same shape with dense fp16 weights (4x the
    # weight bytes, no dequantisation), timed the same way
    w16 = torch.from_numpy(workloads.config_weight("qkv")).to(dev).half()
    w16s = [w16.clone() for _ in range(cold_copies(w16.numel() * 2))]
    del w16
    torch.mm(x, w16s[0].t(), out=y)
    torch.cuda.synchronize()
    gl = capture(torch, [(lambda w=w: torch.mm(x, w.t(), out=y)) for w in w16s])
    us_l = time_graph(torch, gl, reps) * 1e3 / len(w16s)
    out.append({"name": "library_fp16_gemm_qkv", "kind": "reference: torch.mm (hipBLASLt), dense fp16 weights",
                "m": 512, "n": n, "k": k, "us": round(us_l, 2), "TFLOP/s": round(flops / (us_l * 1e-6) / 1e12, 1),
                "frac_mfma_fp16": round(flops / (us_l * 1e-6) / 1e12 / FP16_MFMA_PEAK_TFLOPS, 4)})
    del gl, w16s
    # W8A8 SmoothQuant: QRMSNorm + int8 GEMM, M=2048, K=4096, N=11008
    xh, gamma, wf = workloads.smoothquant_inputs()
    s, gs, wsm = ql.smooth(xh, gamma, wf)
    wq, wsc = ql.w8a8_quant_weight(wsm)
    wq8, wsc8 = ql.fp8_quant_weight(wsm)
    del wf, wsm
    xd = torch.from_numpy(xh).to(dev)
    gd = torch.from_numpy(gs).to(dev)
    copies = cold_copies(wq.nbytes)
    wqs = [torch.from_numpy(wq).to(dev) for _ in range(copies)]
    wsd = torch.from_numpy(wsc).to(dev)
    m, kk = xh.shape
    nn = wq.shape[0]
    xq = torch.empty((m, kk), dtype=torch.int8, device=dev)
    xsc = torch.empty((m,), dtype=torch.float32, device=dev)
    yy = torch.empty((m, nn), dtype=torch.float16, device=dev)
    log("[bench] extra: W8A8 QRMSNorm + GEMM M=2048")
    ql.w8a8_quant_rmsnorm(xd, gd, 1e-6, xq=xq, x_scale=xsc)
    ql.w8a8_gemm(xq, xsc, wqs[0], wsd, out=yy)
    gn = capture(torch, [lambda: ql.w8a8_quant_rmsnorm(xd, gd, 1e-6, xq=xq, x_scale=xsc)] * 8)
    us_n = time_graph(torch, gn, reps) * 1e3 / 8
    gg = capture(torch, [(lambda wqd=wqd: ql.w8a8_gemm(xq, xsc, wqd, wsd, out=yy)) for wqd in wqs])
    us_g = time_graph(torch, gg, reps) * 1e3 / copies
    nb = m * kk * 2 + kk * 2 + m * kk + m * 4
    out.append({"name": "w8a8_quant_rmsnorm", "m": m, "k": kk, "us": round(us_n, 2),
                "GB/s": round(nb / (us_n * 1e-6) / 1e9, 1),
                "frac_hbm": round(nb / (us_n * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)})
    ops = 2.0 * m * nn * kk
    out.append({"name": "w8a8_gemm", "m": m, "n": nn, "k": kk, "us": round(us_g, 2),
                "TOP/s": round(ops / (us_g * 1e-6) / 1e12, 1),
                "frac_mfma_int8": round(ops / (us_g * 1e-6) / 1e12 / INT8_MFMA_PEAK_TOPS, 4)})
    # context: the vendor library's int8 GEMM (torch._int_mm on hipBLASLt) on
    # the same codes, int32 output (no scales, no fp16 epilogue)
    acc32 = torch.empty((m, nn), dtype=torch.int32, device=dev)
    torch._int_mm(xq, wqs[0].t(), out=acc32)
    torch.cuda.synchronize()
    gi = capture(torch, [(lambda wqd=wqd: torch._int_mm(xq, wqd.t(), out=acc32)) for wqd in wqs])
    us_i = time_graph(torch, gi, reps) * 1e3 / copies
    out.append({"name": "library_int8_gemm", "kind": "reference: torch._int_mm (hipBLASLt), int32 output",
                "m": m, "n": nn, "k": kk, "us": round(us_i, 2), "TOP/s": round(ops / (us_i * 1e-6) / 1e12, 1),
                "frac_mfma_int8": round(ops / (us_i * 1e-6) / 1e12 / INT8_MFMA_PEAK_TOPS, 4)})
    del gi, acc32

    # the steps beside the path: residual-fused QRMSNorm, per-token
    # quantisation of a plain activation, the GEMM with bias and residual
    rng = np.random.default_rng(5)
    rd = torch.from_numpy(workloads.activations(rng, m, kk)).to(dev)
    hd = torch.empty_like(xd)
    log("[bench] extra: fused W8A8 steps M=2048")
    ql.w8a8_add_quant_rmsnorm(xd, rd, gd, 1e-6, h_out=hd, xq=xq, x_scale=xsc)
    ga = capture(torch, [lambda: ql.w8a8_add_quant_rmsnorm(xd, rd, gd, 1e-6, h_out=hd, xq=xq, x_scale=xsc)] * 8)
    us_a = time_graph(torch, ga, reps) * 1e3 / 8
    nb = 3 * 2 * m * kk + 2 * kk + m * kk + 4 * m
    out.append({"name": "w8a8_add_quant_rmsnorm", "m": m, "k": kk, "us": round(us_a, 2),
                "GB/s": round(nb / (us_a * 1e-6) / 1e9, 1),
                "frac_hbm": round(nb / (us_a * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)})
    ql.w8a8_quant_per_token(xd, xq=xq, x_scale=xsc)
    gp = capture(torch, [lambda: ql.w8a8_quant_per_token(xd, xq=xq, x_scale=xsc)] * 8)
    us_p = time_graph(torch, gp, reps) * 1e3 / 8
    nb = 2 * m * kk + m * kk + 4 * m
    out.append({"name": "w8a8_quant_per_token", "m": m, "k": kk, "us": round(us_p, 2),
                "GB/s": round(nb / (us_p * 1e-6) / 1e9, 1),
                "frac_hbm": round(nb / (us_p * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)})
    bias = torch.from_numpy(workloads.activations(rng, 1, nn)[0].copy()).to(dev)
    res = torch.from_numpy(workloads.activations(rng, m, nn)).to(dev)
    ql.w8a8_gemm_ex(xq, xsc, wqs[0], wsd, bias=bias, residual=res, out=yy)
    ge = capture(torch, [(lambda wqd=wqd: ql.w8a8_gemm_ex(xq, xsc, wqd, wsd, bias=bias, residual=res, out=yy))
                         for wqd in wqs])
    us_e = time_graph(torch, ge, reps) * 1e3 / copies
    out.append({"name": "w8a8_gemm_bias_residual", "m": m, "n": nn, "k": kk, "us": round(us_e, 2),
                "TOP/s": round(ops / (us_e * 1e-6) / 1e12, 1),
                "frac_mfma_int8": round(ops / (us_e * 1e-6) / 1e12 / INT8_MFMA_PEAK_TOPS, 4)})

    # the same layer with FP8 E4M3 codes
    del wqs, ge, ga, gp
    log("[bench] extra: FP8 QRMSNorm + GEMM M=2048")
    xq8 = torch.empty((m, kk), dtype=torch.uint8, device=dev)
    ql.fp8_quant_rmsnorm(xd, gd, 1e-6, xq=xq8, x_scale=xsc)
    g8n = capture(torch, [lambda: ql.fp8_quant_rmsnorm(xd, gd, 1e-6, xq=xq8, x_scale=xsc)] * 8)
    us_8n = time_graph(torch, g8n, reps) * 1e3 / 8
    nb = m * kk * 2 + kk * 2 + m * kk + m * 4
    out.append({"name": "fp8_quant_rmsnorm", "m": m, "k": kk, "us": round(us_8n, 2),
                "GB/s": round(nb / (us_8n * 1e-6) / 1e9, 1),
                "frac_hbm": round(nb / (us_8n * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)})
    w8s = [torch.from_numpy(wq8).to(dev) for _ in range(copies)]
    w8sc = torch.from_numpy(wsc8).to(dev)
    ql.fp8_gemm(xq8, xsc, w8s[0], w8sc, out=yy)
    g8 = capture(torch, [(lambda w8=w8: ql.fp8_gemm(xq8, xsc, w8, w8sc, out=yy)) for w8 in w8s])
    us_8 = time_graph(torch, g8, reps) * 1e3 / copies
    out.append({"name": "fp8_gemm", "m": m, "n": nn, "k": kk, "us": round(us_8, 2),
                "TFLOP/s": round(ops / (us_8 * 1e-6) / 1e12, 1),
                "frac_mfma_fp8": round(ops / (us_8 * 1e-6) / 1e12 / FP8_MFMA_PEAK_TFLOPS, 4)})
    del g8, w8s, g8n

    # KV cache INT8, groups of 128: one LLaMA-7B layer's K and V for 4096
    # tokens (2 x 4096 x 32 heads x 128), fp16 values of N(0, 1) per head
    # scaled by U(0.1, 10)
    log("[bench] extra: KV cache INT8")
    kv = torch.from_numpy(
        (rng.standard_normal((2 * 4096 * 32, 128)) * rng.uniform(0.1, 10, (2 * 4096 * 32, 1))).astype(np.float16)
    ).to(dev)
    groups = kv.shape[0]
    kq = torch.empty(kv.shape, dtype=torch.int8, device=dev)
    ksc = torch.empty((groups,), dtype=torch.float32, device=dev)
    kout = torch.empty_like(kv)
    ql.kv_quant_int8(kv, 128, q=kq, scale=ksc)
    gq = capture(torch, [lambda: ql.kv_quant_int8(kv, 128, q=kq, scale=ksc)] * 8)
    us_q = time_graph(torch, gq, reps) * 1e3 / 8
    gd_ = capture(torch, [lambda: ql.kv_dequant_int8(kq, ksc, 128, out=kout)] * 8)
    us_d = time_graph(torch, gd_, reps) * 1e3 / 8
    elems = kv.numel()
    for name, us_ in (("kv_quant_int8", us_q), ("kv_dequant_int8", us_d)):
        nb = elems * 2 + elems + groups * 4
        out.append({"name": name, "values": elems, "group": 128, "us": round(us_, 2),
                    "GB/s": round(nb / (us_ * 1e-6) / 1e9, 1),
                    "frac_hbm": round(nb / (us_ * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)})

    # AWQ ratio search, offline: q_proj weights, 128 calibration tokens of the
    # prefill recipe, 20 ratios; host grid, one device GEMM per candidate
    log("[bench] extra: AWQ ratio search (q_proj, 128 tokens, 20 ratios)")
    wq_ = workloads.config_weight("q_proj")
    xc = workloads.config_activations("qkv", 128, wq_.shape[1])
    t0 = time.perf_counter()
    err, best, _, _ = ql.awq_search(xc, wq_, 128, 20)
    secs = time.perf_counter() - t0
    out.append({"name": "awq_search", "t": 128, "n": int(wq_.shape[0]), "k": int(wq_.shape[1]), "group": 128,
                "grid": 20, "s": round(secs, 3), "best_ratio": best / 20,
                "err_vs_ratio_0.5": round(float(err[best] / err[10]), 4)})
    return out


CPU_MIN_SECONDS = 10.0   # oracle time the CPU baseline accumulates at least
CPU_MAX_PASSES = 8


def cpu_baseline(host, shapes, launches, rows_opt, log):
    """The oracle (unmodified) on every launch of one step, restricted to a
    subset of output channels; the rate is scaled by the fraction computed."""
    import oracle
    import workloads

    cores = oracle.num_threads()
    rows_per_opt = rows_opt or max(shapes[name][0] for name in shapes)   # the whole step: ~4 s on 16 cores
    total_bytes = 0.0
    total_s = 0.0
    passes = 0
    # whole passes over the step's launches until at least 10 s of oracle time
    while passes < CPU_MAX_PASSES and (passes == 0 or total_s < CPU_MIN_SECONDS):
        for name, m in launches:
            n, k, g = shapes[name]
            qw, sc, qz = host[name]
            x = workloads.config_activations(name, m, k)
            rows_per = min(rows_per_opt, n)
            rows = np.linspace(0, n - 1, rows_per).astype(np.int64)
            t0 = time.perf_counter()
            oracle.w4a16_forward(x, qw, sc, qz, g, rows=rows)
            total_s += time.perf_counter() - t0
            total_bytes += w4a16_bytes(m, n, k, g) * (rows_per / n)
        passes += 1
        log(f"[bench] cpu baseline: pass {passes}, {total_s:.2f} s for up to {rows_per_opt} channels per launch")
    return {"value": round(total_bytes / total_s / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{passes} pass(es) over one step ({len(launches)} launches), min({rows_per_opt}, N) evenly "
                      f"spaced output channels per launch, {total_s:.1f} s of oracle time"}


def profile_launch(args):
    """One workload, launched `--profile-reps` times eagerly, for rocprofv3
    counter runs; decode launches rotate `--copies` weight copies so each reads
    cold weights.  Then a plain device copy (torch neg on COPY_BYTES of fp16:
    COPY_BYTES read, COPY_BYTES written) whose counter values calibrate them."""
    import torch

    import weight_quantized_amd as ql
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    shape, m = args.profile_launch.split(",")
    m = int(m)
    if shape in ("gate_up", "down", "q_proj"):
        n, k, g = {"gate_up": workloads.C2_GATEUP, "down": workloads.C2_DOWN, "q_proj": workloads.C1}[shape]
        w = workloads.config_weight(shape)
        qw, sc, qz = ql.awq_pack(w, g)
        del w
        base = [torch.from_numpy(a).to(dev) for a in (qw, sc, qz)]
        sets = [base] + [[t.clone() for t in base] for _ in range(args.copies - 1)]
        x = torch.from_numpy(workloads.config_activations(shape, m, k)).to(dev)
        y = torch.empty((m, n), dtype=torch.float16, device=dev)
        ws = torch.zeros(max(ql.w4a16_workspace_bytes(m, n, k, g), 1), dtype=torch.uint8, device=dev)
        for i in range(args.profile_reps):
            d = sets[i % args.copies]
            ql.w4a16_gemm(x, d[0], d[1], d[2], g, out=y, workspace=ws)
        desc = {"shape": f"{shape}_m{m}", "bytes_per_launch": w4a16_bytes(m, n, k, g)}
    elif shape == "qkv":
        n, k, g = workloads.C3
        w = workloads.config_weight("qkv")
        qw, sc, qz = ql.awq_pack(w, g)
        del w
        d = [torch.from_numpy(a).to(dev) for a in (qw, sc, qz)]
        x = torch.from_numpy(workloads.config_activations("qkv", m, k)).to(dev)
        y = torch.empty((m, n), dtype=torch.float16, device=dev)
        for _ in range(args.profile_reps):
            ql.w4a16_gemm(x, *d, g, out=y)
        desc = {"shape": f"qkv_m{m}", "flops_per_launch": 2 * m * n * k}
    elif shape == "w8a8":
        xh, gamma, wf = workloads.smoothquant_inputs(m=m)
        s_, gs, wsm = ql.smooth(xh, gamma, wf)
        wq, wsc = ql.w8a8_quant_weight(wsm)
        del wf, wsm
        xd, gd = torch.from_numpy(xh).to(dev), torch.from_numpy(gs).to(dev)
        wqd, wsd = torch.from_numpy(wq).to(dev), torch.from_numpy(wsc).to(dev)
        xq = torch.empty(xh.shape, dtype=torch.int8, device=dev)
        xsc = torch.empty((m,), dtype=torch.float32, device=dev)
        yy = torch.empty((m, wq.shape[0]), dtype=torch.float16, device=dev)
        for _ in range(args.profile_reps):
            ql.w8a8_quant_rmsnorm(xd, gd, 1e-6, xq=xq, x_scale=xsc)
            ql.w8a8_gemm(xq, xsc, wqd, wsd, out=yy)
        desc = {"shape": f"w8a8_m{m}", "ops_per_launch": 2 * m * wq.shape[0] * xh.shape[1]}
    elif shape == "fp8":
        xh, gamma, wf = workloads.smoothquant_inputs(m=m)
        s_, gs, wsm = ql.smooth(xh, gamma, wf)
        wq8, wsc8 = ql.fp8_quant_weight(wsm)
        del wf, wsm
        xd, gd = torch.from_numpy(xh).to(dev), torch.from_numpy(gs).to(dev)
        wqd, wsd = torch.from_numpy(wq8).to(dev), torch.from_numpy(wsc8).to(dev)
        xq = torch.empty(xh.shape, dtype=torch.uint8, device=dev)
        xsc = torch.empty((m,), dtype=torch.float32, device=dev)
        yy = torch.empty((m, wq8.shape[0]), dtype=torch.float16, device=dev)
        for _ in range(args.profile_reps):
            ql.fp8_quant_rmsnorm(xd, gd, 1e-6, xq=xq, x_scale=xsc)
            ql.fp8_gemm(xq, xsc, wqd, wsd, out=yy)
        desc = {"shape": f"fp8_m{m}", "flops_per_launch": 2 * m * wq8.shape[0] * xh.shape[1]}
    elif shape == "kv":
        # KV cache INT8 codec on m tokens of one LLaMA-7B layer's K and V (2 x m x 32 heads x 128)
        rng = np.random.default_rng(5)
        kv = torch.from_numpy((rng.standard_normal((2 * m * 32, 128)) *
                               rng.uniform(0.1, 10, (2 * m * 32, 1))).astype(np.float16)).to(dev)
        kq = torch.empty(kv.shape, dtype=torch.int8, device=dev)
        ksc = torch.empty((kv.shape[0],), dtype=torch.float32, device=dev)
        kout = torch.empty_like(kv)
        for _ in range(args.profile_reps):
            ql.kv_quant_int8(kv, 128, q=kq, scale=ksc)
            ql.kv_dequant_int8(kq, ksc, 128, out=kout)
        desc = {"shape": f"kv_m{m}", "values": kv.numel(), "bytes_per_launch": kv.numel() * 3 + kv.shape[0] * 4}
    else:
        raise SystemExit(f"unknown workload {shape!r}")
    torch.cuda.synchronize()
    src = torch.ones(COPY_BYTES // 2, dtype=torch.float16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(args.profile_reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    desc.update({"reps": args.profile_reps, "copy_bytes": COPY_BYTES, "source_hash": kernel_source_hash()})
    print(json.dumps(desc), flush=True)


def _counter_rows(path):
    import csv
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
            out[key] = out.get(key, 0.0) + float(r["Counter_Value"])
    return out


def traffic_summary(fetch_csv, write_csv):
    """HBM bytes per launch of the profiled decode kernel from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by the same counter's reading on
    the calibration copy of known size.  Writes TRAFFIC_FILE and prints a
    markdown summary."""
    fetch, write = _counter_rows(fetch_csv), _counter_rows(write_csv)

    def pick(rows, sub):
        return sorted(v for (_, name), v in rows.items() if sub in name)

    def median(v):
        return float(np.median(v)) if v else float("nan")

    dec_f = pick(fetch, "w4a16_decode") + pick(fetch, "w4a16_gemv")
    dec_w = pick(write, "w4a16_decode") + pick(write, "w4a16_gemv")
    cp_f, cp_w = pick(fetch, "neg_kernel"), pick(write, "neg_kernel")
    if not (dec_f and dec_w and cp_f and cp_w):
        raise SystemExit("counter files lack the decode kernel or the calibration copy")
    kib = COPY_BYTES / 1024.0
    f_fac, w_fac = kib / median(cp_f), kib / median(cp_w)
    fetch_b = median(dec_f) * 1024.0 * f_fac
    write_b = median(dec_w) * 1024.0 * w_fac
    # the launch this describes is the one `bench.py --profile-launch` ran: its stdout (a JSON line) is
    # expected as profile_launch.json next to the counter directories
    meta_path = os.path.join(os.path.dirname(os.path.abspath(fetch_csv)), "..", "profile_launch.json")
    meta = {}
    for cand in (meta_path, os.path.join(os.path.dirname(os.path.abspath(fetch_csv)), "profile_launch.json")):
        if os.path.exists(cand):
            with open(cand) as f:
                lines = [ln for ln in f.read().splitlines() if ln.startswith("{")]
            if lines:
                meta = json.loads(lines[-1])
            break
    rec = {"source_hash": meta.get("source_hash", kernel_source_hash()), "shape": meta.get("shape"),
           "kernel": sorted({name for (_, name) in fetch if "w4a16_decode" in name or "w4a16_gemv" in name}),
           "bytes_per_launch": round(fetch_b + write_b), "fetch_bytes": round(fetch_b), "write_bytes": round(write_b),
           "algorithmic_bytes": meta.get("bytes_per_launch"),
           "fetch_kib_raw": median(dec_f), "write_kib_raw": median(dec_w),
           "copy_fetch_kib_raw": median(cp_f), "copy_write_kib_raw": median(cp_w),
           "fetch_scale": round(f_fac, 4), "write_scale": round(w_fac, 4), "dispatches": len(dec_f)}
    records = traffic_records()
    records[rec["shape"]] = rec
    with open(TRAFFIC_FILE, "w") as f:
        json.dump({"records": records}, f, indent=1)
        f.write("\n")
    alg = rec["algorithmic_bytes"]
    print(f"| launch | {rec['shape']} |\n|---|---|")
    print(f"| decode FETCH_SIZE (KiB, median of {len(dec_f)}) | {median(dec_f):.0f} |")
    print(f"| decode WRITE_SIZE (KiB) | {median(dec_w):.0f} |")
    print(f"| copy of {COPY_BYTES >> 20} MiB: FETCH / WRITE (KiB) | {median(cp_f):.0f} / {median(cp_w):.0f} |")
    print(f"| scale factors (known bytes / counter) | {f_fac:.4f} / {w_fac:.4f} |")
    print(f"| decode HBM bytes per launch (fetch + write) | {fetch_b + write_b:,.0f} |")
    if alg:
        print(f"| algorithmic bytes per launch | {alg:,} (traffic / algorithmic = {(fetch_b + write_b) / alg:.3f}) |")


def trace_summary(path):
    """Kernel durations of a rocprofv3 --kernel-trace CSV, grouped by kernel
    name and grid, largest total time first."""
    import csv
    import re
    groups = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            name = re.sub(r"\(anonymous namespace\)::", "", name)
            name = re.sub(r"\(.*$", "", name) if "<" not in name else name[:name.rfind(">") + 1]
            grid = f"{r['Grid_Size_X']}x{r['Grid_Size_Y']}"
            lds = next((r[c] for c in ("LDS_Block_Size", "Group_Segment_Size", "Lds_Size") if c in r), "")
            key = (name, grid, r["Workgroup_Size_X"], lds)
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
            groups.setdefault(key, []).append(dur)
    print("| kernel | grid (threads) | workgroup | LDS bytes | calls | avg us | min us | max us |")
    print("|---|---|---|---|---|---|---|---|")
    for (name, grid, wg, lds), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        print(f"| {name} | {grid} | {wg} | {lds} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")


if __name__ == "__main__":
    main()
