#!/usr/bin/env python3
"""Benchmark of the quantized linear layer on one MI355X.

A step is one pass of the W4A16 decode hot path over the LLaMA-7B MLP
workload: for each batch size M in {1, 4, 8, 16, 32}, the fused gate/up
projection (K=4096, N=22016) and the down projection (K=11008, N=4096), int4
weights in groups of 128 (asymmetric uint4 zero points, fp16 scales), fp16
activations.  Weights are streamed cold: every launch reads one of several
weight copies that together exceed the 256 MB Infinity Cache.

`value` is algorithmic bytes (packed weights + scales + zero points + x + y)
per step divided by the step time, in GB/s.  The `roofline` object covers the
kernel that takes the most time, measured with HIP events on the stream it is
launched on.  `extra` reports the prefill W4A16 GEMM (M=512, fused QKV) and the
W8A8 SmoothQuant layer (QRMSNorm + int8 GEMM, M=2048) against their rooflines.
`cpu_baseline` times the CPU oracle on a bounded sample of the same step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
FP16_MFMA_PEAK_TFLOPS = 2500.0  # dense
INT8_MFMA_PEAK_TOPS = 5000.0    # dense
DECODE_M = (1, 4, 8, 16, 32)
GROUP = 128
METRIC = "W4A16/W8A8 GEMM: HBM GB/s (M<=16), TFLOP/s (M>=512), % of MI355X peak"


def w4a16_bytes(m, n, k, g):
    """Algorithmic bytes: packed codes, fp16 scales, uint4 zeros, fp16 x and y."""
    return n * k // 2 + n * (k // g) * 2 + n * (k // g) // 2 + m * k * 2 + m * n * 2


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--copies", type=int, default=12, help="cold-cache weight copies per shape")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--cpu-sample-rows", type=int, default=0,
                    help="output channels per shape for the oracle sample (0 = auto)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

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
          for name in shapes for m in DECODE_M}
    ys = {(name, m): torch.empty((m, shapes[name][0]), dtype=torch.float16, device=dev)
          for name in shapes for m in DECODE_M}
    need = max(ql.w4a16_workspace_bytes(m, n, k, g) for (n, k, g) in shapes.values() for m in DECODE_M)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    launches = [(name, m) for m in DECODE_M for name in ("gate_up", "down")]
    step_bytes = sum(w4a16_bytes(m, *shapes[name]) for name, m in launches)
    counter = [0]

    def run_step(events=None):
        for name, m in launches:
            n, k, g = shapes[name]
            d = sets[name][counter[0] % args.copies]
            counter[0] += 1
            if events is not None:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
            ql.w4a16_gemm(xs[(name, m)], d[0], d[1], d[2], g, out=ys[(name, m)], workspace=ws)
            if events is not None:
                e1.record()
                events.append((name, m, e0, e1))

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps, bracketed by synchronisation
    log(f"[bench] timing {args.steps} steps")
    events = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_step(events)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # per-launch durations
    per = {}
    for name, m, e0, e1 in events:
        per.setdefault((name, m), []).append(e0.elapsed_time(e1) * 1e3)   # us
    detail = []
    kernel_of = {}
    for (name, m), us in sorted(per.items(), key=lambda kv: (kv[0][1], kv[0][0])):
        n, k, g = shapes[name]
        b = w4a16_bytes(m, n, k, g)
        med = float(np.median(us))
        kname = "w4a16_decode_kernel<16>" if m <= 16 else "w4a16_decode_kernel<32>"
        kernel_of[(name, m)] = kname
        detail.append({"shape": name, "m": m, "n": n, "k": k, "us_median": round(med, 2),
                       "us_p10": round(float(np.percentile(us, 10)), 2),
                       "us_p90": round(float(np.percentile(us, 90)), 2),
                       "GB/s": round(b / (med * 1e-6) / 1e9, 1),
                       "frac_hbm": round(b / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)})
    # dominant kernel (largest total time): bytes per launch / mean launch duration
    tot = {}
    for key, us in per.items():
        kn = kernel_of[key]
        n, k, g = shapes[key[0]]
        t = tot.setdefault(kn, [0.0, 0, 0])
        t[0] += sum(us)
        t[1] += len(us)
        t[2] += len(us) * w4a16_bytes(key[1], n, k, g)
    dom = max(tot, key=lambda kn: tot[kn][0])
    dur_us, cnt, byt = tot[dom]
    achieved = (byt / cnt) / (dur_us / cnt * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "kernel": dom,
                "launches": cnt, "avg_us": round(dur_us / cnt, 3), "avg_bytes": int(byt / cnt)}

    # ---------------- extra: prefill and W8A8 (not part of value)
    extra = []
    if not args.no_extra:
        extra = measure_extra(torch, ql, workloads, dev, log)

    # ---------------- CPU baseline: the oracle on a bounded sample of the step
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(host, shapes, launches, args.cpu_sample_rows, log)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": "W4A16 decode, LLaMA-7B MLP: gate/up K=4096 N=22016 + down K=11008 N=4096, "
                               "M in {1,4,8,16,32}, group 128, asymmetric uint4, fp16 activations",
                   "group": GROUP, "m": list(DECODE_M), "cold_weight_copies": args.copies,
                   "bytes_per_step": step_bytes},
        "roofline": roofline, "cpu_baseline": cpu, "detail": detail, "extra": extra,
    }
    print(json.dumps(line), flush=True)


def _time_launches(torch, fn, iters, warm=3):
    for _ in range(warm):
        fn(0)
    torch.cuda.synchronize()
    evs = []
    for i in range(iters):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn(i)
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 for a, b in evs]


def measure_extra(torch, ql, workloads, dev, log):
    out = []
    # W4A16 prefill, fused QKV M=512, group 64
    n, k, g = workloads.C3
    w = workloads.config_weight("qkv")
    qw, sc, qz = ql.awq_pack(w, g)
    del w
    copies = 8
    ds = [[torch.from_numpy(a).to(dev) for a in (qw, sc, qz)] for _ in range(copies)]
    x = torch.from_numpy(workloads.config_activations("qkv", 512, k)).to(dev)
    y = torch.empty((512, n), dtype=torch.float16, device=dev)
    log("[bench] extra: W4A16 prefill M=512")
    us = _time_launches(torch, lambda i: ql.w4a16_gemm(x, *ds[i % copies], g, out=y), 30)
    med = float(np.median(us))
    flops = 2.0 * 512 * n * k
    out.append({"name": "w4a16_prefill_qkv", "m": 512, "n": n, "k": k, "group": g, "us_median": round(med, 2),
                "TFLOP/s": round(flops / (med * 1e-6) / 1e12, 1),
                "frac_mfma_fp16": round(flops / (med * 1e-6) / 1e12 / FP16_MFMA_PEAK_TFLOPS, 4)})
    del ds
    # W8A8 SmoothQuant: QRMSNorm + int8 GEMM, M=2048, K=4096, N=11008
    xh, gamma, wf = workloads.smoothquant_inputs()
    s, gs, wsm = ql.smooth(xh, gamma, wf)
    wq, wsc = ql.w8a8_quant_weight(wsm)
    del wf, wsm
    xd = torch.from_numpy(xh).to(dev)
    gd = torch.from_numpy(gs).to(dev)
    wqs = [torch.from_numpy(wq).to(dev) for _ in range(6)]
    wsd = torch.from_numpy(wsc).to(dev)
    m, kk = xh.shape
    nn = wq.shape[0]
    xq = torch.empty((m, kk), dtype=torch.int8, device=dev)
    xsc = torch.empty((m,), dtype=torch.float32, device=dev)
    yy = torch.empty((m, nn), dtype=torch.float16, device=dev)
    log("[bench] extra: W8A8 QRMSNorm + GEMM M=2048")
    us_n = _time_launches(torch, lambda i: ql.w8a8_quant_rmsnorm(xd, gd, 1e-6, xq=xq, x_scale=xsc), 30)
    us_g = _time_launches(torch, lambda i: ql.w8a8_gemm(xq, xsc, wqs[i % 6], wsd, out=yy), 30)
    nb = m * kk * 2 + kk * 2 + m * kk + m * 4
    med_n = float(np.median(us_n))
    out.append({"name": "w8a8_quant_rmsnorm", "m": m, "k": kk, "us_median": round(med_n, 2),
                "GB/s": round(nb / (med_n * 1e-6) / 1e9, 1),
                "frac_hbm": round(nb / (med_n * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)})
    ops = 2.0 * m * nn * kk
    med_g = float(np.median(us_g))
    out.append({"name": "w8a8_gemm", "m": m, "n": nn, "k": kk, "us_median": round(med_g, 2),
                "TOP/s": round(ops / (med_g * 1e-6) / 1e12, 1),
                "frac_mfma_int8": round(ops / (med_g * 1e-6) / 1e12 / INT8_MFMA_PEAK_TOPS, 4)})
    return out


def cpu_baseline(host, shapes, launches, rows_opt, log):
    """The oracle (unmodified) on every launch of one step, restricted to a
    subset of output channels; the rate is scaled by the fraction computed."""
    import oracle
    import workloads

    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    rows_per_opt = rows_opt or 2048
    total_bytes = 0.0
    total_s = 0.0
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
    log(f"[bench] cpu baseline: {total_s:.2f} s for up to {rows_per_opt} channels per launch")
    return {"value": round(total_bytes / total_s / 1e9, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"one step (10 launches), min({rows_per_opt}, N) evenly spaced output channels per launch, "
                      f"{total_s:.1f} s of oracle time"}


if __name__ == "__main__":
    main()
