#!/usr/bin/env python3
"""Benchmark of the quantized linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads a,b] [--no-cpu]

A step is one pass of the layer's hot path over one batch of synthetic input:
per-token int8 activation quantization followed by the quantized GEMM
(W4A16 has no activation quantization).  Weights are prepared offline
(fold, quantization) before timing.  Each timed region is one captured HIP
graph of exactly K steps; consecutive steps rotate over enough copies of the
quantized weights (> 512 MB) that every GEMM streams its weights from HBM
rather than from the 256 MB last-level cache.

The JSON line reports the headline workload (W8A8 decode FFN-up, M=8,
K=4096, N=11008) in HBM TB/s, with a "workloads" list holding every workload
(including the M=4096 prefill in INT8 TOP/s), each with the roofline of its
dominant kernel.  `roofline.traffic` is taken from profiles/traffic.json
(rocprofv3 FETCH_SIZE / WRITE_SIZE scaled by a copy-kernel calibration) when
it was measured on the current kernel sources, else null.
The cpu_baseline is the CPU oracle timed on the host's cores on a bounded
sample of the headline workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantized GEMM: HBM TB/s at M≤16, INT8 TOPS at M=4096, % of roofline"
HEADLINE = "w8a8_decode_ffn_up"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0         # MI355X dense int8 MFMA
F16_PEAK_TFLOPS = 2500.0        # MI355X dense fp16/bf16 MFMA
ROTATE_BYTES = 600 * 2 ** 20    # weight copies per rotation: > 2x the 256 MB MALL
KERNEL_SOURCES = {
    "w8a8": ["gemm_w8a8.hip", "qg_device.hpp"],
    "w4a8": ["gemm_w4a8.hip", "qg_device.hpp"],
    "w4a16": ["gemm_w4a16.hip", "qg_device.hpp"],
    "quant": ["quant.hip", "qg_device.hpp"],
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workloads", default="all",
                    help="comma list of workload names, or 'all' (headline first)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the cpu_baseline leg")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain device copy of 512 MiB (counter calibration)")
    return ap.parse_args()


def source_sha(path_key: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[path_key]:
        with open(os.path.join(ROOT, "bit_quantized_gemm_int8_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic():
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return {}
    with open(p) as f:
        return json.load(f)


# ----------------------------------------------------------------- workload

def algorithmic(wl):
    """Bytes the method must move and ops it must do, per GEMM call and per
    activation-quantization call (what the oracle defines, nothing more)."""
    M, K, N, G = wl.M, wl.K, wl.N, wl.K // 128
    out_b = {"f32": 4, "bf16": 2, "f16": 2}[wl.out_dtype]
    x_b = {"f32": 4, "bf16": 2, "f16": 2}[wl.x_dtype]
    if wl.path == "w8a8":
        gemm = N * K + 4 * N + M * K + 4 * M + out_b * M * N
    elif wl.path == "w4a8":
        gemm = N * K // 2 + 4 * N * G + M * K + 4 * M + out_b * M * N
    else:
        gemm = N * K // 2 + 4 * N * G + x_b * M * K + out_b * M * N
    quant = x_b * M * K + M * K + 4 * M if wl.path != "w4a16" else 0
    ops = 2 * M * N * K
    return gemm, quant, ops


def run_workload(wl, steps, warmup, traffic_db):
    import numpy as np
    import torch
    import bit_quantized_gemm_int8_amd as qg
    from workloads import draw, f32_to_bf16_bits, f32_to_f16

    dev = "cuda"
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
    print(f"[bench] {wl.name}: M={wl.M} K={wl.K} N={wl.N} preparing", file=sys.stderr, flush=True)
    d = draw(wl)
    w_d = torch.from_numpy(d["w"]).to(dev)
    if wl.fold:
        xc = torch.from_numpy(d["x_cal"]).to(dev)
        fold = qg.smoothquant_fold if wl.fold == "smoothquant" else qg.awq_fold
        s, w_d = fold(xc, w_d)
        x_in = qg.apply_smoothing(torch.from_numpy(d["x"]).to(dev), s, out_dtype=tdt[wl.x_dtype])
    elif wl.x_dtype == "bf16":
        x_in = torch.from_numpy(f32_to_bf16_bits(d["x"]).view(np.int16)).view(torch.bfloat16).to(dev)
    elif wl.x_dtype == "f16":
        x_in = torch.from_numpy(f32_to_f16(d["x"])).to(dev)
    else:
        x_in = torch.from_numpy(d["x"]).to(dev)

    if wl.path == "w8a8":
        wq, ws = qg.quantize_weight_i8_per_channel(w_d)
        weights = (wq, ws)
    else:
        weights = qg.quantize_weight_u4_g128(w_d)
    del w_d
    wbytes = sum(t.numel() * t.element_size() for t in weights)
    R = max(2, math.ceil(ROTATE_BYTES / wbytes))
    copies = [weights] + [tuple(t.clone() for t in weights) for _ in range(R - 1)]
    xq = torch.empty((wl.M, wl.K), dtype=torch.int8, device=dev)
    xs = torch.empty((wl.M,), dtype=torch.float32, device=dev)
    y = torch.empty((wl.M, wl.N), dtype=tdt[wl.out_dtype], device=dev)

    def quant():
        qg.quantize_per_token_i8(x_in, out=(xq, xs))

    def gemm(i):
        w = copies[i % R]
        if wl.path == "w8a8":
            qg.gemm_w8a8(xq, xs, w[0], w[1], out_dtype=y.dtype, out=y)
        elif wl.path == "w4a8":
            qg.gemm_w4a8_g128(xq, xs, w[0], w[1], w[2], out_dtype=y.dtype, out=y)
        else:
            qg.gemm_w4a16_g128(x_in, w[0], w[1], w[2], out_dtype=y.dtype, out=y)

    def step(i):
        if wl.path != "w4a16":
            quant()
        gemm(i)

    # eager reference output, then graphs
    step(0)
    torch.cuda.synchronize()
    y_ref = y.clone()

    def capture(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i)
        return g

    g_warm = capture(step, max(warmup, 1))
    g_step = capture(step, steps)
    g_gemm = capture(gemm, steps)
    g_quant = capture(lambda i: quant(), steps) if wl.path != "w4a16" else None

    # warmup replays, each checked against the eager result (all copies equal)
    for _ in range(2):
        y.zero_()
        g_warm.replay()
        torch.cuda.synchronize()
        if not torch.equal(y.view(torch.int16) if y.dtype != torch.float32 else y,
                           y_ref.view(torch.int16) if y.dtype != torch.float32 else y_ref):
            raise RuntimeError(f"{wl.name}: graph replay differs from the eager result")

    def timed(g):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return time.perf_counter() - t0, e0.elapsed_time(e1) / 1e3

    wall, gpu = timed(g_step)
    _, gemm_s = timed(g_gemm)
    quant_s = timed(g_quant)[1] if g_quant is not None else 0.0
    if not torch.equal(y.view(torch.int16) if y.dtype != torch.float32 else y,
                       y_ref.view(torch.int16) if y.dtype != torch.float32 else y_ref):
        raise RuntimeError(f"{wl.name}: timed replay differs from the eager result")

    gemm_b, quant_b, ops = algorithmic(wl)
    gemm_us = gemm_s / steps * 1e6
    quant_us = quant_s / steps * 1e6
    step_s = wall / steps
    path_key = wl.path
    tr = traffic_db.get(path_key + ":" + wl.name)
    traffic = None
    if tr and tr.get("source_sha") == source_sha(path_key):
        traffic = tr["bytes_per_launch"]
    if wl.path == "w8a8" and wl.M > 64:
        achieved = ops / (gemm_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": INT8_PEAK_TOPS,
                "unit": "TOP/s", "frac": round(achieved / INT8_PEAK_TOPS, 4), "traffic": traffic}
        value, unit = (ops / step_s / 1e12), "TOP/s"
    else:
        achieved = gemm_b / (gemm_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic}
        value, unit = ((gemm_b + quant_b) / step_s / 1e12), "TB/s"
    res = {
        "workload": wl.name, "path": wl.path, "M": wl.M, "K": wl.K, "N": wl.N,
        "x_dtype": wl.x_dtype, "out_dtype": wl.out_dtype,
        "value": round(value, 4), "unit": unit,
        "ms_per_step": round(step_s * 1e3, 5),
        "gpu_us_per_step": round(gpu / steps * 1e6, 3),
        "gemm_us": round(gemm_us, 3), "quant_us": round(quant_us, 3),
        "gemm_bytes": gemm_b, "quant_bytes": quant_b, "ops": ops,
        "gemm_tops": round(ops / (gemm_us * 1e-6) / 1e12, 2),
        "weight_copies": R, "roofline": roof,
    }
    print(f"[bench] {wl.name}: gemm {gemm_us:.2f} us ({roof['achieved']} {roof['unit']}, "
          f"{100 * roof['frac']:.1f}% of peak), quant {quant_us:.2f} us, "
          f"step {step_s * 1e6:.2f} us", file=sys.stderr, flush=True)
    del copies, g_warm, g_step, g_gemm, g_quant
    torch.cuda.empty_cache()
    return res


def copy_calibration():
    import torch
    n = 512 * 2 ** 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"[bench] copy calibration: 3 copies of {n} bytes", file=sys.stderr, flush=True)


def cpu_baseline(wl, seconds):
    """The oracle, as it stands, on the host cores: quantize the activations and
    run the W8A8 GEMM + epilogue for the headline workload, repeated for about
    `seconds` (weights quantized once beforehand, like the GPU leg)."""
    import numpy as np
    import oracle
    from workloads import draw
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report the visible cores
        threads = os.cpu_count()
    d = draw(wl)
    s = oracle.smoothquant_scales(d["x_cal"], d["w"])
    x_t = oracle.to_f32(oracle.fold_activation(d["x"], s, wl.x_dtype), wl.x_dtype)
    wq, ws = oracle.quantize_weight_i8_per_channel(oracle.fold_weight(d["w"], s))
    gemm_b, quant_b, _ = algorithmic(wl)
    n = 0
    t0 = time.perf_counter()
    while True:
        xq, xs = oracle.quantize_per_token_i8(x_t)
        oracle.gemm_w8a8(xq, xs, wq, ws)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round((gemm_b + quant_b) * n / el / 1e12, 6), "unit": "TB/s",
            "cores": threads, "kind": "oracle",
            "sample": f"{n} full steps of {wl.name} (per-token quantization of {wl.M}x{wl.K} "
                      f"+ {wl.M}x{wl.K}x{wl.N} W8A8 GEMM and epilogue) in {el:.1f} s",
            "ms_per_step": round(el / n * 1e3, 2)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the layer shards column-parallel without collectives; see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from workloads import WORKLOADS, by_name
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import bit_quantized_gemm_int8_amd as qg
    qg.load()
    names = [w.name for w in WORKLOADS] if args.workloads == "all" else args.workloads.split(",")
    names = sorted(names, key=lambda n: n != HEADLINE)
    traffic_db = load_traffic()
    results = [run_workload(by_name(n), args.steps, args.warmup, traffic_db) for n in names]
    if args.copy_calib:
        copy_calibration()
    head = next((r for r in results if r["workload"] == HEADLINE), results[0])
    cpu = None
    if not args.no_cpu and head["workload"] == HEADLINE:
        print("[bench] cpu_baseline: timing the oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(by_name(HEADLINE), args.cpu_seconds)
    line = {
        "metric": METRIC, "value": head["value"], "unit": head["unit"], "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i8",
        "data": "synthetic (seeded; Llama-2-7B-shaped layers, no trained weights)",
        "config": {"workload": head["workload"], "M": head["M"], "K": head["K"], "N": head["N"],
                   "x_dtype": head["x_dtype"], "out_dtype": head["out_dtype"],
                   "step": "quantize_per_token_i8 + gemm_w8a8 (captured HIP graph)",
                   "parallelism": "single GPU"},
        "roofline": head["roofline"], "cpu_baseline": cpu,
        "workloads": results,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
