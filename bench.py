#!/usr/bin/env python3
"""Benchmark of the quantized linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads a,b] [--no-cpu]

A step is one pass of the layer's hot path over one batch of synthetic input:
per-token int8 activation quantization followed by the quantized GEMM
(W4A16 has no activation quantization; W8A8 goes through quantize_gemm_w8a8,
which runs the two as one kernel where the library finds that faster).  Weights are prepared offline
(fold, quantization) before timing.  Each timed region is one captured HIP
graph of exactly K steps; consecutive steps rotate over enough copies of the
quantized weights (> 512 MB) that every GEMM streams its weights from HBM
rather than from the 256 MB last-level cache.

The JSON line reports the headline workload (W8A8 decode FFN-up, M=8,
K=4096, N=11008) in HBM TB/s, with a "workloads" list holding every workload
(including the M=4096 prefill in INT8 TOP/s, and the KV-cache INT8 quantizer
on one layer's 4096-position Llama-2-7B cache), each with the roofline of its
dominant kernel.  `roofline.traffic` is taken from profiles/traffic.json
(rocprofv3 FETCH_SIZE / WRITE_SIZE scaled by a copy-kernel calibration) when
it was measured on the current kernel sources, else null.
The cpu_baseline is the CPU oracle timed on the host's cores on a bounded
sample of the headline workload; each of the five core workloads carries its
own (oracle quantization + GEMM, a few seconds each).  measured_peaks holds
the ceilings measured in the same run: a plain streaming read of each decode
GEMM's byte count, the matrix cores on random operands, the empty launch.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantized GEMM: HBM TB/s at M≤16, INT8 TOPS at M=4096, % of roofline"
HEADLINE = "w8a8_decode_ffn_up"
BENCH_KV = ("kv_llama2_7b_4k",)   # KV-cache workloads in the default run
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0         # MI355X dense int8 MFMA
F16_PEAK_TFLOPS = 2500.0        # MI355X dense fp16/bf16 MFMA
ROTATE_BYTES = 600 * 2 ** 20    # weight copies per rotation: > 2x the 256 MB MALL
KERNEL_REPLAYS = 5              # replays of a per-kernel graph; the median is reported
KERNEL_SOURCES = {
    "w8a8": ["gemm_w8a8.hip", "qg_decode.hpp", "qg_device.hpp"],
    "w8a8_fq": ["gemm_w8a8_fq.hip", "qg_decode.hpp", "qg_device.hpp"],
    "w4a8": ["gemm_w4a8.hip", "gemm_w4a8_fused.hip", "qg_decode.hpp", "qg_device.hpp"],
    "w4a8_outl": ["gemm_w4a8.hip", "gemm_w4a8_fused.hip", "qg_decode.hpp", "qg_device.hpp"],
    "w4a8_sp24": ["gemm_w4a8_sp24.hip", "qg_decode.hpp", "qg_device.hpp"],
    "w4a16": ["gemm_w4a16.hip", "qg_decode.hpp", "qg_device.hpp"],
    "quant": ["quant.hip", "qg_device.hpp"],
    "kv": ["kv.hip", "qg_device.hpp"],
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
    ap.add_argument("--batch-sweep", action="store_true",
                    help="instead of the benchmark line: time every path at M = 1..64 next to "
                         "an fp16 dense GEMM of the same layer, one JSON record per (path, M)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured_peaks leg")
    ap.add_argument("--peaks", action="store_true",
                    help="only the measured_peaks leg (stream read, matrix cores, launch floor)")
    ap.add_argument("--cpu-seconds-each", type=float, default=3.0,
                    help="oracle time per non-headline workload in the per-workload cpu baselines")
    ap.add_argument("--ingest-counters", metavar="DIR",
                    help="summarise rocprofv3 output in DIR/{stats,fetch,write} into profiles/")
    return ap.parse_args()


def median_replay(run):
    """Median over KERNEL_REPLAYS calls of `run` (one timed graph replay each,
    returning seconds): a single replay of a graph of microsecond kernels
    has varied by up to ~15% from one replay to the next."""
    return statistics.median(run() for _ in range(KERNEL_REPLAYS))


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
    elif wl.path == "w4a8_outl":   # plus one 8-byte outlier record per group, s8 per channel
        gemm = N * K // 2 + 4 * N * G + 8 * N * G + 4 * N + M * K + 4 * M + out_b * M * N
    elif wl.path == "w4a8_sp24":   # 48 bytes of kept codes and positions per 128 inputs
        gemm = 48 * N * G + 4 * N * G + M * K + 4 * M + out_b * M * N
    else:
        gemm = N * K // 2 + 4 * N * G + x_b * M * K + out_b * M * N
    quant = x_b * M * K + M * K + 4 * M if wl.path != "w4a16" else 0
    ops = 2 * M * N * K
    return gemm, quant, ops


def fused_step(wl) -> bool:
    """Whether the workload's step runs the one-kernel quantize + W8A8 form,
    or for W4A8 (with or without outliers) the panel pair
    (quantize_per_token_i8_panel + gemm_w4a8_g128[_outliers]_panel): the
    library's own choice for these sizes, asked of the library (host only)."""
    import torch
    import bit_quantized_gemm_int8_amd as qg
    if wl.path == "w4a8":
        return qg.quantize_gemm_w4a8_g128_workspace_bytes(wl.M, wl.N, wl.K) > 0
    if wl.path == "w4a8_outl":
        # the panel pair where it measured faster than the plain outlier kernel
        # (MI355X: 1-8 rows 20-27% faster; 16 rows of K = 11008 slower)
        return wl.M <= 8 and qg.quantize_per_token_i8_panel_bytes(wl.M, wl.K) > 0
    if wl.path != "w8a8":
        return False
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
    return qg.quantize_gemm_w8a8_plan(tdt[wl.x_dtype], wl.M, wl.N, wl.K)


def dominant(wl):
    """(algorithmic bytes, ops, source key) of the workload's dominant kernel:
    the GEMM (for W4A8 on the panel pair, the panel GEMM: its token operands
    are the codes, counted once), or for the one-kernel W8A8 form that
    kernel, which reads the activations and writes their codes and scales
    but never reads the codes back."""
    gemm, quant, ops = algorithmic(wl)
    if fused_step(wl) and wl.path == "w8a8":
        return gemm + quant - (wl.M * wl.K + 4 * wl.M), ops, "w8a8_fq"
    return gemm, ops, wl.path


def kv_algorithmic(wl):
    """Bytes the KV-cache quantizer and dequantizer must move per call: the
    cache in its storage format, the int8 codes and the fp32 scales, each
    once."""
    el = wl.T * wl.H * wl.D
    x_b = {"f32": 4, "bf16": 2, "f16": 2}[wl.dtype]
    scales = 4 * wl.H * ((wl.T + 127) // 128) * wl.D
    return x_b * el + el + scales, el + scales + x_b * el


def run_kv(wl, steps, warmup, traffic_db):
    """KV-cache INT8 quantization of one layer's [T][H][D] cache (and its
    dequantization), each timed as a captured graph of `steps` calls rotating
    over more than 600 MB of cache copies."""
    import numpy as np
    import torch
    import bit_quantized_gemm_int8_amd as qg
    from workloads import draw_kv, f32_to_bf16_bits, f32_to_f16

    dev = "cuda"
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
    print(f"[bench] {wl.name}: T={wl.T} H={wl.H} D={wl.D} preparing", file=sys.stderr, flush=True)
    x = draw_kv(wl)
    if wl.dtype == "bf16":
        kv = torch.from_numpy(f32_to_bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(dev)
    elif wl.dtype == "f16":
        kv = torch.from_numpy(f32_to_f16(x)).to(dev)
    else:
        kv = torch.from_numpy(x).to(dev)
    del x
    q_b, dq_b = kv_algorithmic(wl)
    R = max(2, math.ceil(ROTATE_BYTES / q_b))
    S = (wl.T + 127) // 128
    ins = [kv] + [kv.clone() for _ in range(R - 1)]
    codes = [torch.empty((wl.T, wl.H, wl.D), dtype=torch.int8, device=dev) for _ in range(R)]
    scales = [torch.empty((wl.H, S, wl.D), dtype=torch.float32, device=dev) for _ in range(R)]
    outs = [torch.empty_like(kv) for _ in range(R)]

    def quant(i):
        qg.quantize_kv_i8_segments(ins[i % R], out=(codes[i % R], scales[i % R]))

    def dequant(i):
        qg.dequantize_kv_i8_segments(codes[i % R], scales[i % R], out_dtype=kv.dtype,
                                     out=outs[i % R])

    for i in range(R):
        quant(i)
    torch.cuda.synchronize()
    c_ref, s_ref = codes[0].clone(), scales[0].clone()

    def capture(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i)
        return g

    def timed(g):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3

    g_warm = capture(quant, max(warmup, 1))
    g_q = capture(quant, steps)
    g_dq = capture(dequant, steps)
    g_warm.replay()
    g_q.replay()    # first launch of a graph uploads it: untimed
    g_dq.replay()
    q_s = median_replay(lambda: timed(g_q))
    dq_s = median_replay(lambda: timed(g_dq))
    for i in range(R):
        if not (torch.equal(codes[i], c_ref) and torch.equal(scales[i], s_ref)):
            raise RuntimeError(f"{wl.name}: replayed codes differ from the eager result")
    q_us, dq_us = q_s / steps * 1e6, dq_s / steps * 1e6
    achieved = q_b / (q_us * 1e-6) / 1e9
    tr = traffic_db.get("kv:" + wl.name)
    traffic = tr["bytes_per_launch"] if tr and tr.get("source_sha") == source_sha("kv") else None
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic}
    res = {
        "workload": wl.name, "path": "kv_i8_segments", "T": wl.T, "H": wl.H, "D": wl.D,
        "x_dtype": wl.dtype, "value": round(q_b / (q_us * 1e-6) / 1e12, 4), "unit": "TB/s",
        "ms_per_step": round(q_us / 1e3, 5),
        "quant_us": round(q_us, 3), "dequant_us": round(dq_us, 3),
        "quant_bytes": q_b, "dequant_bytes": dq_b,
        "dequant_TBps": round(dq_b / (dq_us * 1e-6) / 1e12, 4),
        "copies": R, "roofline": roof,
    }
    print(f"[bench] {wl.name}: quant {q_us:.2f} us ({roof['achieved']} GB/s, "
          f"{100 * roof['frac']:.1f}% of peak), dequant {dq_us:.2f} us "
          f"({res['dequant_TBps']} TB/s)", file=sys.stderr, flush=True)
    del ins, codes, scales, outs, g_warm, g_q, g_dq
    torch.cuda.empty_cache()
    return res


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
    elif wl.path == "w4a8_outl":
        weights = qg.quantize_weight_u4_g128_outliers(w_d)
    elif wl.path == "w4a8_sp24":
        weights = qg.quantize_weight_u4_g128_sparse24(w_d)
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
        elif wl.path == "w4a8_outl":
            qg.gemm_w4a8_g128_outliers(xq, xs, *w, out_dtype=y.dtype, out=y)
        elif wl.path == "w4a8_sp24":
            qg.gemm_w4a8_g128_sparse24(xq, xs, *w, out_dtype=y.dtype, out=y)
        else:
            qg.gemm_w4a16_g128(x_in, w[0], w[1], w[2], out_dtype=y.dtype, out=y)

    fused = fused_step(wl)
    ws_bytes = (qg.quantize_gemm_w4a8_g128_workspace_bytes(wl.M, wl.N, wl.K) if wl.path == "w4a8"
                else qg.quantize_per_token_i8_panel_bytes(wl.M, wl.K) if wl.path == "w4a8_outl"
                else 0)
    workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    def layer(i):   # the layer through its one entry point (the library's choice)
        w = copies[i % R]
        if wl.path == "w8a8":
            qg.quantize_gemm_w8a8(x_in, w[0], w[1], out_dtype=y.dtype, out=y, xq_out=(xq, xs))
        else:
            qg.quantize_gemm_w4a8_g128(x_in, w[0], w[1], w[2], out_dtype=y.dtype, out=y,
                                       xq_out=(xq, xs), workspace=workspace)

    def panel_quant():   # the panel pair's two kernels, each alone
        qg.quantize_per_token_i8_panel(x_in, panel=workspace, xq_out=(xq, xs))

    def panel_gemm(i):
        w = copies[i % R]
        if wl.path == "w4a8_outl":
            qg.gemm_w4a8_g128_outliers_panel(workspace, xs, *w, wl.M, out_dtype=y.dtype, out=y)
        else:
            qg.gemm_w4a8_g128_panel(workspace, xs, w[0], w[1], w[2], wl.M, out_dtype=y.dtype, out=y)

    def step(i):
        if wl.path in ("w8a8", "w4a8"):
            layer(i)
            return
        if wl.path == "w4a8_outl" and fused:
            panel_quant()
            panel_gemm(i)
            return
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
    # the dominant kernel alone: the one-kernel W8A8 form is the whole step
    if fused and wl.path in ("w4a8", "w4a8_outl"):
        panel_quant()   # the panel the timed GEMMs read
        g_gemm = capture(panel_gemm, steps)
        g_quant = capture(lambda i: panel_quant(), steps)
    else:
        g_gemm = capture(layer if fused else gemm, steps)
        g_quant = capture(lambda i: quant(), steps) if wl.path != "w4a16" and not fused else None

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

    # one untimed replay of the step graph itself first: a graph's first
    # launch also uploads it to the device, which is not a step's cost
    g_step.replay()
    torch.cuda.synchronize()
    wall, gpu = timed(g_step)
    # per-kernel averages: the median of KERNEL_REPLAYS replays of K launches
    gemm_s = median_replay(lambda: timed(g_gemm)[1])
    quant_s = median_replay(lambda: timed(g_quant)[1]) if g_quant is not None else 0.0
    if not torch.equal(y.view(torch.int16) if y.dtype != torch.float32 else y,
                       y_ref.view(torch.int16) if y.dtype != torch.float32 else y_ref):
        raise RuntimeError(f"{wl.name}: timed replay differs from the eager result")

    gemm_b, quant_b, ops = algorithmic(wl)
    kern_b, _, path_key = dominant(wl)
    gemm_us = gemm_s / steps * 1e6
    quant_us = quant_s / steps * 1e6
    step_s = wall / steps
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
        achieved = kern_b / (gemm_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic}
        value, unit = ((gemm_b + quant_b) / step_s / 1e12), "TB/s"
    res = {
        "workload": wl.name, "path": wl.path, "M": wl.M, "K": wl.K, "N": wl.N,
        "x_dtype": wl.x_dtype, "out_dtype": wl.out_dtype, "fused": fused,
        "value": round(value, 4), "unit": unit,
        "ms_per_step": round(step_s * 1e3, 5),
        "gpu_us_per_step": round(gpu / steps * 1e6, 3),
        "gemm_us": round(gemm_us, 3), "quant_us": round(quant_us, 3),
        "gemm_bytes": gemm_b, "quant_bytes": quant_b, "ops": ops,
        "gemm_tops": round(ops / (gemm_us * 1e-6) / 1e12, 2),
        "weight_copies": R, "roofline": roof,
    }
    if wl.path == "w8a8" and wl.M > 64:
        res["vendor_int8"] = vendor_int8(torch, qg, copies, xq, steps, capture, timed)
    print(f"[bench] {wl.name}: gemm {gemm_us:.2f} us ({roof['achieved']} {roof['unit']}, "
          f"{100 * roof['frac']:.1f}% of peak), quant {quant_us:.2f} us, "
          f"step {step_s * 1e6:.2f} us", file=sys.stderr, flush=True)
    del copies, g_warm, g_step, g_gemm, g_quant
    torch.cuda.empty_cache()
    return res


def vendor_int8(torch, qg, copies, xq, steps, capture, timed):
    """Context for the prefill GEMM: the same int8 x int8 -> int32 product by
    the vendor BLAS (torch._int_mm), next to this library's kernel with int32
    output, on the same operands and weight rotation.  Both results are
    compared element by element."""
    M, N = xq.shape[0], copies[0][0].shape[0]
    acc = torch.empty((M, N), dtype=torch.int32, device=xq.device)

    def ours(i):
        qg.gemm_w8a8(xq, None, copies[i % len(copies)][0], None, out_dtype=torch.int32, out=acc)

    def vendor(i):
        torch._int_mm(xq, copies[i % len(copies)][0].t())

    ours(0)
    ref = torch._int_mm(xq, copies[0][0].t())   # eager first: the BLAS sets itself up
    torch.cuda.synchronize()
    equal = bool(torch.equal(acc, ref))
    del ref
    g_ours, g_vendor = capture(ours, steps), capture(vendor, steps)
    ours_us = median_replay(lambda: timed(g_ours)[1]) / steps * 1e6
    vendor_us = median_replay(lambda: timed(g_vendor)[1]) / steps * 1e6
    del g_ours, g_vendor, acc
    return {"kernel": "torch._int_mm (vendor BLAS), int32 output", "vendor_us": round(vendor_us, 2),
            "ours_int32_us": round(ours_us, 2), "int32_equal": equal}


def copy_calibration():
    """A plain elementwise kernel that reads and writes COPY_BYTES each: the
    known-size reference that HBM byte counters are scaled by."""
    import torch
    a = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        torch.add(a, 1, out=b)
    torch.cuda.synchronize()
    print(f"[bench] copy calibration: 3 passes over {COPY_BYTES} bytes", file=sys.stderr, flush=True)


def cpu_model():
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
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report the visible cores
        return os.cpu_count()


def cpu_baseline_workload(wl, seconds):
    """The oracle, as it stands, on the host cores for one workload's step:
    per-token quantization (O1) and the layer's GEMM with its epilogue
    (O4 W8A8, O5 W4A8, O6 W4A16 -- which has no activation quantization),
    repeated for about `seconds` (at least once).  Offline work (fold, weight
    quantization) is done beforehand, as in the GPU leg.  Reported in the
    workload's own unit: TB/s of algorithmic bytes, or TOP/s for the
    compute-bound prefill."""
    import numpy as np
    import oracle
    from workloads import draw
    d = draw(wl)
    x, w = d["x"], d["w"]
    if wl.fold == "smoothquant":
        s = oracle.smoothquant_scales(d["x_cal"], w)
        x_t = oracle.to_f32(oracle.fold_activation(x, s, wl.x_dtype), wl.x_dtype)
        w = oracle.fold_weight(w, s)
    elif wl.fold == "awq":
        s = oracle.awq_scales(d["x_cal"])
        x_t = oracle.to_f32(oracle.fold_activation(x, s, wl.x_dtype), wl.x_dtype)
        w = oracle.fold_weight(w, s)
    else:
        from workloads import f32_to_bf16_bits, f32_to_f16
        raw = {"bf16": lambda a: f32_to_bf16_bits(a), "f16": f32_to_f16,
               "f32": lambda a: a}[wl.x_dtype](x)
        x_t = oracle.to_f32(raw, wl.x_dtype)
    if wl.path == "w8a8":
        wq, ws = oracle.quantize_weight_i8_per_channel(w)

        def step():
            xq, xs = oracle.quantize_per_token_i8(x_t)
            oracle.gemm_w8a8(xq, xs, wq, ws)
    elif wl.path == "w4a8":
        p, sc, zz = oracle.quantize_weight_u4_g128(w)

        def step():
            xq, xs = oracle.quantize_per_token_i8(x_t)
            oracle.gemm_w4a8_g128(xq, xs, p, sc, zz)
    else:
        p, sc, zz = oracle.quantize_weight_u4_g128(w)
        x64 = x_t.astype(np.float64)

        def step():
            oracle.gemm_w4a16_g128(x64, p, sc, zz)
    gemm_b, quant_b, ops = algorithmic(wl)
    n = 0
    t0 = time.perf_counter()
    while True:
        step()
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per = el / n
    res = {"value": None, "unit": None, "cores": _blas_threads(), "cpu_model": cpu_model(),
           "kind": "oracle", "ms_per_step": round(per * 1e3, 2),
           "GBps": round((gemm_b + quant_b) / per / 1e9, 3), "GOPS": round(ops / per / 1e9, 3),
           "sample": f"{n} full step(s) of {wl.name} ({'per-token quantization + ' if wl.path != 'w4a16' else ''}"
                     f"{wl.M}x{wl.K}x{wl.N} {wl.path.upper()} GEMM and epilogue) in {el:.1f} s"}
    if wl.path == "w8a8" and wl.M > 64:
        res["value"], res["unit"] = round(ops / per / 1e12, 6), "TOP/s"
    else:
        res["value"], res["unit"] = round((gemm_b + quant_b) / per / 1e12, 6), "TB/s"
    print(f"[bench] cpu baseline {wl.name}: {res['ms_per_step']} ms per step "
          f"({res['GBps']} GB/s, {res['GOPS']} GOPS) on {res['cores']} threads", file=sys.stderr,
          flush=True)
    return res


def cpu_baseline(wl, seconds):
    """The oracle, as it stands, on the host cores: quantize the activations and
    run the W8A8 GEMM + epilogue for the headline workload, repeated for about
    `seconds` (weights quantized once beforehand, like the GPU leg)."""
    import oracle
    from workloads import draw
    threads = _blas_threads()
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
            "cores": threads, "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{n} full steps of {wl.name} (per-token quantization of {wl.M}x{wl.K} "
                      f"+ {wl.M}x{wl.K}x{wl.N} W8A8 GEMM and epilogue) in {el:.1f} s",
            "ms_per_step": round(el / n * 1e3, 2)}


# ------------------------------------------------------------ measured peaks

PEAK_READ_BYTES = (("w4a8_ffn_down GEMM bytes", 24260672), ("w4a16_qkv GEMM bytes", 26771456),
                   ("w8a8_decode_ffn_up GEMM bytes", 45341728))
PEAK_MFMA = ((0, "i8 v_mfma_i32_32x32x32_i8", INT8_PEAK_TOPS),
             (1, "i8 v_mfma_i32_16x16x64_i8", INT8_PEAK_TOPS),
             (2, "f16 v_mfma_f32_32x32x16_f16", F16_PEAK_TFLOPS),
             (3, "bf16 v_mfma_f32_32x32x16_bf16", F16_PEAK_TFLOPS))


def measured_peaks(steps):
    """The ceilings measured on this GPU in this run, next to the published
    ones: a plain streaming read of each decode GEMM's algorithmic byte count
    (rotating over more than 600 MB so every read comes from HBM), each
    matrix-core instruction on random register operands (with the clock the
    chip runs under that load, from the per-wave s_memtime / s_memrealtime
    counters), and the fixed cost of an empty launch.  Timed like the
    workloads: captured graphs of `steps` launches, median of 5 replays."""
    import torch
    import bit_quantized_gemm_int8_amd as qg

    def graph_us(fn, n):
        fn(0)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i)
        g.replay()
        torch.cuda.synchronize()

        def once():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / n

        us = median_replay(once)
        del g
        return us

    out = {"method": "captured graphs of K launches timed with HIP events, median of 5 replays; "
                     "reads rotate over > 600 MB of copies; matrix-core operands random full-range"}
    reads = []
    for label, nb in PEAK_READ_BYTES:
        stride = (nb + 4095) // 4096 * 4096
        R = max(2, math.ceil(ROTATE_BYTES / stride))
        buf = torch.randint(0, 255, (R * stride,), dtype=torch.uint8, device="cuda")
        sink = torch.empty((qg.load().qg_peak_stream_read_sink(nb),), dtype=torch.int32, device="cuda")
        views = [buf[i * stride:(i + 1) * stride] for i in range(R)]
        us = graph_us(lambda i: qg.peak_stream_read(views[i % R], nb, sink), steps)
        gbs = nb / (us * 1e-6) / 1e9
        reads.append({"what": label, "bytes": nb, "us": round(us, 3), "GBps": round(gbs, 1),
                      "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)})
        print(f"[bench] peak read {nb} B: {us:.2f} us, {gbs:.0f} GB/s "
              f"({100 * gbs / HBM_PEAK_GBS:.1f}% of {HBM_PEAK_GBS:.0f})", file=sys.stderr, flush=True)
        del buf, views, sink
        torch.cuda.empty_cache()
    out["stream_read"] = reads
    out["empty_launch_us"] = round(graph_us(lambda i: qg.peak_empty(), steps), 3)
    mf = []
    WG, ITERS = 1024, 1500
    clocks = torch.empty((4 * WG, 2), dtype=torch.int64, device="cuda")
    sink = torch.empty((256 * WG,), dtype=torch.int32, device="cuda")
    for kind, label, peak in PEAK_MFMA:
        us = graph_us(lambda i: qg.peak_mfma(kind, ITERS, WG, clocks, sink), 3)
        ops = qg.peak_mfma_ops(kind, ITERS, WG)
        rate = ops / (us * 1e-6) / 1e12
        c = clocks.double()
        ghz = float((c[:, 0] / c[:, 1].clamp(min=1)).mean()) * 0.1   # memtime ticks per 10 ns
        mf.append({"instruction": label, "us": round(us, 1), "rate_T": round(rate, 1),
                   "peak_T": peak, "frac_of_peak": round(rate / peak, 4),
                   "memtime_per_realtime_GHz": round(ghz, 3)})
        print(f"[bench] peak {label}: {rate:.0f} T/s ({100 * rate / peak:.1f}% of {peak:.0f}), "
              f"s_memtime rate {ghz:.2f} GHz", file=sys.stderr, flush=True)
    out["mfma"] = mf
    del clocks, sink
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------ batch sweep

SWEEP_LAYERS = (("w8a8", 4096, 11008, "bf16"), ("w8a8", 11008, 4096, "bf16"),
                ("w4a8", 11008, 4096, "bf16"), ("w4a8", 4096, 11008, "bf16"),
                ("w4a16", 4096, 12288, "f16"), ("w4a16", 11008, 4096, "f16"))
SWEEP_M = (1, 2, 4, 8, 16, 32, 64)


def batch_sweep(steps):
    """Decode-to-prefill crossover: each path's linear layer (activation
    quantization + GEMM through the library's one-call entry points; W4A16
    the GEMM alone) at M = 1..64 tokens, next to an
    fp16 dense GEMM of the same K x N layer (torch.matmul, i.e. the vendor
    BLAS) on fp16 weights.  Seeded random inputs; weights rotate over more
    than 600 MB of copies in both cases so they stream from HBM."""
    import torch
    import bit_quantized_gemm_int8_amd as qg

    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}

    def graph_us(fn, n):
        fn(0)   # eager first: the vendor BLAS sets itself up outside capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i)
        g.replay()
        torch.cuda.synchronize()

        def once():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / n

        return median_replay(once)

    for path, K, N, xd in SWEEP_LAYERS:
        w = torch.randn((K, N), generator=gen, device=dev) * 0.02
        if path == "w8a8":
            weights = qg.quantize_weight_i8_per_channel(w)
        else:
            weights = qg.quantize_weight_u4_g128(w)
        wbytes = sum(t.numel() * t.element_size() for t in weights)
        R = max(2, math.ceil(ROTATE_BYTES / wbytes))
        copies = [weights] + [tuple(t.clone() for t in weights) for _ in range(R - 1)]
        w16 = w.to(torch.float16)
        R16 = max(2, math.ceil(ROTATE_BYTES / (2 * K * N)))
        copies16 = [w16] + [w16.clone() for _ in range(R16 - 1)]
        del w
        for M in SWEEP_M:
            x = torch.randn((M, K), generator=gen, device=dev).to(tdt[xd])
            xq = torch.empty((M, K), dtype=torch.int8, device=dev)
            xs = torch.empty((M,), dtype=torch.float32, device=dev)
            wsp = torch.empty(max(qg.quantize_gemm_w4a8_g128_workspace_bytes(M, N, K), 1),
                              dtype=torch.uint8, device=dev)
            y = torch.empty((M, N), dtype=tdt[xd], device=dev)
            y16 = torch.empty((M, N), dtype=torch.float16, device=dev)
            x16 = x.to(torch.float16)

            def layer(i):
                c = copies[i % R]
                if path == "w4a16":
                    qg.gemm_w4a16_g128(x, c[0], c[1], c[2], out_dtype=y.dtype, out=y)
                    return
                if path == "w8a8":
                    qg.quantize_gemm_w8a8(x, c[0], c[1], out_dtype=y.dtype, out=y, xq_out=(xq, xs))
                    return
                qg.quantize_gemm_w4a8_g128(x, c[0], c[1], c[2], out_dtype=y.dtype, out=y,
                                           xq_out=(xq, xs), workspace=wsp)

            def dense(i):
                torch.matmul(x16, copies16[i % R16], out=y16)

            us = graph_us(layer, steps)
            us16 = graph_us(dense, steps)
            rec = {"path": path, "M": M, "K": K, "N": N, "layer_us": round(us, 3),
                   "fp16_dense_us": round(us16, 3), "speedup_vs_fp16": round(us16 / us, 3),
                   "weight_bytes": wbytes, "weight_TBps": round(wbytes / us / 1e6, 3)}
            print(json.dumps(rec), flush=True)
        del copies, copies16
        torch.cuda.empty_cache()


# ------------------------------------------------------------ counter ingest

# demangled-name patterns of each workload's dominant kernel as bench.py runs it
# (rocprofv3 leaves names with _Float16 mangled, hence the alternatives)
KERNEL_OF = {
    "w8a8_decode_ffn_up": [("k_w8a8_dec<8,", "unsigned short>")],
    "w8a8_tiny": [("k_w8a8_fq<16,", "float>")],
    "w4a8_ffn_down": [("k_w4a8_dec<16, 8, 1, false, unsigned short>",)],
    "w4a8_decode_ffn_up": [("k_w4a8_wide<1, 3, 4, 1, 4, 2, 2, unsigned short>",)],
    "w4a8_outl_ffn_down": [("k_w4a8_dec<16, 8, 1, true, unsigned short>",)],
    "w4a8_sp24_ffn_down": [("k_w4a8_sp24<unsigned short>",)],
    "w4a16_qkv": [("k_w4a16_gemv<4, 2,",), ("k_w4a16_gemvILi4ELi2E",)],
    "w8a8_prefill": [("k_w8a8_tiled<", "unsigned short>")],
    "kv_llama2_7b_4k": [("k_kv_quant_seg<2, 4>",)],
}
# profile file label of each workload's dominant kernel
KERNEL_LABEL = {
    "w8a8_decode_ffn_up": "gemm_w8a8_dec", "w8a8_tiny": "gemm_w8a8_fq",
    "w4a8_ffn_down": "gemm_w4a8_dec", "w4a8_decode_ffn_up": "gemm_w4a8_wide", "w4a16_qkv": "gemm_w4a16_gemv", "w8a8_prefill": "gemm_w8a8_tiled",
    "kv_llama2_7b_4k": "kv_quant_seg", "w4a8_outl_ffn_down": "gemm_w4a8_outl_dec",
    "w4a8_sp24_ffn_down": "gemm_w4a8_sp24",
}
COPY_BYTES = 512 * 2 ** 20
PROFILE_COMMANDS = """\
cd /tmp && export TMPDIR=/tmp
rocprofv3 --kernel-trace --stats -d $OUT/pmc/stats -o run --output-format csv -- python3 $REPO/bench.py --steps 50 --warmup 5 --no-cpu --no-peaks
rocprofv3 --pmc FETCH_SIZE -d $OUT/pmc/fetch -o run --output-format csv -- python3 $REPO/bench.py --steps 10 --warmup 2 --no-cpu --no-peaks --copy-calib
rocprofv3 --pmc WRITE_SIZE -d $OUT/pmc/write -o run --output-format csv -- python3 $REPO/bench.py --steps 10 --warmup 2 --no-cpu --no-peaks --copy-calib
python3 $REPO/bench.py --ingest-counters $OUT/pmc"""


def _csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _match(name, alternatives):
    return any(all(p in name for p in pats) for pats in alternatives)


def _profiled(name):
    """(algorithmic bytes, ops, source key, shape text) of a profiled workload."""
    from workloads import KV_WORKLOADS, by_name
    kv = {w.name: w for w in KV_WORKLOADS}
    if name in kv:
        wl = kv[name]
        return kv_algorithmic(wl)[0], 0, "kv", f"T={wl.T}, H={wl.H}, D={wl.D}, {wl.dtype}"
    wl = by_name(name)
    kern_b, ops, key = dominant(wl)
    return kern_b, ops, key, f"M={wl.M}, K={wl.K}, N={wl.N}"


def ingest_counters(d):
    """rocprofv3 CSVs -> profiles/traffic.json + per-kernel summaries.

    d/stats: --kernel-trace --stats run; d/fetch: --pmc FETCH_SIZE run;
    d/write: --pmc WRITE_SIZE run (both with --copy-calib).  FETCH_SIZE and
    WRITE_SIZE are KiB per dispatch; each is scaled by known copy bytes over
    what the same counter reads for the 512 MiB device copy.
    """
    import glob
    stats = _csv_rows(glob.glob(os.path.join(d, "stats", "*kernel_stats.csv"))[0])
    per = {}
    for ctr, sub in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        rows = _csv_rows(glob.glob(os.path.join(d, sub, "*counter_collection.csv"))[0])
        vals = {}
        for r in rows:
            if r["Counter_Name"] != ctr:
                continue
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        # the calibration copy is the only dispatch of that size in the run
        copy = [v for vs in vals.values() for v in vs if 0.5 < v * 1024 / COPY_BYTES < 2.0]
        factor = (COPY_BYTES / (sum(copy) / len(copy) * 1024)) if copy else None
        per[ctr] = (vals, factor, len(copy))
    out, lines = {}, []
    for wl_name, pats in KERNEL_OF.items():
        gemm_b, ops, key, _ = _profiled(wl_name)
        srow = next((r for r in stats if _match(r["Name"], pats)), None)
        rec = {"kernel": srow["Name"].split("(")[0] if srow else None,
               "calls": int(srow["Calls"]) if srow else 0,
               "avg_ns": float(srow["AverageNs"]) if srow else None,
               "algorithmic_bytes": gemm_b, "ops": ops}
        total = 0.0
        ok = True
        for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
            vals, factor, ncopy = per[ctr]
            v = [x for k, xs in vals.items() if _match(k, pats) for x in xs]
            if not v or factor is None:
                ok = False
                continue
            mean_kib = sum(v) / len(v)
            rec[ctr.lower() + "_kib_mean"] = round(mean_kib, 1)
            rec[ctr.lower() + "_copy_factor"] = round(factor, 4)
            total += mean_kib * 1024 * factor
        rec["bytes_per_launch"] = round(total) if ok else None
        rec["source_sha"] = source_sha(key)
        out[key + ":" + wl_name] = rec
        lines.append(rec)
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    for key, rec in out.items():
        path, wl_name = key.split(":")
        shape = _profiled(wl_name)[3]
        kname = KERNEL_LABEL[wl_name]
        fn = os.path.join(ROOT, "profiles", f"{kname}.{wl_name}.md")
        avg = rec["avg_ns"]
        lines = [f"# {kname} on {wl_name} ({shape})", "",
                 "rocprofv3 summary of the benchmark's dominant kernel for this workload.", "",
                 "Commands (repository root as $REPO, an output directory as $OUT, one MI355X):", "", "```",
                 PROFILE_COMMANDS, "```", "",
                 "| quantity | value |", "|---|---|",
                 f"| kernel | `{rec['kernel']}` |",
                 f"| dispatches traced | {rec['calls']} |",
                 f"| average duration (kernel trace) | {avg / 1e3:.3f} us |" if avg else "| average duration | n/a |",
                 f"| algorithmic bytes per launch | {rec['algorithmic_bytes']} |",
                 f"| algorithmic ops per launch | {rec['ops']} |"]
        if avg:
            lines.append(f"| algorithmic GB/s at that duration | {rec['algorithmic_bytes'] / avg:.1f} |")
            lines.append(f"| algorithmic TOP/s at that duration | {rec['ops'] / avg / 1e3:.1f} |")
        for ctr in ("fetch_size", "write_size"):
            if ctr + "_kib_mean" in rec:
                lines.append(f"| {ctr.upper()} mean (KiB per dispatch) | {rec[ctr + '_kib_mean']} |")
                lines.append(f"| {ctr.upper()} copy-kernel scale factor | {rec[ctr + '_copy_factor']} |")
        lines.append(f"| HBM traffic per launch (scaled FETCH + WRITE) | {rec['bytes_per_launch']} |")
        if rec["bytes_per_launch"]:
            lines.append(f"| traffic / algorithmic bytes | {rec['bytes_per_launch'] / rec['algorithmic_bytes']:.3f} |")
        lines.append(f"| kernel source hash | {rec['source_sha']} |")
        lines += ["", "The scale factor is the 512 MiB known-size elementwise copy's true bytes over",
                  "what the same counter reported for it in the same run."]
        with open(fn, "w") as f:
            f.write("\n".join(lines) + "\n")
    # every library kernel the benchmark ran, from the kernel trace
    rows = [r for r in stats if "qg::" in r["Name"] or "_ZN2qg" in r["Name"]]
    lines = ["# Kernel trace of the benchmark (all workloads)", "",
             "Commands (repository root as $REPO, an output directory as $OUT, one MI355X):",
             "", "```", PROFILE_COMMANDS.splitlines()[0], PROFILE_COMMANDS.splitlines()[1], "```", "",
             "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{r['Name'].split('(')[0]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} "
                     f"| {float(r['MinNs']) / 1e3:.3f} | {float(r['MaxNs']) / 1e3:.3f} |")
    with open(os.path.join(ROOT, "profiles", "kernel_trace.bench_all_workloads.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps(out, indent=1))


STEP_TEXT = {
    "w8a8": lambda h: "quantize_gemm_w8a8: " + ("one fused kernel" if h["fused"] else
                                                  "quantize_per_token_i8 + gemm_w8a8 kernels"),
    "w4a8": lambda h: "quantize_gemm_w4a8_g128: " + (
        "quantize_per_token_i8_panel + gemm_w4a8_g128_panel kernels" if h["fused"] else
        "quantize_per_token_i8 + gemm_w4a8_g128 kernels"),
    "w4a8_outl": lambda h: ("quantize_per_token_i8_panel + gemm_w4a8_g128_outliers_panel"
                            if h["fused"] else "quantize_per_token_i8 + gemm_w4a8_g128_outliers"),
    "w4a8_sp24": lambda h: "quantize_per_token_i8 + gemm_w4a8_g128_sparse24",
    "w4a16": lambda h: "gemm_w4a16_g128",
}


def _config(head):
    if "T" in head:   # a KV-cache workload run on its own
        return {"workload": head["workload"], "T": head["T"], "H": head["H"], "D": head["D"],
                "x_dtype": head["x_dtype"],
                "step": "quantize_kv_i8_segments (captured HIP graph)",
                "parallelism": "single GPU"}
    return {"workload": head["workload"], "M": head["M"], "K": head["K"], "N": head["N"],
            "x_dtype": head["x_dtype"], "out_dtype": head["out_dtype"],
            "step": STEP_TEXT[head["path"]](head) + " (captured HIP graph)",
            "parallelism": "single GPU"}


def main():
    args = parse()
    if args.batch_sweep:
        batch_sweep(args.steps)
        return
    if args.peaks:
        import torch
        print(json.dumps({"measured_peaks": measured_peaks(args.steps),
                          "device": torch.cuda.get_device_name(0)}), flush=True)
        return
    if args.ingest_counters:
        ingest_counters(args.ingest_counters)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the layer shards column-parallel without collectives; see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from workloads import KV_WORKLOADS, VARIANT_WORKLOADS, WORKLOADS, by_name
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import bit_quantized_gemm_int8_amd as qg
    qg.load()
    kv_wls = {w.name: w for w in KV_WORKLOADS if w.name in BENCH_KV}
    names = [w.name for w in WORKLOADS + VARIANT_WORKLOADS] + list(kv_wls) \
        if args.workloads == "all" else args.workloads.split(",")
    names = sorted(names, key=lambda n: n != HEADLINE)
    traffic_db = load_traffic()
    results = [run_kv(kv_wls[n], args.steps, args.warmup, traffic_db) if n in kv_wls
               else run_workload(by_name(n), args.steps, args.warmup, traffic_db) for n in names]
    if args.copy_calib:
        copy_calibration()
    head = next((r for r in results if r["workload"] == HEADLINE), results[0])
    peaks = None if args.no_peaks else measured_peaks(args.steps)
    cpu = None
    if not args.no_cpu and head["workload"] == HEADLINE:
        print("[bench] cpu_baseline: timing the oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(by_name(HEADLINE), args.cpu_seconds)
        core = {w.name for w in WORKLOADS}
        for r in results:
            if r["workload"] in core:
                r["cpu_baseline"] = (cpu if r["workload"] == HEADLINE else
                                     cpu_baseline_workload(by_name(r["workload"]),
                                                           args.cpu_seconds_each))
    line = {
        "metric": METRIC, "value": head["value"], "unit": head["unit"], "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i8",
        "data": "synthetic (seeded; Llama-2-7B-shaped layers, no trained weights)",
        "config": _config(head),
        "roofline": head["roofline"], "cpu_baseline": cpu,
        "measured_peaks": peaks,
        "workloads": results,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
