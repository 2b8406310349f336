"""Seeded synthetic inputs for the quantized linear layer.

This module holds random draws, shapes and plain dtype casts only.  It does
no quantization, no contraction and no smoothing arithmetic, so that the CPU
oracle and the GPU path, which both take their inputs from here, share no step
of the method.  The shapes stand in for the Llama-2-7B layers the pages talk
about (hidden 4096, FFN 11008, fused QKV 12288): 「LLM推理降本五要素」 §2.1
measures a Llama-2-7B FFN layer; 「第4章：量化」 §2.2 and
「Quantization & Flash Attention」 §2.2 give the smoothing folds applied to
workloads 2, 4 and 5.

Value distributions (readings of the pages where they are silent):
  * activations ~ N(0, 1), weights ~ N(0, 0.02) with 0.02 the standard
    deviation;
  * "1% outlier channels x50": round(0.01*K) input channels picked by a seeded
    permutation, multiplied by 50 after sampling (the same channels in the
    calibration batch);
  * calibration batch for the offline folds: 512 tokens from the same
    generator family with its own seed.
Seeds: X = 1000*i, W = 1000*i + 1, outlier choice = 1000*i + 2,
calibration = 1000*i + 3, with i the workload number (1..5).
Draws are made in float64 and rounded to float32 (round to nearest even).
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "by_name", "draw", "f32_to_bf16_bits",
           "f32_to_f16", "bf16_bits_to_f32", "ragged", "KVWorkload", "KV_WORKLOADS",
           "draw_kv", "VARIANT_WORKLOADS"]


@dataclass(frozen=True)
class Workload:
    """One synthetic quantized-linear workload: Y[M,N] = X[M,K] @ W[K,N]."""
    index: int
    name: str
    path: str            # "w8a8" | "w4a8" | "w4a16"
    M: int
    K: int
    N: int
    x_dtype: str         # dtype handed to the layer: "f32" | "bf16" | "f16"
    out_dtype: str       # "f32" | "bf16" | "f16"
    outlier_cols: int    # number of outlier input channels
    outlier_scale: float
    fold: Optional[str]  # None | "smoothquant" | "awq"  (alpha = 0.5)
    calib_tokens: int = 512

    @property
    def groups(self) -> int:
        return self.K // 128


WORKLOADS = (
    Workload(1, "w8a8_tiny", "w8a8", 16, 512, 512, "f32", "f32", 4, 30.0, None),
    Workload(2, "w8a8_decode_ffn_up", "w8a8", 8, 4096, 11008, "bf16", "bf16",
             41, 50.0, "smoothquant"),
    Workload(3, "w4a8_ffn_down", "w4a8", 16, 11008, 4096, "bf16", "bf16", 0, 1.0, None),
    Workload(4, "w4a16_qkv", "w4a16", 1, 4096, 12288, "f16", "f16", 0, 1.0, "awq"),
    Workload(5, "w8a8_prefill", "w8a8", 4096, 4096, 11008, "bf16", "bf16",
             41, 50.0, "smoothquant"),
)


# Variants of a workload on another path, with the same draws (same index and
# seeds): the FFN-down layer with the top 3 weights of each group kept in INT8
# (「LLM推理降本五要素」 §2.2), and pruned 2:4 before 4-bit quantization (§3.2);
# the decode FFN-up layer of workload 2 with W4A8 weights (§2.2).
VARIANT_WORKLOADS = (
    replace(WORKLOADS[2], name="w4a8_outl_ffn_down", path="w4a8_outl"),
    replace(WORKLOADS[2], name="w4a8_sp24_ffn_down", path="w4a8_sp24"),
    replace(WORKLOADS[1], name="w4a8_decode_ffn_up", path="w4a8"),
)


def by_name(name: str) -> Workload:
    for wl in WORKLOADS + VARIANT_WORKLOADS:
        if wl.name == name or str(wl.index) == str(name):
            return wl
    raise KeyError(name)


def ragged(wl: Workload, M: int, K: int, N: int) -> Workload:
    """Same distributions and path, other sizes (for ragged/edge cases)."""
    oc = min(wl.outlier_cols, K) if wl.outlier_cols else 0
    return replace(wl, M=M, K=K, N=N, outlier_cols=oc)


def _normal(seed: int, shape, std: float) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal(shape, dtype=np.float64) * std


def draw(wl: Workload, seed_offset: int = 0, rows: Optional[int] = None) -> dict:
    """Raw draws for workload `wl` (float32, before any fold or cast).

    Returns a dict with
      x      float32 [M, K]   activations (outlier channels already scaled)
      w      float32 [K, N]   weights, logical Y = X @ W
      x_cal  float32 [T, K]   calibration batch (only when wl.fold is set)
      outliers int64 [n]      sorted outlier channel indices
    `rows` overrides M (a smaller slice of the same distribution).
    """
    base = 1000 * wl.index + seed_offset
    M = wl.M if rows is None else rows
    out = {}
    if wl.outlier_cols:
        rng = np.random.Generator(np.random.PCG64(base + 2))
        idx = np.sort(rng.permutation(wl.K)[: wl.outlier_cols])
    else:
        idx = np.zeros(0, np.int64)
    out["outliers"] = idx.astype(np.int64)
    x = _normal(base + 0, (M, wl.K), 1.0)
    x[:, idx] *= wl.outlier_scale
    out["x"] = x.astype(np.float32)
    out["w"] = _normal(base + 1, (wl.K, wl.N), 0.02).astype(np.float32)
    if wl.fold is not None:
        xc = _normal(base + 3, (wl.calib_tokens, wl.K), 1.0)
        xc[:, idx] *= wl.outlier_scale
        out["x_cal"] = xc.astype(np.float32)
    return out


# --- KV cache ------------------------------------------------------------------
# One layer of one sequence's key (or value) cache, [T][H][D] position-major.
# 「LLM推理降本五要素」 §5.2 quantizes a Llama-2-7B cache (32 heads of 128
# dims; 4096 positions is that model's context length).  Value recipe (a
# reading: the pages give none): N(0, 1) per element, times a per-(head,
# channel) magnitude exp(N(0, 0.5^2)), and 2 outlier channels per head
# (seeded choice) times 10 -- keys vary by channel, the reason for per-channel
# scales.  Seeds: values 7000 + i, magnitudes 7000 + i + 100, outliers
# 7000 + i + 200.


@dataclass(frozen=True)
class KVWorkload:
    index: int
    name: str
    T: int
    H: int
    D: int
    dtype: str           # "f32" | "bf16" | "f16"


KV_WORKLOADS = (
    KVWorkload(1, "kv_small", 300, 4, 128, "bf16"),
    KVWorkload(2, "kv_llama2_7b_4k", 4096, 32, 128, "bf16"),
)


def draw_kv(wl: KVWorkload, T: Optional[int] = None, H: Optional[int] = None,
            D: Optional[int] = None) -> np.ndarray:
    """float32 [T, H, D] cache values (before the cast to wl.dtype)."""
    T = wl.T if T is None else T
    H = wl.H if H is None else H
    D = wl.D if D is None else D
    base = 7000 + wl.index
    x = _normal(base, (T, H, D), 1.0)
    mag = np.exp(_normal(base + 100, (H, D), 0.5))
    rng = np.random.Generator(np.random.PCG64(base + 200))
    for h in range(H):
        mag[h, rng.permutation(D)[:2]] *= 10.0
    return (x * mag[None]).astype(np.float32)


# --- plain storage-format casts (inputs are handed over in these formats) ----

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    Input values must be finite.  Used to build bf16 inputs only.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 (exact)."""
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_f16(x: np.ndarray) -> np.ndarray:
    """float32 -> float16 (IEEE round to nearest even)."""
    return np.asarray(x, np.float32).astype(np.float16)
