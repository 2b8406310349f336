"""Oracle offline smoothing folds (test infrastructure; see oracle/__init__.py).

Both folds rescale input channel j:  X W = (X diag(s)^-1)(diag(s) W).
  SmoothQuant, 「第4章：量化」 §2.2: s_j = max|X_j|^a / max|W_j|^(1-a);
  AWQ, 「Quantization & Flash Attention」 §2.2-2.3: s_c = mean|X_c|^a.
Only a = 0.5 (the value both pages use as the common choice) is defined,
so the power is a square root.  Precision readings: channel maxima are exact;
the AWQ mean sums |x| over the calibration tokens in float64, in token order;
square roots and the quotient are float32, correctly rounded.  A channel
whose statistic is 0 keeps s = 1.  max|W_j| runs over row j of W [K, N]
(input channel j, all outputs), matching diag(s) scaling the rows of W.
"""
from __future__ import annotations

import numpy as np


def smoothquant_scales(x_cal: np.ndarray, w: np.ndarray) -> np.ndarray:
    """s_j = sqrt(max_t |x_cal[t, j]|) / sqrt(max_n |w[j, n]|), float32 [K]."""
    a = np.max(np.abs(np.asarray(x_cal, np.float32)), axis=0)
    b = np.max(np.abs(np.asarray(w, np.float32)), axis=1)
    ok = (a > 0) & (b > 0)
    ra = np.sqrt(a).astype(np.float32)
    rb = np.sqrt(np.where(ok, b, np.float32(1.0))).astype(np.float32)
    s = (ra / rb).astype(np.float32)
    return np.where(ok, s, np.float32(1.0)).astype(np.float32)


def awq_scales(x_cal: np.ndarray) -> np.ndarray:
    """s_c = sqrt(mean_t |x_cal[t, c]|), float32 [K].

    The mean: float64 sum in token order t = 0 .. T-1, divided by T in
    float64, rounded to float32; then a float32 square root.
    """
    x = np.asarray(x_cal, np.float32)
    T, K = x.shape
    total = np.zeros(K, np.float64)
    for t in range(T):
        total += np.abs(x[t]).astype(np.float64)
    m = (total / np.float64(T)).astype(np.float32)
    s = np.sqrt(m).astype(np.float32)
    return np.where(m > 0, s, np.float32(1.0)).astype(np.float32)


def fold_weight(w: np.ndarray, s: np.ndarray) -> np.ndarray:
    """W~ = diag(s) W: row j of w [K, N] times s_j, float32."""
    return (np.asarray(s, np.float32)[:, None] * np.asarray(w, np.float32)).astype(np.float32)


def _f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def fold_activation(x: np.ndarray, s: np.ndarray, out_dtype: str) -> np.ndarray:
    """X~ = X diag(s)^-1: column j of x [M, K] divided by s_j (float32),
    then stored in `out_dtype` ("f32", "f16", or "bf16" as uint16 bits),
    rounding to nearest even."""
    y = (np.asarray(x, np.float32) / np.asarray(s, np.float32)[None, :]).astype(np.float32)
    if out_dtype == "f32":
        return y
    if out_dtype == "f16":
        return y.astype(np.float16)
    if out_dtype == "bf16":
        return _f32_to_bf16_bits(y)
    raise ValueError(out_dtype)
