"""Oracle for KV-cache INT8 quantization (test infrastructure; see oracle/__init__.py).

「LLM推理降本五要素」 §5.2: the cached keys/values are quantized in position
segments of 128 tokens, each segment with its own scale per embedding channel
(head dimension), kept in a buffer indexed [layer, kv head, position // 128,
head dim]; a value is quantized as round(k / scale) clamped to int8.
「第4章：量化」 §1.2 gives the symmetric scale s = max|x| / 127, §1.1 the
quantize / dequantize pair x_int = round(x / s), x_hat = x_int * s.

Readings (also listed with the other readings of the pages):
  * The cache tensor of one layer is token-major, [T][H][D] (T positions,
    H kv heads, D head dim) -- the grouped layout [L/G][G][H][D] with G = 128
    of 「现代AI加速技术全景解析」 §5.2 for one sequence.
  * Symmetric per (head, segment, channel): s = fl32(max|x| / 127) over the
    segment's positions (a last, partial segment uses the positions it has);
    codes clamp(rne(fl32(x / s)), -127, 127); a channel of a segment whose
    s is 0 (all zero, or max|x| / 127 below binary32's range) gets zero
    codes.  The pages' code clamps to [-128, 127]; while s is a normal number
    the quotient never leaves [-127, 127] up to one rounding, so either clamp
    gives the same codes; with a subnormal s the quotient can pass 127.5 and
    the [-127, 127] clamp binds (the rule of the symmetric quantizer).
  * Scales are fp32, [H][ceil(T / 128)][D].
  * The per-token variant (one scale per position and head, over the head
    dim) is per-token quantization of the [T*H][D] matrix.
"""
from __future__ import annotations

import numpy as np

from .quant import _symmetric_i8

SEG = 128


def quantize_kv_segments(kv_f32: np.ndarray, seg: int = SEG):
    """kv_f32: float32 [T, H, D].  Returns (codes int8 [T, H, D],
    scales float32 [H, ceil(T / seg), D])."""
    kv = np.asarray(kv_f32, np.float32)
    T, H, D = kv.shape
    S = (T + seg - 1) // seg
    codes = np.zeros((T, H, D), np.int8)
    scales = np.zeros((H, S, D), np.float32)
    for si in range(S):
        t0, t1 = si * seg, min(T, (si + 1) * seg)
        q, s = _symmetric_i8(kv[t0:t1], axis=0)      # one scale per (head, channel)
        codes[t0:t1] = q
        scales[:, si, :] = s
    return codes, scales


def dequantize_kv_segments(codes: np.ndarray, scales: np.ndarray, seg: int = SEG) -> np.ndarray:
    """x_hat = x_int * s (「第4章：量化」 §1.1), exactly, in float64 [T, H, D]."""
    T = codes.shape[0]
    pos_seg = np.arange(T) // seg                                      # [T]
    s = np.transpose(scales, (1, 0, 2))[pos_seg].astype(np.float64)   # [T, H, D]
    return codes.astype(np.float64) * s
