"""Oracle quantizers (test infrastructure; see oracle/__init__.py).

Notation: fl32(e) is e evaluated in IEEE binary32 with correct rounding
(NumPy float32 arithmetic); rne(v) rounds half to even (np.rint).
"""
from __future__ import annotations

import numpy as np

G128 = 128


def to_f32(x, dtype: str) -> np.ndarray:
    """Upcast a layer input to float32 exactly.

    dtype "f32": float32 array; "f16": float16 array; "bf16": uint16 bit
    patterns of bfloat16 (the upper half of a float32).
    """
    if dtype == "f32":
        return np.asarray(x, np.float32)
    if dtype == "f16":
        return np.asarray(x, np.float16).astype(np.float32)
    if dtype == "bf16":
        return (np.asarray(x, np.uint16).astype(np.uint32) << 16).view(np.float32)
    raise ValueError(dtype)


def _symmetric_i8(x: np.ndarray, axis: int):
    """Symmetric int8 codes of x with one scale per slice along `axis`.

    「第4章：量化」 §1.2: s = max|x| / 127, z = 0; §1.1: x_int = round(x/s);
    「LLM推理降本五要素」 §5.2: round, then clamp to the int8 range.
    Readings: the scale and the quotient are fl32; round is half-to-even;
    codes are clamped to [-127, 127].  With a normal s the clamp never binds
    (|x|/s <= 127 up to one rounding); a subnormal s has fewer significant
    bits, so max|x|/s can exceed 127.5 and the clamp binds (max|x| =
    316 * 2^-149 gives s = 2 * 2^-149 and 158 -> 127).  A slice whose fl32
    scale is 0 -- all zero, or max|x| so small that max|x|/127 rounds to 0 --
    gets s = 0 and all-zero codes (no division; x_hat = q s = 0 either way).
    """
    x = np.asarray(x, np.float32)
    amax = np.max(np.abs(x), axis=axis, keepdims=True)            # exact
    s = (amax / np.float32(127.0)).astype(np.float32)               # fl32
    ok = s > 0
    nz = np.broadcast_to(ok, x.shape)
    safe = np.where(ok, s, np.float32(1.0)).astype(np.float32)
    quot = (x / safe).astype(np.float32)                            # fl32(x/s)
    q = np.clip(np.rint(quot), -127, 127)
    q = np.where(nz, q, 0).astype(np.int8)
    return q, np.squeeze(s, axis=axis)


def quantize_per_token_i8(x_f32: np.ndarray):
    """Per-token dynamic symmetric int8 activation quantization.

    「第4章：量化」 §1.3 (per-token, dynamic: one scale per token),
    §1.2 (symmetric scale), §1.1 (x_int = round(x/s));
    「LLM推理降本五要素」 §5.2 (round then clamp to int8).
    x_f32: float32 [M, K].  Returns (codes int8 [M, K], scale float32 [M]).
    """
    return _symmetric_i8(x_f32, axis=1)


def quantize_weight_i8_per_channel(w_f32: np.ndarray):
    """Per-output-channel symmetric int8 weight quantization.

    「第4章：量化」 §1.3 (per-channel: one scale per output channel), §1.2.
    w_f32: float32 [K, N] (Y = X @ W).  Returns (codes int8 [N, K] stored
    K-contiguous per output channel, scale float32 [N]).
    """
    q, s = _symmetric_i8(w_f32, axis=0)          # q [K, N], s [N]
    return np.ascontiguousarray(q.T), s


def f16_round_up(t: np.ndarray) -> np.ndarray:
    """Smallest float16 that is >= t (t: float32, finite, >= 0).

    Reading: the u4 group scale is stored in fp16 ("fp16 scale+zero per
    group"); rounding it upward (never below (max - min)/15) keeps every code
    of the group inside [0, 15], so the round-trip error stays within s/2;
    round-to-nearest would let 0.1% of N(0, 0.02) groups need a code of 16.
    """
    t = np.asarray(t, np.float32)
    h = t.astype(np.float16)                                         # RNE
    below = h.astype(np.float32) < t
    with np.errstate(over="ignore"):        # nextafter(65504) is only taken if below
        up = np.nextafter(h, np.float16(np.inf))
    return np.where(below, up, h).astype(np.float16)


def quantize_weight_u4_g128(w_f32: np.ndarray):
    """Group-wise (g=128 along K) asymmetric uint4 weight quantization.

    「第4章：量化」 §1.1 (x_int = round(x/s) + z, round first then add z),
    §1.2 (asymmetric: s from max - min, z adjusts the offset; for 4 bits the
    range is 2**4 - 1 = 15), §1.3 (per-group), §3.2/§3.3 (bits=4,
    group_size=128, contiguous groups, zero point on);
    「LLM推理降本五要素」 §2.2 (each group has its own scale and zero point).

    Per output column n and group g (k in [128g, 128g+128)):
      lo, hi = min, max of the 128 weights
      t  = fl32(fl32(hi - lo) / 15);  s16 = smallest fp16 >= t;  s = float(s16)
      z  = clamp(rne(fl32(-lo / s)), 0, 15)
      q  = clamp(rne(fl32(w / s)) + z, 0, 15)
    A constant group (t == 0) gets s16 = 0, z = 0, q = 0.
    w_f32: float32 [K, N], K % 128 == 0.
    Returns (packed int32 [N, K/8], scale float16 [N, K/128],
             zero float16 [N, K/128]).
    """
    w = np.asarray(w_f32, np.float32)
    K, N = w.shape
    if K % G128:
        raise ValueError("K must be a multiple of 128")
    G = K // G128
    wg = w.reshape(G, G128, N)                                     # [G,128,N]
    lo = wg.min(axis=1)
    hi = wg.max(axis=1)                                            # [G, N]
    t = ((hi - lo).astype(np.float32) / np.float32(15.0)).astype(np.float32)
    if not np.all(np.isfinite(t)) or np.any(t > np.float32(65504.0)):
        raise ValueError("group range does not fit an fp16 scale")
    s16 = f16_round_up(t)                                          # [G, N]
    s = s16.astype(np.float32)
    ok = s > 0
    safe = np.where(ok, s, np.float32(1.0)).astype(np.float32)
    z = np.clip(np.rint((-lo / safe).astype(np.float32)), 0, 15)
    z = np.where(ok, z, 0.0)
    q = np.rint((wg / safe[:, None, :]).astype(np.float32)) + z[:, None, :]
    q = np.clip(q, 0, 15)
    q = np.where(ok[:, None, :], q, 0).astype(np.uint8)           # [G,128,N]
    codes = np.ascontiguousarray(q.reshape(K, N).T)                # [N, K]
    return (pack_u4(codes), np.ascontiguousarray(s16.T),
            np.ascontiguousarray(z.astype(np.float16).T))


def pack_u4(codes: np.ndarray) -> np.ndarray:
    """Pack 4-bit codes [N, K] (values 0..15) into int32 [N, K/8].

    Format reading ("8 codes packed per int32"): word i of a row holds the
    codes of k = 8i .. 8i+7, the code of k = 8i + j in bits 4j .. 4j+3.
    """
    c = np.asarray(codes, np.uint8).astype(np.uint32)
    N, K = c.shape
    if K % 8:
        raise ValueError("K must be a multiple of 8")
    c = c.reshape(N, K // 8, 8)
    word = np.zeros((N, K // 8), np.uint32)
    for j in range(8):
        word |= c[:, :, j] << np.uint32(4 * j)
    return word.view(np.int32)


def unpack_u4(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_u4: int32 [N, K/8] -> uint8 codes [N, K]."""
    w = np.asarray(packed, np.int32).view(np.uint32)
    N, W = w.shape
    out = np.empty((N, W, 8), np.uint8)
    for j in range(8):
        out[:, :, j] = (w >> np.uint32(4 * j)) & np.uint32(0xF)
    return out.reshape(N, W * 8)


def dequant_u4_g128(packed, scale16, zero16) -> np.ndarray:
    """x_hat = (x_int - z) * s  (「第4章：量化」 §1.1), float64 [K, N]."""
    codes = unpack_u4(packed).astype(np.float64)                  # [N, K]
    N, K = codes.shape
    s = np.repeat(np.asarray(scale16, np.float16).astype(np.float64), G128, axis=1)
    z = np.repeat(np.asarray(zero16, np.float16).astype(np.float64), G128, axis=1)
    return ((codes - z) * s).T
