"""Oracle for 2:4 structured-sparse uint4 weights with int8 activations (test
infrastructure; see oracle/__init__.py).

「LLM推理降本五要素」 §3.2: of every 4 weights the 2 largest are kept (2:4
structured sparsity), then the kept weights are quantized to 4 bits with
group size 128 and a zero point (the page's settings: 4-bit, group 128,
zero point, sparsity 0.5), computed with int8 activations (W4A8); the codes
take 1/8 of the fp16 volume.  「现代AI加速技术全景解析」 §3.1 names the 2:4
pattern (2 nonzeros in every 4 elements).

Readings (also listed with the other readings of the pages):
  * "Every 4 weights" are 4 consecutive input channels k = 4t .. 4t+3 of one
    output channel; "the 2 largest" by |w|, equal magnitudes to the lower
    index.  Exactly 2 are kept in every 4.
  * The 4-bit scale and zero point of a group of 128 inputs come from its 64
    kept weights, with the rules of the dense g=128 quantizer (「第4章：量化」
    §1.1-1.2, fp16 scale rounded up); a pruned weight is 0 and has no code.
  * Product: y[m,n] = s_x[m] sum_g s[n,g] sum_{kept k in g} xq[m,k] (q - z).
  * Storage (a format of this library, laid out for the matrix cores' 2:4
    operand): per (output channel n, group g) four 12-byte blocks, one per 32
    inputs (block b: k = 128 g + 32 b + [0, 32)), each three little-endian
    32-bit words: two words of codes, one word of positions.  The 16 kept
    weights of a block, in ascending k, are values j = 0..15; value j sits in
    code word j // 8, at bits 8 i .. 8 i + 3 for i = j % 8 < 4 and at bits
    8 (i - 4) + 4 .. 8 (i - 4) + 7 for i >= 4; its position within its 4
    inputs (0..3) sits at bits 2 j .. 2 j + 1 of the position word.
"""
from __future__ import annotations

import numpy as np

from .quant import G128, f16_round_up

WORDS_PER_GROUP = 12


def prune_2_4(w_f32: np.ndarray) -> np.ndarray:
    """Kept positions: bool [K, N], the 2 largest |w| of every 4 consecutive k of
    each column (ties to the lower index)."""
    w = np.asarray(w_f32, np.float32)
    K, N = w.shape
    if K % 4:
        raise ValueError("K must be a multiple of 4")
    q = np.abs(w).reshape(K // 4, 4, N)
    order = np.argsort(-q, axis=1, kind="stable")[:, :2, :]          # [K/4, 2, N]
    keep = np.zeros(q.shape, bool)
    np.put_along_axis(keep, order, True, axis=1)
    return keep.reshape(K, N)


def quantize_weight_u4_g128_sparse24(w_f32: np.ndarray):
    """w float32 [K, N] -> (packed int32 [N, (K/128) * 12], scale float16 [N, G],
    zero float16 [N, G]); K % 128 == 0."""
    w = np.asarray(w_f32, np.float32)
    K, N = w.shape
    if K % G128:
        raise ValueError("K must be a multiple of 128")
    G = K // G128
    keep = prune_2_4(w)
    wg = w.reshape(G, G128, N)
    kg = keep.reshape(G, G128, N)
    lo = np.where(kg, wg, np.float32(np.inf)).min(axis=1)                 # [G, N]
    hi = np.where(kg, wg, np.float32(-np.inf)).max(axis=1)
    t = ((hi - lo).astype(np.float32) / np.float32(15.0)).astype(np.float32)
    if not np.all(np.isfinite(t)) or np.any(t > np.float32(65504.0)):
        raise ValueError("group range does not fit an fp16 scale")
    s16 = f16_round_up(t)
    s = s16.astype(np.float32)
    ok = s > 0
    safe = np.where(ok, s, np.float32(1.0)).astype(np.float32)
    z = np.clip(np.rint((-lo / safe).astype(np.float32)), 0, 15)
    z = np.where(ok, z, 0.0)
    q = np.rint((wg / safe[:, None, :]).astype(np.float32)) + z[:, None, :]
    q = np.where(ok[:, None, :], np.clip(q, 0, 15), 0).astype(np.int64)    # [G, 128, N]
    pos = np.tile(np.arange(4), G128 // 4)                                  # position within 4

    packed = np.zeros((N, G, WORDS_PER_GROUP), np.uint32)
    for g in range(G):
        for b in range(4):
            ks = np.arange(32 * b, 32 * b + 32)
            for n in range(N):
                kk = ks[kg[g, ks, n]]                                       # 16 kept, ascending
                codes, where = q[g, kk, n], pos[kk]
                w0 = w1 = pw = 0
                for j in range(16):
                    i = j % 8
                    sh = 8 * i if i < 4 else 8 * (i - 4) + 4
                    if j < 8:
                        w0 |= int(codes[j]) << sh
                    else:
                        w1 |= int(codes[j]) << sh
                    pw |= int(where[j]) << (2 * j)
                packed[n, g, 3 * b:3 * b + 3] = (w0, w1, pw)
    return (packed.reshape(N, G * WORDS_PER_GROUP).view(np.int32),
            np.ascontiguousarray(s16.T), np.ascontiguousarray(z.astype(np.float16).T))


def expand_sparse24(packed) -> np.ndarray:
    """Inverse of the storage format: int32 [N, G*12] -> dense codes int64
    [N, K] with -1 at pruned positions."""
    p = np.asarray(packed, np.int32).view(np.uint32)
    N, W = p.shape
    G = W // WORDS_PER_GROUP
    out = np.full((N, G * G128), -1, np.int64)
    p = p.reshape(N, G, 4, 3).astype(np.int64)
    for g in range(G):
        for b in range(4):
            for j in range(16):
                i = j % 8
                sh = 8 * i if i < 4 else 8 * (i - 4) + 4
                code = (p[:, g, b, j // 8] >> sh) & 0xF
                where = (p[:, g, b, 2] >> (2 * j)) & 3
                k = G128 * g + 32 * b + 4 * (j // 2) + where
                out[np.arange(N), k] = code
    return out


def gemm_w4a8_g128_sparse24_acc(xq, packed, zero16) -> np.ndarray:
    """acc[m, g, n] = sum over the kept k of group g of xq[m,k] (q[n,k] - z[n,g]),
    exact int64 [M, G, N]."""
    codes = expand_sparse24(packed)                                        # [N, K]
    N, K = codes.shape
    G = K // G128
    z = np.repeat(np.asarray(zero16, np.float16).astype(np.int64), G128, axis=1)
    wz = np.where(codes >= 0, codes - z, 0)                                 # pruned: no term
    xq = np.asarray(xq).astype(np.int64)
    acc = np.empty((xq.shape[0], G, N), np.int64)
    for g in range(G):
        sl = slice(G128 * g, G128 * (g + 1))
        acc[:, g, :] = xq[:, sl] @ wz[:, sl].T
    return acc


def gemm_w4a8_g128_sparse24(xq, x_scale, packed, scale16, zero16) -> np.ndarray:
    """y_exact = s_x[m] sum_g s[n,g] acc[m,g,n] in float64 (「LLM推理降本五要素」 §3.2)."""
    acc = gemm_w4a8_g128_sparse24_acc(xq, packed, zero16).astype(np.float64)
    s = np.asarray(scale16, np.float16).astype(np.float64).T                # [G, N]
    return np.asarray(x_scale, np.float32).astype(np.float64)[:, None] * \
        np.einsum("mgn,gn->mn", acc, s)
