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
    Channels are stored in tiles of 16: [ceil(N/16)][G][16][12] words, the
    channels past N of the last tile zero, so that the 16 channels' words of
    one group are 768 contiguous bytes.
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


def tile16(rows: np.ndarray) -> np.ndarray:
    """[N, G*12] words per channel -> the stored tiles [ceil(N/16), G, 16, 12]."""
    r = np.asarray(rows)
    N, W = r.shape
    G = W // WORDS_PER_GROUP
    T = (N + 15) // 16
    out = np.zeros((T * 16, G, WORDS_PER_GROUP), r.dtype)
    out[:N] = r.reshape(N, G, WORDS_PER_GROUP)
    return np.ascontiguousarray(out.reshape(T, 16, G, WORDS_PER_GROUP).transpose(0, 2, 1, 3))


def untile16(tiles: np.ndarray, N: int) -> np.ndarray:
    """Inverse of tile16: [T, G, 16, 12] -> [N, G*12]."""
    t = np.asarray(tiles)
    T, G = t.shape[0], t.shape[1]
    return np.ascontiguousarray(t.transpose(0, 2, 1, 3).reshape(T * 16, G * WORDS_PER_GROUP)[:N])


def quantize_weight_u4_g128_sparse24(w_f32: np.ndarray):
    """w float32 [K, N] -> (packed int32 [ceil(N/16), K/128, 16, 12] (the stored
    tiles), scale float16 [N, G], zero float16 [N, G]); K % 128 == 0."""
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
    # the two kept places of every 4 inputs, in ascending order: [G, 32, N]
    k4 = kg.reshape(G, G128 // 4, 4, N)
    pa = np.argmax(k4, axis=2)                                              # first kept
    pb = 3 - np.argmax(k4[:, :, ::-1, :], axis=2)                           # last kept
    t4 = np.arange(G128 // 4)[None, :, None]
    qa = np.take_along_axis(q, (4 * t4 + pa)[:, :, None, :].reshape(G, -1, N), axis=1)
    qb = np.take_along_axis(q, (4 * t4 + pb)[:, :, None, :].reshape(G, -1, N), axis=1)
    # kept values in ascending k: value 2t is pa's, 2t + 1 is pb's  -> [G, 64, N]
    vals = np.stack([qa, qb], axis=2).reshape(G, 64, N).astype(np.uint64)
    wher = np.stack([pa, pb], axis=2).reshape(G, 64, N).astype(np.uint64)

    packed = np.zeros((N, G, WORDS_PER_GROUP), np.uint32)
    for b in range(4):
        w0 = np.zeros((G, N), np.uint64)
        w1 = np.zeros((G, N), np.uint64)
        pw = np.zeros((G, N), np.uint64)
        for j in range(16):
            i = j % 8
            sh = np.uint64(8 * i if i < 4 else 8 * (i - 4) + 4)
            v = vals[:, 16 * b + j, :]
            if j < 8:
                w0 |= v << sh
            else:
                w1 |= v << sh
            pw |= wher[:, 16 * b + j, :] << np.uint64(2 * j)
        packed[:, :, 3 * b] = w0.T
        packed[:, :, 3 * b + 1] = w1.T
        packed[:, :, 3 * b + 2] = pw.T
    return (tile16(packed.reshape(N, G * WORDS_PER_GROUP).view(np.int32)),
            np.ascontiguousarray(s16.T), np.ascontiguousarray(z.astype(np.float16).T))


def expand_sparse24(packed, N: int) -> np.ndarray:
    """Inverse of the storage format: the stored tiles -> dense codes int64
    [N, K] with -1 at pruned positions."""
    p = untile16(np.asarray(packed, np.int32), N).view(np.uint32)
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
    codes = expand_sparse24(packed, np.asarray(zero16).shape[0])          # [N, K]
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
