"""Oracle for W4A8 with per-group INT8 outlier retention (test infrastructure;
see oracle/__init__.py).

「LLM推理降本五要素」 §2.2, second measure: in each weight group the weights
of largest magnitude (the top 2%) are found offline, kept at INT8 precision
in a separate store, and computed on a side path next to the 4-bit group
product.

Readings (also listed with the other readings of the pages):
  * "Top 2% of each group" with g = 128 is ceil(0.02 * 128) = 3 weights per
    (output channel, group), chosen by |w|, ties to the lower input index.
    Every group has exactly 3 (the page's rule is per group, not a global
    threshold).  The page's pseudo-code branches on a per-group flag; it is
    read as an illustration of the side path, not as whole groups in INT8.
  * The group's uint4 scale and zero point are formed from the other 125
    weights, with the same rules as the plain g=128 quantizer; an outlier
    position gets the code q = z, so it adds nothing to the 4-bit product.
  * Outliers are stored as symmetric INT8 codes with one binary32 scale per
    output channel, s8 = fl32(max |outlier| / 127) over the channel's
    outliers (「第4章：量化」 §1.2 and §1.3), codes clamped to [-127, 127]; a
    channel whose s8 is 0 (outliers all zero, or too small for max/127 to
    stay above 0 in binary32) gets zero codes.
  * Store: per (output channel, group) one 64-bit record of four 16-bit slots
    (index << 8 | code byte), the three outliers by ascending index in slots
    0-2 and 0xFFFF in slot 3.
  * Product:  y[m,n] = s_x[m] * ( sum_g s[n,g] acc[m,g,n] + s8[n] acc_o[m,n] )
    with acc as in the plain W4A8 product and
    acc_o[m,n] = sum over the channel's outliers of xq[m,k] * code.
"""
from __future__ import annotations

import numpy as np

from .quant import G128, f16_round_up, pack_u4
from .gemm import gemm_w4a8_g128_acc

N_OUT = 3          # outliers per group of 128: ceil(0.02 * 128)
EMPTY_SLOT = 0xFFFF


def select_outliers(w_f32: np.ndarray, n_out: int = N_OUT) -> np.ndarray:
    """Indices (within the group, ascending) of the n_out largest |w| of every
    (group, column): float32 [K, N] -> int64 [G, n_out, N]; ties in |w| go to
    the lower index (stable sort)."""
    w = np.asarray(w_f32, np.float32)
    K, N = w.shape
    wg = w.reshape(K // G128, G128, N)
    order = np.argsort(-np.abs(wg), axis=1, kind="stable")          # [G, 128, N]
    return np.sort(order[:, :n_out, :], axis=1)


def quantize_weight_u4_g128_outliers(w_f32: np.ndarray, n_out: int = N_OUT):
    """w float32 [K, N] -> (packed int32 [N, K/8], scale f16 [N, G],
    zero f16 [N, G], records uint64 [N, G], outlier scale float32 [N]).

    Per (column n, group g): the outliers are select_outliers'; the uint4
    scale and zero point come from the remaining weights exactly as in
    quantize_weight_u4_g128 (「第4章：量化」 §1.1-1.2: t = fl32(fl32(hi - lo)/15),
    s = the smallest fp16 >= t, z = clamp(rne(fl32(-lo/s)), 0, 15),
    q = clamp(rne(fl32(w/s)) + z, 0, 15); a constant remainder gets s = z = 0);
    outlier positions get q = z.
    """
    w = np.asarray(w_f32, np.float32)
    K, N = w.shape
    if K % G128:
        raise ValueError("K must be a multiple of 128")
    G = K // G128
    wg = w.reshape(G, G128, N)
    idx = select_outliers(w, n_out)                                 # [G, n_out, N]
    is_out = np.zeros(wg.shape, bool)
    for i in range(n_out):
        np.put_along_axis(is_out, idx[:, i:i + 1, :], True, axis=1)

    # 4-bit part over the remaining weights
    lo = np.where(is_out, np.float32(np.inf), wg).min(axis=1)        # [G, N]
    hi = np.where(is_out, np.float32(-np.inf), wg).max(axis=1)
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
    q = np.clip(q, 0, 15)
    q = np.where(ok[:, None, :], q, 0)
    q = np.where(is_out, z[:, None, :], q).astype(np.uint8)          # outliers: q = z
    codes = np.ascontiguousarray(q.reshape(K, N).T)

    # INT8 side store, one scale per output channel
    ov = np.take_along_axis(wg, idx, axis=1)                          # [G, n_out, N]
    amax = np.abs(ov).max(axis=(0, 1))                                # [N]
    s8 = (amax / np.float32(127.0)).astype(np.float32)
    s8_safe = np.where(s8 > 0, s8, np.float32(1.0)).astype(np.float32)
    oc = np.clip(np.rint((ov / s8_safe[None, None, :]).astype(np.float32)), -127, 127)
    oc = np.where(s8[None, None, :] > 0, oc, 0).astype(np.int64)

    rec = np.zeros((G, N), np.uint64)
    for i in range(n_out):
        slot = (idx[:, i, :].astype(np.uint64) << np.uint64(8)) | (oc[:, i, :] & 0xFF).astype(np.uint64)
        rec |= slot << np.uint64(16 * i)
    for i in range(n_out, 4):
        rec |= np.uint64(EMPTY_SLOT) << np.uint64(16 * i)
    return (pack_u4(codes), np.ascontiguousarray(s16.T),
            np.ascontiguousarray(z.astype(np.float16).T), np.ascontiguousarray(rec.T), s8)


def decode_records(rec: np.ndarray):
    """uint64 [N, G] -> (index int64 [N, G, 4], code int64 [N, G, 4],
    valid bool [N, G, 4]); a slot is valid when its index is below 128."""
    r = np.asarray(rec, np.uint64)
    slots = np.stack([(r >> np.uint64(16 * i)) & np.uint64(0xFFFF) for i in range(4)], axis=-1)
    slots = slots.astype(np.int64)
    index = slots >> 8
    code = ((slots & 0xFF) ^ 0x80) - 0x80                              # two's complement byte
    return index, code, index < G128


def gemm_w4a8_g128_outlier_acc(xq, rec) -> np.ndarray:
    """acc_o[m, n] = sum over the channel's outlier slots of xq[m, 128 g + index] * code,
    exact int64 [M, N]."""
    xq = np.asarray(xq).astype(np.int64)
    index, code, valid = decode_records(rec)                          # [N, G, 4]
    N, G, _ = index.shape
    acc = np.zeros((xq.shape[0], N), np.int64)
    for g in range(G):
        for i in range(4):
            k = np.where(valid[:, g, i], G128 * g + index[:, g, i], 0)   # [N]
            c = np.where(valid[:, g, i], code[:, g, i], 0)
            acc += xq[:, k] * c[None, :]
    return acc


def gemm_w4a8_g128_outliers(xq, x_scale, packed, scale16, zero16, rec, s8) -> np.ndarray:
    """y_exact[m, n] = s_x[m] (sum_g s[n,g] acc[m,g,n] + s8[n] acc_o[m,n]) in float64
    from the exact integer accumulators (「LLM推理降本五要素」 §2.2)."""
    acc = gemm_w4a8_g128_acc(xq, packed, zero16).astype(np.float64)       # [M, G, N]
    s = np.asarray(scale16, np.float16).astype(np.float64).T               # [G, N]
    dense = np.einsum("mgn,gn->mn", acc, s)
    side = gemm_w4a8_g128_outlier_acc(xq, rec).astype(np.float64) * \
        np.asarray(s8, np.float32).astype(np.float64)[None, :]
    return np.asarray(x_scale, np.float32).astype(np.float64)[:, None] * (dense + side)
