"""Oracle contractions and epilogues (test infrastructure; see oracle/__init__.py).

Integer accumulators are exact.  The float64 matmul used below is applied to
integer-valued matrices whose every partial sum is an integer of magnitude
below 2**53, so it is exact whatever order the BLAS library sums in; the
pure-integer variants (`exact_int=True`) use int64 NumPy matmul instead and
must agree bit for bit.
"""
from __future__ import annotations

import numpy as np

from .quant import unpack_u4, G128


def _int_matmul(a: np.ndarray, b: np.ndarray, exact_int: bool) -> np.ndarray:
    """a [M, K] @ b [K, N] for small integers, returned as int64."""
    if exact_int:
        return np.asarray(a, np.int64) @ np.asarray(b, np.int64)
    bound = (np.abs(np.asarray(a, np.int64)).max(initial=0)
             * np.abs(np.asarray(b, np.int64)).max(initial=0) * a.shape[1])
    assert bound < 2 ** 53, "float64 path would not be exact"
    return (np.asarray(a, np.float64) @ np.asarray(b, np.float64)).astype(np.int64)


def gemm_w8a8_acc(xq: np.ndarray, wq: np.ndarray, exact_int: bool = False) -> np.ndarray:
    """acc[m, n] = sum_k xq[m, k] * wq[n, k]  (int8 x int8 -> exact integer).

    「第4章：量化」 §2.3 (W8A8: the GEMM runs on INT8 units);
    「LLM推理降本五要素」 §2.1.  xq int8 [M, K]; wq int8 [N, K].
    The result must fit int32 (|acc| <= K * 127**2), which is asserted.
    """
    acc = _int_matmul(xq, np.asarray(wq).T, exact_int)
    assert np.abs(acc).max(initial=0) < 2 ** 31
    return acc


def gemm_w8a8(xq, x_scale, wq, w_scale) -> np.ndarray:
    """y_exact[m, n] = acc[m, n] * s_x[m] * s_w[n]  (float64).

    Dequantization x_hat = x_int * s (「第4章：量化」 §1.1, z = 0) applied to
    both operands of the contraction: X_hat W_hat = diag(s_x) acc diag(s_w).
    """
    acc = gemm_w8a8_acc(xq, wq).astype(np.float64)
    return acc * np.asarray(x_scale, np.float64)[:, None] * np.asarray(w_scale, np.float64)[None, :]


def _codes_minus_zero(packed, zero16) -> np.ndarray:
    """(q - z) per weight as int64 [N, G, 128] (「第4章：量化」 §1.1)."""
    codes = unpack_u4(packed).astype(np.int64)                  # [N, K]
    N, K = codes.shape
    z = np.asarray(zero16, np.float16).astype(np.float64)
    assert np.all(z == np.rint(z)) and z.min(initial=0) >= 0 and z.max(initial=0) <= 15
    return codes.reshape(N, K // G128, G128) - z.astype(np.int64)[:, :, None]


def gemm_w4a8_g128_acc(xq, packed, zero16, exact_int: bool = False) -> np.ndarray:
    """Per-group int accumulators acc[m, g, n] = sum_{k in g} xq[m,k] (q[n,k] - z[n,g]).

    「LLM推理降本五要素」 §2.2 (W4A8, group size 128, per-group scale and
    zero point); 「第4章：量化」 §1.1 (dequantize subtracts z).
    xq int8 [M, K]; packed int32 [N, K/8]; zero16 float16 [N, G].
    Returns int64 [M, G, N] (each |acc| <= 128 * 127 * 15).
    """
    wz = _codes_minus_zero(packed, zero16)                        # [N, G, 128]
    xq = np.asarray(xq)
    M, K = xq.shape
    N, G, _ = wz.shape
    acc = np.empty((M, G, N), np.int64)
    for g in range(G):
        acc[:, g, :] = _int_matmul(xq[:, g * G128:(g + 1) * G128], wz[:, g, :].T, exact_int)
    return acc


def gemm_w4a8_g128(xq, x_scale, packed, scale16, zero16) -> np.ndarray:
    """y_exact[m, n] = s_x[m] * sum_g s[n, g] * acc[m, g, n]  (float64).

    The scale of a group multiplies only that group's partial sum, since
    x_hat w_hat summed over a group is s_x s_g sum (x_int)(q - z)
    (「第4章：量化」 §1.1 applied per group, §1.3 per-group granularity).
    """
    acc = gemm_w4a8_g128_acc(xq, packed, zero16).astype(np.float64)   # [M,G,N]
    s = np.asarray(scale16, np.float16).astype(np.float64).T          # [G, N]
    y = (acc * s[None, :, :]).sum(axis=1)
    return y * np.asarray(x_scale, np.float64)[:, None]


def gemm_w4a16_g128_partials(x_f64, packed, zero16) -> np.ndarray:
    """p[m, g, n] = sum_{k in g} x[m, k] * (q[n, k] - z[n, g])  (float64).

    Weight-only 4-bit: activations stay in 16-bit floats
    (「第4章：量化」 §3.1), codes dequantized inside the contraction
    (§3.5, the fused idea).  With fp16 x every term is a multiple of 2**-24
    and |p| < 2**27, so the float64 sum is exact.
    x_f64: float64 [M, K] holding the exact values of the fp16/bf16 input.
    """
    wz = _codes_minus_zero(packed, zero16).astype(np.float64)     # [N, G, 128]
    x = np.asarray(x_f64, np.float64)
    M, K = x.shape
    N, G, _ = wz.shape
    p = np.empty((M, G, N), np.float64)
    for g in range(G):
        p[:, g, :] = x[:, g * G128:(g + 1) * G128] @ wz[:, g, :].T
    return p


def gemm_w4a16_g128(x_f64, packed, scale16, zero16) -> np.ndarray:
    """y_exact[m, n] = sum_g s[n, g] * p[m, g, n]  (float64)."""
    p = gemm_w4a16_g128_partials(x_f64, packed, zero16)
    s = np.asarray(scale16, np.float16).astype(np.float64).T      # [G, N]
    return (p * s[None, :, :]).sum(axis=1)
