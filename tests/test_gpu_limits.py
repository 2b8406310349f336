"""GPU parity at the largest K the g=128 uint4 GEMMs accept (65535 groups),
where the oracle's general routines would be too slow: every packed word is
0x76543210, so the code of k is k mod 8, and each group's sum has a closed
form, acc[m,g,n] = sum_{k in g} x[m,k] (k mod 8) - z[n,g] sum_{k in g} x[m,k]
(exact in int64 / float64).  W4A8 compares its int32 per-group sums bit for
bit; W4A16 its outputs within the W4A16 bound."""
import numpy as np
import torch

import bit_quantized_gemm_int8_amd as qg
from tests.gpu_util import to_dev, to_np, out_f64
from tests.tolerance import assert_close
from workloads import f32_to_f16

import pytest

pytestmark = pytest.mark.gpu

G_MAX = 65535
K_MAX = 128 * G_MAX


def _codes_k_mod_8(N, K):
    return np.full((N, K // 8), 0x76543210, dtype=np.uint32).view(np.int32)


def _zeros(rng, N, G):
    return rng.integers(0, 16, (N, G)).astype(np.float16)


def test_w4a8_max_groups():
    M, N, K = 2, 16, K_MAX
    rng = np.random.default_rng(1)
    xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    zz = _zeros(rng, N, G_MAX)
    print(f"limits w4a8 M={M} N={N} K={K}", flush=True)
    acc = qg.gemm_w4a8_g128(to_dev(xq), None, to_dev(_codes_k_mod_8(N, K)), None, to_dev(zz),
                            out_dtype=torch.int32)
    torch.cuda.synchronize()
    xg = xq.astype(np.int64).reshape(M, G_MAX, 128)
    s1 = (xg * (np.arange(128) % 8)).sum(-1)                      # [M, G]
    s0 = xg.sum(-1)
    ref = s1[:, :, None] - zz.astype(np.int64).T[None] * s0[:, :, None]   # [M, G, N]
    np.testing.assert_array_equal(to_np(acc), ref)


def test_w4a16_max_groups():
    M, N, K = 1, 16, K_MAX
    rng = np.random.default_rng(2)
    xh = f32_to_f16(rng.standard_normal((M, K)).astype(np.float32))
    zz = _zeros(rng, N, G_MAX)
    sc = (rng.random((N, G_MAX)) * 0.01 + 1e-3).astype(np.float16)
    print(f"limits w4a16 M={M} N={N} K={K}", flush=True)
    y = qg.gemm_w4a16_g128(to_dev(xh), to_dev(_codes_k_mod_8(N, K)), to_dev(sc), to_dev(zz),
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    xg = xh.astype(np.float64).reshape(M, G_MAX, 128)
    c = np.arange(128) % 8
    p1 = (xg * c).sum(-1)                                         # exact: fp16 x small integers
    p0 = xg.sum(-1)
    z64, s64 = zz.astype(np.float64).T[None], sc.astype(np.float64).T[None]   # [1, G, N]
    p = p1[:, :, None] - z64 * p0[:, :, None]                     # [M, G, N]
    yref = (p * s64).sum(1)
    # the bound's B = sum_g s sum_k |x| |code - z|: per group, |x| summed by code
    ax = np.abs(xg).reshape(M, G_MAX, 16, 8).sum(2)               # [M, G, code]
    dist = np.abs(np.arange(8)[None, None, :, None] - z64[:, :, None, :])   # [1, G, code, N]
    B = (np.einsum("mgc,xgcn->mgn", ax, dist) * s64).sum(1)
    assert_close(out_f64(y), yref, "f32", floor=(128 + G_MAX + 10) * 2.0 ** -24 * B,
                 what="w4a16 at 65535 groups")
