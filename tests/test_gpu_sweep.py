"""GPU parity on seeded random shapes, every entry point of the linear layer.

The hand-picked cases elsewhere sit on the kernel-selection thresholds; these
draw (M, N, K) at random across the bands the launchers tell apart (up to 8,
9-16, 17-64 and more token rows; short and long K; narrow and wide N, ragged
everywhere), from fixed seeds so that every run checks the same shapes.
Integer results (codes, scales, int32 accumulators) must match the oracle bit
for bit; W4A16 outputs meet the W4A16 bound; the fused quantize + W8A8 call
must match the two-kernel path bit for bit.
"""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_int8_amd as qg
import oracle
from tests.gpu_util import to_dev, to_np, out_f64
from tests.test_gpu_gemm import _w4a16_floor
from tests.test_gpu_quant import _check_per_token
from tests.tolerance import assert_close
from workloads import f32_to_f16

pytestmark = pytest.mark.gpu


def _draw_shapes(seed, n, k_step, k_max, cap, kn_cap=None, n_max=3000, m_max=600,
                 wide_n=True):
    """n shapes (M, N, K): K a multiple of k_step up to k_max (4096 beyond 64
    token rows), M N K <= cap and K N <= kn_cap."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        band = int(rng.integers(0, 4))
        lo, hi = [(1, 8), (9, 16), (17, 64), (65, m_max)][band]
        M = int(rng.integers(lo, hi + 1))
        if wide_n and M <= 16 and rng.random() < 0.4:
            N = int(rng.integers(4000, 14000))           # decode-sized layers
        else:
            N = int(rng.integers(1, n_max + 1))
        kk = k_max if M <= 64 else min(k_max, 4096)
        K = k_step * int(rng.integers(1, kk // k_step + 1))
        if M * N * K <= cap and (kn_cap is None or K * N <= kn_cap):
            out.append((M, N, K))
    return out


def _ids(shapes):
    return [f"{m}x{n}x{k}" for m, n, k in shapes]


def _codes(rng, shape):
    return rng.integers(-127, 128, shape).astype(np.int8)


def _u4(rng, K, N):
    return oracle.quantize_weight_u4_g128((rng.standard_normal((K, N)) * 0.02).astype(np.float32))


W8A8 = _draw_shapes(101, 48, 16, 16384, 1e9)


@pytest.mark.parametrize("M,N,K", W8A8, ids=_ids(W8A8))
def test_w8a8(M, N, K):
    rng = np.random.default_rng(M + 3 * N + 7 * K)
    xq, wq = _codes(rng, (M, K)), _codes(rng, (N, K))
    print(f"sweep w8a8 M={M} N={N} K={K}", flush=True)
    acc = qg.gemm_w8a8(to_dev(xq), None, to_dev(wq), None, out_dtype=torch.int32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(acc), oracle.gemm_w8a8_acc(xq, wq))


W4A8 = _draw_shapes(202, 40, 128, 16384, 4e8, kn_cap=4e7)


@pytest.mark.parametrize("M,N,K", W4A8, ids=_ids(W4A8))
def test_w4a8(M, N, K):
    rng = np.random.default_rng(M + 5 * N + 3 * K)
    packed, sc, zz = _u4(rng, K, N)
    xq = _codes(rng, (M, K))
    print(f"sweep w4a8 M={M} N={N} K={K}", flush=True)
    acc = qg.gemm_w4a8_g128(to_dev(xq), None, to_dev(packed), None, to_dev(zz),
                            out_dtype=torch.int32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(acc), oracle.gemm_w4a8_g128_acc(xq, packed, zz))


W4A16 = _draw_shapes(303, 32, 128, 8192, 2e8, kn_cap=4e7)


@pytest.mark.parametrize("M,N,K", W4A16, ids=_ids(W4A16))
def test_w4a16(M, N, K):
    rng = np.random.default_rng(M + 11 * N + K)
    packed, sc, zz = _u4(rng, K, N)
    xh = f32_to_f16(rng.standard_normal((M, K)).astype(np.float32))
    x64 = xh.astype(np.float64)
    print(f"sweep w4a16 M={M} N={N} K={K}", flush=True)
    y = qg.gemm_w4a16_g128(to_dev(xh), to_dev(packed), to_dev(sc), to_dev(zz),
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    yref = oracle.gemm_w4a16_g128(x64, packed, sc, zz)
    assert_close(out_f64(y), yref, "f32", floor=_w4a16_floor(x64, packed, sc, zz), what="w4a16")


OUTL = _draw_shapes(404, 24, 128, 4096, 1e8, kn_cap=4e6, n_max=1500, wide_n=False)


@pytest.mark.parametrize("M,N,K", OUTL, ids=_ids(OUTL))
def test_w4a8_outliers(M, N, K):
    rng = np.random.default_rng(M + 13 * N + K)
    w = rng.standard_normal((K, N)) * 0.02
    w[rng.random((K, N)) < 0.01] *= 8.0
    p, s, z, r, s8 = oracle.quantize_weight_u4_g128_outliers(w.astype(np.float32))
    xq = _codes(rng, (M, K))
    print(f"sweep w4a8 outliers M={M} N={N} K={K}", flush=True)
    acc = qg.gemm_w4a8_g128_outliers(to_dev(xq), None, to_dev(p), None, to_dev(z),
                                     to_dev(r.view(np.int64)), None, out_dtype=torch.int32)
    torch.cuda.synchronize()
    got, G = to_np(acc), K // 128
    np.testing.assert_array_equal(got[:, :G, :], oracle.gemm_w4a8_g128_acc(xq, p, z))
    np.testing.assert_array_equal(got[:, G, :], oracle.gemm_w4a8_g128_outlier_acc(xq, r))


SP24 = _draw_shapes(505, 24, 128, 4096, 1e8, kn_cap=4e6, n_max=1500, wide_n=False)


@pytest.mark.parametrize("M,N,K", SP24, ids=_ids(SP24))
def test_w4a8_sparse24(M, N, K):
    rng = np.random.default_rng(M + 17 * N + K)
    w = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    p, s, z = oracle.quantize_weight_u4_g128_sparse24(w)
    xq = _codes(rng, (M, K))
    print(f"sweep w4a8 2:4 M={M} N={N} K={K}", flush=True)
    acc = qg.gemm_w4a8_g128_sparse24(to_dev(xq), None, to_dev(p), None, to_dev(z),
                                     out_dtype=torch.int32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(acc), oracle.gemm_w4a8_g128_sparse24_acc(xq, p, z))


def _quant_cases(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(rng.integers(1, 2000))
        K = 16 * int(rng.integers(1, 70000 // 16))
        if M * K <= 4e6:
            out.append((M, K, ["f32", "bf16", "f16"][int(rng.integers(0, 3))]))
    return out


QUANT = _quant_cases(606, 40)


@pytest.mark.parametrize("M,K,fmt", QUANT, ids=[f"{m}x{k}-{f}" for m, k, f in QUANT])
def test_per_token(M, K, fmt):
    rng = np.random.default_rng(M * 7 + K)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.integers(0, K, 2)] *= 30.0
    print(f"sweep per-token M={M} K={K} {fmt}", flush=True)
    _check_per_token(x, fmt)


def _fused_cases(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(rng.integers(1, 17))
        mr = 1 if M <= 1 else 2 if M <= 2 else 4 if M <= 4 else 8 if M <= 8 else 16
        K = 16 * int(rng.integers(1, (4096 * 8 // mr) // 16 + 1))   # codes fit the fused kernel
        N = int(rng.integers(4000, 14000)) if rng.random() < 0.5 else int(rng.integers(1, 3000))
        if M * N * K <= 2e8:
            out.append((M, N, K))
    return out


FUSED = _fused_cases(707, 32)


@pytest.mark.parametrize("M,N,K", FUSED, ids=_ids(FUSED))
def test_fused_matches_two_kernels(M, N, K):
    g = torch.Generator(device="cuda")
    g.manual_seed(M * 3 + N + K)
    xdt = [torch.bfloat16, torch.float16, torch.float32][(M + N + K) % 3]
    x = torch.randn((M, K), generator=g, device="cuda").to(xdt)
    w = torch.randn((K, N), generator=g, device="cuda") * 0.02
    wq, ws = qg.quantize_weight_i8_per_channel(w)
    print(f"sweep fused M={M} N={N} K={K} x={xdt}", flush=True)
    y, xq, xs = qg.quantize_gemm_w8a8(x, wq, ws, out_dtype=torch.bfloat16, fuse=True)
    y2, xq2, xs2 = qg.quantize_gemm_w8a8(x, wq, ws, out_dtype=torch.bfloat16, fuse=False)
    torch.cuda.synchronize()
    assert torch.equal(xs, xs2) and torch.equal(xq, xq2)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
