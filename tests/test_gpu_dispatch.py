"""GPU parity on both sides of every kernel-selection threshold of the GEMM
entry points.  The launchers pick among several kernels and launch shapes by
M, N, K and the LDS their token rows need; each case below names the choice it
lands on, and its neighbour lands on the other one.  W8A8 and W4A8 compare
their int32 accumulators with the oracle bit for bit, W4A16 its outputs within
the W4A16 bound, the fused call its codes, scales and outputs with the
two-step path bit for bit."""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_int8_amd as qg
import oracle
from tests.gpu_util import to_dev, to_np, out_f64
from tests.tolerance import assert_close
from workloads import f32_to_f16

pytestmark = pytest.mark.gpu


def _codes(rng, shape):
    return rng.integers(-127, 128, shape).astype(np.int8)


W8A8_CASES = [
    # (M, N, K): kernel chosen
    (8, 16, 4096),       # decode, 8 waves (N/16 <= 384, K >= 4096)
    (9, 4096, 4096),     # decode with 16 token rows (N/16 = 256, K >= 2048)
    (16, 4096, 2048),    # same, 4 waves (K < 4096)
    (16, 4096, 2032),    # wide (K < 2048)
    (16, 4112, 4096),    # wide (N/16 = 257)
    (17, 64, 4096),      # wide (M > 16), one block per workgroup: K split over 4 waves
    (64, 64, 1024),      # wide, 4 tiles of 16 rows, K split over 4 waves
    (17, 8192, 1024),    # wide, 2 blocks per workgroup, one wave per block (2 m-tiles)
    (33, 8192, 1024),    # wide, 2 blocks per workgroup, K split over 4 waves (3 m-tiles)
    (33, 16400, 1024),   # wide, 4 blocks per workgroup, one wave per block
    (65, 64, 1024),      # LDS-tiled prefill kernel
    (8, 6144, 4096),     # decode, 8 waves (N/16 = 384)
    (8, 6160, 4096),     # decode, 4 waves (N/16 = 385)
    (8, 6144, 4080),     # decode, 4 waves (K < 4096)
    (8, 12288, 4096),    # decode, 768 one-block workgroups, all resident
    (8, 12304, 4096),    # multi-block workgroups (769 blocks > 3 x 256)
    (8, 16384, 4096),    # multi-block, 4 blocks per workgroup
    (8, 16400, 4096),    # one-block workgroups again (over 1024 blocks)
    (8, 6160, 10112),    # token rows at 80 KB of LDS: 4 waves
    (8, 6160, 10240),    # token rows past 80 KB: one workgroup per CU, 8 waves
    (8, 64, 14208),      # one phase at the 112 KB limit
    (8, 64, 14224),      # two phases
    (16, 64, 7040),      # 16 rows, one phase
    (16, 64, 7168),      # 16 rows, two phases
]


@pytest.mark.parametrize("M,N,K", W8A8_CASES)
def test_w8a8_boundaries(M, N, K):
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    xq, wq = _codes(rng, (M, K)), _codes(rng, (N, K))
    print(f"dispatch w8a8 M={M} N={N} K={K}", flush=True)
    acc = qg.gemm_w8a8(to_dev(xq), None, to_dev(wq), None, out_dtype=torch.int32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(acc), oracle.gemm_w8a8_acc(xq, wq))


W4A8_CASES = [
    (16, 64, 1024),      # decode kernel (M <= 16)
    (4, 6128, 1024),     # decode kernel (383 blocks of 16 rows)
    (4, 6144, 1024),     # wide kernel (384 blocks: 2 per workgroup, K split over 4 waves)
    (16, 6144, 1024),    # wide kernel, 16 rows
    (2, 12304, 1024),    # wide kernel, 3 blocks per workgroup, the last workgroup ragged
    (8, 16400, 1024),    # wide kernel, 4 blocks per workgroup (K split over 2 waves)
    (17, 6128, 1024),    # one weight stream, 2 tiles of 16 rows (383 blocks)
    (17, 6144, 1024),    # wide kernel, 2 m-tiles
    (33, 6144, 1024),    # wide kernel, 4 m-tiles (K and m-tiles split over 2 waves each)
    (17, 64, 1024),      # one weight stream, 2 tiles of 16 rows
    (32, 64, 1024),      # 2 tiles, both full
    (33, 64, 1024),      # 4 tiles
    (64, 64, 1024),      # 4 tiles, all full
    (65, 64, 1024),      # direct-load kernel (M > 64)
    (2, 16, 163712),     # decode kernel with 1279 groups (scales at 80 KB of LDS)
    (2, 16, 163840),     # 1280 groups: direct-load kernel
    (20, 16, 163712),    # 2 tiles with 1279 groups
    (1, 64, 4096),       # one token row: int8 dot-product kernel, 2 KB weight rows, 4 per wave
    (1, 50, 3200),       # same, second kilobyte of each row ragged, last wave 2 rows
    (1, 12304, 1024),    # same, 1 KB rows, 8 per wave
    (1, 37, 1152),       # same, 576-byte rows (lanes past the row end idle)
    (1, 16, 128),        # same, one group
    (1, 4100, 11008),    # same, 6 KB rows, one per wave
    (1, 24, 16384),      # same, 8 KB rows (the longest it takes)
    (1, 24, 16512),      # rows past 8 KB: the matrix-core decode kernel
    (2, 50, 4096),       # two token rows: the int8 dot-product kernel (K <= 4096)
    (2, 37, 1152),       # same, ragged rows
    (2, 50, 4224),       # two rows past K = 4096: the matrix-core decode kernel
]


@pytest.mark.parametrize("M,N,K", W4A8_CASES)
def test_w4a8_boundaries(M, N, K):
    rng = np.random.default_rng(M * 11 + N + K)
    w = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    packed, sc, zz = oracle.quantize_weight_u4_g128(w)
    xq = _codes(rng, (M, K))
    print(f"dispatch w4a8 M={M} N={N} K={K}", flush=True)
    acc = qg.gemm_w4a8_g128(to_dev(xq), None, to_dev(packed), None, to_dev(zz), out_dtype=torch.int32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(acc), oracle.gemm_w4a8_g128_acc(xq, packed, zz))


W4A16_CASES = [
    (8, 8192, 4096),     # decode, 512 one-block workgroups (2 per CU)
    (8, 8208, 4096),     # multi-block workgroups (513 blocks)
    (8, 16400, 4096),    # one-block workgroups again (over 1024 blocks)
    (8, 6144, 1024),     # decode, 8 waves (N/16 = 384)
    (8, 6160, 1024),     # decode, 4 waves
    (8, 64, 4864),       # decode with token rows near 80 KB
    (8, 64, 4992),       # rows past 80 KB: decode kernel in 2 phases of K
    (4, 64, 11008),      # 4 rows of K = 11008 (86 KB): 2 phases
    (2, 64, 11008),      # 2 rows (43 KB): one phase
    (9, 64, 1024),       # wide kernel (9..16 rows), one block per workgroup, K split in 4
    (16, 4096, 1536),    # wide kernel, 256 blocks
    (16, 8192, 2048),    # wide kernel, 2 blocks per workgroup, K split in 2
    (12, 12304, 4096),   # wide kernel, 3 blocks per workgroup, the last ragged
    (10, 4096, 11008),   # wide kernel, long K (86 groups)
    (17, 4096, 1024),    # wide kernel, 2 m-tiles, one block per workgroup: 2 x 2 waves
    (48, 12288, 512),    # wide kernel, 3 m-tiles, K split in 2
    (64, 6144, 256),     # wide kernel, 4 m-tiles split over 2 waves
    (65, 40, 256),       # direct-load kernel (M > 64)
    (1, 64, 4096),       # one token row: vector-ALU kernel, 2 KB weight rows, 4 per wave
    (1, 50, 3200),       # same, second kilobyte of each row ragged, last wave 2 rows
    (1, 37, 2048),       # same, 1 KB rows, 8 per wave
    (1, 37, 1152),       # same, 576-byte rows (lanes past the row end idle)
    (1, 16, 128),        # same, one group
    (1, 12300, 4096),    # same, 3075 waves
    (1, 64, 4224),       # rows past 2 KB: the matrix-core decode kernel
]


def _w4a16_floor(x64, packed, sc, zz):
    codes = oracle.unpack_u4(packed).astype(np.float64)
    N, K = codes.shape
    G = K // 128
    wz = np.abs(codes.reshape(N, G, 128) - zz.astype(np.float64)[:, :, None])
    B = np.zeros((x64.shape[0], N))
    for g in range(G):
        B += (np.abs(x64[:, 128 * g:128 * (g + 1)]) @ wz[:, g, :].T) * sc.astype(np.float64)[:, g]
    return (128 + G + 10) * 2.0 ** -24 * B


@pytest.mark.parametrize("M,N,K", W4A16_CASES)
def test_w4a16_boundaries(M, N, K):
    rng = np.random.default_rng(M * 13 + N + K)
    w = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    packed, sc, zz = oracle.quantize_weight_u4_g128(w)
    xh = f32_to_f16(rng.standard_normal((M, K)).astype(np.float32))
    x64 = xh.astype(np.float64)
    print(f"dispatch w4a16 M={M} N={N} K={K}", flush=True)
    y = qg.gemm_w4a16_g128(to_dev(xh), to_dev(packed), to_dev(sc), to_dev(zz), out_dtype=torch.float32)
    torch.cuda.synchronize()
    yref = oracle.gemm_w4a16_g128(x64, packed, sc, zz)
    assert_close(out_f64(y), yref, "f32", floor=_w4a16_floor(x64, packed, sc, zz), what="w4a16")


FUSED_CASES = [
    # (M, N, K, fuse): path taken
    (4, 8192, 4096, None),    # automatic choice: fused (M <= 4, N K = 2^25)
    (4, 8192, 4080, None),    # automatic choice: two kernels (N K < 2^25)
    (5, 8192, 4096, None),    # automatic choice: two kernels (M > 4)
    (1, 64, 32768, True),     # fused: a row of 4096 chunks, one per thread of 16 waves x 4
    (1, 64, 32784, True),     # past that: two kernels even when asked to fuse
    (8, 64, 4096, True),      # fused: 8 rows of 512 chunks
    (8, 64, 4112, True),      # past that: two kernels
    (16, 64, 2048, True),     # fused: 16 rows of 256 chunks, one row per wave
    (16, 64, 2064, True),     # past that: two kernels
    (16, 512, 768, None),     # automatic choice: fused (9..16 rows, K <= 768)
    (16, 512, 784, None),     # automatic choice: two kernels (K > 768)
    (8, 512, 512, None),      # automatic choice: two kernels (8 rows, N K < 2^25)
]


@pytest.mark.parametrize("M,N,K,fuse", FUSED_CASES)
def test_fused_boundaries(M, N, K, fuse):
    g = torch.Generator(device="cuda")
    g.manual_seed(M + N + K)
    x = torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16)
    w = torch.randn((K, N), generator=g, device="cuda") * 0.02
    wq, ws = qg.quantize_weight_i8_per_channel(w)
    print(f"dispatch fused M={M} N={N} K={K} fuse={fuse}", flush=True)
    y, xq, xs = qg.quantize_gemm_w8a8(x, wq, ws, out_dtype=torch.bfloat16, fuse=fuse)
    xq2, xs2 = qg.quantize_per_token_i8(x)
    y2 = qg.gemm_w8a8(xq2, xs2, wq, ws, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(xs, xs2) and torch.equal(xq, xq2)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
