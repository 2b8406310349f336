"""GPU parity of the three GEMMs against the oracle.

Integer accumulators (the QG_I32 outputs) must match bit for bit; scaled
outputs must meet tests/tolerance.py.  Operand codes come from the oracle so
that the GEMMs are checked on their own; the chained runs live in
test_gpu_workloads.py.
"""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_int8_amd as qg
import oracle
from tests.gpu_util import to_dev, to_np, out_f64
from tests.tolerance import assert_close
from workloads import f32_to_bf16_bits, f32_to_f16

pytestmark = pytest.mark.gpu

TORCH_OUT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}

W8A8_SHAPES = [(16, 512, 512), (1, 16, 16), (3, 17, 48), (8, 11008, 4096), (17, 40, 528),
               (33, 100, 1024), (64, 64, 64), (65, 300, 272), (100, 257, 4096),
               (300, 520, 1040), (257, 1000, 1936),
               # decode kernel: odd 16-byte chunk count per row (LDS pitch), several
               # token-row staging rounds, and a K whose rows overflow the LDS budget
               (5, 33, 4112), (12, 100, 9008), (16, 40, 8192),
               # wide decode kernel: three weight blocks per workgroup with the last
               # workgroup partly past N, and the full 64-token FFN-up shape
               (40, 10256, 512), (64, 11008, 4096),
               # each weight block's K split over 4 waves: 2 blocks per workgroup
               # with K not a multiple of 128 (ragged last phase) and an odd chunk
               # count, one block per workgroup (narrow layers) with long K
               (48, 8200, 1040), (64, 6144, 272), (20, 2048, 11008), (57, 3000, 4112),
               # decode kernel with long token rows (above 80 KB of LDS, one
               # workgroup per compute unit), the last size that fits and the first
               # that does not; 8 and 4 waves per workgroup on either side of 384
               # weight blocks
               (8, 40, 11008), (6, 1040, 13824), (8, 24, 14336), (3, 5000, 20000),
               (4, 6144, 1024), (2, 6160, 4096),
               # 9..16 token rows on the decode kernel (N/16 <= 256), at its LDS
               # limit, and just past 256 weight blocks (wide kernel)
               (16, 4096, 4096), (9, 300, 6912), (13, 4112, 1024),
               # decode kernel walking K in phases: 2, 3 (K not a multiple of
               # 128) and 10 token-row slices, and the longest K the API takes
               (16, 200, 11008), (9, 48, 20016), (16, 64, 65536), (1, 32, 133136),
               # more 16-row blocks than one-block workgroups can be resident:
               # 12-wave workgroups over 3 or 4 blocks, the last one ragged
               (5, 13830, 5120), (7, 16384, 4096)]


def _codes(rng, shape):
    return rng.integers(-127, 128, shape).astype(np.int8)


@pytest.mark.parametrize("M,N,K", W8A8_SHAPES)
def test_w8a8_acc_bitwise(M, N, K):
    rng = np.random.default_rng(M * 31 + N * 7 + K)
    xq, wq = _codes(rng, (M, K)), _codes(rng, (N, K))
    acc = qg.gemm_w8a8(to_dev(xq), None, to_dev(wq), None, out_dtype=torch.int32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(acc), oracle.gemm_w8a8_acc(xq, wq))


@pytest.mark.parametrize("M", [8, 300])
def test_w8a8_acc_extremes(M):
    K, N = 4096, 48
    xq = np.full((M, K), 127, np.int8)
    xq[1::2] = -127
    wq = np.full((N, K), -127, np.int8)
    wq[::3] = 127
    acc = to_np(qg.gemm_w8a8(to_dev(xq), None, to_dev(wq), None, out_dtype=torch.int32))
    np.testing.assert_array_equal(acc, oracle.gemm_w8a8_acc(xq, wq))
    assert np.abs(acc).max() == K * 127 * 127


@pytest.mark.parametrize("fmt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("M,N,K", [(16, 512, 512), (8, 11008, 4096), (100, 257, 4096), (3, 17, 48)])
def test_w8a8_scaled(fmt, M, N, K):
    rng = np.random.default_rng(M + N + K)
    xq, wq = _codes(rng, (M, K)), _codes(rng, (N, K))
    sx = (rng.random(M) * 0.05 + 1e-3).astype(np.float32)
    sw = (rng.random(N) * 1e-3 + 1e-5).astype(np.float32)
    y = qg.gemm_w8a8(to_dev(xq), to_dev(sx), to_dev(wq), to_dev(sw), out_dtype=TORCH_OUT[fmt])
    assert_close(out_f64(y), oracle.gemm_w8a8(xq, sx, wq, sw), fmt, what=f"w8a8 {fmt}")


@pytest.mark.parametrize("M,N,K", [(16, 512, 512), (200, 300, 1024)])
def test_w8a8_power_of_two_scales_bitwise(M, N, K):
    rng = np.random.default_rng(5)
    xq, wq = _codes(rng, (M, K)), _codes(rng, (N, K))
    sx = (2.0 ** rng.integers(-10, -2, M)).astype(np.float32)
    sw = (2.0 ** rng.integers(-14, -6, N)).astype(np.float32)
    y = qg.gemm_w8a8(to_dev(xq), to_dev(sx), to_dev(wq), to_dev(sw), out_dtype=torch.float32)
    np.testing.assert_array_equal(out_f64(y), oracle.gemm_w8a8(xq, sx, wq, sw))


def test_w8a8_prefill_full():
    """4096 x 11008 x 4096 in the launch configuration the benchmark times,
    full-range random codes: every int32 accumulator and every bf16 output
    against the oracle (float64 BLAS on integer operands is exact here)."""
    M, N, K = 4096, 11008, 4096
    g = torch.Generator(device="cuda").manual_seed(1234)
    xq = torch.randint(-127, 128, (M, K), dtype=torch.int8, device="cuda", generator=g)
    wq = torch.randint(-127, 128, (N, K), dtype=torch.int8, device="cuda", generator=g)
    sx = torch.rand(M, device="cuda", generator=g) * 0.05 + 1e-3
    sw = torch.rand(N, device="cuda", generator=g) * 1e-3 + 1e-5
    acc = qg.gemm_w8a8(xq, None, wq, None, out_dtype=torch.int32)
    y = qg.gemm_w8a8(xq, sx, wq, sw, out_dtype=torch.bfloat16)
    xq_n, wq_n = to_np(xq), to_np(wq)
    ref = oracle.gemm_w8a8_acc(xq_n, wq_n)
    np.testing.assert_array_equal(to_np(acc), ref)
    yref = oracle.gemm_w8a8(xq_n, to_np(sx), wq_n, to_np(sw))
    assert_close(out_f64(y), yref, "bf16", what="prefill bf16")
    # run-to-run determinism
    y2 = qg.gemm_w8a8(xq, sx, wq, sw, out_dtype=torch.bfloat16)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


# ---------------------------------------------------------------- W4A8 / W4A16

def _u4_weights(rng, K, N):
    w = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    return oracle.quantize_weight_u4_g128(w)


def _w4_devs(packed, sc, zz):
    return to_dev(packed), to_dev(sc), to_dev(zz)


W4_SHAPES = [(16, 4096, 11008), (1, 16, 128), (5, 17, 256), (16, 300, 1024), (17, 64, 384),
             (33, 40, 640), (1, 12288, 4096), (3, 100, 2048), (2, 48, 14336),
             # 17..64 token rows on 2 or 4 tiles of one weight stream: partial
             # last tiles, an odd group count, the full FFN-down shape
             (32, 4096, 11008), (64, 40, 256), (48, 300, 640), (20, 16, 128), (57, 33, 1152),
             # two weight blocks per wave on wide layers (N / 32 >= 256): full,
             # ragged last pair of blocks with an odd group count, 16 rows
             (1, 8192, 1024), (3, 8200, 384), (16, 11008, 4096),
             # 17-64 rows on wide layers (2-4 weight blocks per workgroup, the
             # token rows staged once): 2 and 4 m-tiles, ragged rows and last
             # workgroup, odd group counts, a group count past one phase ring
             (32, 11008, 4096), (48, 11008, 4096), (17, 6160, 1152), (33, 12288, 4224),
             (64, 16400, 256), (40, 7000, 640), (20, 14400, 1024), (24, 12288, 2048)]


@pytest.mark.parametrize("M,N,K", W4_SHAPES)
def test_w4a8_group_acc_bitwise(M, N, K):
    rng = np.random.default_rng(M * 13 + N + K)
    packed, sc, zz = _u4_weights(rng, K, N)
    xq = _codes(rng, (M, K))
    wqd, scd, zzd = _w4_devs(packed, sc, zz)
    acc = qg.gemm_w4a8_g128(to_dev(xq), None, wqd, None, zzd, out_dtype=torch.int32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(acc), oracle.gemm_w4a8_g128_acc(xq, packed, zz))


@pytest.mark.parametrize("M,K", [(24, 36864), (40, 40960), (8, 65536)])
def test_w4a8_long_k_sampled(M, K):
    """A wide layer whose K is too long for the wide kernel's LDS with float
    outputs (scales of 288-512 groups per weight row): that launch takes the
    multi-tile kernel (17-64 rows) or the two-blocks-per-wave decode kernel
    (up to 16) instead, while the int32 per-group outputs, whose kernel keeps
    no partial sums in LDS, still fit the wide kernel.  Seeded random codes,
    zero points and scales; per-group sums exact and scaled outputs checked
    on sampled columns (the first, the last and 46 drawn)."""
    N = 12288
    G = K // 128
    rng = np.random.default_rng(M * 7 + 1)
    packed = rng.integers(0, 2 ** 32, (N, K // 8), dtype=np.uint64).astype(np.uint32).view(np.int32)
    zz = rng.integers(0, 16, (N, G)).astype(np.float16)
    sc = (rng.random((N, G)) * 1e-3 + 1e-4).astype(np.float16)
    xq = _codes(rng, (M, K))
    sx = (rng.random(M) * 0.05 + 1e-3).astype(np.float32)
    cols = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 46, replace=False)]))
    wqd, scd, zzd = _w4_devs(packed, sc, zz)
    xqd = to_dev(xq)
    acc = qg.gemm_w4a8_g128(xqd, None, wqd, None, zzd, out_dtype=torch.int32)
    y = qg.gemm_w4a8_g128(xqd, to_dev(sx), wqd, scd, zzd, out_dtype=torch.float32)
    torch.cuda.synchronize()
    idx = torch.from_numpy(cols).to(acc.device)
    p, s, z = packed[cols], sc[cols], zz[cols]
    np.testing.assert_array_equal(to_np(acc.index_select(2, idx)), oracle.gemm_w4a8_g128_acc(xq, p, z))
    assert_close(out_f64(y.index_select(1, idx)), oracle.gemm_w4a8_g128(xq, sx, p, s, z), "f32",
                 floor=_w4a8_floor(xq, sx, p, s, z), what="w4a8 long K")


def _w4a8_floor(xq, sx, packed, sc, zz):
    acc = oracle.gemm_w4a8_g128_acc(xq, packed, zz).astype(np.float64)       # [M, G, N]
    s = sc.astype(np.float64).T                                              # [G, N]
    B = np.abs(sx.astype(np.float64))[:, None] * np.abs(acc * s[None]).sum(axis=1)
    G = acc.shape[1]
    return (G + 10) * 2.0 ** -24 * B


@pytest.mark.parametrize("fmt", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("M,N,K", [(16, 4096, 11008), (5, 17, 256), (33, 40, 640), (2, 48, 14336),
                                   (64, 300, 1024), (4, 8200, 1024), (16, 11008, 4096),
                                   (32, 11008, 4096), (57, 7000, 1152),
                                   # one and two token rows (int8 dot-product kernel)
                                   (1, 4096, 11008), (1, 777, 4224), (2, 4100, 4096)])
def test_w4a8_scaled(fmt, M, N, K):
    rng = np.random.default_rng(M + 3 * N + K)
    packed, sc, zz = _u4_weights(rng, K, N)
    xq = _codes(rng, (M, K))
    sx = (rng.random(M) * 0.05 + 1e-3).astype(np.float32)
    wqd, scd, zzd = _w4_devs(packed, sc, zz)
    y = qg.gemm_w4a8_g128(to_dev(xq), to_dev(sx), wqd, scd, zzd, out_dtype=TORCH_OUT[fmt])
    yref = oracle.gemm_w4a8_g128(xq, sx, packed, sc, zz)
    n = assert_close(out_f64(y), yref, fmt, floor=_w4a8_floor(xq, sx, packed, sc, zz),
                     what=f"w4a8 {fmt}")
    print(f"w4a8 {fmt} {M}x{N}x{K}: {n} of {yref.size} outputs within the cancellation floor only")


def _w4a16_floor(x64, packed, sc, zz):
    codes = oracle.unpack_u4(packed).astype(np.float64)                    # [N, K]
    N, K = codes.shape
    G = K // 128
    wz = np.abs(codes.reshape(N, G, 128) - zz.astype(np.float64)[:, :, None])
    B = np.zeros((x64.shape[0], N))
    for g in range(G):
        B += (np.abs(x64[:, 128 * g:128 * (g + 1)]) @ wz[:, g, :].T) * sc.astype(np.float64)[:, g]
    return (128 + G + 10) * 2.0 ** -24 * B


@pytest.mark.parametrize("xfmt", ["f16", "bf16"])
@pytest.mark.parametrize("fmt", ["f16", "f32", "bf16"])
@pytest.mark.parametrize("M,N,K", [(1, 12288, 4096), (5, 17, 256), (16, 300, 1024), (33, 40, 640),
                                   (2, 48, 14336), (48, 10256, 512), (64, 512, 4096),
                                   # 12-wave workgroups over 3 and 4 weight blocks
                                   # (more blocks than 2 per CU), the last ragged
                                   (8, 12288, 4096), (6, 11000, 4096), (7, 16384, 4096),
                                   # 1-4 rows: one group, odd group counts, a ragged
                                   # last block past 256 blocks, long K
                                   (1, 17, 128), (3, 40, 640), (4, 4100, 4096),
                                   (1, 4096, 11008), (2, 1000, 4224), (1, 40, 12288),
                                   (4, 64, 1152),
                                   # 9-64 rows on wide layers, 2-4 weight blocks per
                                   # workgroup, each block's K split over 2 waves
                                   # (2-3 m-tiles) or its m-tiles (4): odd group
                                   # counts, ragged rows and last block, one phase
                                   (24, 6160, 1152), (40, 12304, 640), (64, 14400, 512),
                                   (17, 16400, 384), (12, 14336, 1024), (49, 7000, 1152)])
def test_w4a16(xfmt, fmt, M, N, K):
    rng = np.random.default_rng(M * 5 + N + K)
    packed, sc, zz = _u4_weights(rng, K, N)
    x32 = rng.standard_normal((M, K)).astype(np.float32)
    if xfmt == "f16":
        xh = f32_to_f16(x32)
        xd, x64 = to_dev(xh), xh.astype(np.float64)
    else:
        xb = f32_to_bf16_bits(x32)
        xd, x64 = to_dev(xb, "bf16"), oracle.to_f32(xb, "bf16").astype(np.float64)
    wqd, scd, zzd = _w4_devs(packed, sc, zz)
    y = qg.gemm_w4a16_g128(xd, wqd, scd, zzd, out_dtype=TORCH_OUT[fmt])
    yref = oracle.gemm_w4a16_g128(x64, packed, sc, zz)
    n = assert_close(out_f64(y), yref, fmt, floor=_w4a16_floor(x64, packed, sc, zz),
                     what=f"w4a16 x{xfmt} {fmt}")
    print(f"w4a16 x{xfmt}->{fmt} {M}x{N}x{K}: {n} of {yref.size} within the floor only")


@pytest.mark.parametrize("M,N,K", [(4, 48, 512), (1, 48, 512), (1, 40, 4096)])
def test_w4a16_exact_case_bitwise(M, N, K):
    """Power-of-two scales and small-integer activations make every partial sum
    exact in binary32, so the fp32 output must equal y_exact bit for bit (one
    token row runs the vector-ALU kernel, four rows the matrix cores)."""
    rng = np.random.default_rng(9 + M + K)
    codes = rng.integers(0, 16, (N, K)).astype(np.uint8)
    packed = oracle.pack_u4(codes)
    G = K // 128
    zz = rng.integers(0, 16, (N, G)).astype(np.float16)
    sc = (2.0 ** rng.integers(-8, -2, (N, G))).astype(np.float16)
    xh = rng.integers(-8, 9, (M, K)).astype(np.float16)
    y = qg.gemm_w4a16_g128(to_dev(xh), to_dev(packed), to_dev(sc), to_dev(zz),
                           out_dtype=torch.float32)
    np.testing.assert_array_equal(out_f64(y), oracle.gemm_w4a16_g128(xh.astype(np.float64),
                                                                     packed, sc, zz))


@pytest.mark.parametrize("M,K", [(1, 4096), (1, 2048), (4, 1024)])
def test_w4a16_subnormal_activations_bitwise(M, K):
    """fp16 subnormal activations k 2^-24 (|k| <= 8) must enter the products
    unflushed.  With scales 2^-4 or 2^-3 every partial sum is an integer
    multiple of 2^-28 below 2^24 units, so the fp32 output is exact and must
    equal y_exact bit for bit; a flushed subnormal would change it."""
    rng = np.random.default_rng(17 + M + K)
    N = 72
    G = K // 128
    codes = rng.integers(0, 16, (N, K)).astype(np.uint8)
    packed = oracle.pack_u4(codes)
    zz = rng.integers(0, 16, (N, G)).astype(np.float16)
    sc = (2.0 ** rng.integers(-4, -2, (N, G))).astype(np.float16)
    xh = (rng.integers(-8, 9, (M, K)) * 2.0 ** -24).astype(np.float16)
    assert np.count_nonzero(np.abs(xh) < 2.0 ** -14) > K // 2   # mostly subnormal
    y = qg.gemm_w4a16_g128(to_dev(xh), to_dev(packed), to_dev(sc), to_dev(zz),
                           out_dtype=torch.float32)
    np.testing.assert_array_equal(out_f64(y), oracle.gemm_w4a16_g128(xh.astype(np.float64),
                                                                     packed, sc, zz))


def test_gemm_empty_shapes():
    xq = torch.zeros((0, 64), dtype=torch.int8, device="cuda")
    wq = torch.zeros((32, 64), dtype=torch.int8, device="cuda")
    y = qg.gemm_w8a8(xq, torch.zeros(0, device="cuda"), wq, torch.zeros(32, device="cuda"))
    assert y.shape == (0, 32)
