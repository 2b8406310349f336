"""Pins for the oracle contractions and epilogues (CPU only).

  * pure-Python integer loops on tiny shapes, with an unpack of the packed
    words written independently (hex digits of each word);
  * int64 matmul (no BLAS) equals the float64-BLAS path bit for bit;
  * special cases: all-ones codes give acc = K (128 per group), one-hot rows
    select one weight code;
  * power-of-two scales make the fp32-representable product exact;
  * the whole chain against a library routine: torch.matmul in float64 of
    the dequantized operands (x_hat = (x_int - z) s) equals y_exact.
"""
from fractions import Fraction

import numpy as np
import torch

import oracle
from workloads import by_name, draw, f32_to_bf16_bits


def _unpack_hex(packed_row):
    """Codes of one packed row, read from the hex digits (last digit = k 8i)."""
    out = []
    for w in packed_row:
        h = f"{int(w) & 0xffffffff:08x}"
        out.extend(int(d, 16) for d in reversed(h))
    return out


def test_w8a8_acc_brute_force():
    rng = np.random.default_rng(0)
    for M, N, K in [(1, 1, 16), (3, 5, 48), (4, 4, 256)]:
        xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
        wq = rng.integers(-127, 128, (N, K)).astype(np.int8)
        acc = oracle.gemm_w8a8_acc(xq, wq)
        for m in range(M):
            for n in range(N):
                assert acc[m, n] == sum(int(xq[m, k]) * int(wq[n, k]) for k in range(K))


def test_w8a8_acc_extremes_and_paths_agree():
    K = 4096
    xq = np.full((2, K), 127, np.int8)
    xq[1] = -127
    wq = np.full((3, K), -127, np.int8)
    acc = oracle.gemm_w8a8_acc(xq, wq)
    assert acc[0, 0] == -K * 127 * 127 and acc[1, 2] == K * 127 * 127
    ones = oracle.gemm_w8a8_acc(np.ones((2, 512), np.int8), np.ones((5, 512), np.int8))
    assert np.all(ones == 512)
    wl = by_name("w8a8_tiny")
    d = draw(wl)
    xq, _ = oracle.quantize_per_token_i8(d["x"])
    wq, _ = oracle.quantize_weight_i8_per_channel(d["w"])
    assert np.array_equal(oracle.gemm_w8a8_acc(xq, wq),
                          oracle.gemm_w8a8_acc(xq, wq, exact_int=True))


def test_w8a8_one_hot_selects_code():
    rng = np.random.default_rng(2)
    wq = rng.integers(-127, 128, (6, 64)).astype(np.int8)
    xq = np.zeros((64, 64), np.int8)
    xq[np.arange(64), np.arange(64)] = 1
    assert np.array_equal(oracle.gemm_w8a8_acc(xq, wq), wq.T.astype(np.int64))


def test_w8a8_epilogue_power_of_two_exact():
    rng = np.random.default_rng(4)
    xq = rng.integers(-127, 128, (4, 64)).astype(np.int8)
    wq = rng.integers(-127, 128, (8, 64)).astype(np.int8)
    sx = (2.0 ** rng.integers(-8, 0, 4)).astype(np.float32)
    sw = (2.0 ** rng.integers(-12, -4, 8)).astype(np.float32)
    y = oracle.gemm_w8a8(xq, sx, wq, sw)
    for m in range(4):
        for n in range(8):
            exact = Fraction(sum(int(xq[m, k]) * int(wq[n, k]) for k in range(64))) \
                * Fraction(float(sx[m])) * Fraction(float(sw[n]))
            assert Fraction(float(y[m, n])) == exact
            assert float(np.float32(y[m, n])) == float(y[m, n])   # fits fp32


def test_w8a8_whole_chain_vs_torch_float64():
    wl = by_name("w8a8_tiny")
    d = draw(wl)
    xq, sx = oracle.quantize_per_token_i8(d["x"])
    wq, sw = oracle.quantize_weight_i8_per_channel(d["w"])
    y = oracle.gemm_w8a8(xq, sx, wq, sw)
    x_hat = torch.from_numpy(xq.astype(np.float64) * sx[:, None].astype(np.float64))
    w_hat = torch.from_numpy((wq.astype(np.float64) * sw[:, None].astype(np.float64)).T.copy())
    ref = torch.matmul(x_hat, w_hat).numpy()
    bound = 2.0 ** -50 * (np.abs(x_hat.numpy()) @ np.abs(w_hat.numpy()))
    assert np.all(np.abs(y - ref) <= bound)
    # and the quantized layer approximates the float layer
    yf = d["x"].astype(np.float64) @ d["w"].astype(np.float64)
    assert np.abs(y - yf).max() < 0.05 * np.abs(yf).max()


def _u4_case(seed, M, K, N):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    x = rng.standard_normal((M, K)).astype(np.float32)
    packed, sc, zz = oracle.quantize_weight_u4_g128(w)
    return x, w, packed, sc, zz


def test_w4a8_acc_brute_force():
    x, _, packed, sc, zz = _u4_case(8, 3, 256, 5)
    xq, _ = oracle.quantize_per_token_i8(x)
    acc = oracle.gemm_w4a8_g128_acc(xq, packed, zz)
    assert acc.shape == (3, 2, 5)
    for n in range(5):
        codes = _unpack_hex(packed[n])
        for g in range(2):
            z = int(zz[n, g])
            for m in range(3):
                ref = sum(int(xq[m, k]) * (codes[k] - z) for k in range(128 * g, 128 * g + 128))
                assert acc[m, g, n] == ref
    assert np.array_equal(acc, oracle.gemm_w4a8_g128_acc(xq, packed, zz, exact_int=True))


def test_w4a8_all_ones_and_one_hot():
    N, K = 4, 256
    codes = np.ones((N, K), np.uint8)
    packed = oracle.pack_u4(codes)
    zero = np.zeros((N, 2), np.float16)
    acc = oracle.gemm_w4a8_g128_acc(np.ones((2, K), np.int8), packed, zero)
    assert np.all(acc == 128)
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 16, (N, K)).astype(np.uint8)
    zero = rng.integers(0, 16, (N, 2)).astype(np.float16)
    xq = np.zeros((1, K), np.int8)
    xq[0, 200] = 1
    acc = oracle.gemm_w4a8_g128_acc(xq, oracle.pack_u4(codes), zero)
    assert np.all(acc[0, 0] == 0)
    assert np.array_equal(acc[0, 1], codes[:, 200].astype(np.int64) - zero[:, 1].astype(np.int64))


def test_w4a8_whole_chain_vs_torch_float64():
    x, w, packed, sc, zz = _u4_case(12, 4, 512, 24)
    xq, sx = oracle.quantize_per_token_i8(x)
    y = oracle.gemm_w4a8_g128(xq, sx, packed, sc, zz)
    codes = np.array([_unpack_hex(r) for r in packed], np.float64)       # [N, K]
    s = np.repeat(sc.astype(np.float64), 128, axis=1)
    z = np.repeat(zz.astype(np.float64), 128, axis=1)
    w_hat = torch.from_numpy(((codes - z) * s).T.copy())
    x_hat = torch.from_numpy(xq.astype(np.float64) * sx[:, None].astype(np.float64))
    ref = torch.matmul(x_hat, w_hat).numpy()
    bound = 2.0 ** -48 * (np.abs(x_hat.numpy()) @ np.abs(w_hat.numpy()))
    assert np.all(np.abs(y - ref) <= bound)
    yf = x.astype(np.float64) @ w.astype(np.float64)
    # 4-bit weights: the layer error stays a small fraction of the output RMS
    assert np.sqrt(np.mean((y - yf) ** 2)) < 0.15 * np.sqrt(np.mean(yf ** 2))


def test_w4a16_partials_exact_and_chain():
    x, w, packed, sc, zz = _u4_case(13, 2, 256, 6)
    x16 = x.astype(np.float16)
    x64 = x16.astype(np.float64)
    p = oracle.gemm_w4a16_g128_partials(x64, packed, zz)
    for n in range(6):
        codes = _unpack_hex(packed[n])
        for g in range(2):
            for m in range(2):
                exact = sum(Fraction(float(x16[m, k])) * (codes[k] - int(zz[n, g]))
                            for k in range(128 * g, 128 * g + 128))
                assert Fraction(float(p[m, g, n])) == exact
    y = oracle.gemm_w4a16_g128(x64, packed, sc, zz)
    w_hat = torch.from_numpy(oracle.dequant_u4_g128(packed, sc, zz).copy())
    ref = torch.matmul(torch.from_numpy(x64), w_hat).numpy()
    bound = 2.0 ** -48 * (np.abs(x64) @ np.abs(w_hat.numpy()))
    assert np.all(np.abs(y - ref) <= bound)


def test_bf16_input_path_through_oracle():
    x = np.array([[1.0, -2.0, 0.5, 3.0] * 32], np.float32)
    b = f32_to_bf16_bits(x)
    assert np.array_equal(oracle.to_f32(b, "bf16"), x)
