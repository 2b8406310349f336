"""Pins of the W4A8 outlier-retention oracle (「LLM推理降本五要素」 §2.2) against a
hand-worked fixture, brute force, invariants of the selection and reductions to
the plain W4A8 and W8A8 oracles."""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.outlier import (N_OUT, decode_records, gemm_w4a8_g128_outlier_acc,
                            gemm_w4a8_g128_outliers, quantize_weight_u4_g128_outliers,
                            select_outliers)

GOLD = os.path.join(os.path.dirname(__file__), "golden", "outlier_groups.txt")
POS = [0, 5, 15, 16, 31, 77, 100, 120]


def _fixture_weights():
    k = np.arange(128)
    a = (0.01 * ((k % 16) - 8)).astype(np.float64)
    a[5], a[77], a[100] = 1.27, -0.5, 0.3
    b = (0.001 * ((k % 8) - 4)).astype(np.float64)
    b[3], b[40], b[90], b[120] = 0.5, -0.5, 0.5, -0.5
    return np.stack([a, b], axis=1).astype(np.float32)               # [128, 2]


def test_golden_groups():
    rows = {}
    for line in open(GOLD):
        line = line.strip()
        if line and not line.startswith("#"):
            col, sbits, z, idx, slots, codes = [p.strip() for p in line.split("|")]
            rows[col] = (int(sbits, 16), int(z), [int(v) for v in idx.split()],
                         [int(v, 16) for v in slots.split()], [int(v) for v in codes.split()])
    packed, s16, z16, rec, s8 = quantize_weight_u4_g128_outliers(_fixture_weights())
    codes = oracle.unpack_u4(packed)
    for n, col in enumerate(("A", "B")):
        sbits, z, idx, slots, cs = rows[col]
        assert int(s16[n, 0].view(np.uint16)) == sbits
        assert float(z16[n, 0]) == z
        index, code, valid = decode_records(rec)
        assert list(index[n, 0, :3]) == idx and valid[n, 0, :3].all() and not valid[n, 0, 3]
        got_slots = [int((int(rec[n, 0]) >> (16 * i)) & 0xFFFF) for i in range(4)]
        assert got_slots == slots
        assert [int(codes[n, p]) for p in POS] == cs
    assert s8[0] == np.float32(0.01) and s8[1] == np.float32(np.float32(0.5) / np.float32(127))


def _random_w(seed, K, N):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((K, N)) * 0.02
    spikes = rng.random((K, N)) < 0.01
    w[spikes] *= 8.0
    return w.astype(np.float32)


def test_selection_invariants():
    w = _random_w(1, 512, 37)
    idx = select_outliers(w)                                          # [G, 3, N]
    G = 4
    wg = w.reshape(G, 128, 37)
    for g in range(G):
        for n in range(37):
            sel = set(idx[g, :, n].tolist())
            assert len(sel) == N_OUT
            mags = np.abs(wg[g, :, n])
            m_in = min(mags[list(sel)])
            rest = [mags[k] for k in range(128) if k not in sel]
            assert max(rest) <= m_in
    # ties go to the lower index
    t = np.zeros((128, 1), np.float32)
    t[[9, 20, 64, 99, 127], 0] = [0.7, -0.7, 0.7, 0.7, -0.7]
    assert select_outliers(t)[0, :, 0].tolist() == [9, 20, 64]


def test_round_trip_bounds_and_outlier_positions():
    w = _random_w(2, 1024, 48)
    packed, s16, z16, rec, s8 = quantize_weight_u4_g128_outliers(w)
    codes = oracle.unpack_u4(packed).astype(np.float64)              # [N, K]
    index, code, valid = decode_records(rec)
    N, K = codes.shape
    s = np.repeat(s16.astype(np.float64), 128, axis=1)
    z = np.repeat(z16.astype(np.float64), 128, axis=1)
    is_out = np.zeros((N, K), bool)
    for g in range(K // 128):
        for i in range(N_OUT):
            is_out[np.arange(N), 128 * g + index[:, g, i]] = True
    wt = w.T.astype(np.float64)
    err = np.abs(wt - (codes - z) * s)
    # one binary32 rounding of w / s may push a value a hair past s / 2
    assert np.all(err[~is_out] <= s[~is_out] * (0.5 + 2.0 ** -20))
    assert np.all(codes[is_out] == z[is_out])                        # outliers: q = z
    for n in range(N):
        for g in range(K // 128):
            for i in range(N_OUT):
                k = 128 * g + index[n, g, i]
                assert abs(wt[n, k] - code[n, g, i] * float(s8[n])) <= float(s8[n]) * (0.5 + 2.0 ** -20)
    assert np.all(np.abs(code[valid]) <= 127)
    assert np.any(np.abs(code[valid]) == 127)


def test_group_range_shrinks():
    w = _random_w(3, 512, 64)
    _, s_plain, _ = oracle.quantize_weight_u4_g128(w)
    _, s_out, _, _, _ = quantize_weight_u4_g128_outliers(w)
    assert np.all(s_out.astype(np.float64) <= s_plain.astype(np.float64))
    assert np.mean(s_out.astype(np.float64) < s_plain.astype(np.float64)) > 0.5


def test_outlier_acc_brute_force():
    rng = np.random.default_rng(4)
    M, K, N = 3, 256, 5
    w = _random_w(5, K, N)
    xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    packed, s16, z16, rec, s8 = quantize_weight_u4_g128_outliers(w)
    acc = gemm_w4a8_g128_outlier_acc(xq, rec)
    for m in range(M):
        for n in range(N):
            tot = 0
            for g in range(K // 128):
                r = int(rec[n, g])
                for i in range(4):
                    slot = (r >> (16 * i)) & 0xFFFF
                    kk, c = slot >> 8, slot & 0xFF
                    if kk < 128:
                        c = c - 256 if c >= 128 else c
                        tot += int(xq[m, 128 * g + kk]) * c
            assert acc[m, n] == tot


def test_product_matches_dequantized_weights_exactly():
    """y_exact equals s_x (xq . w_hat) with w_hat the dequantized weights, in exact
    rationals, up to float64's own rounding of the oracle's sum."""
    rng = np.random.default_rng(6)
    M, K, N = 2, 256, 4
    w = _random_w(7, K, N)
    xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    xs = (rng.random(M) * 0.1 + 0.01).astype(np.float32)
    packed, s16, z16, rec, s8 = quantize_weight_u4_g128_outliers(w)
    y = gemm_w4a8_g128_outliers(xq, xs, packed, s16, z16, rec, s8)
    codes = oracle.unpack_u4(packed)
    index, code, valid = decode_records(rec)
    for m in range(M):
        for n in range(N):
            tot, mag = Fraction(0), Fraction(0)
            for k in range(K):
                g = k // 128
                t = Fraction(int(xq[m, k])) * (int(codes[n, k]) - Fraction(float(z16[n, g]))) * \
                    Fraction(float(s16[n, g]))
                tot += t
                mag += abs(t)
            for g in range(K // 128):
                for i in range(4):
                    if valid[n, g, i]:
                        t = Fraction(int(xq[m, 128 * g + index[n, g, i]])) * int(code[n, g, i]) * \
                            Fraction(float(s8[n]))
                        tot += t
                        mag += abs(t)
            exact = Fraction(float(xs[m])) * tot
            assert abs(Fraction(float(y[m, n])) - exact) <= Fraction(float(xs[m])) * mag * Fraction(1, 2 ** 48)


def test_reduces_to_plain_w4a8_without_side_codes():
    rng = np.random.default_rng(8)
    M, K, N = 3, 384, 6
    w = _random_w(9, K, N)
    xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    xs = (rng.random(M) * 0.1).astype(np.float32)
    packed, s16, z16, rec, s8 = quantize_weight_u4_g128_outliers(w)
    zero_codes = rec & np.uint64(0xFF00FF00FF00FF00)          # keep indices, codes 0
    y = gemm_w4a8_g128_outliers(xq, xs, packed, s16, z16, zero_codes, s8)
    np.testing.assert_array_equal(y, oracle.gemm_w4a8_g128(xq, xs, packed, s16, z16))


def test_three_nonzeros_per_group_is_w8a8():
    """A weight matrix with exactly three nonzero weights per (column, group): the
    4-bit part is constant (s = z = q = 0) and the product is the per-channel
    INT8 product of the plain W8A8 oracle on the same codes."""
    rng = np.random.default_rng(10)
    M, K, N = 4, 512, 7
    w = np.zeros((K, N), np.float32)
    for n in range(N):
        for g in range(K // 128):
            ks = rng.choice(128, 3, replace=False)
            w[128 * g + ks, n] = rng.standard_normal(3).astype(np.float32)
    xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    xs = (rng.random(M) * 0.1).astype(np.float32)
    packed, s16, z16, rec, s8 = quantize_weight_u4_g128_outliers(w)
    assert not np.any(s16.astype(np.float64)) and not np.any(oracle.unpack_u4(packed))
    wq8, ws8 = oracle.quantize_weight_i8_per_channel(w)
    np.testing.assert_array_equal(ws8, s8)
    y = gemm_w4a8_g128_outliers(xq, xs, packed, s16, z16, rec, s8)
    y8 = oracle.gemm_w8a8(xq, xs, wq8, ws8)
    np.testing.assert_allclose(y, y8, rtol=1e-12, atol=0)


def test_rejects_bad_k():
    with pytest.raises(ValueError):
        quantize_weight_u4_g128_outliers(np.zeros((100, 2), np.float32))


def test_error_vs_plain_u4():
    """Keeping the 3 largest weights of each group in INT8 lowers the weight
    round-trip error of the layer (the reason the page gives)."""
    w = _random_w(11, 1024, 256)
    p, s, z, r, s8 = oracle.quantize_weight_u4_g128_outliers(w)
    index, code, valid = oracle.decode_records(r)
    what = oracle.dequant_u4_g128(p, s, z).T                       # [N, K]
    for g in range(1024 // 128):
        for i in range(3):
            what[np.arange(256), 128 * g + index[:, g, i]] = code[:, g, i] * s8.astype(np.float64)
    pp, ps, pz = oracle.quantize_weight_u4_g128(w)
    plain = oracle.dequant_u4_g128(pp, ps, pz).T
    e_out = np.abs(what - w.T).mean()
    e_plain = np.abs(plain - w.T).mean()
    assert e_out < e_plain
    print(f"mean |w - w_hat|: plain u4 {e_plain:.3e}, with INT8 outliers {e_out:.3e}")
