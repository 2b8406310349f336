"""Pins of the 2:4 sparse uint4 oracle (「LLM推理降本五要素」 §3.2) against a hand-worked
group, the pruning invariants, the format's inverse, brute force, the page's
volume figure and a reduction to the dense W4A8 oracle."""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.sparse24 import (expand_sparse24, gemm_w4a8_g128_sparse24,
                             gemm_w4a8_g128_sparse24_acc, prune_2_4,
                             quantize_weight_u4_g128_sparse24)

GOLD = os.path.join(os.path.dirname(__file__), "golden", "sparse24_group.txt")


def _w(seed, K, N):
    return (np.random.default_rng(seed).standard_normal((K, N)) * 0.02).astype(np.float32)


def test_golden_groups():
    rows = {}
    for line in open(GOLD):
        if line.strip() and not line.startswith("#"):
            name, sbits, z, words = [p.strip() for p in line.split("|")]
            rows[name] = (int(sbits, 16), int(z), [int(x, 16) for x in words.split()])
    P = {0: [1, -3, 2, 0], 1: [0, 0, 5, -5], 2: [2, -2, 2, 1]}
    a = [0.01 * P[(k // 4) % 3][k % 4] for k in range(128)]
    b = [0.01 * [-5, -4, 3, 0][k % 4] for k in range(128)]
    w = np.array([a, b]).T.astype(np.float32)                         # [128, 2]
    packed, s16, z16 = quantize_weight_u4_g128_sparse24(w)
    for n, name in enumerate(("A", "B")):
        sbits, z, words = rows[name]
        assert int(s16[n, 0].view(np.uint16)) == sbits
        assert float(z16[n, 0]) == z
        assert [int(v) for v in packed[0, 0, n].view(np.uint32)] == words
    assert not packed[0, 0, 2:].any()                                   # tile rows past N are zero


def test_pruning_invariants_and_ties():
    w = _w(1, 512, 33)
    keep = prune_2_4(w)
    k4 = keep.reshape(128, 4, 33)
    assert (k4.sum(axis=1) == 2).all()
    a = np.abs(w).reshape(128, 4, 33)
    kept_min = np.where(k4, a, np.inf).min(axis=1)
    pruned_max = np.where(k4, -np.inf, a).max(axis=1)
    assert (kept_min >= pruned_max).all()
    t = np.array([[0.5], [-0.5], [0.5], [0.1], [0.0], [0.0], [0.0], [0.0]], np.float32)
    assert prune_2_4(t)[:, 0].tolist() == [True, True, False, False, True, True, False, False]


def test_format_inverse_and_round_trip():
    w = _w(2, 1024, 40)
    packed, s16, z16 = quantize_weight_u4_g128_sparse24(w)
    codes = expand_sparse24(packed, 40)                                 # [N, K], -1 = pruned
    keep = prune_2_4(w).T
    assert ((codes >= 0) == keep).all()
    assert codes.max() <= 15
    s = np.repeat(s16.astype(np.float64), 128, axis=1)
    z = np.repeat(z16.astype(np.float64), 128, axis=1)
    err = np.abs(w.T.astype(np.float64) - (codes - z) * s)
    assert (err[keep] <= s[keep] * (0.5 + 2.0 ** -20)).all()


def test_volume_is_one_eighth_of_fp16_for_codes():
    """「LLM推理降本五要素」 §3.2: 2:4 then 4 bits leaves 1/8 of the fp16 volume (the
    codes); the positions add 2 bits per kept weight."""
    K, N = 4096, 64
    packed, _, _ = quantize_weight_u4_g128_sparse24(_w(3, K, N))
    code_bytes = packed.nbytes * 8 // 12          # two of every three words are codes
    assert code_bytes * 8 == K * N * 2            # fp16 bytes / 8 (N a multiple of 16: no padding)
    assert packed.nbytes == K * N * 3 // 8        # codes + positions: 3 bits per dense weight


def test_reduces_to_dense_w4a8():
    """Pruned positions given the code z are the dense W4A8 product with the same
    scales and zero points, exactly."""
    rng = np.random.default_rng(4)
    M, K, N = 5, 384, 24
    w = _w(5, K, N)
    xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    xs = (rng.random(M) * 0.1 + 1e-3).astype(np.float32)
    packed, s16, z16 = quantize_weight_u4_g128_sparse24(w)
    codes = expand_sparse24(packed, N)
    z = np.repeat(z16.astype(np.int64), 128, axis=1)
    dense = oracle.pack_u4(np.where(codes >= 0, codes, z).astype(np.uint8))
    np.testing.assert_array_equal(gemm_w4a8_g128_sparse24_acc(xq, packed, z16),
                                  oracle.gemm_w4a8_g128_acc(xq, dense, z16))
    np.testing.assert_allclose(gemm_w4a8_g128_sparse24(xq, xs, packed, s16, z16),
                               oracle.gemm_w4a8_g128(xq, xs, dense, s16, z16), rtol=1e-15, atol=0)


def test_product_brute_force():
    rng = np.random.default_rng(6)
    M, K, N = 2, 256, 3
    w = _w(7, K, N)
    xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    xs = (rng.random(M) * 0.1 + 0.01).astype(np.float32)
    packed, s16, z16 = quantize_weight_u4_g128_sparse24(w)
    y = gemm_w4a8_g128_sparse24(xq, xs, packed, s16, z16)
    keep = prune_2_4(w)
    for m in range(M):
        for n in range(N):
            tot, mag = Fraction(0), Fraction(0)
            for k in range(K):
                if not keep[k, n]:
                    continue
                g = k // 128
                sg, zg = Fraction(float(s16[n, g])), Fraction(float(z16[n, g]))
                q = int(np.clip(np.rint(np.float32(w[k, n] / np.float32(s16[n, g]))) + float(zg), 0, 15)) \
                    if sg else 0
                t = int(xq[m, k]) * (q - zg) * sg
                tot += t
                mag += abs(t)
            exact = Fraction(float(xs[m])) * tot
            assert abs(Fraction(float(y[m, n])) - exact) <= Fraction(float(xs[m])) * mag * Fraction(1, 2 ** 48)


def test_tiles_round_trip():
    rows = np.arange(37 * 24, dtype=np.int32).reshape(37, 24)          # 37 channels, 2 groups
    from oracle.sparse24 import tile16, untile16
    t = tile16(rows)
    assert t.shape == (3, 2, 16, 12) and not t[2, :, 5:].any()
    np.testing.assert_array_equal(untile16(t, 37), rows)
    assert t[1, 1, 3, 7] == rows[16 + 3, 12 + 7]


def test_rejects_bad_k():
    with pytest.raises(ValueError):
        quantize_weight_u4_g128_sparse24(np.zeros((96, 2), np.float32))
