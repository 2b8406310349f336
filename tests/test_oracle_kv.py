"""Pins of the KV-cache INT8 oracle (oracle/kv.py) against what the pages and
the arithmetic fix, independently of the oracle's own code:

  * exact-rational brute force (tests/exact.py) on tiny caches, including a
    partial last segment;
  * round-half-to-even ties with a power-of-two scale;
  * the round-trip bound |x - x_hat| <= s/2 (「第4章：量化」 §1.1-1.2);
  * every channel of every segment reaches code +-127 at its max;
  * zero channels, one-token segments and segment independence
    (「LLM推理降本五要素」 §5.2: each 128-token segment has its own scales);
  * the size arithmetic: int8 codes are half the fp16 cache.
"""
import numpy as np
import pytest

import oracle
from tests.exact import fl32, frac, rne_int


def _brute(kv, seg=128):
    T, H, D = kv.shape
    S = (T + seg - 1) // seg
    codes = np.zeros((T, H, D), np.int64)
    scales = [[[None] * D for _ in range(S)] for _ in range(H)]
    for h in range(H):
        for si in range(S):
            ts = range(si * seg, min(T, (si + 1) * seg))
            for d in range(D):
                a = max(abs(frac(kv[t, h, d])) for t in ts)
                s = fl32(a / 127)
                scales[h][si][d] = s
                for t in ts:
                    codes[t, h, d] = 0 if a == 0 else max(-127, min(127, rne_int(fl32(frac(kv[t, h, d]) / s))))
    return codes, scales


def _cache(rng, T, H, D):
    kv = rng.standard_normal((T, H, D)).astype(np.float32)
    kv[:, :, rng.integers(0, D)] *= 40.0          # an outlier channel
    return kv


def test_brute_force_tiny_with_partial_segment():
    rng = np.random.default_rng(11)
    kv = _cache(rng, 131, 2, 3)
    codes, scales = oracle.quantize_kv_segments(kv)
    bc, bs = _brute(kv)
    np.testing.assert_array_equal(codes.astype(np.int64), bc)
    for h in range(2):
        for si in range(2):
            for d in range(3):
                assert frac(scales[h, si, d]) == bs[h][si][d]


def test_rne_ties_with_power_of_two_scale():
    # segment max 127 * 2^-3 makes s exactly 2^-3; (j + 1/2) * 2^-3 are ties
    kv = np.zeros((128, 1, 4), np.float32)
    kv[0, 0, :] = 127 * 0.125
    kv[1, 0, :] = [2.5 * 0.125, 3.5 * 0.125, -2.5 * 0.125, 0.5 * 0.125]
    codes, scales = oracle.quantize_kv_segments(kv)
    assert np.all(scales == np.float32(0.125))
    assert codes[1, 0].tolist() == [2, 4, -2, 0]


def test_round_trip_within_half_scale():
    rng = np.random.default_rng(12)
    kv = _cache(rng, 300, 4, 64)
    codes, scales = oracle.quantize_kv_segments(kv)
    xhat = oracle.dequantize_kv_segments(codes, scales)
    s = np.transpose(scales, (1, 0, 2))[np.arange(300) // 128].astype(np.float64)
    assert np.all(np.abs(kv.astype(np.float64) - xhat) <= s / 2 * (1 + 2.0 ** -20))


def test_every_channel_reaches_127():
    rng = np.random.default_rng(13)
    kv = _cache(rng, 257, 3, 32)
    codes, scales = oracle.quantize_kv_segments(kv)
    for si in range(3):
        seg = codes[si * 128:(si + 1) * 128].astype(np.int64)
        assert np.all(np.abs(seg).max(axis=0) == 127)
    assert np.abs(codes.astype(np.int64)).max() <= 127


def test_zero_channel_one_token_segment_and_independence():
    rng = np.random.default_rng(14)
    kv = _cache(rng, 129, 2, 16)
    kv[:128, 1, 5] = 0.0                               # an all-zero channel in segment 0
    codes, scales = oracle.quantize_kv_segments(kv)
    assert scales[1, 0, 5] == 0 and np.all(codes[:128, 1, 5] == 0)
    # segment 1 holds one token: every nonzero value is its own max
    last = codes[128].astype(np.int64)
    assert np.all((np.abs(last) == 127) | (kv[128] == 0))
    # changing segment 1 leaves segment 0 untouched
    kv2 = kv.copy()
    kv2[128] *= 1000.0
    c2, s2 = oracle.quantize_kv_segments(kv2)
    np.testing.assert_array_equal(c2[:128], codes[:128])
    np.testing.assert_array_equal(s2[:, 0], scales[:, 0])


def test_size_arithmetic():
    # 8-bit codes are exactly half of an fp16 cache; fp32 scales per 128
    # positions add 4/128 bytes per code byte
    T, H, D = 4096, 32, 128
    codes, scales = oracle.quantize_kv_segments(np.ones((T, 1, 1), np.float32))
    assert codes.nbytes * 2 == 2 * T * 1 * 1 and scales.nbytes == 4 * (T // 128)
    assert (T * H * D) / (2 * T * H * D) == 0.5
    assert 4 * H * (T // 128) * D / (T * H * D) == pytest.approx(1 / 32)
