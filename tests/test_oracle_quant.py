"""Pins for the oracle quantizers (CPU only).

What pins what:
  * brute force in exact rationals with explicitly written IEEE roundings
    (tests/exact.py) -> float32 division / RNE / fp16 round-up semantics;
  * hand-worked tie and clamp cases (tests/golden) -> rounding mode, order of
    round and +z, clamp ranges, scale formulas (/127, /15);
  * round-trip bound |x - x_hat| <= s/2 (up to one fp32 rounding of x/s),
    which a wrong scale denominator, a wrong sign or a dropped z breaks;
  * structural invariants: a +-127 code in every row with a normal scale,
    q = 0 at the group minimum, the code range;
  * hand-worked subnormal-scale rows (the clamp binding, a scale that
    underflows to 0) and exact-rational brute force across that range;
  * the packing order from a hand-written word table.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.exact import fl32, f16_up, rne_int, frac
from workloads import by_name, draw

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(fname):
    with open(os.path.join(GOLD, fname)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield [p.split() for p in line.split("|")]


# ---------------------------------------------------------------- per-token i8

def test_per_token_golden_ties():
    for (e,), vals, codes in _rows("per_token_ties.txt"):
        s = 2.0 ** int(e)
        x = (np.array([float(v) for v in vals]) * s).astype(np.float32)[None, :]
        q, sc = oracle.quantize_per_token_i8(x)
        assert sc[0] == np.float32(s)
        assert q[0].tolist() == [int(c) for c in codes]


def _brute_per_token(row):
    xs = [frac(v) for v in row]
    amax = max(abs(v) for v in xs)
    s = fl32(amax / 127)
    if s == 0:
        return [0] * len(xs), 0.0
    return [max(-127, min(127, rne_int(fl32(v / s)))) for v in xs], float(s)


def test_per_token_brute_force_random():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((6, 40)) * rng.choice([1e-3, 1.0, 40.0], (6, 1))).astype(np.float32)
    x[2, :] = 0.0
    x[3, 5] = 1e-30                     # tiny amax row
    x[3, np.arange(40) != 5] = 0.0
    q, s = oracle.quantize_per_token_i8(x)
    for m in range(x.shape[0]):
        bq, bs = _brute_per_token(x[m])
        assert q[m].tolist() == bq
        assert float(s[m]) == bs


def test_per_token_golden_subnormal_scales():
    """Hand-worked rows whose scale is subnormal: the clamp binds (158 -> 127,
    127.5 -> 127), a scale that underflows to 0 gives zero codes."""
    u = 2.0 ** -149
    n = 0
    for (su,), vals, codes in _rows("per_token_subnormal.txt"):
        x = np.zeros((1, 16), np.float32)
        x[0, : len(vals)] = np.array([int(v) for v in vals], np.float64) * u
        q, sc = oracle.quantize_per_token_i8(x)
        assert float(sc[0]) == int(su) * u
        assert q[0, : len(vals)].tolist() == [int(c) for c in codes]
        assert not q[0, len(vals):].any()
        n += 1
    assert n == 5


def test_per_token_brute_force_subnormal():
    """Rows with max|x| from 2^-149 to past 127 * 2^-128 (subnormal and
    underflowing scales, finite and infinite reciprocals) against exact
    rationals."""
    rng = np.random.default_rng(11)
    u = 2.0 ** -149
    amax_units = [1, 2, 63, 64, 127, 150, 190, 191, 300, 316, 400, 444, 1000, 12345, 2 ** 20, 127 * 2 ** 21,
                  127 * 2 ** 21 + 12345, 2 ** 23 + 1]
    rows = []
    for k in amax_units:
        v = rng.integers(-k, k + 1, 24).astype(np.float64)
        v[rng.integers(0, 24)] = k * rng.choice([-1, 1])
        rows.append(v * u)
    x = np.array(rows).astype(np.float32)
    q, s = oracle.quantize_per_token_i8(x)
    clamped = 0
    for m in range(x.shape[0]):
        bq, bs = _brute_per_token(x[m])
        assert q[m].tolist() == bq
        assert float(s[m]) == bs
        clamped += int(bs > 0 and frac(np.max(np.abs(x[m]))) / frac(bs) > Fraction(255, 2))
    assert clamped >= 6      # the clamp binds on several of these rows


def test_per_token_round_trip_and_range():
    wl = by_name("w8a8_decode_ffn_up")
    x = draw(wl, rows=64)["x"]
    q, s = oracle.quantize_per_token_i8(x)
    assert q.dtype == np.int8 and s.dtype == np.float32
    err = np.abs(x.astype(np.float64) - q.astype(np.float64) * s[:, None])
    # |x/s| <= 127(1+2^-24), so one fp32 rounding of x/s adds < 2^-17 s
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 2.0 ** -16))
    assert np.all(np.abs(q).max(axis=1) == 127)
    assert q.min() >= -127


def test_per_token_zero_row_and_empty():
    q, s = oracle.quantize_per_token_i8(np.zeros((3, 16), np.float32))
    assert np.all(q == 0) and np.all(s == 0)
    q, s = oracle.quantize_per_token_i8(np.zeros((0, 16), np.float32))
    assert q.shape == (0, 16) and s.shape == (0,)


def test_input_upcast_is_exact():
    b = np.array([0x3F80, 0xC040, 0x0001, 0x7F7F], np.uint16)   # 1, -3, tiny, max
    f = oracle.to_f32(b, "bf16")
    assert f[0] == 1.0 and f[1] == -3.0 and f[2] == np.float32(2.0 ** -133)
    h = np.array([1.5, -2.0, 6.1e-5], np.float16)
    assert np.all(oracle.to_f32(h, "f16") == h.astype(np.float32))


# --------------------------------------------------------- per-channel i8

def test_per_channel_is_per_token_of_transpose():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((96, 24)) * 0.02).astype(np.float32)
    q, s = oracle.quantize_weight_i8_per_channel(w)
    assert q.shape == (24, 96) and s.shape == (24,)
    for n in range(24):
        bq, bs = _brute_per_token(w[:, n])
        assert q[n].tolist() == bq and float(s[n]) == bs
    err = np.abs(w.T.astype(np.float64) - q * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None] * (0.5 + 2.0 ** -16))


# ------------------------------------------------------------- u4 g128

def _brute_u4_group(vals):
    xs = [frac(v) for v in vals]
    lo, hi = min(xs), max(xs)
    t = fl32(fl32(hi - lo) / 15)
    s = f16_up(t)
    if s == 0:
        return 0, 0.0, [0] * len(xs)
    z = max(0, min(15, rne_int(fl32(-lo / s))))
    q = [max(0, min(15, rne_int(fl32(v / s)) + z)) for v in xs]
    return z, float(s), q


def _group_from_units(listed, s):
    g = np.zeros(128, np.float64)
    g[: len(listed)] = listed
    return (g * s).astype(np.float32)


def test_u4_golden_groups():
    s = 2.0 ** -6
    for (lo, hi), listed, (z,), codes in _rows("u4_groups.txt"):
        listed = [float(v) for v in listed]
        assert min(listed) == float(lo) and max(listed) == float(hi)
        col = _group_from_units(listed, s)
        w = np.stack([col, col[::-1].copy()], axis=1)               # [128, 2]
        packed, sc, zz = oracle.quantize_weight_u4_g128(w)
        c = oracle.unpack_u4(packed)
        assert sc[0, 0] == np.float16(s) and zz[0, 0] == float(z)
        assert c[0, : len(listed)].tolist() == [int(v) for v in codes]
        assert c[1].tolist() == c[0][::-1].tolist()
        bz, bs, bq = _brute_u4_group(col)
        assert bz == int(z) and bs == s and bq == c[0].tolist()


def test_u4_brute_force_random():
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((256, 6)) * 0.02).astype(np.float32)
    w[:128, 3] += 0.5            # all-positive group: z clamps to 0
    w[128:, 4] -= 0.5            # all-negative group: z clamps to 15
    w[:128, 5] = 0.125           # constant group: s = 0, z = 0, q = 0
    packed, sc, zz = oracle.quantize_weight_u4_g128(w)
    codes = oracle.unpack_u4(packed)
    for n in range(6):
        for g in range(2):
            bz, bs, bq = _brute_u4_group(w[128 * g:128 * (g + 1), n])
            assert float(sc[n, g]) == bs and float(zz[n, g]) == bz
            assert codes[n, 128 * g:128 * (g + 1)].tolist() == bq
    assert zz[3, 0] == 0 and zz[4, 1] == 15 and sc[5, 0] == 0 and np.all(codes[5, :128] == 0)


def test_u4_round_trip_and_code_range():
    rng = np.random.default_rng(5)
    K, N = 128 * 8, 2048                      # 16384 groups of N(0, 0.02)
    w = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    packed, sc, zz = oracle.quantize_weight_u4_g128(w)
    assert packed.dtype == np.int32 and packed.shape == (N, K // 8)
    assert sc.dtype == np.float16 and sc.shape == (N, K // 128)
    codes = oracle.unpack_u4(packed).reshape(N, K // 128, 128)
    s = sc.astype(np.float64)
    # the stored scale is never below the exact range / 15
    wg = w.T.reshape(N, K // 128, 128).astype(np.float64)
    rng15 = (wg.max(axis=2) - wg.min(axis=2)) / 15
    assert np.all(s >= rng15 * (1 - 2.0 ** -23))
    assert np.all((zz >= 0) & (zz <= 15)) and np.all(zz == np.rint(zz))
    assert zz.min() > 0 and zz.max() < 15        # z never clamps on N(0, 0.02)
    # q = 0 at the group minimum, top code 14 or 15
    assert np.all(codes.min(axis=2) == 0)
    assert np.all(codes.max(axis=2) >= 14)
    w_hat = (codes - zz.astype(np.float64)[:, :, None]) * s[:, :, None]
    err = np.abs(wg - w_hat)
    assert np.all(err <= s[:, :, None] * (0.5 + 2.0 ** -18))
    deq = oracle.dequant_u4_g128(packed, sc, zz)
    assert np.array_equal(deq, w_hat.reshape(N, K).T)


def test_f16_round_up():
    t = np.array([2.0 ** -6, 0.1, 1.0 + 2.0 ** -12, 3e-8, 0.0, 65504.0], np.float32)
    h = oracle.f16_round_up(t)
    for ti, hi in zip(t, h):
        assert float(hi) == float(f16_up(frac(ti)))
        assert float(hi) >= float(ti)
    assert float(h[0]) == 2.0 ** -6


def test_pack_order_golden():
    for codes, words in _rows("pack_order.txt"):
        c = np.array([[int(v) for v in codes]], np.uint8)
        p = oracle.pack_u4(c)
        assert [f"{int(v) & 0xffffffff:08x}" for v in p[0]] == words
        assert np.array_equal(oracle.unpack_u4(p), c)


def test_pack_unpack_round_trip():
    rng = np.random.default_rng(1)
    c = rng.integers(0, 16, (7, 256), dtype=np.uint8)
    assert np.array_equal(oracle.unpack_u4(oracle.pack_u4(c)), c)


def test_u4_rejects_partial_groups():
    with pytest.raises(ValueError):
        oracle.quantize_weight_u4_g128(np.zeros((100, 4), np.float32))
