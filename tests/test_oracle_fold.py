"""Pins for the oracle smoothing folds (CPU only).

  * the identity X W = (X diag(s)^-1)(diag(s) W) (「第4章：量化」 §2.2,
    「Quantization & Flash Attention」 §2.2) in float64: bit-exact with
    power-of-two s (exact sums via math.fsum), within float64 rounding
    otherwise, for the scales both folds produce;
  * the SmoothQuant closed form at alpha = 0.5: after the fold, on the
    calibration batch the scale was computed from,
    max|X~_j| = max|W~_j| = sqrt(max|X_j| max|W_j|);
  * AWQ: s_c^2 equals mean|X_c| (to rounding), constant columns give
    sqrt(c) exactly; the in-order float64 sum agrees with an exact sum;
  * the elementwise folds are correctly rounded float32 / bf16 / fp16 results.
"""
import math

import numpy as np

import oracle
from tests.exact import frac, fl32
from workloads import by_name, draw


def _fsum_matmul(a, b):
    M, K = a.shape
    _, N = b.shape
    out = np.empty((M, N), np.float64)
    for m in range(M):
        for n in range(N):
            out[m, n] = math.fsum(float(a[m, k]) * float(b[k, n]) for k in range(K))
    return out


def test_identity_bit_exact_power_of_two():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((4, 32))
    w = rng.standard_normal((32, 6)) * 0.02
    s = 2.0 ** rng.integers(-5, 6, 32)
    lhs = _fsum_matmul(x, w)
    rhs = _fsum_matmul(x / s[None, :], s[:, None] * w)
    assert np.array_equal(lhs, rhs)


def test_identity_float64_with_fold_scales():
    wl = by_name("w8a8_decode_ffn_up")
    d = draw(wl, rows=4)
    w = d["w"][:, :64].astype(np.float64)
    for s in (oracle.smoothquant_scales(d["x_cal"], d["w"][:, :64]),
              oracle.awq_scales(d["x_cal"])):
        s = s.astype(np.float64)
        x = d["x"].astype(np.float64)
        lhs = x @ w
        rhs = (x / s[None, :]) @ (s[:, None] * w)
        bound = 4 * wl.K * 2.0 ** -52 * (np.abs(x) @ np.abs(w))
        assert np.all(np.abs(lhs - rhs) <= bound)


def test_smoothquant_closed_form():
    wl = by_name("w8a8_decode_ffn_up")
    d = draw(wl, rows=2)
    x_cal, w = d["x_cal"], d["w"]
    s = oracle.smoothquant_scales(x_cal, w)
    a = np.abs(x_cal).max(axis=0).astype(np.float64)
    b = np.abs(w).max(axis=1).astype(np.float64)
    target = np.sqrt(a * b)
    xt = np.abs(x_cal.astype(np.float64) / s.astype(np.float64)[None, :]).max(axis=0)
    wt = np.abs(s.astype(np.float64)[:, None] * w.astype(np.float64)).max(axis=1)
    assert np.allclose(xt, target, rtol=2.0 ** -21, atol=0)
    assert np.allclose(wt, target, rtol=2.0 ** -21, atol=0)
    # the outlier channels are the ones whose activations shrink the most
    idx = d["outliers"]
    assert s[idx].min() > np.delete(s, idx).max()


def test_smoothquant_scale_rounding_brute_force():
    rng = np.random.default_rng(3)
    x_cal = rng.standard_normal((5, 8)).astype(np.float32)
    w = (rng.standard_normal((8, 3)) * 0.02).astype(np.float32)
    x_cal[:, 7] = 0.0
    s = oracle.smoothquant_scales(x_cal, w)
    for j in range(8):
        a = max(abs(frac(v)) for v in x_cal[:, j])
        b = max(abs(frac(v)) for v in w[j])
        if a == 0:
            assert s[j] == 1.0
            continue
        # float64 sqrt then rounding to float32 equals the correctly rounded
        # float32 sqrt (53 >= 2*24 + 2, so the double rounding is innocuous)
        ra = fl32(frac(math.sqrt(float(a))))
        rb = fl32(frac(math.sqrt(float(b))))
        assert frac(s[j]) == fl32(ra / rb)


def test_awq_scales():
    x = np.ones((16, 4), np.float32)
    x[:, 1] = -4.0
    x[:, 2] = 0.0
    x[::2, 3] = 2.0
    x[1::2, 3] = -0.5
    s = oracle.awq_scales(x)
    assert s[0] == 1.0 and s[1] == 2.0 and s[2] == 1.0
    assert s[3] == np.float32(math.sqrt(1.25))
    wl = by_name("w4a16_qkv")
    d = draw(wl, rows=1)
    s = oracle.awq_scales(d["x_cal"])
    exact_mean = np.array([math.fsum(abs(float(v)) for v in d["x_cal"][:, c]) / 512
                           for c in range(0, wl.K, 97)])
    assert np.allclose(s[::97].astype(np.float64) ** 2, exact_mean, rtol=2.0 ** -21)


def test_fold_elementwise_correctly_rounded():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((3, 10)).astype(np.float32) * 30
    w = rng.standard_normal((10, 4)).astype(np.float32) * 0.02
    s = (rng.random(10) * 3 + 0.1).astype(np.float32)
    wt = oracle.fold_weight(w, s)
    for j in range(10):
        for n in range(4):
            assert frac(wt[j, n]) == fl32(frac(s[j]) * frac(w[j, n]))
    xt = oracle.fold_activation(x, s, "f32")
    for m in range(3):
        for j in range(10):
            assert frac(xt[m, j]) == fl32(frac(x[m, j]) / frac(s[j]))
    xb = oracle.fold_activation(x, s, "bf16")
    back = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    # nearest bf16: within half a bf16 ulp (2^-8 relative) of the fp32 quotient
    assert np.all(np.abs(back - xt) <= np.abs(xt) * 2.0 ** -8)
    xh = oracle.fold_activation(x, s, "f16")
    assert np.array_equal(xh, xt.astype(np.float16))
