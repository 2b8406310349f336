"""GPU parity of every symmetric int8 quantizer on inputs whose scale is
subnormal in binary32 (max|x| below 127 * 2^-126): per-token activations,
per-channel weights, the fused quantize + W8A8 call, the KV-cache segments
and the INT8 outlier side store.  There the scale carries fewer significant
bits, so max|x| / s can pass 127.5 and the clamp to [-127, 127] binds; below
127 * 2^-128 the reciprocal of s overflows and every code comes from the
division; below 63.5 * 2^-149 the scale itself underflows to 0 and the codes
are 0.  Codes and scales must equal the oracle's bit for bit
(「第4章：量化」 §1.1-1.2; 「LLM推理降本五要素」 §5.2: round, then clamp)."""
import os

import numpy as np
import pytest
import torch

import bit_quantized_gemm_int8_amd as qg
import oracle
from tests.gpu_util import to_dev, to_np
from workloads import f32_to_bf16_bits

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")
U = 2.0 ** -149          # smallest binary32 subnormal

# max|x| in units of U: scale underflows (<= 63), subnormal scale with the
# clamp binding (128-190, 256-317, 383-444), subnormal scale without it,
# infinite reciprocal up to 127 * 2^21, finite reciprocal above, normal scale
AMAX_UNITS = [1, 2, 63, 64, 127, 150, 190, 191, 300, 316, 400, 444, 1000, 12345, 2 ** 20,
              127 * 2 ** 21, 127 * 2 ** 21 + 12345, 2 ** 23 + 1, 127 * 2 ** 23 + 5]


def _rows(n_per, K, seed):
    """[len(AMAX_UNITS) * n_per, K] float32 rows, row i with max|x| exactly
    AMAX_UNITS[i // n_per] units, integer multiples of U (all exact)."""
    rng = np.random.default_rng(seed)
    rows = []
    for k in AMAX_UNITS:
        for _ in range(n_per):
            v = rng.integers(-k, k + 1, K).astype(np.float64)
            v[rng.integers(0, K)] = k * rng.choice([-1, 1])
            rows.append(v * U)
    return np.array(rows).astype(np.float32)


def _act(x32, fmt):
    if fmt == "f32":
        return to_dev(x32), x32
    b = f32_to_bf16_bits(x32)
    return to_dev(b, "bf16"), oracle.to_f32(b, "bf16")


def _golden():
    out = []
    for line in open(os.path.join(GOLD, "per_token_subnormal.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            su, vals, codes = [p.split() for p in line.split("|")]
            out.append((int(su[0]), [int(v) for v in vals], [int(c) for c in codes]))
    return out


def test_per_token_golden_subnormal():
    for su, vals, codes in _golden():
        x = np.zeros((1, 16), np.float32)
        x[0, : len(vals)] = np.array(vals, np.float64) * U
        print(f"per-token golden s={su}u {vals}", flush=True)
        xq, xs = qg.quantize_per_token_i8(to_dev(x))
        torch.cuda.synchronize()
        assert float(to_np(xs)[0]) == su * U
        assert to_np(xq)[0, : len(vals)].tolist() == codes


@pytest.mark.parametrize("fmt", ["f32", "bf16"])
@pytest.mark.parametrize("K", [48, 4096, 11008, 20000])
def test_per_token_subnormal(fmt, K):
    x = _rows(2, K, seed=K)
    xd, xo = _act(x, fmt)
    print(f"per-token subnormal M={x.shape[0]} K={K} {fmt}", flush=True)
    xq, xs = qg.quantize_per_token_i8(xd)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_per_token_i8(xo)
    np.testing.assert_array_equal(to_np(xs), s_ref)
    np.testing.assert_array_equal(to_np(xq), q_ref)
    if fmt == "f32":   # the clamp binds on the rows built for it
        assert np.sum(np.abs(xo) / np.where(s_ref > 0, s_ref, 1)[:, None] > 127.5) > 0


@pytest.mark.parametrize("fmt", ["f32", "bf16"])
@pytest.mark.parametrize("K", [48, 4096])
def test_per_token_subnormal_many_rows(fmt, K):
    """The same rows, repeated past 1024 of them: the one-wave-per-row form."""
    x = np.tile(_rows(2, K, seed=K + 1), (28, 1))
    xd, xo = _act(x, fmt)
    print(f"per-token subnormal many rows M={x.shape[0]} K={K} {fmt}", flush=True)
    xq, xs = qg.quantize_per_token_i8(xd)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_per_token_i8(xo)
    np.testing.assert_array_equal(to_np(xs), s_ref)
    np.testing.assert_array_equal(to_np(xq), q_ref)


@pytest.mark.parametrize("K", [64, 4096])
def test_weight_i8_subnormal(K):
    w = _rows(2, K, seed=K).T.copy()              # [K, N]: one subnormal case per column
    print(f"weight i8 subnormal K={K} N={w.shape[1]}", flush=True)
    wq, ws = qg.quantize_weight_i8_per_channel(to_dev(w))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_weight_i8_per_channel(w)
    np.testing.assert_array_equal(to_np(ws), s_ref)
    np.testing.assert_array_equal(to_np(wq), q_ref)


@pytest.mark.parametrize("fuse", [True, False])
@pytest.mark.parametrize("fmt", ["f32", "bf16"])
@pytest.mark.parametrize("M0,K,N", [(1, 512, 64), (2, 4096, 11008), (4, 768, 100)])
def test_fused_w8a8_subnormal(fuse, fmt, M0, K, N):
    """Quantize + W8A8 in one call (the fused kernel where it covers the
    shape, the two kernels otherwise): codes, scales and int32 accumulators."""
    x_all = _rows(1, K, seed=3 * K + N)
    rng = np.random.default_rng(K)
    wq = to_dev(rng.integers(-127, 128, (N, K)).astype(np.int8))
    for r0 in range(0, x_all.shape[0], M0):
        x = x_all[r0:r0 + M0]
        xd, xo = _act(x, fmt)
        print(f"fused subnormal rows {r0}..{r0 + x.shape[0]} K={K} N={N} {fmt} fuse={fuse}",
              flush=True)
        y, xq, xs = qg.quantize_gemm_w8a8(xd, wq, None, out_dtype=torch.int32, fuse=fuse)
        torch.cuda.synchronize()
        q_ref, s_ref = oracle.quantize_per_token_i8(xo)
        np.testing.assert_array_equal(to_np(xs), s_ref)
        np.testing.assert_array_equal(to_np(xq), q_ref)
        acc = oracle.gemm_w8a8_acc(q_ref, to_np(wq))
        np.testing.assert_array_equal(to_np(y).astype(np.int64), acc)


@pytest.mark.parametrize("fmt", ["f32", "bf16"])
def test_kv_subnormal(fmt):
    """Each (head, channel) of each segment gets its own max|x| from the
    subnormal range; T = 300 gives two whole segments and a ragged one."""
    T, H, D = 300, 2, len(AMAX_UNITS) - len(AMAX_UNITS) % 16 + 16
    rng = np.random.default_rng(5)
    kv = np.zeros((T, H, D), np.float64)
    for h in range(H):
        for d in range(D):
            k = AMAX_UNITS[(d + 7 * h) % len(AMAX_UNITS)]
            for s0 in range(0, T, 128):
                t1 = min(T, s0 + 128)
                v = rng.integers(-k, k + 1, t1 - s0).astype(np.float64)
                v[rng.integers(0, t1 - s0)] = k * rng.choice([-1, 1])
                kv[s0:t1, h, d] = v
    kv = (kv * U).astype(np.float32)
    kd, ko = _act(kv.reshape(T, -1), fmt)
    kd = kd.view(T, H, D)
    ko = ko.reshape(T, H, D)
    print(f"kv subnormal T,H,D={T},{H},{D} {fmt}", flush=True)
    kq, ks = qg.quantize_kv_i8_segments(kd)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_kv_segments(ko)
    np.testing.assert_array_equal(to_np(ks), s_ref)
    np.testing.assert_array_equal(to_np(kq), q_ref)


def test_outlier_side_store_subnormal():
    """Columns whose outliers are subnormal: the side store's s8 and codes
    (the clamp binds on some), with the uint4 part of the same columns."""
    K = 256
    w = _rows(1, K, seed=17).T.copy()            # [K, N]
    print(f"outlier subnormal K={K} N={w.shape[1]}", flush=True)
    wq, sc, zz, rec, s8 = qg.quantize_weight_u4_g128_outliers(to_dev(w))
    torch.cuda.synchronize()
    p_ref, s_ref, z_ref, r_ref, s8_ref = oracle.quantize_weight_u4_g128_outliers(w)
    np.testing.assert_array_equal(to_np(s8), s8_ref)
    np.testing.assert_array_equal(to_np(rec).view(np.uint64), r_ref)
    np.testing.assert_array_equal(to_np(sc).view(np.uint16), s_ref.view(np.uint16))
    np.testing.assert_array_equal(to_np(zz).view(np.uint16), z_ref.view(np.uint16))
    np.testing.assert_array_equal(to_np(wq), p_ref)
