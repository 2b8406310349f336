"""GPU parity of the quantizers against the oracle: bit-exact codes, scales and
zero points (all three decide integers in binary32 on both sides)."""
import os

import numpy as np
import pytest
import torch

import bit_quantized_gemm_int8_amd as qg
import oracle
from tests.gpu_util import to_dev, to_np, f16_bits
from workloads import by_name, draw, f32_to_bf16_bits, f32_to_f16

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _act(x32, fmt):
    """Stored activation in `fmt` plus the exact float32 values the oracle sees."""
    if fmt == "f32":
        return to_dev(x32), x32
    if fmt == "bf16":
        b = f32_to_bf16_bits(x32)
        return to_dev(b, "bf16"), oracle.to_f32(b, "bf16")
    h = f32_to_f16(x32)
    return to_dev(h), oracle.to_f32(h, "f16")


def _check_per_token(x32, fmt):
    xd, xo = _act(x32, fmt)
    xq, xs = qg.quantize_per_token_i8(xd)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_per_token_i8(xo)
    np.testing.assert_array_equal(to_np(xs), s_ref)
    np.testing.assert_array_equal(to_np(xq), q_ref)


@pytest.mark.parametrize("fmt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("M,K", [(16, 512), (8, 4096), (16, 11008), (3, 16), (5, 48),
                                 (2, 4112), (7, 12304), (2, 16400), (3, 20000), (4, 16384),
                                 (2, 8208)])
def test_per_token_parity(fmt, M, K):
    rng = np.random.default_rng(M * 100003 + K)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.integers(0, K, 3)] *= 30.0
    if M > 2:
        x[1] = 0.0                                  # all-zero token
    _check_per_token(x, fmt)


# many rows: the one-wave-per-row form (M >= 1024, rows of at most 16 KB),
# ragged K (a row's last kilobyte partly past its end), every input format,
# zero rows and rows with huge and tiny maxima
@pytest.mark.parametrize("fmt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("M,K", [(1024, 4096), (1027, 48), (1500, 1040), (2049, 4112), (1024, 16),
                                 (1030, 8192), (1024, 2064)])
def test_per_token_many_rows(fmt, M, K):
    if fmt == "f32" and K > 4096:
        K = 4096 - 16          # keep rows within 16 KB
    rng = np.random.default_rng(M * 7 + K)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.integers(0, K, 2)] *= 40.0
    x[3] = 0.0                                          # all-zero token
    x[5] *= 1e-30 if fmt == "f32" else 1e-3             # tiny maximum (subnormal scale for f32)
    x[7, -1] = 3e4 if fmt != "bf16" else 3e30           # the maximum in the row's last element
    _check_per_token(x, fmt)


def test_per_token_workload_inputs():
    for name in ("w8a8_tiny", "w4a8_ffn_down"):
        wl = by_name(name)
        d = draw(wl)
        _check_per_token(d["x"], wl.x_dtype)


def test_per_token_prefill_full():
    wl = by_name("w8a8_prefill")
    d = draw(wl)
    _check_per_token(d["x"], "bf16")


def test_per_token_golden_ties():
    rows = []
    for line in open(os.path.join(GOLD, "per_token_ties.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            e, vals, codes = [p.split() for p in line.split("|")]
            rows.append((int(e[0]), [float(v) for v in vals], [int(c) for c in codes]))
    for e, vals, codes in rows:
        K = 16 * ((len(vals) + 15) // 16)
        x = np.zeros((1, K), np.float32)
        x[0, : len(vals)] = np.array(vals) * 2.0 ** e
        for fmt in ("f32", "bf16"):
            xd, _ = _act(x, fmt)
            xq, xs = qg.quantize_per_token_i8(xd)
            torch.cuda.synchronize()
            assert float(to_np(xs)[0]) == 2.0 ** e
            assert to_np(xq)[0, : len(vals)].tolist() == codes


def test_per_token_empty_and_out():
    xd = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    xq, xs = qg.quantize_per_token_i8(xd)
    assert xq.shape == (0, 64) and xs.shape == (0,)


@pytest.mark.parametrize("K,N", [(512, 512), (48, 100), (4096, 11008), (1040, 70)])
def test_weight_i8_parity(K, N):
    rng = np.random.default_rng(K + N)
    w = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    w[:, 0] = 0.0                                   # zero column
    wq, ws = qg.quantize_weight_i8_per_channel(to_dev(w))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_weight_i8_per_channel(w)
    np.testing.assert_array_equal(to_np(ws), s_ref)
    np.testing.assert_array_equal(to_np(wq), q_ref)


@pytest.mark.parametrize("K,N", [(11008, 4096), (4096, 12288), (128, 70), (384, 65)])
def test_weight_u4_parity(K, N):
    rng = np.random.default_rng(K * 7 + N)
    w = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    w[:128, 1] = 0.25                               # constant group
    w[:128, 2] += 0.5                               # z clamps to 0
    w[:128, 3] -= 0.5                               # z clamps to 15
    wq, sc, zz = qg.quantize_weight_u4_g128(to_dev(w))
    torch.cuda.synchronize()
    p_ref, s_ref, z_ref = oracle.quantize_weight_u4_g128(w)
    np.testing.assert_array_equal(f16_bits(sc), s_ref.view(np.uint16))
    np.testing.assert_array_equal(f16_bits(zz), z_ref.view(np.uint16))
    np.testing.assert_array_equal(to_np(wq), p_ref)


def test_weight_u4_golden_groups():
    s = 2.0 ** -6
    cols = []
    for line in open(os.path.join(GOLD, "u4_groups.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            _, listed, _, _ = [p.split() for p in line.split("|")]
            col = np.zeros(128)
            col[: len(listed)] = [float(v) for v in listed]
            cols.append(col * s)
    w = np.stack(cols, axis=1).astype(np.float32)
    wq, sc, zz = qg.quantize_weight_u4_g128(to_dev(w))
    torch.cuda.synchronize()
    p_ref, s_ref, z_ref = oracle.quantize_weight_u4_g128(w)
    np.testing.assert_array_equal(to_np(wq), p_ref)
    np.testing.assert_array_equal(f16_bits(zz), z_ref.view(np.uint16))
    np.testing.assert_array_equal(f16_bits(sc), s_ref.view(np.uint16))
