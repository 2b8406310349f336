"""GPU parity of W4A8 with the INT8 outlier side path (「LLM推理降本五要素」 §2.2)
against the oracle: codes, scale and zero bits, outlier records and INT8
scales bit for bit; per-group and side int32 accumulators bit for bit; scaled
outputs within the W4A8 tolerance (one ulp, or the cancellation floor of the
binary32 group sums, two more roundings for the side term)."""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_int8_amd as qg
import oracle
from tests.gpu_util import to_dev, to_np, out_f64
from tests.tolerance import assert_close
from workloads import by_name, draw

pytestmark = pytest.mark.gpu

TORCH_OUT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _weights(seed, K, N, spikes=True):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((K, N)) * 0.02
    if spikes:
        mask = rng.random((K, N)) < 0.01
        w[mask] *= 8.0
    return w.astype(np.float32)


def _check_quant(w):
    K, N = w.shape
    print(f"outlier quant K={K} N={N}", flush=True)
    wq, sc, zz, rec, s8 = qg.quantize_weight_u4_g128_outliers(to_dev(w))
    torch.cuda.synchronize()
    p_ref, s_ref, z_ref, r_ref, s8_ref = oracle.quantize_weight_u4_g128_outliers(w)
    np.testing.assert_array_equal(to_np(rec).view(np.uint64), r_ref)
    np.testing.assert_array_equal(to_np(s8), s8_ref)
    np.testing.assert_array_equal(to_np(sc).view(np.uint16), s_ref.view(np.uint16))
    np.testing.assert_array_equal(to_np(zz).view(np.uint16), z_ref.view(np.uint16))
    np.testing.assert_array_equal(to_np(wq), p_ref)
    return (wq, sc, zz, rec, s8), (p_ref, s_ref, z_ref, r_ref, s8_ref)


@pytest.mark.parametrize("K,N", [(128, 2), (512, 37), (384, 64), (2048, 100)])
def test_quant_parity(K, N):
    _check_quant(_weights(K + N, K, N))


def test_quant_golden_fixture():
    k = np.arange(128)
    a = (0.01 * ((k % 16) - 8)).astype(np.float64)
    a[5], a[77], a[100] = 1.27, -0.5, 0.3
    b = (0.001 * ((k % 8) - 4)).astype(np.float64)
    b[3], b[40], b[90], b[120] = 0.5, -0.5, 0.5, -0.5
    w = np.stack([a, b], axis=1).astype(np.float32)
    dev, _ = _check_quant(w)
    rec = to_np(dev[3]).view(np.uint64)
    assert int(rec[0, 0]) == 0xFFFF641E4DCE057F and int(rec[1, 0]) == 0xFFFF5A7F2881037F


def test_quant_ties_and_degenerate_groups():
    rng = np.random.default_rng(3)
    K, N = 512, 24
    # a coarse grid makes equal magnitudes common: ties must go to the lower index
    w = (np.rint(rng.standard_normal((K, N)) * 2) * 0.01).astype(np.float32)
    w[:, 0] = 0.0                                    # all-zero column: s = z = q = 0, s8 = 0
    w[:, 1] = 0.0
    w[[3, 70, 100], 1] = [0.5, -0.25, 0.125]         # group 0 of column 1: three nonzeros only
    w[128 + 7, 2] = 4.0                              # one large spike
    _check_quant(w)


def test_quant_full_size():
    wl = by_name("w4a8_ffn_down")
    _check_quant(draw(wl)["w"])


def _codes(rng, shape):
    return rng.integers(-127, 128, shape).astype(np.int8)


SHAPES = [(1, 16, 128), (3, 33, 384), (16, 64, 1024), (17, 40, 640), (40, 48, 256),
          (5, 100, 2048), (16, 4096, 11008)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_acc_bitwise(M, N, K):
    w = _weights(M + N + K, K, N)
    rng = np.random.default_rng(K + 7 * M)
    xq = _codes(rng, (M, K))
    p, s, z, r, s8 = oracle.quantize_weight_u4_g128_outliers(w)
    print(f"outlier gemm acc M={M} N={N} K={K}", flush=True)
    acc = qg.gemm_w4a8_g128_outliers(to_dev(xq), None, to_dev(p), None, to_dev(z),
                                     to_dev(r.view(np.int64)), None, out_dtype=torch.int32)
    torch.cuda.synchronize()
    got = to_np(acc)
    G = K // 128
    np.testing.assert_array_equal(got[:, :G, :], oracle.gemm_w4a8_g128_acc(xq, p, z))
    np.testing.assert_array_equal(got[:, G, :], oracle.gemm_w4a8_g128_outlier_acc(xq, r))


def _floor(xq, sx, p, s, z, r, s8):
    acc = oracle.gemm_w4a8_g128_acc(xq, p, z).astype(np.float64)               # [M, G, N]
    sg = s.astype(np.float64).T
    side = oracle.gemm_w4a8_g128_outlier_acc(xq, r).astype(np.float64) * s8.astype(np.float64)
    B = np.abs(sx.astype(np.float64))[:, None] * (np.abs(acc * sg[None]).sum(axis=1) + np.abs(side))
    G = acc.shape[1]
    return (G + 12) * 2.0 ** -24 * B


@pytest.mark.parametrize("fmt", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (3, 33, 384), (17, 40, 640), (16, 4096, 11008)])
def test_gemm_scaled(fmt, M, N, K):
    w = _weights(M * 3 + N + K, K, N)
    rng = np.random.default_rng(N + K)
    xq = _codes(rng, (M, K))
    sx = (rng.random(M) * 0.05 + 1e-3).astype(np.float32)
    p, s, z, r, s8 = oracle.quantize_weight_u4_g128_outliers(w)
    y = qg.gemm_w4a8_g128_outliers(to_dev(xq), to_dev(sx), to_dev(p), to_dev(s), to_dev(z),
                                   to_dev(r.view(np.int64)), to_dev(s8), out_dtype=TORCH_OUT[fmt])
    yref = oracle.gemm_w4a8_g128_outliers(xq, sx, p, s, z, r, s8)
    n = assert_close(out_f64(y), yref, fmt, floor=_floor(xq, sx, p, s, z, r, s8),
                     what=f"w4a8 outliers {fmt}")
    print(f"w4a8 outliers {fmt} {M}x{N}x{K}: {n} of {yref.size} outputs within the floor only")


def test_workload_end_to_end():
    """The FFN-down workload through the library only: GPU weight quantization,
    GPU activation quantization, fused GEMM; every intermediate against the
    oracle."""
    wl = by_name("w4a8_ffn_down")
    d = draw(wl)
    dev, ref = _check_quant(d["w"])
    x16 = torch.from_numpy(d["x"]).to("cuda").to(torch.bfloat16)
    xq, sx = qg.quantize_per_token_i8(x16)
    y = qg.gemm_w4a8_g128_outliers(xq, sx, *dev, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    xq_ref, sx_ref = oracle.quantize_per_token_i8(oracle.to_f32(to_np(x16), "bf16"))
    np.testing.assert_array_equal(to_np(xq), xq_ref)
    yref = oracle.gemm_w4a8_g128_outliers(xq_ref, sx_ref, *ref)
    assert_close(out_f64(y), yref, "bf16", floor=_floor(xq_ref, sx_ref, *ref), what="ffn_down")
    # the side path matters: without it the output moves by far more than the tolerance
    y_plain = oracle.gemm_w4a8_g128(xq_ref, sx_ref, ref[0], ref[1], ref[2])
    assert np.abs(y_plain - yref).max() > 0.01 * np.abs(yref).max()


def test_graph_replay():
    w = _weights(5, 1024, 1040)
    rng = np.random.default_rng(9)
    xq = to_dev(_codes(rng, (8, 1024)))
    sx = to_dev((rng.random(8) * 0.05 + 1e-3).astype(np.float32))
    dev = qg.quantize_weight_u4_g128_outliers(to_dev(w))
    y = qg.gemm_w4a8_g128_outliers(xq, sx, *dev, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qg.gemm_w4a8_g128_outliers(xq, sx, *dev, out_dtype=torch.bfloat16, out=y)
    for _ in range(3):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16))


# the panel form: the same accumulators (and side sum) bit for bit, from the
# token panel of quantize_per_token_i8_panel
PANEL_SHAPES = [(1, 16, 128), (3, 33, 384), (16, 64, 1024), (5, 100, 2048), (16, 4096, 11008),
                (2, 4100, 4096), (8, 40, 16384), (1, 12288, 4096)]


@pytest.mark.parametrize("M,N,K", PANEL_SHAPES)
def test_panel_gemm_acc_bitwise(M, N, K):
    w = _weights(M + N + K + 1, K, N)
    p, s, z, r, s8 = oracle.quantize_weight_u4_g128_outliers(w)
    g = torch.Generator(device="cuda")
    g.manual_seed(M * 7 + K)
    x = (torch.randn((M, K), generator=g, device="cuda") * 3).to(torch.bfloat16)
    print(f"outlier panel gemm acc M={M} N={N} K={K}", flush=True)
    panel, xq, xs = qg.quantize_per_token_i8_panel(x)
    acc = qg.gemm_w4a8_g128_outliers_panel(panel, None, to_dev(p), None, to_dev(z),
                                           to_dev(r.view(np.int64)), None, M,
                                           out_dtype=torch.int32)
    acc2 = qg.gemm_w4a8_g128_outliers(xq, None, to_dev(p), None, to_dev(z),
                                      to_dev(r.view(np.int64)), None, out_dtype=torch.int32)
    torch.cuda.synchronize()
    assert torch.equal(acc, acc2)
    if M * N * K <= 16 * 4096 * 4096:
        got, xq_np = to_np(acc), to_np(xq)
        G = K // 128
        np.testing.assert_array_equal(got[:, :G, :], oracle.gemm_w4a8_g128_acc(xq_np, p, z))
        np.testing.assert_array_equal(got[:, G, :], oracle.gemm_w4a8_g128_outlier_acc(xq_np, r))


@pytest.mark.parametrize("fmt", ["bf16", "f32"])
@pytest.mark.parametrize("M,N,K", [(3, 33, 384), (16, 4096, 11008)])
def test_panel_gemm_scaled(fmt, M, N, K):
    w = _weights(M + 2 * N + K, K, N)
    p, s, z, r, s8 = oracle.quantize_weight_u4_g128_outliers(w)
    g = torch.Generator(device="cuda")
    g.manual_seed(M + K)
    x = (torch.randn((M, K), generator=g, device="cuda") * 3).to(torch.bfloat16)
    print(f"outlier panel gemm scaled M={M} N={N} K={K} {fmt}", flush=True)
    panel, xq, xs = qg.quantize_per_token_i8_panel(x)
    out = {"bf16": torch.bfloat16, "f32": torch.float32}[fmt]
    y = qg.gemm_w4a8_g128_outliers_panel(panel, xs, to_dev(p), to_dev(s), to_dev(z),
                                         to_dev(r.view(np.int64)), to_dev(s8), M, out_dtype=out)
    torch.cuda.synchronize()
    xq_np, xs_np = to_np(xq), to_np(xs)
    yref = oracle.gemm_w4a8_g128_outliers(xq_np, xs_np, p, s, z, r, s8)
    assert_close(out_f64(y), yref, fmt, floor=_floor(xq_np, xs_np, p, s, z, r, s8),
                 what=f"outlier panel {fmt}")
