"""GPU parity of the 2:4 sparse W4A8 path (「LLM推理降本五要素」 §3.2) against the
oracle: the sparse weight words, scale and zero bits bit for bit; per-group
int32 accumulators of the sparse matrix-core product bit for bit; scaled
outputs within the W4A8 tolerance."""
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


def _w(seed, K, N):
    return (np.random.default_rng(seed).standard_normal((K, N)) * 0.02).astype(np.float32)


def _check_quant(w):
    K, N = w.shape
    print(f"sparse24 quant K={K} N={N}", flush=True)
    dev = qg.quantize_weight_u4_g128_sparse24(to_dev(w))
    torch.cuda.synchronize()
    ref = oracle.quantize_weight_u4_g128_sparse24(w)
    np.testing.assert_array_equal(to_np(dev[1]).view(np.uint16), ref[1].view(np.uint16))
    np.testing.assert_array_equal(to_np(dev[2]).view(np.uint16), ref[2].view(np.uint16))
    np.testing.assert_array_equal(to_np(dev[0]), ref[0])
    return dev, ref


@pytest.mark.parametrize("K,N", [(128, 2), (256, 37), (1024, 64)])
def test_quant_parity(K, N):
    _check_quant(_w(K + N, K, N))


def test_quant_golden_and_ties():
    P = {0: [1, -3, 2, 0], 1: [0, 0, 5, -5], 2: [2, -2, 2, 1]}
    a = [0.01 * P[(k // 4) % 3][k % 4] for k in range(128)]
    b = [0.01 * [-5, -4, 3, 0][k % 4] for k in range(128)]
    c = [0.0] * 128                                             # all zero: s = z = q = 0
    rng = np.random.default_rng(1)
    d = list(np.rint(rng.standard_normal(128) * 2) * 0.01)      # coarse grid: many ties
    w = np.array([a, b, c, d]).T.astype(np.float32)
    dev, _ = _check_quant(w)
    words = to_np(dev[0]).view(np.uint32)
    assert [hex(v) for v in words[0, 0, 0, :3]] == ["0xa03e4aa3", "0x4eaa03e", "0xe94e94e9"]


def test_quant_full_size():
    _check_quant(draw(by_name("w4a8_ffn_down"))["w"])


def _codes(rng, shape):
    return rng.integers(-127, 128, shape).astype(np.int8)


SHAPES = [(1, 16, 128), (3, 33, 384), (16, 64, 1024), (17, 40, 640), (40, 48, 256),
          (5, 100, 2048), (16, 4096, 11008), (64, 24, 512)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_acc_bitwise(M, N, K):
    w = _w(M + N + K, K, N)
    rng = np.random.default_rng(K + 5 * M)
    xq = _codes(rng, (M, K))
    p, s, z = oracle.quantize_weight_u4_g128_sparse24(w)
    print(f"sparse24 gemm acc M={M} N={N} K={K}", flush=True)
    acc = qg.gemm_w4a8_g128_sparse24(to_dev(xq), None, to_dev(p), None, to_dev(z),
                                     out_dtype=torch.int32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(acc), oracle.gemm_w4a8_g128_sparse24_acc(xq, p, z))


def test_gemm_acc_extremes():
    """Full-range codes and activations: |x (q - z)| up to 127 * 15 per term."""
    K, N, M = 512, 32, 16
    rng = np.random.default_rng(2)
    w = (rng.integers(0, 2, (K, N)) * 2 - 1).astype(np.float32) * rng.random((K, N)).astype(np.float32)
    xq = np.where(rng.random((M, K)) < 0.5, -127, 127).astype(np.int8)
    p, s, z = oracle.quantize_weight_u4_g128_sparse24(w)
    acc = qg.gemm_w4a8_g128_sparse24(to_dev(xq), None, to_dev(p), None, to_dev(z),
                                     out_dtype=torch.int32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(acc), oracle.gemm_w4a8_g128_sparse24_acc(xq, p, z))


def _floor(xq, sx, p, s, z):
    acc = oracle.gemm_w4a8_g128_sparse24_acc(xq, p, z).astype(np.float64)
    sg = s.astype(np.float64).T
    B = np.abs(sx.astype(np.float64))[:, None] * np.abs(acc * sg[None]).sum(axis=1)
    return (acc.shape[1] + 10) * 2.0 ** -24 * B


@pytest.mark.parametrize("fmt", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (3, 33, 384), (17, 40, 640), (16, 4096, 11008)])
def test_gemm_scaled(fmt, M, N, K):
    w = _w(7 * M + N + K, K, N)
    rng = np.random.default_rng(N + 3 * K)
    xq = _codes(rng, (M, K))
    sx = (rng.random(M) * 0.05 + 1e-3).astype(np.float32)
    p, s, z = oracle.quantize_weight_u4_g128_sparse24(w)
    y = qg.gemm_w4a8_g128_sparse24(to_dev(xq), to_dev(sx), to_dev(p), to_dev(s), to_dev(z),
                                   out_dtype=TORCH_OUT[fmt])
    yref = oracle.gemm_w4a8_g128_sparse24(xq, sx, p, s, z)
    n = assert_close(out_f64(y), yref, fmt, floor=_floor(xq, sx, p, s, z),
                     what=f"w4a8 2:4 {fmt}")
    print(f"w4a8 2:4 {fmt} {M}x{N}x{K}: {n} of {yref.size} outputs within the floor only")


def test_workload_end_to_end():
    wl = by_name("w4a8_ffn_down")
    d = draw(wl)
    dev, ref = _check_quant(d["w"])
    x16 = torch.from_numpy(d["x"]).to("cuda").to(torch.bfloat16)
    xq, sx = qg.quantize_per_token_i8(x16)
    y = qg.gemm_w4a8_g128_sparse24(xq, sx, *dev, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    xq_ref, sx_ref = oracle.quantize_per_token_i8(oracle.to_f32(to_np(x16), "bf16"))
    np.testing.assert_array_equal(to_np(xq), xq_ref)
    yref = oracle.gemm_w4a8_g128_sparse24(xq_ref, sx_ref, *ref)
    assert_close(out_f64(y), yref, "bf16", floor=_floor(xq_ref, sx_ref, *ref), what="ffn_down 2:4")


def test_graph_replay():
    w = _w(5, 1024, 1040)
    rng = np.random.default_rng(9)
    xq = to_dev(_codes(rng, (8, 1024)))
    sx = to_dev((rng.random(8) * 0.05 + 1e-3).astype(np.float32))
    dev = qg.quantize_weight_u4_g128_sparse24(to_dev(w))
    y = qg.gemm_w4a8_g128_sparse24(xq, sx, *dev, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qg.gemm_w4a8_g128_sparse24(xq, sx, *dev, out_dtype=torch.bfloat16, out=y)
    for _ in range(3):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16))
