"""The Python binding refuses operands the kernels would index out of bounds:
an `out=` tensor on the host or of the wrong shape, and scale, zero-point or
record tensors whose shapes disagree with M, N and K/128.  Every check fires
before the library is called, so nothing is launched."""
import pytest
import torch

import bit_quantized_gemm_int8_amd as qg

pytestmark = pytest.mark.gpu
D = "cuda"


def _w8():
    xq = torch.zeros((4, 256), dtype=torch.int8, device=D)
    xs = torch.ones((4,), dtype=torch.float32, device=D)
    wq = torch.zeros((32, 256), dtype=torch.int8, device=D)
    ws = torch.ones((32,), dtype=torch.float32, device=D)
    return xq, xs, wq, ws


def _w4(N=32, K=256):
    wq = torch.zeros((N, K // 8), dtype=torch.int32, device=D)
    sc = torch.ones((N, K // 128), dtype=torch.float16, device=D)
    zz = torch.zeros((N, K // 128), dtype=torch.float16, device=D)
    return wq, sc, zz


def test_host_out_refused():
    xq, xs, wq, ws = _w8()
    with pytest.raises(ValueError):
        qg.gemm_w8a8(xq, xs, wq, ws, out_dtype=torch.float32,
                     out=torch.empty((4, 32), dtype=torch.float32))
    x = torch.zeros((4, 256), dtype=torch.bfloat16, device=D)
    with pytest.raises(ValueError):
        qg.quantize_per_token_i8(x, out=(torch.empty((4, 256), dtype=torch.int8),
                                         torch.empty((4,), dtype=torch.float32, device=D)))
    with pytest.raises(ValueError):
        qg.quantize_gemm_w8a8(x, wq, ws, out_dtype=torch.float32,
                              xq_out=(torch.empty((4, 256), dtype=torch.int8, device=D),
                                      torch.empty((4,), dtype=torch.float32)))


def test_misshaped_scales_refused():
    xq, xs, wq, ws = _w8()
    with pytest.raises(ValueError):
        qg.gemm_w8a8(xq, xs[:3].contiguous(), wq, ws)
    with pytest.raises(ValueError):
        qg.gemm_w8a8(xq, xs, wq, torch.ones((31,), dtype=torch.float32, device=D))
    with pytest.raises(ValueError):
        qg.gemm_w8a8(xq, xs, wq[:, :128].contiguous(), ws)            # K disagrees
    x = torch.zeros((4, 256), dtype=torch.bfloat16, device=D)
    with pytest.raises(ValueError):
        qg.quantize_gemm_w8a8(x, wq, torch.ones((16,), dtype=torch.float32, device=D))
    p4, s4, z4 = _w4()
    with pytest.raises(ValueError):
        qg.gemm_w4a8_g128(xq, xs, p4, s4[:, :1].contiguous(), z4)
    with pytest.raises(ValueError):
        qg.gemm_w4a8_g128(xq, xs, p4, s4, z4[:16].contiguous())
    with pytest.raises(ValueError):
        qg.gemm_w4a8_g128(xq, torch.ones((5,), dtype=torch.float32, device=D), p4, s4, z4)
    xh = torch.zeros((4, 256), dtype=torch.float16, device=D)
    with pytest.raises(ValueError):
        qg.gemm_w4a16_g128(xh, p4, s4.reshape(64, 1).contiguous()[:32].contiguous(), z4)
    rec = torch.zeros((32, 2), dtype=torch.int64, device=D)
    s8 = torch.ones((32,), dtype=torch.float32, device=D)
    with pytest.raises(ValueError):
        qg.gemm_w4a8_g128_outliers(xq, xs, p4, s4, z4, rec, s8[:8].contiguous())
    with pytest.raises(ValueError):
        qg.gemm_w4a8_g128_outliers(xq, xs, p4, s4, z4, rec[:, :1].contiguous(), s8)
    wsp = torch.zeros((2, 2, 16, 12), dtype=torch.int32, device=D)
    with pytest.raises(ValueError):
        qg.gemm_w4a8_g128_sparse24(xq, xs, wsp, s4[:, :1].contiguous(), z4)
    kq = torch.zeros((200, 2, 64), dtype=torch.int8, device=D)
    with pytest.raises(ValueError):
        qg.dequantize_kv_i8_segments(kq, torch.ones((2, 1, 64), dtype=torch.float32, device=D))


def test_well_formed_calls_still_run():
    xq, xs, wq, ws = _w8()
    y = qg.gemm_w8a8(xq, xs, wq, ws, out_dtype=torch.float32)
    p4, s4, z4 = _w4()
    y4 = qg.gemm_w4a8_g128(xq, xs, p4, s4, z4, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert not y.any() and not y4.any()
