"""GPU parity of the fused quantize + W8A8 call: it must give the results of
quantize_per_token_i8 followed by gemm_w8a8 bit for bit (codes, scales and
outputs), inside the fused kernel's range and on the two-step fallback, and
the headline decode workload must match the oracle."""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_int8_amd as qg
import oracle
from tests.gpu_util import to_np, out_f64
from tests.tolerance import assert_close
from workloads import by_name, draw

pytestmark = pytest.mark.gpu

XDT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
YDT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32, "i32": torch.int32}


def _bits(t):
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t


def _case(M, N, K, xdt, ydt, seed, fuse=True):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.randn((M, K), generator=g, device="cuda")
    x[:, :3] *= 20.0                                        # a few large channels
    if M > 2:
        x[1] = 0.0                                          # an all-zero token
    x = x.to(XDT[xdt])
    w = torch.randn((K, N), generator=g, device="cuda") * 0.02
    wq, ws = qg.quantize_weight_i8_per_channel(w)
    print(f"fused M={M} N={N} K={K} x={xdt} y={ydt}", flush=True)
    y, xq, xs = qg.quantize_gemm_w8a8(x, wq, ws, out_dtype=YDT[ydt], fuse=fuse)
    xq2, xs2 = qg.quantize_per_token_i8(x)
    y2 = qg.gemm_w8a8(xq2, xs2, wq, ws, out_dtype=YDT[ydt])
    torch.cuda.synchronize()
    assert torch.equal(xs, xs2)
    assert torch.equal(xq, xq2)
    assert torch.equal(_bits(y), _bits(y2))


# inside the fused range (M <= 16, m K <= 32768 with m = M rounded up to a
# power of two), one kernel forced: every MR class, ragged K (units past K,
# a row's chunks split over waves), N tails, and grids of 1, 2 and 4 weight
# blocks per workgroup
@pytest.mark.parametrize("M,N,K", [(1, 16, 16), (1, 11008, 4096), (2, 17, 512), (3, 100, 4112),
                                   (4, 64, 8192), (5, 1040, 2000), (8, 11008, 4096), (8, 40, 4096),
                                   (7, 33, 1024), (8, 4096, 2048), (2, 5136, 1024), (1, 4096, 11008),
                                   (6, 10256, 4096), (9, 64, 1024), (16, 512, 512), (12, 300, 2048),
                                   (16, 11008, 768), (13, 1000, 384)])
@pytest.mark.parametrize("xdt", ["bf16", "f16", "f32"])
def test_fused_matches_two_steps(M, N, K, xdt):
    _case(M, N, K, xdt, "bf16", seed=M * 1000 + N + K)


@pytest.mark.parametrize("ydt", ["f32", "f16", "i32"])
@pytest.mark.parametrize("M", [8, 16])
def test_fused_output_dtypes(ydt, M):
    _case(M, 1040, 1024, "bf16", ydt, seed=5 + M)


# outside it (M > 16, or rows whose codes exceed 4096 chunks), asked to fuse
# or not: the two kernels
@pytest.mark.parametrize("M,N,K,xdt", [(17, 64, 512, "bf16"), (16, 100, 4096, "bf16"),
                                       (8, 64, 8192, "f32"), (16, 64, 2064, "f32"),
                                       (300, 1040, 1024, "bf16")])
@pytest.mark.parametrize("fuse", [True, False])
def test_fallback_matches_two_steps(M, N, K, xdt, fuse):
    _case(M, N, K, xdt, "bf16", seed=M + N + K, fuse=fuse)


# the library's own choice, on both sides of its thresholds
@pytest.mark.parametrize("M,N,K,xdt", [(1, 11008, 4096, "bf16"), (4, 8192, 4096, "bf16"),
                                       (4, 8192, 4080, "bf16"), (8, 11008, 4096, "bf16"),
                                       (2, 64, 512, "bf16"), (16, 512, 512, "f32"),
                                       (9, 4096, 768, "bf16"), (9, 4096, 784, "bf16")])
def test_auto_matches_two_steps(M, N, K, xdt):
    _case(M, N, K, xdt, "bf16", seed=3 * M + N + K, fuse=None)


def test_tiny_workload_fused_against_oracle():
    """The 16 x 512 x 512 fp32 workload, which the library runs fused."""
    wl = by_name("w8a8_tiny")
    d = draw(wl)
    x = torch.from_numpy(d["x"]).to("cuda")
    wq, ws = qg.quantize_weight_i8_per_channel(torch.from_numpy(d["w"]).to("cuda"))
    assert qg.quantize_gemm_w8a8_plan(torch.float32, wl.M, wl.N, wl.K)
    y, xq, xs = qg.quantize_gemm_w8a8(x, wq, ws, out_dtype=torch.float32)
    torch.cuda.synchronize()
    xq_ref, xs_ref = oracle.quantize_per_token_i8(d["x"])
    wq_ref, ws_ref = oracle.quantize_weight_i8_per_channel(d["w"])
    np.testing.assert_array_equal(to_np(xq), xq_ref)
    np.testing.assert_array_equal(to_np(xs), xs_ref)
    np.testing.assert_array_equal(to_np(wq), wq_ref)
    yref = oracle.gemm_w8a8(xq_ref, xs_ref, wq_ref, ws_ref)
    assert_close(out_f64(y), yref, "f32", what="fused tiny")


def test_headline_workload_against_oracle():
    wl = by_name("w8a8_decode_ffn_up")
    d = draw(wl)
    s = oracle.smoothquant_scales(d["x_cal"], d["w"])
    xb = oracle.fold_activation(d["x"], s, "bf16")                    # bf16 bits
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to("cuda")
    wf = oracle.fold_weight(d["w"], s)
    wq, ws = qg.quantize_weight_i8_per_channel(torch.from_numpy(wf).to("cuda"))
    y, xq, xs = qg.quantize_gemm_w8a8(x, wq, ws, out_dtype=torch.bfloat16, fuse=True)
    torch.cuda.synchronize()
    xq_ref, xs_ref = oracle.quantize_per_token_i8(oracle.to_f32(xb, "bf16"))
    wq_ref, ws_ref = oracle.quantize_weight_i8_per_channel(wf)
    np.testing.assert_array_equal(to_np(xq), xq_ref)
    np.testing.assert_array_equal(to_np(xs), xs_ref)
    np.testing.assert_array_equal(to_np(wq), wq_ref)
    yref = oracle.gemm_w8a8(xq_ref, xs_ref, wq_ref, ws_ref)
    assert_close(out_f64(y), yref, "bf16", what="fused headline")


def test_codes_only_when_n_is_zero():
    x = torch.randn((4, 256), device="cuda").to(torch.bfloat16)
    wq = torch.empty((0, 256), dtype=torch.int8, device="cuda")
    y, xq, xs = qg.quantize_gemm_w8a8(x, wq, None)
    xq2, xs2 = qg.quantize_per_token_i8(x)
    torch.cuda.synchronize()
    assert y.shape == (4, 0) and torch.equal(xq, xq2) and torch.equal(xs, xs2)


def test_graph_replay():
    x = torch.randn((8, 4096), device="cuda").to(torch.bfloat16)
    w = torch.randn((4096, 2048), device="cuda") * 0.02
    wq, ws = qg.quantize_weight_i8_per_channel(w)
    y, xq, xs = qg.quantize_gemm_w8a8(x, wq, ws, fuse=True)
    torch.cuda.synchronize()
    ref = y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qg.quantize_gemm_w8a8(x, wq, ws, out=y, xq_out=(xq, xs), fuse=True)
    for _ in range(3):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16))
