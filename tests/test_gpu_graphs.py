"""Captured HIP graphs of the linear layer replay to the eager result.

Every path (activation quantization + GEMM, or the W4A16 GEMM alone) is run
eagerly, then captured into a graph that is replayed several times with other
eager work between the replays; each replay must reproduce the eager output
bit for bit.  This is a property of the GPU path on its own (no oracle): the
kernels keep no state between calls and use no memset nodes.
"""
import pytest
import torch

import bit_quantized_gemm_int8_amd as qg

pytestmark = pytest.mark.gpu

# M values: the decode kernels (1, 8), the wide decode kernel (40) and the
# tiled prefill kernel (300)
CASES = [(path, M) for path in ("w8a8", "w4a8", "w4a16") for M in (1, 8, 40, 300)]


def _layer(path, M, K, N, gen):
    dev = "cuda"
    w = torch.randn((K, N), generator=gen, device=dev) * 0.02
    xdt = torch.float16 if path == "w4a16" else torch.bfloat16
    x = torch.randn((M, K), generator=gen, device=dev).to(xdt)
    if path == "w8a8":
        weights = qg.quantize_weight_i8_per_channel(w)
    else:
        weights = qg.quantize_weight_u4_g128(w)
    xq = torch.empty((M, K), dtype=torch.int8, device=dev)
    xs = torch.empty((M,), dtype=torch.float32, device=dev)
    y = torch.empty((M, N), dtype=xdt, device=dev)

    def step():
        if path == "w4a16":
            qg.gemm_w4a16_g128(x, *weights, out_dtype=y.dtype, out=y)
            return
        qg.quantize_per_token_i8(x, out=(xq, xs))
        if path == "w8a8":
            qg.gemm_w8a8(xq, xs, weights[0], weights[1], out_dtype=y.dtype, out=y)
        else:
            qg.gemm_w4a8_g128(xq, xs, *weights, out_dtype=y.dtype, out=y)

    return step, y


@pytest.mark.parametrize("path,M", CASES)
def test_graph_replay_matches_eager(path, M):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1000 + M)
    K, N = 1024, 1040
    step, y = _layer(path, M, K, N, gen)
    step()
    torch.cuda.synchronize()
    ref = y.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    scratch = torch.randn((512, 512), generator=gen, device="cuda")
    for _ in range(4):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16))
        scratch = scratch @ scratch.t().contiguous() * 1e-3   # unrelated eager work between replays
        torch.cuda.synchronize()
