"""The allocation-free quantize + W4A8 entry point against the one that takes
a workspace: codes, scales, int32 group accumulators and scaled outputs bit
for bit (the same kernels run on the library's own panel array), on two
calls in a row, the second with a smaller input, and the accumulators
against the oracle."""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_int8_amd as qg
import oracle
from tests.gpu_util import to_dev, to_np

pytestmark = pytest.mark.gpu


def _case(M, N, K, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    packed, sc, zz = oracle.quantize_weight_u4_g128(w)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = (torch.randn((M, K), generator=g, device="cuda") * 2.0).to(torch.bfloat16)
    return x, packed, sc, zz


def _bits(t):
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t


def test_noalloc_matches_workspace_entry_point():
    # second call smaller: fewer rows, shorter K, narrower N (both on the
    # panel pair: 257-383 weight blocks)
    for M, N, K, seed in ((16, 6128, 4096, 1), (3, 4160, 2048, 2)):
        x, packed, sc, zz = _case(M, N, K, seed)
        wq, s_d, z_d = to_dev(packed), to_dev(sc), to_dev(zz)
        assert qg.quantize_gemm_w4a8_g128_workspace_bytes(M, N, K) > 0   # the panel pair runs
        print(f"noalloc M={M} N={N} K={K}", flush=True)
        for ydt in (torch.int32, torch.bfloat16):
            w_scale = None if ydt == torch.int32 else s_d
            y, xq, xs = qg.quantize_gemm_w4a8_g128_noalloc(x, wq, w_scale, z_d, out_dtype=ydt)
            y2, xq2, xs2 = qg.quantize_gemm_w4a8_g128(x, wq, w_scale, z_d, out_dtype=ydt)
            torch.cuda.synchronize()
            assert torch.equal(xq, xq2) and torch.equal(xs, xs2)
            assert torch.equal(_bits(y), _bits(y2))
            if ydt == torch.int32:
                np.testing.assert_array_equal(to_np(y),
                                              oracle.gemm_w4a8_g128_acc(to_np(xq), packed, zz))


def test_noalloc_two_kernel_shapes():
    """Where the plain kernels run (17 rows) no array is used; same results."""
    M, N, K = 17, 256, 1024
    x, packed, sc, zz = _case(M, N, K, 3)
    wq, z_d = to_dev(packed), to_dev(zz)
    y, xq, xs = qg.quantize_gemm_w4a8_g128_noalloc(x, wq, None, z_d, out_dtype=torch.int32)
    y2, xq2, xs2 = qg.quantize_gemm_w4a8_g128(x, wq, None, z_d, out_dtype=torch.int32)
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(xq, xq2) and torch.equal(xs, xs2)
