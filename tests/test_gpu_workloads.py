"""The five workloads end to end on the GPU, stage by stage against the oracle.

Each chain runs the library exactly as the benchmark does (offline fold and
weight quantization, per-token activation quantization, GEMM) at the
workloads' full sizes; every integer / binary32 intermediate must match the
oracle bit for bit, the final outputs within tests/tolerance.py.  For the
4096-token prefill the GEMM output is checked on sampled rows.
"""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_int8_amd as qg
import oracle
from tests.gpu_util import to_dev, to_np, out_f64, f16_bits
from tests.tolerance import assert_close
from tests.test_gpu_gemm import _w4a8_floor, _w4a16_floor
from workloads import WORKLOADS, by_name, draw, f32_to_bf16_bits

pytestmark = pytest.mark.gpu
TORCH_OUT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _fold_both(wl, d):
    """GPU fold and oracle fold; asserts they agree; returns the folded operands."""
    xc, w = d["x_cal"], d["w"]
    fn = qg.smoothquant_fold if wl.fold == "smoothquant" else qg.awq_fold
    s_d, w_d = fn(to_dev(xc), to_dev(w))
    x_d = qg.apply_smoothing(to_dev(d["x"]), s_d, out_dtype=TORCH_OUT[wl.x_dtype])
    torch.cuda.synchronize()
    s = oracle.smoothquant_scales(xc, w) if wl.fold == "smoothquant" else oracle.awq_scales(xc)
    np.testing.assert_array_equal(to_np(s_d), s)
    wt = oracle.fold_weight(w, s)
    np.testing.assert_array_equal(to_np(w_d), wt)
    xt = oracle.fold_activation(d["x"], s, wl.x_dtype)
    np.testing.assert_array_equal(to_np(x_d).view(np.uint16), np.asarray(xt).view(np.uint16))
    return x_d, w_d, oracle.to_f32(xt, wl.x_dtype), wt


def _input(wl, d):
    if wl.fold:
        return _fold_both(wl, d)
    if wl.x_dtype == "bf16":
        b = f32_to_bf16_bits(d["x"])
        return to_dev(b, "bf16"), to_dev(d["w"]), oracle.to_f32(b, "bf16"), d["w"]
    return to_dev(d["x"]), to_dev(d["w"]), d["x"], d["w"]


@pytest.mark.parametrize("name", [w.name for w in WORKLOADS])
def test_workload_chain(name):
    wl = by_name(name)
    d = draw(wl)
    x_d, w_d, x_o, w_o = _input(wl, d)
    out = TORCH_OUT[wl.out_dtype]
    if wl.path == "w8a8":
        xq, xs = qg.quantize_per_token_i8(x_d)
        wq, ws = qg.quantize_weight_i8_per_channel(w_d)
        y = qg.gemm_w8a8(xq, xs, wq, ws, out_dtype=out)
        torch.cuda.synchronize()
        xq_o, xs_o = oracle.quantize_per_token_i8(x_o)
        wq_o, ws_o = oracle.quantize_weight_i8_per_channel(w_o)
        np.testing.assert_array_equal(to_np(xs), xs_o)
        np.testing.assert_array_equal(to_np(xq), xq_o)
        np.testing.assert_array_equal(to_np(ws), ws_o)
        np.testing.assert_array_equal(to_np(wq), wq_o)
        # every output, the prefill's 4096 x 11008 included (float64 BLAS on
        # integer operands: exact)
        yref = oracle.gemm_w8a8(xq_o, xs_o, wq_o, ws_o)
        assert_close(out_f64(y), yref, wl.out_dtype, what=name)
        if wl.M > 64:
            acc = qg.gemm_w8a8(xq, None, wq, None, out_dtype=torch.int32)
            np.testing.assert_array_equal(to_np(acc), oracle.gemm_w8a8_acc(xq_o, wq_o))
    elif wl.path == "w4a8":
        xq, xs = qg.quantize_per_token_i8(x_d)
        wq, sc, zz = qg.quantize_weight_u4_g128(w_d)
        y = qg.gemm_w4a8_g128(xq, xs, wq, sc, zz, out_dtype=out)
        acc = qg.gemm_w4a8_g128(xq, None, wq, None, zz, out_dtype=torch.int32)
        torch.cuda.synchronize()
        xq_o, xs_o = oracle.quantize_per_token_i8(x_o)
        p_o, s_o, z_o = oracle.quantize_weight_u4_g128(w_o)
        np.testing.assert_array_equal(to_np(xq), xq_o)
        np.testing.assert_array_equal(to_np(xs), xs_o)
        np.testing.assert_array_equal(to_np(wq), p_o)
        np.testing.assert_array_equal(f16_bits(sc), s_o.view(np.uint16))
        np.testing.assert_array_equal(f16_bits(zz), z_o.view(np.uint16))
        np.testing.assert_array_equal(to_np(acc), oracle.gemm_w4a8_g128_acc(xq_o, p_o, z_o))
        yref = oracle.gemm_w4a8_g128(xq_o, xs_o, p_o, s_o, z_o)
        assert_close(out_f64(y), yref, wl.out_dtype,
                     floor=_w4a8_floor(xq_o, xs_o, p_o, s_o, z_o), what=name)
    else:
        wq, sc, zz = qg.quantize_weight_u4_g128(w_d)
        y = qg.gemm_w4a16_g128(x_d, wq, sc, zz, out_dtype=out)
        torch.cuda.synchronize()
        p_o, s_o, z_o = oracle.quantize_weight_u4_g128(w_o)
        np.testing.assert_array_equal(to_np(wq), p_o)
        np.testing.assert_array_equal(f16_bits(sc), s_o.view(np.uint16))
        np.testing.assert_array_equal(f16_bits(zz), z_o.view(np.uint16))
        x64 = x_o.astype(np.float64)
        yref = oracle.gemm_w4a16_g128(x64, p_o, s_o, z_o)
        assert_close(out_f64(y), yref, wl.out_dtype, floor=_w4a16_floor(x64, p_o, s_o, z_o),
                     what=name)


@pytest.mark.parametrize("fold", ["smoothquant", "awq"])
def test_fold_edge_cases(fold):
    rng = np.random.default_rng(2)
    T, K, N = 7, 64, 40
    xc = rng.standard_normal((T, K)).astype(np.float32)
    w = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    xc[:, 3] = 0.0           # silent channel: s = 1
    w[5, :] = 0.0            # zero weight row: s = 1 for SmoothQuant
    fn = qg.smoothquant_fold if fold == "smoothquant" else qg.awq_fold
    s_d, w_d = fn(to_dev(xc), to_dev(w))
    torch.cuda.synchronize()
    s = oracle.smoothquant_scales(xc, w) if fold == "smoothquant" else oracle.awq_scales(xc)
    np.testing.assert_array_equal(to_np(s_d), s)
    np.testing.assert_array_equal(to_np(w_d), oracle.fold_weight(w, s))
    assert s[3] == 1.0
