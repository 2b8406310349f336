"""The C-ABI library loads without a GPU, exports every function the headers
(include/*.h) declare, and rejects bad arguments on the host (nothing is
launched).

Failure handling is forced from the host: every call below fails validation
before any HIP call, so no GPU is needed.
"""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemm.h")
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def _lib():
    import bit_quantized_gemm_int8_amd as q
    if not os.path.exists(q.LIB_PATH):
        from bit_quantized_gemm_int8_amd.build import build
        build()
    return q.load()


def _declared(headers=None):
    names = []
    for h in headers or HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)
    return names


def test_header_declares_the_entry_points():
    names = set(_declared([HEADER]))
    for n in ["quantize_per_token_i8", "quantize_weight_i8_per_channel",
              "quantize_weight_u4_g128", "gemm_w8a8", "gemm_w4a8_g128", "gemm_w4a16_g128",
              "smoothquant_fold", "awq_fold", "apply_smoothing", "qg_status_string",
              "qg_abi_version", "quantize_kv_i8_segments", "dequantize_kv_i8_segments",
              "quantize_weight_u4_g128_outliers", "gemm_w4a8_g128_outliers",
              "quantize_weight_u4_g128_sparse24", "gemm_w4a8_g128_sparse24",
              "quantize_gemm_w8a8", "quantize_gemm_w8a8_plan", "quantize_gemm_w4a8_g128",
              "quantize_gemm_w4a8_g128_workspace_bytes", "quantize_gemm_w4a8_g128_noalloc",
              "quantize_per_token_i8_panel", "gemm_w4a8_g128_panel",
              "gemm_w4a8_g128_outliers_panel"]:
        assert n in names, n


def test_library_exports_every_declared_symbol():
    lib = _lib()
    names = _declared()
    assert {"qg_peak_stream_read", "qg_peak_mfma", "qg_peak_empty"} <= set(names)
    for name in names:
        assert hasattr(lib, name), f"{name} declared in include/*.h but not exported"
    assert lib.qg_abi_version() == 1


P = ctypes.c_void_p
A = P(4096)          # aligned dummy address, never dereferenced: validation fails first
MIS = P(4097)        # misaligned


def test_validation_codes():
    lib = _lib()
    OK, NULL, SHAPE, ALIGN, DTYPE = 0, 1, 2, 3, 4
    q = lib.quantize_per_token_i8
    assert q(None, 0, 4, 16, None, None, None) == NULL
    assert q(A, 0, 4, 17, A, A, None) == SHAPE
    assert q(A, 0, 4, 0, A, A, None) == SHAPE
    assert q(A, 0, -1, 16, A, A, None) == SHAPE
    assert q(A, 3, 4, 16, A, A, None) == DTYPE
    assert q(MIS, 0, 4, 16, A, A, None) == ALIGN
    assert q(None, 0, 0, 16, None, None, None) == OK          # empty: nothing to do
    g = lib.gemm_w8a8
    assert g(A, A, A, A, 4, 4, 16, None, 2, None) == NULL
    assert g(A, None, A, None, 4, 4, 16, A, 2, None) == NULL   # scales needed unless I32
    assert g(A, A, A, A, 4, 4, 24, A, 2, None) == SHAPE
    assert g(A, A, A, A, 4, 4, 16 * 8400, A, 2, None) == SHAPE  # acc would overflow int32
    assert g(A, A, A, A, 4, 4, 16, A, 9, None) == DTYPE
    assert g(A, A, MIS, A, 4, 4, 16, A, 2, None) == ALIGN
    assert g(None, None, None, None, 0, 4, 16, None, 2, None) == OK
    assert g(None, None, None, None, 4, 0, 16, None, 2, None) == OK
    w4 = lib.gemm_w4a8_g128
    assert w4(A, A, A, A, A, 4, 4, 192, A, 2, None) == SHAPE
    assert w4(A, A, A, A, None, 4, 4, 128, A, 2, None) == NULL
    w16 = lib.gemm_w4a16_g128
    assert w16(A, 0, A, A, A, 4, 4, 128, A, 1, None) == DTYPE  # fp32 activations
    assert w16(A, 1, A, A, A, 4, 4, 128, A, 3, None) == DTYPE  # int32 output
    assert w16(A, 1, A, A, A, 4, 4, 100, A, 1, None) == SHAPE
    u4 = lib.quantize_weight_u4_g128
    assert u4(A, 130, 8, A, A, A, None) == SHAPE
    assert u4(A, 128, 8, A, None, A, None) == NULL
    i8 = lib.quantize_weight_i8_per_channel
    assert i8(A, 20, 8, A, A, None) == SHAPE
    assert lib.smoothquant_fold(A, 0, A, 16, 4, A, A, None) == SHAPE
    assert lib.awq_fold(A, 4, A, 18, 4, A, A, None) == SHAPE
    assert lib.apply_smoothing(A, 4, 16, A, A, 3, None) == DTYPE
    kq = lib.quantize_kv_i8_segments
    assert kq(None, 2, 256, 8, 128, A, A, None) == NULL
    assert kq(A, 2, 256, 8, 120, A, A, None) == SHAPE     # D not a multiple of 16
    assert kq(A, 2, 256, 8, 272, A, A, None) == SHAPE     # D > 256
    assert kq(A, 2, 256, 0, 128, A, A, None) == SHAPE     # no heads
    assert kq(A, 2, 256, 2 ** 15 + 1, 128, A, A, None) == SHAPE   # H * D > 2^22
    assert kq(A, 2, -1, 8, 128, A, A, None) == SHAPE
    assert kq(A, 3, 256, 8, 128, A, A, None) == DTYPE
    assert kq(A, 2, 256, 8, 128, A, MIS, None) == ALIGN
    assert kq(None, 2, 0, 8, 128, None, None, None) == OK   # empty cache
    kd = lib.dequantize_kv_i8_segments
    assert kd(A, A, 256, 8, 128, None, 2, None) == NULL
    assert kd(A, A, 256, 8, 8, A, 2, None) == SHAPE
    assert kd(A, A, 256, 8, 128, A, 3, None) == DTYPE
    assert kd(MIS, A, 256, 8, 128, A, 2, None) == ALIGN
    uo = lib.quantize_weight_u4_g128_outliers
    assert uo(A, 130, 8, A, A, A, A, A, None) == SHAPE
    assert uo(A, 128 * 1280, 8, A, A, A, A, A, None) == SHAPE   # too many groups to stage
    assert uo(A, 128, 8, A, A, A, None, A, None) == NULL
    assert uo(A, 128, 8, A, A, A, MIS, A, None) == ALIGN
    assert uo(None, 128, 0, None, None, None, None, None, None) == OK
    go = lib.gemm_w4a8_g128_outliers
    assert go(A, A, A, A, A, A, A, 4, 4, 192, A, 2, None) == SHAPE
    assert go(A, A, A, A, A, A, None, 4, 4, 128, A, 2, None) == NULL   # s8 needed unless I32
    assert go(A, A, A, A, A, None, A, 4, 4, 128, A, 2, None) == NULL
    assert go(A, A, A, A, A, A, A, 4, 4, 128, A, 9, None) == DTYPE
    assert go(A, A, A, A, A, MIS, A, 4, 4, 128, A, 2, None) == ALIGN
    assert go(None, None, None, None, None, None, None, 0, 4, 128, None, 2, None) == OK
    us = lib.quantize_weight_u4_g128_sparse24
    assert us(A, 130, 8, A, A, A, None) == SHAPE
    assert us(A, 128, 8, A, None, A, None) == NULL
    assert us(A, 128, 8, MIS, A, A, None) == ALIGN
    gs = lib.gemm_w4a8_g128_sparse24
    assert gs(A, A, A, A, A, 4, 4, 192, A, 2, None) == SHAPE
    assert gs(A, A, A, A, A, 16 * 65535 + 1, 4, 128, A, 2, None) == SHAPE
    assert gs(A, None, A, A, A, 4, 4, 128, A, 2, None) == NULL
    assert gs(A, A, A, A, A, 4, 4, 128, A, 7, None) == DTYPE
    assert gs(A, A, MIS, A, A, 4, 4, 128, A, 2, None) == ALIGN
    assert gs(None, None, None, None, None, 4, 0, 128, None, 2, None) == OK
    fq = lib.quantize_gemm_w8a8
    assert fq(A, 2, A, A, 8, 16, 4096, A, 2, None, A, 0, None) == NULL     # xq needed
    assert fq(A, 2, A, None, 8, 16, 4096, A, 2, A, A, 0, None) == NULL     # w_scale needed unless I32
    assert fq(A, 2, A, A, 8, 16, 4100, A, 2, A, A, 0, None) == SHAPE
    assert fq(A, 3, A, A, 8, 16, 4096, A, 2, A, A, 0, None) == DTYPE
    assert fq(MIS, 2, A, A, 8, 16, 4096, A, 2, A, A, 0, None) == ALIGN
    assert fq(A, 2, A, A, 8, 16, 4096, A, 2, A, A, 3, None) == 6          # QG_ERR_ARG
    assert fq(A, 2, A, A, 8, 16, 4096, A, 2, A, A, -1, None) == 6
    assert fq(None, 2, None, None, 0, 16, 4096, None, 2, None, None, 2, None) == OK
    f4 = lib.quantize_gemm_w4a8_g128
    f4.argtypes = [P, ctypes.c_int, P, P, P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, P,
                   ctypes.c_int, P, P, P, ctypes.c_int64, P]
    ws = 32 * 2112                                                   # 16 x 4160 x 4096 needs it
    assert f4(A, 2, A, A, A, 16, 4160, 4096, A, 2, A, A, A, ws - 16, None) == SHAPE
    assert f4(A, 2, A, A, A, 16, 4160, 4096, A, 2, A, A, None, ws, None) == NULL
    assert f4(A, 2, A, A, A, 16, 4160, 4096, A, 2, A, A, MIS, ws, None) == ALIGN
    assert f4(A, 2, A, A, A, 16, 4160, 4096, A, 2, A, A, A, -1, None) == SHAPE
    assert f4(A, 2, A, A, A, 8, 16, 192, A, 2, A, A, A, ws, None) == SHAPE      # K % 128
    assert f4(A, 3, A, A, A, 8, 16, 4096, A, 2, A, A, A, ws, None) == DTYPE
    assert f4(A, 2, A, A, A, 8, 16, 4096, A, 9, A, A, A, ws, None) == DTYPE
    assert f4(A, 2, A, None, A, 8, 16, 4096, A, 2, A, A, A, ws, None) == NULL   # scales unless I32
    assert f4(A, 2, A, A, None, 8, 16, 4096, A, 2, A, A, A, ws, None) == NULL   # zero points
    assert f4(A, 2, A, A, A, 8, 16, 4096, A, 2, None, A, A, ws, None) == NULL   # xq
    assert f4(MIS, 2, A, A, A, 8, 16, 4096, A, 2, A, A, A, ws, None) == ALIGN
    assert f4(None, 2, None, None, None, 0, 16, 4096, None, 2, None, None, None, 0, None) == OK
    # the g=128 uint4 GEMMs take at most 65535 groups per row, as the quantizer
    g4, g16 = lib.gemm_w4a8_g128, lib.gemm_w4a16_g128
    assert g4(A, A, A, A, A, 1, 16, 65536 * 128, A, 2, None) == SHAPE
    assert g16(A, 1, A, A, A, 1, 16, 65536 * 128, A, 1, None) == SHAPE
    assert lib.quantize_weight_u4_g128(A, 65536 * 128, 16, A, A, A, None) == SHAPE
    assert "ARG" in lib.qg_status_string(6).decode()
    assert "SHAPE" in lib.qg_status_string(2).decode()


def test_fused_plan_on_the_host():
    """quantize_gemm_w8a8_plan: the automatic choice on both sides of each of
    its thresholds, the forced modes and the fused kernel's coverage (a host
    query: nothing is launched)."""
    import torch
    import bit_quantized_gemm_int8_amd as q
    _lib()
    plan = q.quantize_gemm_w8a8_plan
    bf, f32 = torch.bfloat16, torch.float32
    assert plan(bf, 4, 8192, 4096)                  # few rows, N K = 2^25
    assert not plan(bf, 4, 8192, 4080)              # N K < 2^25
    assert not plan(bf, 5, 8192, 4096)              # 5..8 rows
    assert plan(f32, 16, 512, 512)                  # 9..16 short rows
    assert plan(bf, 9, 11008, 768)
    assert not plan(bf, 9, 11008, 784)              # K > 768
    assert not plan(f32, 8, 512, 512)
    assert not plan(bf, 17, 512, 512, fuse=True)    # past the kernel's 16 rows
    assert plan(bf, 16, 64, 2048, fuse=True)        # 16 rows x 256 chunks: covered
    assert not plan(bf, 16, 64, 2064, fuse=True)    # past 4096 chunks
    assert plan(f32, 1, 64, 32768, fuse=True)
    assert not plan(f32, 1, 64, 32784, fuse=True)
    assert not plan(bf, 1, 11008, 4096, fuse=False)
    assert not plan(bf, 0, 11008, 4096) and not plan(bf, 1, 0, 4096)
    lib = q.load()
    out = ctypes.c_int(7)
    assert lib.quantize_gemm_w8a8_plan(2, 4, 16, 100, 0, ctypes.byref(out)) == 2   # SHAPE
    assert lib.quantize_gemm_w8a8_plan(3, 4, 16, 128, 0, ctypes.byref(out)) == 4   # DTYPE
    assert lib.quantize_gemm_w8a8_plan(2, 4, 16, 128, 5, ctypes.byref(out)) == 6   # ARG
    assert lib.quantize_gemm_w8a8_plan(2, 4, 16, 128, 0, None) == 1                # NULL
    assert out.value == 7                                                         # untouched


def test_w4a8_workspace_on_the_host():
    """quantize_gemm_w4a8_g128_workspace_bytes: (K / 128) x 2112 bytes where
    the panel pair runs (2..16 rows, K <= 16384, 257-383 blocks of 16
    channels, not where the plain GEMM is the dot-product kernel), 0 where
    the call runs the two plain kernels; the panel's own size."""
    import bit_quantized_gemm_int8_amd as q
    _lib()
    wb = q.quantize_gemm_w4a8_g128_workspace_bytes
    assert wb(16, 4112, 11008) == 86 * 2112           # 257 weight blocks: the panel pair
    assert wb(16, 6128, 4096) == 32 * 2112            # 383 blocks
    assert wb(16, 6144, 4096) == 0                    # 384 blocks: the wide GEMM
    assert wb(16, 11008, 4096) == 0 and wb(1, 12288, 4096) == 0
    assert wb(2, 4112, 16384) == 128 * 2112           # the longest K
    assert wb(2, 4112, 16512) == 0
    assert wb(1, 4112, 4096) == 0                     # one row: the dot-product GEMM
    assert wb(2, 4112, 4096) == 0                     # two rows, K <= 4096: likewise
    assert wb(2, 4112, 4224) == 33 * 2112             # two rows past K = 4096: the pair
    assert wb(16, 4096, 11008) == 0                   # 256 blocks: the plain kernels
    assert wb(1, 4096, 4096) == 0 and wb(3, 100, 2048) == 0
    assert wb(17, 8192, 4096) == 0                    # past 16 rows
    assert wb(0, 8192, 4096) == 0 and wb(4, 0, 4096) == 0
    assert wb(4, 8192, 200) == 0 and wb(-1, 8192, 256) == 0
    pb = q.quantize_per_token_i8_panel_bytes
    assert pb(1, 128) == 2112 and pb(16, 16384) == 128 * 2112 and pb(5, 4096) == 32 * 2112
    assert pb(17, 4096) == 0 and pb(0, 4096) == 0 and pb(4, 16512) == 0 and pb(4, 200) == 0


def test_noalloc_validation_codes():
    lib = _lib()
    OK, NULL, SHAPE, ALIGN, DTYPE = 0, 1, 2, 3, 4
    I64 = ctypes.c_int64
    na = lib.quantize_gemm_w4a8_g128_noalloc
    na.argtypes = [P, ctypes.c_int, P, P, P, I64, I64, I64, P, ctypes.c_int, P, P, P]
    assert na(A, 2, A, A, A, 8, 16, 192, A, 2, A, A, None) == SHAPE       # K % 128
    assert na(A, 2, A, A, A, -1, 16, 4096, A, 2, A, A, None) == SHAPE
    assert na(A, 3, A, A, A, 8, 16, 4096, A, 2, A, A, None) == DTYPE
    assert na(A, 2, A, A, A, 8, 16, 4096, A, 9, A, A, None) == DTYPE
    assert na(A, 2, A, None, A, 8, 16, 4096, A, 2, A, A, None) == NULL    # scales unless I32
    assert na(A, 2, A, A, A, 8, 16, 4096, A, 2, None, A, None) == NULL    # xq
    assert na(A, 2, A, A, None, 8, 16, 4096, A, 2, A, A, None) == NULL    # zero points
    assert na(MIS, 2, A, A, A, 8, 16, 4096, A, 2, A, A, None) == ALIGN
    assert na(None, 2, None, None, None, 0, 16, 4096, None, 2, None, None, None) == OK


def test_panel_validation_codes():
    lib = _lib()
    OK, NULL, SHAPE, ALIGN, DTYPE = 0, 1, 2, 3, 4
    I64 = ctypes.c_int64
    qp = lib.quantize_per_token_i8_panel
    qp.argtypes = [P, ctypes.c_int, I64, I64, P, P, P, I64, P]
    pbytes = 32 * 2112
    assert qp(A, 2, 4, 4096, A, A, A, pbytes - 1, None) == SHAPE
    assert qp(A, 2, 17, 4096, A, A, A, 10 ** 7, None) == SHAPE        # past 16 rows
    assert qp(A, 2, 4, 16512, A, A, A, 10 ** 7, None) == SHAPE        # K > 16384
    assert qp(A, 2, 4, 4000, A, A, A, 10 ** 7, None) == SHAPE         # K % 128
    assert qp(A, 3, 4, 4096, A, A, A, pbytes, None) == DTYPE
    assert qp(A, 2, 4, 4096, A, None, A, pbytes, None) == NULL        # x_scale
    assert qp(A, 2, 4, 4096, A, A, None, pbytes, None) == NULL        # panel
    assert qp(A, 2, 4, 4096, MIS, A, A, pbytes, None) == ALIGN
    assert qp(A, 2, 4, 4096, A, A, MIS, pbytes, None) == ALIGN
    assert qp(None, 2, 0, 4096, None, None, None, 0, None) == OK
    gp = lib.gemm_w4a8_g128_panel
    gp.argtypes = [P, I64, P, P, P, P, I64, I64, I64, P, ctypes.c_int, P]
    assert gp(A, pbytes - 16, A, A, A, A, 4, 64, 4096, A, 2, None) == SHAPE
    assert gp(A, 10 ** 7, A, A, A, A, 17, 64, 4096, A, 2, None) == SHAPE
    assert gp(A, pbytes, A, A, A, A, 4, 64, 4096, A, 9, None) == DTYPE
    assert gp(A, pbytes, None, A, A, A, 4, 64, 4096, A, 2, None) == NULL   # x_scale unless I32
    assert gp(A, pbytes, A, A, A, None, 4, 64, 4096, A, 2, None) == NULL   # zero points
    assert gp(MIS, pbytes, A, A, A, A, 4, 64, 4096, A, 2, None) == ALIGN
    assert gp(None, 0, None, None, None, None, 4, 0, 4096, None, 2, None) == OK
    go = lib.gemm_w4a8_g128_outliers_panel
    go.argtypes = [P, I64, P, P, P, P, P, P, I64, I64, I64, P, ctypes.c_int, P]
    assert go(A, pbytes - 16, A, A, A, A, A, A, 4, 64, 4096, A, 2, None) == SHAPE
    assert go(A, 10 ** 7, A, A, A, A, A, A, 4, 64, 16512, A, 2, None) == SHAPE   # K > 16384
    assert go(A, pbytes, A, A, A, A, A, A, 4, 64, 4096, A, 9, None) == DTYPE
    assert go(A, pbytes, A, A, A, A, None, A, 4, 64, 4096, A, 2, None) == NULL   # records
    assert go(A, pbytes, A, A, A, A, A, None, 4, 64, 4096, A, 2, None) == NULL   # s8 unless I32
    assert go(A, pbytes, A, A, A, A, MIS, A, 4, 64, 4096, A, 2, None) == ALIGN
    assert go(None, 0, None, None, None, None, None, None, 0, 64, 4096, None, 2, None) == OK


def test_binding_rejects_host_tensors():
    import torch
    import bit_quantized_gemm_int8_amd as q
    _lib()
    with pytest.raises(TypeError):
        q.quantize_per_token_i8(torch.zeros(4, 16))


def test_peak_probe_validation():
    """The measurement probes check their arguments on the host too."""
    lib = _lib()
    NULL, SHAPE, ALIGN, ARG = 1, 2, 3, 6
    r = lib.qg_peak_stream_read
    r.argtypes = [P, ctypes.c_int64, P, P]
    assert r(None, 1024, A, None) == NULL
    assert r(A, 0, A, None) == SHAPE
    assert r(A, (1 << 31) + 1, A, None) == SHAPE
    assert r(MIS, 1024, A, None) == ALIGN
    sink = lib.qg_peak_stream_read_sink
    sink.argtypes, sink.restype = [ctypes.c_int64], ctypes.c_int64
    assert sink(0) == 0
    # at most 256 workgroups of 8 waves: 24 MB needs 12 KB per wave
    assert sink(24260672) == 8 * ((24260672 + 8 * 12 * 1024 - 1) // (8 * 12 * 1024))
    assert sink(24260672) <= 256 * 8
    m = lib.qg_peak_mfma
    m.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, P, P, P]
    assert m(0, 10, 4, None, A, None) == NULL
    assert m(4, 10, 4, A, A, None) == ARG
    assert m(0, 0, 4, A, A, None) == SHAPE
    assert m(0, 10, 65536, A, A, None) == SHAPE
    ops = lib.qg_peak_mfma_ops
    ops.argtypes, ops.restype = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64], ctypes.c_int64
    assert ops(0, 1, 1) == 16 * 2 * 32 * 32 * 32
    assert ops(2, 3, 5) == 3 * 5 * 16 * 2 * 32 * 32 * 16
    assert ops(9, 1, 1) == -1
