"""Quantized linear layer for AMD MI355X (gfx950): thin Python binding.

Every function here marshals torch tensors into the C ABI of libqgemm.so
(include/qgemm.h) and enqueues the library's HIP kernels on the current torch
stream; no step of the computation runs in Python.  Functions that return
tensors allocate them with torch (or fill `out=` when given).  If the library
is not built, the first call raises RuntimeError -- there is no fallback.

Entry points (same names as the C ABI):
  quantize_per_token_i8(x)                      -> (xq int8 [M,K], x_scale f32 [M])
  quantize_weight_i8_per_channel(w)             -> (wq int8 [N,K], w_scale f32 [N])
  quantize_weight_u4_g128(w)                    -> (wq int32 [N,K/8], scale f16 [N,G], zero f16 [N,G])
  gemm_w8a8(xq, x_scale, wq, w_scale, out_dtype)
  quantize_gemm_w8a8(x, wq, w_scale, out_dtype)  -> (y, xq, x_scale): both steps in one call
  gemm_w4a8_g128(xq, x_scale, wq, w_scale, w_zero, out_dtype)
  quantize_per_token_i8_panel(x)                -> (panel uint8, xq, x_scale): codes + W4A8 token panel
  gemm_w4a8_g128_panel(panel, x_scale, wq, w_scale, w_zero, M, out_dtype)
  quantize_gemm_w4a8_g128(x, wq, w_scale, w_zero, out_dtype) -> (y, xq, x_scale): both steps in one call
  quantize_gemm_w4a8_g128_workspace_bytes(M, N, K) -> bytes of device workspace that call needs
  quantize_gemm_w4a8_g128_noalloc(x, wq, w_scale, w_zero, out_dtype) -> (y, xq, x_scale): the library's own panel
  gemm_w4a16_g128(x, wq, w_scale, w_zero, out_dtype)
  smoothquant_fold(x_cal, w) / awq_fold(x_cal, w) -> (s f32 [K], w_folded f32 [K,N])
  apply_smoothing(x, s, out_dtype)
  quantize_weight_u4_g128_outliers(w)           -> (wq, scale, zero, records int64 [N,G], s8 f32 [N])
  gemm_w4a8_g128_outliers(xq, x_scale, wq, w_scale, w_zero, records, s8, out_dtype)
  gemm_w4a8_g128_outliers_panel(panel, x_scale, wq, w_scale, w_zero, records, s8, M, out_dtype)
  quantize_weight_u4_g128_sparse24(w)           -> (wsp int32 [N/16,G,16,12], scale f16 [N,G], zero f16 [N,G])
  gemm_w4a8_g128_sparse24(xq, x_scale, wsp, w_scale, w_zero, out_dtype)
  quantize_kv_i8_segments(kv)                   -> (kv_q int8 [T,H,D], kv_scale f32 [H,ceil(T/128),D])
  dequantize_kv_i8_segments(kv_q, kv_scale, out_dtype) -> [T,H,D]
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "LIB_PATH", "load", "QG_F32", "QG_F16", "QG_BF16", "QG_I32",
    "quantize_per_token_i8", "quantize_weight_i8_per_channel", "quantize_weight_u4_g128",
    "gemm_w8a8", "gemm_w4a8_g128", "gemm_w4a16_g128", "quantize_gemm_w8a8",
    "quantize_gemm_w8a8_plan", "quantize_gemm_w4a8_g128",
    "quantize_gemm_w4a8_g128_workspace_bytes", "quantize_per_token_i8_panel",
    "quantize_per_token_i8_panel_bytes", "gemm_w4a8_g128_panel",
    "gemm_w4a8_g128_outliers_panel",
    "quantize_gemm_w4a8_g128_noalloc",
    "smoothquant_fold", "awq_fold", "apply_smoothing", "status_string",
    "quantize_kv_i8_segments", "dequantize_kv_i8_segments", "KV_SEGMENT",
    "quantize_weight_u4_g128_outliers", "gemm_w4a8_g128_outliers",
    "quantize_weight_u4_g128_sparse24", "gemm_w4a8_g128_sparse24",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqgemm.so")

QG_F32, QG_F16, QG_BF16, QG_I32 = 0, 1, 2, 3
_DTYPE_CODE = {torch.float32: QG_F32, torch.float16: QG_F16, torch.bfloat16: QG_BF16,
               torch.int32: QG_I32}

_vp, _i64, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
_SIGNATURES = {
    "quantize_per_token_i8": [_vp, _int, _i64, _i64, _vp, _vp, _vp],
    "quantize_weight_i8_per_channel": [_vp, _i64, _i64, _vp, _vp, _vp],
    "quantize_weight_u4_g128": [_vp, _i64, _i64, _vp, _vp, _vp, _vp],
    "gemm_w8a8": [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _int, _vp],
    "quantize_gemm_w8a8": [_vp, _int, _vp, _vp, _i64, _i64, _i64, _vp, _int, _vp, _vp, _int, _vp],
    "quantize_gemm_w8a8_plan": [_int, _i64, _i64, _i64, _int, _vp],
    "gemm_w4a8_g128": [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _int, _vp],
    "quantize_gemm_w4a8_g128": [_vp, _int, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _int, _vp, _vp,
                                _vp, _i64, _vp],
    "quantize_per_token_i8_panel": [_vp, _int, _i64, _i64, _vp, _vp, _vp, _i64, _vp],
    "quantize_gemm_w4a8_g128_noalloc": [_vp, _int, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _int,
                                        _vp, _vp, _vp],
    "gemm_w4a8_g128_panel": [_vp, _i64, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _int, _vp],
    "gemm_w4a8_g128_outliers_panel": [_vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64,
                                      _vp, _int, _vp],
    "gemm_w4a16_g128": [_vp, _int, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _int, _vp],
    "smoothquant_fold": [_vp, _i64, _vp, _i64, _i64, _vp, _vp, _vp],
    "awq_fold": [_vp, _i64, _vp, _i64, _i64, _vp, _vp, _vp],
    "apply_smoothing": [_vp, _i64, _i64, _vp, _vp, _int, _vp],
    "quantize_kv_i8_segments": [_vp, _int, _i64, _i64, _i64, _vp, _vp, _vp],
    "quantize_weight_u4_g128_outliers": [_vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp],
    "gemm_w4a8_g128_outliers": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _int,
                                _vp],
    "quantize_weight_u4_g128_sparse24": [_vp, _i64, _i64, _vp, _vp, _vp, _vp],
    "gemm_w4a8_g128_sparse24": [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _int, _vp],
    "dequantize_kv_i8_segments": [_vp, _vp, _i64, _i64, _i64, _vp, _int, _vp],
}

# measurement probes (include/qgemm_peaks.h)
_PEAK_SIGNATURES = {
    "qg_peak_stream_read_sink": [_i64],
    "qg_peak_stream_read": [_vp, _i64, _vp, _vp],
    "qg_peak_mfma": [_int, _i64, _i64, _vp, _vp, _vp],
    "qg_peak_mfma_ops": [_int, _i64, _i64],
    "qg_peak_empty": [_vp],
}

_lib: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    """Load libqgemm.so (once).  Raises RuntimeError if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m bit_quantized_gemm_int8_amd.build` "
                "(hipcc, gfx950).  There is no non-HIP fallback.")
        lib = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        for name, args in _PEAK_SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int64 if name.endswith(("_sink", "_ops")) else ctypes.c_int
        lib.quantize_gemm_w4a8_g128_workspace_bytes.argtypes = [_i64, _i64, _i64]
        lib.quantize_gemm_w4a8_g128_workspace_bytes.restype = ctypes.c_int64
        lib.quantize_per_token_i8_panel_bytes.argtypes = [_i64, _i64]
        lib.quantize_per_token_i8_panel_bytes.restype = ctypes.c_int64
        lib.qg_status_string.argtypes = [ctypes.c_int]
        lib.qg_status_string.restype = ctypes.c_char_p
        lib.qg_abi_version.restype = ctypes.c_int
        _lib = lib
    return _lib


def status_string(rc: int) -> str:
    return load().qg_status_string(rc).decode()


def _call(name: str, *args) -> None:
    rc = getattr(load(), name)(*args)
    if rc != 0:
        raise RuntimeError(f"{name}: {status_string(rc)}")


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor, name: str, dtypes, shape=None, device=None) -> int:
    """Device pointer of a contiguous GPU tensor, after checking its dtype and,
    when given, its shape and that it lives on `device` (the kernels index
    every operand by M, N, K and the group count, so a mis-shaped tensor would
    be read or written past its allocation)."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other operands on {device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype in {dtypes}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _opt(t, name, dtypes, shape, device):
    """_dev for an operand that may be None (passed to the library as NULL)."""
    return None if t is None else _dev(t, name, dtypes, shape, device)


def _out(out, shape, dtype, device, name="out"):
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if not isinstance(out, torch.Tensor) or not out.is_cuda or out.device != device:
        raise ValueError(f"{name} must be a tensor on {device}")
    if tuple(out.shape) != tuple(shape) or out.dtype != dtype or not out.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}")
    return out


def _2d(t, name):
    if not isinstance(t, torch.Tensor) or t.dim() != 2:
        raise ValueError(f"{name} must be a 2-D tensor")
    return t.shape


_FLOATS = (torch.float32, torch.float16, torch.bfloat16)


def quantize_per_token_i8(x: torch.Tensor, out=None):
    """x [M, K] (f32/f16/bf16) -> (xq int8 [M, K], x_scale f32 [M])."""
    px = _dev(x, "x", _FLOATS)
    M, K = _2d(x, "x")
    xq, xs = out if out is not None else (None, None)
    xq = _out(xq, (M, K), torch.int8, x.device, "xq out")
    xs = _out(xs, (M,), torch.float32, x.device, "x_scale out")
    _call("quantize_per_token_i8", px, _DTYPE_CODE[x.dtype], M, K, xq.data_ptr(), xs.data_ptr(),
          _stream())
    return xq, xs


def quantize_weight_i8_per_channel(w: torch.Tensor):
    """w f32 [K, N] -> (wq int8 [N, K], w_scale f32 [N])."""
    pw = _dev(w, "w", (torch.float32,))
    K, N = _2d(w, "w")
    wq = torch.empty((N, K), dtype=torch.int8, device=w.device)
    ws = torch.empty((N,), dtype=torch.float32, device=w.device)
    _call("quantize_weight_i8_per_channel", pw, K, N, wq.data_ptr(), ws.data_ptr(), _stream())
    return wq, ws


def quantize_weight_u4_g128(w: torch.Tensor):
    """w f32 [K, N] -> (wq int32 [N, K/8], scale f16 [N, K/128], zero f16 [N, K/128])."""
    pw = _dev(w, "w", (torch.float32,))
    K, N = _2d(w, "w")
    wq = torch.empty((N, K // 8), dtype=torch.int32, device=w.device)
    sc = torch.empty((N, K // 128), dtype=torch.float16, device=w.device)
    zz = torch.empty((N, K // 128), dtype=torch.float16, device=w.device)
    _call("quantize_weight_u4_g128", pw, K, N, wq.data_ptr(), sc.data_ptr(), zz.data_ptr(),
          _stream())
    return wq, sc, zz


def gemm_w8a8(xq, x_scale, wq, w_scale, out_dtype=torch.bfloat16, out=None):
    """y [M, N] = (xq @ wq^T) * x_scale[:, None] * w_scale[None, :] (int32 if out_dtype is int32)."""
    pxq = _dev(xq, "xq", (torch.int8,))
    M, K = _2d(xq, "xq")
    dev = xq.device
    N = _2d(wq, "wq")[0]
    pwq = _dev(wq, "wq", (torch.int8,), (N, K), dev)
    pxs = _opt(x_scale, "x_scale", (torch.float32,), (M,), dev)
    pws = _opt(w_scale, "w_scale", (torch.float32,), (N,), dev)
    y = _out(out, (M, N), out_dtype, dev)
    _call("gemm_w8a8", pxq, pxs, pwq, pws, M, N, K, y.data_ptr(), _DTYPE_CODE[out_dtype],
          _stream())
    return y


_FUSE = {None: 0, False: 1, True: 2}


def quantize_gemm_w8a8(x, wq, w_scale, out_dtype=torch.bfloat16, out=None, xq_out=None, fuse=None):
    """x [M, K] (f32/f16/bf16) -> (y [M, N], xq int8 [M, K], x_scale f32 [M]):
    per-token quantization and the W8A8 product in one call.  fuse: None lets
    the library choose, True runs the one-kernel form wherever it covers the
    shape, False the two kernels; the results are the same."""
    px = _dev(x, "x", _FLOATS)
    M, K = _2d(x, "x")
    dev = x.device
    N = _2d(wq, "wq")[0]
    pwq = _dev(wq, "wq", (torch.int8,), (N, K), dev)
    pws = _opt(w_scale, "w_scale", (torch.float32,), (N,), dev)
    y = _out(out, (M, N), out_dtype, dev)
    xq, xs = xq_out if xq_out is not None else (None, None)
    xq = _out(xq, (M, K), torch.int8, dev, "xq out")
    xs = _out(xs, (M,), torch.float32, dev, "x_scale out")
    _call("quantize_gemm_w8a8", px, _DTYPE_CODE[x.dtype], pwq, pws, M, N, K, y.data_ptr(),
          _DTYPE_CODE[out_dtype], xq.data_ptr(), xs.data_ptr(), _FUSE[fuse], _stream())
    return y, xq, xs


def quantize_gemm_w8a8_plan(x_dtype, M, N, K, fuse=None) -> bool:
    """True when quantize_gemm_w8a8 with activations of x_dtype and these
    sizes runs the one-kernel form, False for the two kernels (host only)."""
    fused = ctypes.c_int(0)
    _call("quantize_gemm_w8a8_plan", _DTYPE_CODE[x_dtype], M, N, K, _FUSE[fuse],
          ctypes.byref(fused))
    return bool(fused.value)


def gemm_w4a8_g128(xq, x_scale, wq, w_scale, w_zero, out_dtype=torch.bfloat16, out=None):
    """W4A8 with g=128 uint4 weights; int32 out_dtype returns per-group acc [M, K/128, N]."""
    pxq = _dev(xq, "xq", (torch.int8,))
    M, K = _2d(xq, "xq")
    dev = xq.device
    N = _2d(wq, "wq")[0]
    pwq = _dev(wq, "wq", (torch.int32,), (N, K // 8), dev)
    pwz = _dev(w_zero, "w_zero", (torch.float16,), (N, K // 128), dev)
    pxs = _opt(x_scale, "x_scale", (torch.float32,), (M,), dev)
    pws = _opt(w_scale, "w_scale", (torch.float16,), (N, K // 128), dev)
    shape = (M, K // 128, N) if out_dtype == torch.int32 else (M, N)
    y = _out(out, shape, out_dtype, dev)
    _call("gemm_w4a8_g128", pxq, pxs, pwq, pws, pwz, M, N, K, y.data_ptr(),
          _DTYPE_CODE[out_dtype], _stream())
    return y


def quantize_per_token_i8_panel_bytes(M: int, K: int) -> int:
    """Bytes of the W4A8 token panel for M rows of K (0 where unsupported)."""
    return int(load().quantize_per_token_i8_panel_bytes(M, K))


def quantize_per_token_i8_panel(x, panel=None, xq_out=None, write_xq=True):
    """x [M, K] (f32/f16/bf16, M <= 16, K <= 16384) -> (panel uint8, xq, x_scale):
    the codes and scales of quantize_per_token_i8 plus the token panel that
    gemm_w4a8_g128_panel reads.  write_xq=False skips xq (returned as None)."""
    px = _dev(x, "x", _FLOATS)
    M, K = _2d(x, "x")
    dev = x.device
    need = quantize_per_token_i8_panel_bytes(M, K)
    if panel is None:
        panel = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    pp = _dev(panel, "panel", (torch.uint8,), None, dev)
    xq, xs = xq_out if xq_out is not None else (None, None)
    xq = _out(xq, (M, K), torch.int8, dev, "xq out") if write_xq else None
    xs = _out(xs, (M,), torch.float32, dev, "x_scale out")
    _call("quantize_per_token_i8_panel", px, _DTYPE_CODE[x.dtype], M, K,
          xq.data_ptr() if xq is not None else None, xs.data_ptr(), pp, panel.numel(), _stream())
    return panel, xq, xs


def gemm_w4a8_g128_panel(panel, x_scale, wq, w_scale, w_zero, M, out_dtype=torch.bfloat16,
                         out=None):
    """W4A8 g=128 on a token panel of M rows (quantize_per_token_i8_panel);
    int32 out_dtype returns per-group acc [M, K/128, N]."""
    dev = panel.device
    pp = _dev(panel, "panel", (torch.uint8,), None, dev)
    N, K8 = _2d(wq, "wq")
    K = K8 * 8
    pwq = _dev(wq, "wq", (torch.int32,), (N, K // 8), dev)
    pwz = _dev(w_zero, "w_zero", (torch.float16,), (N, K // 128), dev)
    pxs = _opt(x_scale, "x_scale", (torch.float32,), (M,), dev)
    pws = _opt(w_scale, "w_scale", (torch.float16,), (N, K // 128), dev)
    shape = (M, K // 128, N) if out_dtype == torch.int32 else (M, N)
    y = _out(out, shape, out_dtype, dev)
    _call("gemm_w4a8_g128_panel", pp, panel.numel(), pxs, pwq, pws, pwz, M, N, K, y.data_ptr(),
          _DTYPE_CODE[out_dtype], _stream())
    return y


def quantize_gemm_w4a8_g128_workspace_bytes(M: int, N: int, K: int) -> int:
    """Device workspace (bytes) quantize_gemm_w4a8_g128 needs for these sizes
    (0: it runs the two kernels in sequence and needs none)."""
    return int(load().quantize_gemm_w4a8_g128_workspace_bytes(M, N, K))


def quantize_gemm_w4a8_g128(x, wq, w_scale, w_zero, out_dtype=torch.bfloat16, out=None,
                            xq_out=None, workspace=None):
    """x [M, K] (f32/f16/bf16) -> (y, xq int8 [M, K], x_scale f32 [M]):
    per-token quantization and the W4A8 g=128 product in one call, the same
    results as quantize_per_token_i8 then gemm_w4a8_g128.  workspace: a
    contiguous uint8 device tensor of at least
    quantize_gemm_w4a8_g128_workspace_bytes(M, N, K) bytes, allocated here
    when None."""
    px = _dev(x, "x", _FLOATS)
    M, K = _2d(x, "x")
    dev = x.device
    N = _2d(wq, "wq")[0]
    pwq = _dev(wq, "wq", (torch.int32,), (N, K // 8), dev)
    pwz = _dev(w_zero, "w_zero", (torch.float16,), (N, K // 128), dev)
    pws = _opt(w_scale, "w_scale", (torch.float16,), (N, K // 128), dev)
    shape = (M, K // 128, N) if out_dtype == torch.int32 else (M, N)
    y = _out(out, shape, out_dtype, dev)
    xq, xs = xq_out if xq_out is not None else (None, None)
    xq = _out(xq, (M, K), torch.int8, dev, "xq out")
    xs = _out(xs, (M,), torch.float32, dev, "x_scale out")
    need = quantize_gemm_w4a8_g128_workspace_bytes(M, N, K)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    pw = _dev(workspace, "workspace", (torch.uint8,), None, dev)
    _call("quantize_gemm_w4a8_g128", px, _DTYPE_CODE[x.dtype], pwq, pws, pwz, M, N, K,
          y.data_ptr(), _DTYPE_CODE[out_dtype], xq.data_ptr(), xs.data_ptr(), pw,
          workspace.numel(), _stream())
    return y, xq, xs


def quantize_gemm_w4a8_g128_noalloc(x, wq, w_scale, w_zero, out_dtype=torch.bfloat16, out=None,
                                    xq_out=None):
    """quantize_gemm_w4a8_g128 with the library's own per-GPU panel array
    instead of a workspace: the C call allocates nothing (outputs given as
    out / xq_out are filled in place; calls overlapping on one GPU race)."""
    px = _dev(x, "x", _FLOATS)
    M, K = _2d(x, "x")
    dev = x.device
    N = _2d(wq, "wq")[0]
    pwq = _dev(wq, "wq", (torch.int32,), (N, K // 8), dev)
    pwz = _dev(w_zero, "w_zero", (torch.float16,), (N, K // 128), dev)
    pws = _opt(w_scale, "w_scale", (torch.float16,), (N, K // 128), dev)
    shape = (M, K // 128, N) if out_dtype == torch.int32 else (M, N)
    y = _out(out, shape, out_dtype, dev)
    xq, xs = xq_out if xq_out is not None else (None, None)
    xq = _out(xq, (M, K), torch.int8, dev, "xq out")
    xs = _out(xs, (M,), torch.float32, dev, "x_scale out")
    _call("quantize_gemm_w4a8_g128_noalloc", px, _DTYPE_CODE[x.dtype], pwq, pws, pwz, M, N, K,
          y.data_ptr(), _DTYPE_CODE[out_dtype], xq.data_ptr(), xs.data_ptr(), _stream())
    return y, xq, xs


def gemm_w4a16_g128(x, wq, w_scale, w_zero, out_dtype=None, out=None):
    """W4A16: x f16/bf16 [M, K]; returns y [M, N] (default dtype: that of x)."""
    px = _dev(x, "x", (torch.float16, torch.bfloat16))
    M, K = _2d(x, "x")
    dev = x.device
    N = _2d(wq, "wq")[0]
    pwq = _dev(wq, "wq", (torch.int32,), (N, K // 8), dev)
    pws = _dev(w_scale, "w_scale", (torch.float16,), (N, K // 128), dev)
    pwz = _dev(w_zero, "w_zero", (torch.float16,), (N, K // 128), dev)
    out_dtype = out_dtype or x.dtype
    y = _out(out, (M, N), out_dtype, dev)
    _call("gemm_w4a16_g128", px, _DTYPE_CODE[x.dtype], pwq, pws, pwz, M, N, K, y.data_ptr(),
          _DTYPE_CODE[out_dtype], _stream())
    return y


def quantize_weight_u4_g128_outliers(w: torch.Tensor):
    """w f32 [K, N] -> (wq int32 [N, K/8], scale f16 [N, G], zero f16 [N, G],
    records int64 [N, G] (the uint64 bit patterns), s8 f32 [N]): uint4 groups
    of 128 with each group's 3 largest weights in an INT8 side store."""
    pw = _dev(w, "w", (torch.float32,))
    K, N = _2d(w, "w")
    G = K // 128
    wq = torch.empty((N, K // 8), dtype=torch.int32, device=w.device)
    sc = torch.empty((N, G), dtype=torch.float16, device=w.device)
    zz = torch.empty((N, G), dtype=torch.float16, device=w.device)
    rec = torch.empty((N, G), dtype=torch.int64, device=w.device)
    s8 = torch.empty((N,), dtype=torch.float32, device=w.device)
    _call("quantize_weight_u4_g128_outliers", pw, K, N, wq.data_ptr(), sc.data_ptr(),
          zz.data_ptr(), rec.data_ptr(), s8.data_ptr(), _stream())
    return wq, sc, zz, rec, s8


def gemm_w4a8_g128_outliers(xq, x_scale, wq, w_scale, w_zero, records, s8,
                            out_dtype=torch.bfloat16, out=None):
    """W4A8 g=128 with the INT8 outlier side path; int32 out_dtype returns the
    per-group accumulators and the side sum, [M, K/128 + 1, N]."""
    pxq = _dev(xq, "xq", (torch.int8,))
    M, K = _2d(xq, "xq")
    dev = xq.device
    N = _2d(wq, "wq")[0]
    pwq = _dev(wq, "wq", (torch.int32,), (N, K // 8), dev)
    pwz = _dev(w_zero, "w_zero", (torch.float16,), (N, K // 128), dev)
    prc = _dev(records, "records", (torch.int64,), (N, K // 128), dev)
    pxs = _opt(x_scale, "x_scale", (torch.float32,), (M,), dev)
    pws = _opt(w_scale, "w_scale", (torch.float16,), (N, K // 128), dev)
    ps8 = _opt(s8, "s8", (torch.float32,), (N,), dev)
    shape = (M, K // 128 + 1, N) if out_dtype == torch.int32 else (M, N)
    y = _out(out, shape, out_dtype, dev)
    _call("gemm_w4a8_g128_outliers", pxq, pxs, pwq, pws, pwz, prc, ps8, M, N, K, y.data_ptr(),
          _DTYPE_CODE[out_dtype], _stream())
    return y


def gemm_w4a8_g128_outliers_panel(panel, x_scale, wq, w_scale, w_zero, records, s8, M,
                                  out_dtype=torch.bfloat16, out=None):
    """gemm_w4a8_g128_outliers on a token panel of M rows
    (quantize_per_token_i8_panel); int32 out_dtype returns [M, K/128 + 1, N]."""
    dev = panel.device
    pp = _dev(panel, "panel", (torch.uint8,), None, dev)
    N, K8 = _2d(wq, "wq")
    K = K8 * 8
    pwq = _dev(wq, "wq", (torch.int32,), (N, K // 8), dev)
    pwz = _dev(w_zero, "w_zero", (torch.float16,), (N, K // 128), dev)
    prc = _dev(records, "records", (torch.int64,), (N, K // 128), dev)
    pxs = _opt(x_scale, "x_scale", (torch.float32,), (M,), dev)
    pws = _opt(w_scale, "w_scale", (torch.float16,), (N, K // 128), dev)
    ps8 = _opt(s8, "s8", (torch.float32,), (N,), dev)
    shape = (M, K // 128 + 1, N) if out_dtype == torch.int32 else (M, N)
    y = _out(out, shape, out_dtype, dev)
    _call("gemm_w4a8_g128_outliers_panel", pp, panel.numel(), pxs, pwq, pws, pwz, prc, ps8, M, N,
          K, y.data_ptr(), _DTYPE_CODE[out_dtype], _stream())
    return y


def quantize_weight_u4_g128_sparse24(w: torch.Tensor):
    """w f32 [K, N] -> (wsp int32 [ceil(N/16), K/128, 16, 12], scale f16 [N, G],
    zero f16 [N, G]): 2:4 structured-sparse uint4 groups of 128."""
    pw = _dev(w, "w", (torch.float32,))
    K, N = _2d(w, "w")
    G = K // 128
    wsp = torch.empty(((N + 15) // 16, G, 16, 12), dtype=torch.int32, device=w.device)
    sc = torch.empty((N, G), dtype=torch.float16, device=w.device)
    zz = torch.empty((N, G), dtype=torch.float16, device=w.device)
    _call("quantize_weight_u4_g128_sparse24", pw, K, N, wsp.data_ptr(), sc.data_ptr(),
          zz.data_ptr(), _stream())
    return wsp, sc, zz


def gemm_w4a8_g128_sparse24(xq, x_scale, wsp, w_scale, w_zero, out_dtype=torch.bfloat16,
                            out=None):
    """W4A8 on 2:4 sparse uint4 weights; int32 out_dtype returns per-group acc [M, K/128, N]."""
    pxq = _dev(xq, "xq", (torch.int8,))
    M, K = _2d(xq, "xq")
    dev = xq.device
    N = _2d(w_zero, "w_zero")[0]
    pwz = _dev(w_zero, "w_zero", (torch.float16,), (N, K // 128), dev)
    pws_ = _dev(wsp, "wsp", (torch.int32,), ((N + 15) // 16, K // 128, 16, 12), dev)
    pxs = _opt(x_scale, "x_scale", (torch.float32,), (M,), dev)
    pws = _opt(w_scale, "w_scale", (torch.float16,), (N, K // 128), dev)
    shape = (M, K // 128, N) if out_dtype == torch.int32 else (M, N)
    y = _out(out, shape, out_dtype, dev)
    _call("gemm_w4a8_g128_sparse24", pxq, pxs, pws_, pws, pwz, M, N, K, y.data_ptr(),
          _DTYPE_CODE[out_dtype], _stream())
    return y


def _fold(name, x_cal, w):
    pxc = _dev(x_cal, "x_cal", (torch.float32,))
    T, K = _2d(x_cal, "x_cal")
    N = _2d(w, "w")[1]
    pw = _dev(w, "w", (torch.float32,), (K, N), x_cal.device)
    s = torch.empty((K,), dtype=torch.float32, device=w.device)
    wo = torch.empty_like(w)
    _call(name, pxc, T, pw, K, N, s.data_ptr(), wo.data_ptr(), _stream())
    return s, wo


def smoothquant_fold(x_cal: torch.Tensor, w: torch.Tensor):
    """SmoothQuant alpha=0.5 fold -> (s [K], diag(s) w)."""
    return _fold("smoothquant_fold", x_cal, w)


def awq_fold(x_cal: torch.Tensor, w: torch.Tensor):
    """AWQ alpha=0.5 fold -> (s [K], diag(s) w)."""
    return _fold("awq_fold", x_cal, w)


def apply_smoothing(x: torch.Tensor, s: torch.Tensor, out_dtype=torch.bfloat16):
    """x f32 [M, K] / s[K] per column, stored as out_dtype."""
    px = _dev(x, "x", (torch.float32,))
    M, K = _2d(x, "x")
    ps = _dev(s, "s", (torch.float32,), (K,), x.device)
    y = torch.empty((M, K), dtype=out_dtype, device=x.device)
    _call("apply_smoothing", px, M, K, ps, y.data_ptr(), _DTYPE_CODE[out_dtype], _stream())
    return y


KV_SEGMENT = 128   # positions per KV-cache scale segment


def quantize_kv_i8_segments(kv: torch.Tensor, out=None):
    """kv [T, H, D] (f32/f16/bf16) -> (kv_q int8 [T, H, D],
    kv_scale f32 [H, ceil(T/128), D]): one scale per head, 128-position
    segment and channel."""
    pk = _dev(kv, "kv", _FLOATS)
    if kv.dim() != 3:
        raise ValueError("kv must be [T, H, D]")
    T, H, D = kv.shape
    S = (T + KV_SEGMENT - 1) // KV_SEGMENT
    kq, ks = out if out is not None else (None, None)
    kq = _out(kq, (T, H, D), torch.int8, kv.device, "kv_q out")
    ks = _out(ks, (H, S, D), torch.float32, kv.device, "kv_scale out")
    _call("quantize_kv_i8_segments", pk, _DTYPE_CODE[kv.dtype], T, H, D, kq.data_ptr(),
          ks.data_ptr(), _stream())
    return kq, ks


def dequantize_kv_i8_segments(kv_q: torch.Tensor, kv_scale: torch.Tensor,
                              out_dtype=torch.bfloat16, out=None):
    """kv_q int8 [T, H, D] * kv_scale [H, t // 128, D] -> [T, H, D] of out_dtype."""
    pq = _dev(kv_q, "kv_q", (torch.int8,))
    if kv_q.dim() != 3:
        raise ValueError("kv_q must be [T, H, D]")
    T, H, D = kv_q.shape
    S = (T + KV_SEGMENT - 1) // KV_SEGMENT
    ps = _dev(kv_scale, "kv_scale", (torch.float32,), (H, S, D), kv_q.device)
    y = _out(out, (T, H, D), out_dtype, kv_q.device)
    _call("dequantize_kv_i8_segments", pq, ps, T, H, D, y.data_ptr(), _DTYPE_CODE[out_dtype],
          _stream())
    return y


# ------------------------------------------------------ measurement probes
# Not part of the layer: the ceilings its kernels are compared against.

def peak_stream_read(buf: torch.Tensor, nbytes: int, sink: torch.Tensor = None):
    """Read the first `nbytes` bytes of `buf` once (qg_peak_stream_read);
    returns the int32 sink tensor the kernel writes."""
    _dev(buf, "buf", (torch.uint8, torch.int8))
    if nbytes > buf.numel():
        raise ValueError("nbytes exceeds the buffer")
    n = load().qg_peak_stream_read_sink(nbytes)
    sink = _out(sink, (n,), torch.int32, buf.device, "sink")
    _call("qg_peak_stream_read", buf.data_ptr(), nbytes, sink.data_ptr(), _stream())
    return sink


def peak_mfma(kind: int, iters: int, workgroups: int, clocks=None, sink=None):
    """Matrix-core loop (qg_peak_mfma); returns (clocks uint64-as-int64
    [4 * workgroups, 2], sink) -- per wave the shader-clock and 100 MHz
    real-time counters elapsed over its loop."""
    dev = torch.device("cuda", torch.cuda.current_device())
    clocks = _out(clocks, (4 * workgroups, 2), torch.int64, dev, "clocks")
    sink = _out(sink, (256 * workgroups,), torch.int32, dev, "sink")
    _call("qg_peak_mfma", kind, iters, workgroups, clocks.data_ptr(), sink.data_ptr(), _stream())
    return clocks, sink


def peak_mfma_ops(kind: int, iters: int, workgroups: int) -> int:
    return int(load().qg_peak_mfma_ops(kind, iters, workgroups))


def peak_empty():
    """One empty workgroup (qg_peak_empty): the fixed cost of a launch."""
    _call("qg_peak_empty", _stream())
