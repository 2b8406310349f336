"""GPU parity of the KV-cache INT8 quantizer (128-position segments x per-channel
scales) against the oracle: codes and scales bit for bit (both sides decide
them in binary32 with correctly rounded division and half-to-even rounding);
dequantized values within one rounding of the output format of the exact
product code * scale."""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_int8_amd as qg
import oracle
from tests.gpu_util import to_dev, to_np, out_f64
from tests.tolerance import ulp
from workloads import KV_WORKLOADS, draw_kv, f32_to_bf16_bits, f32_to_f16

pytestmark = pytest.mark.gpu

_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _cache(x32, fmt):
    """Stored cache in `fmt` plus the exact float32 values the oracle sees."""
    if fmt == "f32":
        return to_dev(x32), x32
    if fmt == "bf16":
        b = f32_to_bf16_bits(x32)
        return to_dev(b, "bf16"), oracle.to_f32(b, "bf16")
    h = f32_to_f16(x32)
    return to_dev(h), oracle.to_f32(h, "f16")


def _check(x32, fmt):
    kd, ko = _cache(x32, fmt)
    print(f"kv quant T,H,D={tuple(x32.shape)} {fmt}", flush=True)
    kq, ks = qg.quantize_kv_i8_segments(kd)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_kv_segments(ko)
    np.testing.assert_array_equal(to_np(ks), s_ref)
    np.testing.assert_array_equal(to_np(kq), q_ref)
    return kq, ks, q_ref, s_ref


def _draw(T, H, D, seed):
    return draw_kv(KV_WORKLOADS[0], T=T, H=H, D=D) if seed is None else \
        np.random.default_rng(seed).standard_normal((T, H, D)).astype(np.float32)


# (T, H, D, fmt): several segments with ragged last ones, every supported
# head dim class (D / 8 dividing 256 or not: idle threads), one position,
# exactly one segment, one position past a segment
CASES = [
    (300, 4, 128, "bf16"), (128, 2, 128, "bf16"), (129, 3, 128, "f16"), (1, 2, 128, "f32"),
    (257, 2, 64, "bf16"), (200, 2, 256, "bf16"), (131, 3, 16, "f32"), (140, 2, 32, "f16"),
    (200, 2, 96, "bf16"), (150, 3, 80, "f32"), (260, 1, 112, "f16"), (384, 5, 240, "bf16"),
    (127, 7, 48, "bf16"),
    # three 64-channel slices per head (D = 192) and a head count that is not
    # a power of two: the work-item index is divided by both
    (300, 3, 192, "bf16"), (129, 5, 192, "f16"), (130, 40, 128, "bf16"),
]


@pytest.mark.parametrize("T,H,D,fmt", CASES)
def test_kv_quant_parity(T, H, D, fmt):
    _check(_draw(T, H, D, None), fmt)


def test_kv_quant_zero_channels_and_segments():
    x = _draw(300, 3, 128, None)
    x[:, 1, 5] = 0.0                 # a channel zero in every segment
    x[128:256, 2, :] = 0.0           # a whole (segment, head) zero
    x[256:, 0, 7] = 0.0              # zero only in the last, partial segment
    kq, ks, _, s_ref = _check(x, "bf16")
    s = to_np(ks)
    assert (s[1, :, 5] == 0).all() and (s[2, 1, :] == 0).all() and s[0, 2, 7] == 0
    assert (to_np(kq)[128:256, 2, :] == 0).all()


def test_kv_quant_every_channel_reaches_127():
    x = _draw(256, 2, 128, 5)
    kq, _, _, _ = _check(x, "f32")
    q = to_np(kq).astype(np.int32).reshape(2, 128, 2, 128)    # [segment, position, head, channel]
    assert (np.abs(q).max(axis=1) == 127).all()


def test_kv_quant_full_size():
    wl = KV_WORKLOADS[1]
    _check(draw_kv(wl), wl.dtype)


def test_kv_value_per_token_variant():
    """Values quantized per position and head over the head dim: the per-token
    quantizer on the cache viewed as [T*H][D]."""
    x = _draw(200, 4, 128, 11)
    kd, ko = _cache(x, "bf16")
    vq, vs = qg.quantize_per_token_i8(kd.view(200 * 4, 128))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_per_token_i8(ko.reshape(200 * 4, 128))
    np.testing.assert_array_equal(to_np(vs), s_ref)
    np.testing.assert_array_equal(to_np(vq), q_ref)


@pytest.mark.parametrize("T,H,D", [(300, 4, 128), (129, 3, 80), (1, 1, 16), (4096, 32, 128)])
@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
def test_kv_dequant(T, H, D, out):
    x = draw_kv(KV_WORKLOADS[0], T=T, H=H, D=D)
    kd, ko = _cache(x, "bf16")
    kq, ks = qg.quantize_kv_i8_segments(kd)
    y = qg.dequantize_kv_i8_segments(kq, ks, out_dtype=_TORCH[out])
    torch.cuda.synchronize()
    exact = oracle.dequantize_kv_segments(to_np(kq), to_np(ks))
    got = out_f64(y)
    d = np.abs(got - exact)
    if out == "f32":
        bound = np.abs(exact) * 2.0 ** -24          # one binary32 rounding
    else:
        bound = ulp(exact, out)                      # binary32 then the output format
    bad = d > bound
    assert not bad.any(), f"{int(bad.sum())} of {bad.size} values out of tolerance"


def test_kv_empty_cache():
    kd = torch.empty((0, 4, 128), dtype=torch.bfloat16, device="cuda")
    kq, ks = qg.quantize_kv_i8_segments(kd)
    y = qg.dequantize_kv_i8_segments(kq, ks)
    torch.cuda.synchronize()
    assert kq.shape == (0, 4, 128) and ks.shape == (4, 0, 128) and y.shape == (0, 4, 128)


def test_kv_rejects_bad_head_dim():
    kd = torch.zeros((4, 2, 120), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError, match="SHAPE"):
        qg.quantize_kv_i8_segments(kd)


def test_kv_graph_replay_matches_eager():
    x = draw_kv(KV_WORKLOADS[0])
    kd, _ = _cache(x, "bf16")
    kq, ks = qg.quantize_kv_i8_segments(kd)
    y = qg.dequantize_kv_i8_segments(kq, ks)
    torch.cuda.synchronize()
    rq, rs, ry = kq.clone(), ks.clone(), y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qg.quantize_kv_i8_segments(kd, out=(kq, ks))
        qg.dequantize_kv_i8_segments(kq, ks, out=y)
    for _ in range(3):
        kq.zero_(); ks.zero_(); y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(kq, rq) and torch.equal(ks, rs)
        assert torch.equal(y.view(torch.int16), ry.view(torch.int16))


def test_kv_quant_golden_ties():
    """The hand-worked tie cases (s = 2^e, x/s exact) laid along the positions of
    one channel: half-way values round to even."""
    import os
    rows = []
    for line in open(os.path.join(os.path.dirname(__file__), "golden", "per_token_ties.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            e, vals, codes = [p.split() for p in line.split("|")]
            rows.append((int(e[0]), [float(v) for v in vals], [int(c) for c in codes]))
    x = np.zeros((128, 1, 16), np.float32)
    for ch, (e, vals, codes) in enumerate(rows):
        x[: len(vals), 0, ch] = np.array(vals) * 2.0 ** e
    for fmt in ("f32", "bf16"):
        kd, _ = _cache(x, fmt)
        kq, ks = qg.quantize_kv_i8_segments(kd)
        torch.cuda.synchronize()
        for ch, (e, vals, codes) in enumerate(rows):
            assert float(to_np(ks)[0, 0, ch]) == 2.0 ** e
            assert to_np(kq)[: len(vals), 0, ch].tolist() == codes


def test_kv_quant_near_ties():
    """Values on and within a few ulps of x/s = k + 1/2 for scales that are not
    powers of two: the range where the fast reciprocal path must hand over to
    the correctly rounded division."""
    rng = np.random.default_rng(77)
    T, H, D = 256, 2, 64
    x = np.zeros((T, H, D), np.float32)
    for h in range(H):
        for d in range(D):
            amax = np.float32(rng.uniform(0.01, 100.0))
            s = np.float32(amax / np.float32(127.0))
            k = rng.integers(-126, 126, T).astype(np.float64) + 0.5
            ties = (k * np.float64(s)).astype(np.float32)              # nearest float to (k + 1/2) s
            ulps = rng.integers(-4, 5, T).astype(np.int32)
            ties = (ties.view(np.int32) + ulps * np.sign(ties).astype(np.int32)).view(np.float32)
            ties = np.clip(ties, -amax, amax)
            ties[0] = amax                                              # position 0 (segment 0) and
            ties[128] = -amax                                           # 128 (segment 1) set the max
            x[:, h, d] = ties
    _check(x, "f32")
