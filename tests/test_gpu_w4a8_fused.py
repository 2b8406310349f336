"""GPU parity of the quantize + W4A8 call (quantize_gemm_w4a8_g128).

Its codes and scales must be those of quantize_per_token_i8 and its int32
per-group accumulators those of gemm_w4a8_g128, bit for bit, whichever form
the library picks (the panel pair quantize_per_token_i8_panel +
gemm_w4a8_g128_panel on layers of 257-383 weight blocks, the plain
kernels otherwise); the panel pair is also run explicitly on every shape the
panel takes.  Scaled outputs are held to the oracle with the W4A8 rounding
bound.  The panel's layout is checked byte for byte against its documented
definition.
"""
import numpy as np
import pytest
import torch

import bit_quantized_gemm_int8_amd as qg
import oracle
from tests.gpu_util import to_dev, to_np, out_f64
from tests.tolerance import assert_close

pytestmark = pytest.mark.gpu

XDT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
YDT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def _weights(rng, K, N):
    w = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    return oracle.quantize_weight_u4_g128(w)


def _x(seed, M, K, xdt):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.randn((M, K), generator=g, device="cuda")
    x[:, :3] *= 20.0                                        # a few large channels
    if M > 2:
        x[1] = 0.0                                          # an all-zero token
    return x.to(XDT[xdt])


def _floor(xq, sx, packed, sc, zz):
    acc = oracle.gemm_w4a8_g128_acc(xq, packed, zz).astype(np.float64)       # [M, G, N]
    s = sc.astype(np.float64).T
    B = np.abs(sx.astype(np.float64))[:, None] * np.abs(acc * s[None]).sum(axis=1)
    return (acc.shape[1] + 10) * 2.0 ** -24 * B


# every panel row class (1, 2, 4, 8, 16 rows), 16, 8, 4, 2 and 1 waves,
# runs of 1..4 units, odd group counts (a unit's second group past K), half a
# unit (K = 128), more and fewer than 256 weight blocks, ragged N, the longest
# K the panel takes (16384); past it: 17 rows, K > 16384
SHAPES = [(16, 4096, 11008), (16, 11008, 4096), (1, 12288, 4096), (3, 100, 2048),
          (5, 17, 1152), (2, 48, 14336), (8, 33, 16384), (4, 8200, 16384), (12, 300, 1024),
          (7, 1000, 896), (9, 520, 4224), (6, 16, 2432), (9, 40, 640), (3, 40, 256),
          (2, 30, 128), (16, 5000, 384),
          (1, 4096, 11008), (17, 64, 1024), (2, 40, 16512)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("xdt", ["bf16", "f32"])
def test_codes_and_group_acc_bitwise(M, N, K, xdt):
    rng = np.random.default_rng(M * 7 + N + K)
    packed, sc, zz = _weights(rng, K, N)
    wq, s_d, z_d = to_dev(packed), to_dev(sc), to_dev(zz)
    x = _x(M * 1000 + N + K, M, K, xdt)
    need = qg.quantize_gemm_w4a8_g128_workspace_bytes(M, N, K)
    print(f"w4a8 fused M={M} N={N} K={K} x={xdt} workspace={need}", flush=True)
    acc, xq, xs = qg.quantize_gemm_w4a8_g128(x, wq, None, z_d, out_dtype=torch.int32)
    xq2, xs2 = qg.quantize_per_token_i8(x)
    acc2 = qg.gemm_w4a8_g128(xq2, None, wq, None, z_d, out_dtype=torch.int32)
    torch.cuda.synchronize()
    assert torch.equal(xs, xs2)
    assert torch.equal(xq, xq2)
    assert torch.equal(acc, acc2)
    if qg.quantize_per_token_i8_panel_bytes(M, K):   # the panel pair, whatever the choice
        panel, xq3, xs3 = qg.quantize_per_token_i8_panel(x)
        acc3 = qg.gemm_w4a8_g128_panel(panel, None, wq, None, z_d, M, out_dtype=torch.int32)
        torch.cuda.synchronize()
        assert torch.equal(xq3, xq2) and torch.equal(xs3, xs2)
        assert torch.equal(acc3, acc2)
    if M * N * K <= 16 * 4096 * 4096:
        np.testing.assert_array_equal(to_np(acc), oracle.gemm_w4a8_g128_acc(to_np(xq), packed, zz))


@pytest.mark.parametrize("ydt", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("M,N,K", [(8, 11008, 4096), (1, 12288, 4096), (4, 8200, 16384),
                                   (16, 4096, 11008), (9, 40, 640)])
def test_scaled_against_oracle(ydt, M, N, K):
    rng = np.random.default_rng(3 * M + N + K)
    packed, sc, zz = _weights(rng, K, N)
    x = _x(M + N + K, M, K, "bf16")
    print(f"w4a8 fused scaled M={M} N={N} K={K} y={ydt}", flush=True)
    y, xq, xs = qg.quantize_gemm_w4a8_g128(x, to_dev(packed), to_dev(sc), to_dev(zz),
                                           out_dtype=YDT[ydt])
    torch.cuda.synchronize()
    xq_ref, xs_ref = oracle.quantize_per_token_i8(x.float().cpu().numpy())
    np.testing.assert_array_equal(to_np(xq), xq_ref)
    np.testing.assert_array_equal(to_np(xs), xs_ref)
    yref = oracle.gemm_w4a8_g128(xq_ref, xs_ref, packed, sc, zz)
    n = assert_close(out_f64(y), yref, ydt, floor=_floor(xq_ref, xs_ref, packed, sc, zz),
                     what=f"fused w4a8 {ydt}")
    print(f"fused w4a8 {ydt} {M}x{N}x{K}: {n} of {yref.size} outputs within the floor only")


@pytest.mark.parametrize("xdt", ["f16", "f32"])
def test_input_dtypes(xdt):
    M, N, K = 8, 4096, 4096
    rng = np.random.default_rng(11)
    packed, sc, zz = _weights(rng, K, N)
    x = _x(12, M, K, xdt)
    acc, xq, xs = qg.quantize_gemm_w4a8_g128(x, to_dev(packed), None, to_dev(zz),
                                             out_dtype=torch.int32)
    xq2, xs2 = qg.quantize_per_token_i8(x)
    torch.cuda.synchronize()
    assert torch.equal(xq, xq2) and torch.equal(xs, xs2)
    np.testing.assert_array_equal(to_np(acc), oracle.gemm_w4a8_g128_acc(to_np(xq), packed, zz))


def test_dirty_workspace_and_smaller_second_call():
    """Panel rows past M are written by the quantizer, not left over: a
    workspace full of stale bytes, then reused by a call with fewer rows,
    gives the same accumulators (one-call form and the explicit pair)."""
    N, K = 4160, 4096
    rng = np.random.default_rng(5)
    packed, sc, zz = _weights(rng, K, N)
    wq, z_d = to_dev(packed), to_dev(zz)
    nbytes = qg.quantize_gemm_w4a8_g128_workspace_bytes(16, N, K)
    assert nbytes == qg.quantize_per_token_i8_panel_bytes(16, K) > 0
    ws = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda")
    for M in (16, 3):
        x = _x(40 + M, M, K, "bf16")
        acc, xq, _ = qg.quantize_gemm_w4a8_g128(x, wq, None, z_d, out_dtype=torch.int32,
                                                workspace=ws)
        torch.cuda.synchronize()
        ref = oracle.gemm_w4a8_g128_acc(to_np(xq), packed, zz)
        np.testing.assert_array_equal(to_np(acc), ref)
        ws.random_(0, 256)
        qg.quantize_per_token_i8_panel(x, panel=ws)
        acc2 = qg.gemm_w4a8_g128_panel(ws, None, wq, None, z_d, M, out_dtype=torch.int32)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_np(acc2), ref)


def test_workspace_too_small_is_rejected():
    M, N, K = 4, 4160, 4096
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    wq = torch.zeros((N, K // 8), dtype=torch.int32, device="cuda")
    z = torch.zeros((N, K // 128), dtype=torch.float16, device="cuda")
    need = qg.quantize_gemm_w4a8_g128_workspace_bytes(M, N, K)
    assert need == 32 * 2112
    ws = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(RuntimeError, match="SHAPE"):
        qg.quantize_gemm_w4a8_g128(x, wq, z, z, workspace=ws)


def test_codes_only_when_n_is_zero():
    x = torch.randn((4, 256), device="cuda").to(torch.bfloat16)
    wq = torch.empty((0, 32), dtype=torch.int32, device="cuda")
    z = torch.empty((0, 2), dtype=torch.float16, device="cuda")
    y, xq, xs = qg.quantize_gemm_w4a8_g128(x, wq, z, z)
    xq2, xs2 = qg.quantize_per_token_i8(x)
    torch.cuda.synchronize()
    assert y.shape == (4, 0) and torch.equal(xq, xq2) and torch.equal(xs, xs2)


@pytest.mark.parametrize("N", [4160, 11008])   # the panel pair; the plain quantizer + wide GEMM
def test_graph_replay(N):
    M, K = 8, 4096
    rng = np.random.default_rng(9)
    packed, sc, zz = _weights(rng, K, N)
    wq, s_d, z_d = to_dev(packed), to_dev(sc), to_dev(zz)
    x = _x(77, M, K, "bf16")
    ws = torch.empty(max(qg.quantize_gemm_w4a8_g128_workspace_bytes(M, N, K), 1), dtype=torch.uint8,
                     device="cuda")
    y, xq, xs = qg.quantize_gemm_w4a8_g128(x, wq, s_d, z_d, workspace=ws)
    torch.cuda.synchronize()
    ref = y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qg.quantize_gemm_w4a8_g128(x, wq, s_d, z_d, out=y, xq_out=(xq, xs), workspace=ws)
    for _ in range(3):
        y.zero_()
        ws.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16))


def _panel_expected(xq, M, K):
    """The documented panel layout, assembled from the codes: entries
    [g][h][r][j] of the 16 codes at k = 128 g + 32 j + 16 h + i in the order
    i = 0 2 4 6 1 3 5 7 8 10 12 14 9 11 13 15, rows up to M rounded to a
    power of two (zeros past M), then int32 sums [g][16]."""
    G = K // 128
    m = 1 if M <= 1 else 2 if M <= 2 else 4 if M <= 4 else 8 if M <= 8 else 16
    order = np.array([0, 2, 4, 6, 1, 3, 5, 7, 8, 10, 12, 14, 9, 11, 13, 15])
    rows = np.zeros((m, K), np.int8)
    rows[:M] = xq
    t = rows.reshape(m, G, 4, 2, 16)[..., order]           # [r][g][j][h][i]
    panel = t.transpose(1, 3, 0, 2, 4).reshape(-1)          # [g][h][r][j][i]
    sums = np.zeros((G, 16), np.int32)
    sums[:, :M] = xq.astype(np.int32).reshape(M, G, 128).sum(axis=2).T
    return panel.view(np.uint8), sums


@pytest.mark.parametrize("M,K,xdt", [(1, 128, "bf16"), (2, 4096, "f16"), (3, 1152, "f32"),
                                     (8, 16384, "bf16"), (13, 11008, "bf16"), (16, 4096, "f32")])
def test_panel_layout(M, K, xdt):
    x = _x(M * 3 + K, M, K, xdt)
    need = qg.quantize_per_token_i8_panel_bytes(M, K)
    print(f"panel layout M={M} K={K} x={xdt} bytes={need}", flush=True)
    panel = torch.randint(0, 256, (need,), dtype=torch.uint8, device="cuda")   # stale bytes
    panel, xq, xs = qg.quantize_per_token_i8_panel(x, panel=panel)
    xq2, xs2 = qg.quantize_per_token_i8(x)
    torch.cuda.synchronize()
    assert torch.equal(xq, xq2) and torch.equal(xs, xs2)
    codes, sums = _panel_expected(to_np(xq), M, K)
    got = to_np(panel)
    G = K // 128
    np.testing.assert_array_equal(got[:codes.size], codes)
    np.testing.assert_array_equal(got[2048 * G:2048 * G + 64 * G].view(np.int32).reshape(G, 16),
                                  sums)


def test_one_panel_feeds_several_gemms():
    """Quantize once, then the projections sharing that input (three weight
    matrices of different widths, int32 and bf16 outputs)."""
    M, K = 4, 4096
    x = _x(321, M, K, "bf16")
    panel, xq, xs = qg.quantize_per_token_i8_panel(x, write_xq=True)
    panel2, xq_none, xs2 = qg.quantize_per_token_i8_panel(x, write_xq=False)
    rng = np.random.default_rng(8)
    for N in (4096, 1024, 11008):
        packed, sc, zz = _weights(rng, K, N)
        wq, s_d, z_d = to_dev(packed), to_dev(sc), to_dev(zz)
        print(f"panel gemm M={M} N={N} K={K}", flush=True)
        acc = qg.gemm_w4a8_g128_panel(panel2, None, wq, None, z_d, M, out_dtype=torch.int32)
        acc2 = qg.gemm_w4a8_g128(xq, None, wq, None, z_d, out_dtype=torch.int32)
        y = qg.gemm_w4a8_g128_panel(panel, xs, wq, s_d, z_d, M, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(acc, acc2)
        xq_np, xs_np = to_np(xq), to_np(xs)
        yref = oracle.gemm_w4a8_g128(xq_np, xs_np, packed, sc, zz)
        assert_close(out_f64(y), yref, "bf16", floor=_floor(xq_np, xs_np, packed, sc, zz),
                     what="panel w4a8")
    assert xq_none is None and torch.equal(xs, xs2)
