"""The seeded input generator: determinism, shapes and stated structure."""
import numpy as np

from workloads import WORKLOADS, by_name, draw, ragged, f32_to_bf16_bits, bf16_bits_to_f32


def test_workload_table():
    assert [w.index for w in WORKLOADS] == [1, 2, 3, 4, 5]
    assert by_name("w8a8_prefill").M == 4096
    assert by_name("w4a8_ffn_down").groups == 86
    assert by_name("w4a16_qkv").groups == 32


def test_draw_deterministic_and_structured():
    wl = by_name("w8a8_tiny")
    a, b = draw(wl), draw(wl)
    assert np.array_equal(a["x"], b["x"]) and np.array_equal(a["w"], b["w"])
    assert a["x"].shape == (16, 512) and a["w"].shape == (512, 512)
    assert len(a["outliers"]) == 4
    col_amax = np.abs(a["x"]).max(axis=0)
    assert set(np.argsort(col_amax)[-4:]) == set(a["outliers"].tolist())
    assert 0.018 < a["w"].std() < 0.022
    c = draw(wl, seed_offset=1)
    assert not np.array_equal(a["x"], c["x"])


def test_outlier_channels_shared_with_calibration():
    wl = ragged(by_name("w8a8_decode_ffn_up"), 4, 4096, 64)
    d = draw(wl)
    assert len(d["outliers"]) == 41 and d["x_cal"].shape == (512, 4096)
    top = np.argsort(np.abs(d["x_cal"]).max(axis=0))[-41:]
    assert set(top.tolist()) == set(d["outliers"].tolist())


def test_bf16_cast_rne():
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5], np.float32)
    b = f32_to_bf16_bits(x)
    assert bf16_bits_to_f32(b).tolist() == [1.0, 1.0, 1.0 + 2.0 ** -6, -2.5]
