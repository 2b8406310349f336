"""Pin the storage formats against the weight-size figures the pages print.

The packed uint4 codes the oracle produces take exactly a quarter of the
fp16 bytes and int8 codes exactly half; scaled to a 70B-parameter model that
gives the 140 GB -> 35 GB (-75%) and /2 figures in tests/golden/size_claims.txt.
The g=128 fp16 scale and zero add 32 bits per 128 weights (4.25 bits per
weight in total), which the pages leave out of their figure.
"""
import os

import numpy as np

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "size_claims.txt")


def _claims():
    out = {}
    for line in open(GOLD):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            out[k] = float(v)
    return out


def test_size_claims():
    c = _claims()
    K, N = 1024, 384
    w = (np.random.default_rng(0).standard_normal((K, N)) * 0.02).astype(np.float32)
    packed, sc, zz = oracle.quantize_weight_u4_g128(w)
    q8, s8 = oracle.quantize_weight_i8_per_channel(w)
    fp16_bytes = K * N * 2
    assert packed.nbytes * 4 == fp16_bytes
    assert q8.nbytes * 2 == fp16_bytes
    bits_per_weight_codes = packed.nbytes * 8 / (K * N)
    bits_per_weight_meta = (sc.nbytes + zz.nbytes) * 8 / (K * N)
    assert bits_per_weight_codes == 4.0 and bits_per_weight_meta == 0.25
    P = c["params"]
    assert P * 16 / 8 / 1e9 == c["fp16_GB"]
    assert P * bits_per_weight_codes / 8 / 1e9 == c["int4_GB"]
    assert P * 8 / 8 / 1e9 == c["int8_GB"]
    assert 1 - c["int4_GB"] / c["fp16_GB"] == c["int4_reduction"]
    # with the group metadata the 70B model needs 37.1875 GB
    assert P * (bits_per_weight_codes + bits_per_weight_meta) / 8 / 1e9 == 37.1875
