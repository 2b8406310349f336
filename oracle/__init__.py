"""CPU oracle for the quantized linear layer -- TEST INFRASTRUCTURE ONLY.

Plain, slow and obviously correct NumPy code written from the pages.  It is
imported only by tests/, by __graft_entry__.smoke() and by the cpu_baseline
leg of bench.py; the library under bit_quantized_gemm_int8_amd/ never uses it
and shares no code with it.

Every value is the plain definition of what the method computes:
  * quantization (codes, scales, zero points) in IEEE float32 with correctly
    rounded division and round-half-to-even, as the GPU path decides the same
    integers in the same precision;
  * contractions exactly in integers (int64, or float64 on integer-valued
    operands where every partial sum is an integer below 2**53);
  * epilogues in float64 from the exact accumulators ("y_exact").

Sources (cited by page title and section):
  「第4章：量化」 §1.1 (affine quantize/dequantize), §1.2 (symmetric and
  asymmetric scale), §1.3 (per-channel / per-group / per-token granularity),
  §2.2 (SmoothQuant fold), §3.2-3.3 (4-bit, group 128, zero point configs);
  「Quantization & Flash Attention」 §2.2-2.3 (AWQ per-channel fold);
  「LLM推理降本五要素」 §2.2 (group-wise W4A8 with per-group scale and zero;
  the top 2% of each group kept in INT8 on a side path; §3.2 2:4 structured
  sparsity followed by 4-bit group quantization),
  §5.2 (round-then-clamp to int8; KV-cache position segments of 128 tokens
  with per-channel scales).

Parity status: every function here is pinned by tests/test_oracle_*.py
against closed forms, invariants, brute force on tiny inputs and the
size figures the pages print; none is "parity unpinned".
"""
from .quant import (quantize_per_token_i8, quantize_weight_i8_per_channel,
                    quantize_weight_u4_g128, pack_u4, unpack_u4,
                    f16_round_up, dequant_u4_g128, to_f32)
from .gemm import (gemm_w8a8_acc, gemm_w8a8, gemm_w4a8_g128_acc, gemm_w4a8_g128,
                   gemm_w4a16_g128_partials, gemm_w4a16_g128)
from .fold import (smoothquant_scales, awq_scales, fold_weight, fold_activation)

__all__ = [
    "quantize_per_token_i8", "quantize_weight_i8_per_channel",
    "quantize_weight_u4_g128", "pack_u4", "unpack_u4", "f16_round_up",
    "dequant_u4_g128", "to_f32",
    "gemm_w8a8_acc", "gemm_w8a8", "gemm_w4a8_g128_acc", "gemm_w4a8_g128",
    "gemm_w4a16_g128_partials", "gemm_w4a16_g128",
    "smoothquant_scales", "awq_scales", "fold_weight", "fold_activation",
]
from .kv import quantize_kv_segments, dequantize_kv_segments
from .outlier import (quantize_weight_u4_g128_outliers, gemm_w4a8_g128_outliers,
                      gemm_w4a8_g128_outlier_acc, decode_records, select_outliers)
from .sparse24 import (quantize_weight_u4_g128_sparse24, gemm_w4a8_g128_sparse24,
                       gemm_w4a8_g128_sparse24_acc, expand_sparse24, prune_2_4)
