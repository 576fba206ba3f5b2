"""CPU oracle for block-quantized FlashAttention -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg
may import this package. The product path (``block_quantized_flashattention_amd``)
never imports it, and this package imports nothing from the product path: the
two share no code.

What it computes is the plain definition of the method, slowly and in the
open:

* ``quant``      -- symmetric per-block amax quantization to INT8, FP8 e4m3fn or
                    nibble-packed INT4, with the quotient formed in IEEE fp32,
                    optionally after an exact rotation rounded once to 16 bits,
                    and the append of one token into a quantized KV cache;
* ``attention``  -- exact softmax attention in float64 on the dequantized values
                    (prefill, causal or not, grouped-query heads);
* ``decode``     -- one query token against a quantized KV cache of per-sequence
                    length, in float64.

Pages cited in docstrings (by title and section; titles shortened):

* [FA-INT8/INT4]  "FlashAttention INT8/INT4 quantization" blog post on the
                   ops-transformer library (hwcomputing.csdn.net/6a140ce2...).
* [Edge-FA]       "FlashAttention在端侧设备的部署：手机/IoT优化" (ai6s.net/6a157c77...).
* [OT-Quant]      ops-transformer INT8/INT4 quantized-inference article
                   (2048ai.net/6989721354...).
* [Ascend-INT8]   "INT8 量化算子：让大模型在昇腾NPU上减肥不掉肉"
                   (hwcomputing.csdn.net/6a0dcc10...).
* [MindIE-SD]     MindIE-SD "量化" feature doc, FA quantization part
                   (gitcode.com/Ascend/MindIE-SD, docs/zh/features/quantization.md).

Every function here is pinned by ``tests/test_oracle_*.py`` against values the
pages fix, hand-computed cases, library routines and closed forms.
"""
from .quant import (QMAX, bf16_round, block_quant, code_values, dequantize, e4m3fn_decode,
                    e4m3fn_encode, fp16_round, kv_append, pack_int4, quantize_with_scale,
                    rotate16, rotate_block_quant, unpack_int4)
from .attention import attention, attention_rows, decode

__all__ = [
    "QMAX", "bf16_round", "block_quant", "code_values", "dequantize", "e4m3fn_decode",
    "e4m3fn_encode", "fp16_round", "kv_append", "pack_int4", "quantize_with_scale",
    "rotate16", "rotate_block_quant", "unpack_int4", "attention",
    "attention_rows", "decode",
]
