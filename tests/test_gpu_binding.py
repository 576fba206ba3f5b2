"""The Python binding refuses tensors whose shapes or dtypes disagree with the
sizes it passes to the library (which trusts them), before any launch."""
import pytest
import torch

import block_quantized_flashattention_amd as qfa

pytestmark = pytest.mark.gpu


def _t(shape, dtype):
    return torch.zeros(shape, dtype=dtype, device="cuda")


def test_fwd_rejects_mismatched_tensors():
    i8, u8, f32, f16 = torch.int8, torch.uint8, torch.float32, torch.float16
    good = dict(q_codes=_t((1, 2, 300, 128), i8), q_scales=_t((1, 2, 3), f32),
                k_codes=_t((1, 2, 300, 128), i8), k_scales=_t((1, 2, 2), f32),
                v_codes=_t((1, 2, 300, 128), i8), v_scales=_t((1, 2, 2), f32))
    kw = dict(q_qtype="int8", k_qtype="int8", v_qtype="int8", q_block=128, kv_block=256,
              softmax_scale=0.1, causal=True)
    qfa.fwd(**good, **kw)  # the well-formed call runs
    torch.cuda.synchronize()
    bad = [
        dict(q_scales=_t((1, 2, 2), f32)),                    # too few Q blocks
        dict(k_scales=_t((1, 2, 3), f32)),                    # wrong K block count
        dict(v_scales=_t((1, 2, 2), f16)),                    # V scale dtype != K scale dtype
        dict(v_codes=_t((1, 2, 299, 128), i8)),               # V rows != K rows
        dict(v_codes=_t((1, 2, 300, 64), u8)),                # INT4-shaped V with INT8 v_qtype
        dict(k_codes=_t((1, 2, 300, 128), u8)),               # code dtype vs qtype
    ]
    for b in bad:
        with pytest.raises(ValueError):
            qfa.fwd(**{**good, **b}, **kw)
    with pytest.raises(ValueError):
        qfa.fwd(**good, **kw, out=_t((1, 2, 300, 64), f16))   # output shape
    with pytest.raises(ValueError):
        qfa.fwd(**{**good, "v_codes": _t((1, 2, 300, 64), u8)}, **{**kw, "v_qtype": "int4"},
                out=_t((1, 2, 299, 128), f16))


def test_decode_and_append_reject_mismatched_tensors():
    f16 = torch.float16
    q = _t((2, 4, 1, 128), f16)
    kc = _t((2, 2, 2048, 128), torch.int8)
    ks = _t((2, 2, 8), f16)
    lens = torch.full((2,), 100, dtype=torch.int32, device="cuda")
    kw = dict(kv_qtype="int8", kv_block=256, softmax_scale=0.1)
    qfa.decode(q, kc, kc, ks, ks, lens, **kw)
    torch.cuda.synchronize()
    with pytest.raises(ValueError):
        qfa.decode(q, kc, kc, ks, _t((2, 2, 8), torch.float32), lens, **kw)
    with pytest.raises(ValueError):
        qfa.decode(q, kc, kc, _t((2, 2, 7), f16), ks, lens, **kw)
    with pytest.raises(ValueError):
        qfa.decode(q, kc, kc, ks, ks, lens[:1], **kw)
    with pytest.raises(ValueError):
        qfa.decode(q, kc, kc, ks, ks, lens, kv_qtype="int4", kv_block=256, softmax_scale=0.1)
    x = _t((2, 2, 128), f16)
    pos = torch.zeros(2, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        qfa.kv_append(x, pos, kc, _t((2, 2, 9), f16), 256, "int8")
    with pytest.raises(ValueError):
        qfa.kv_append(x, pos, kc, ks, 256, "int4")


def test_block_quant_rejects_mismatched_outputs():
    x = _t((1, 2, 300, 128), torch.float16)
    with pytest.raises(ValueError):
        qfa.block_quant(x, 128, "int8", scales=_t((1, 2, 2), torch.float32))
    with pytest.raises(ValueError):
        qfa.block_quant(x, 128, "int4", codes=_t((1, 2, 300, 128), torch.uint8))
    with pytest.raises(ValueError):
        qfa.block_quant(x, 128, "fp8", codes=_t((1, 2, 300, 128), torch.int8))
