"""GPU parity of qfa_fwd against the oracle's float64 attention on the same
codes: small cases spanning several tiles with ragged tails, both layouts,
every code type, and the full-size workloads on sampled rows."""
import numpy as np
import pytest
import torch

import block_quantized_flashattention_amd as qfa
import oracle
import qfa_workloads as wl
from gpu_util import assert_close, prefill_parity, say

pytestmark = pytest.mark.gpu


def test_tiny_workload_all_rows():
    prefill_parity(wl.TINY)


SMALL = [
    wl.scaled(wl.INT8_CAUSAL, name="int8_causal_h2_s300", Hq=2, Hkv=2, S=300),
    wl.scaled(wl.INT8_CAUSAL, name="int8_causal_h2_s300_d64", Hq=2, Hkv=2, S=300, D=64,
              softmax_scale=0.125, k_outlier_channels=2),
    wl.scaled(wl.INT8_CAUSAL, name="int8_noncausal_s257", Hq=3, Hkv=3, S=257, causal=False),
    wl.scaled(wl.FP8_ROT, name="fp8_rot_b1_h2_s333", B=1, Hq=2, Hkv=2, S=333),
    wl.scaled(wl.FP8_ROT, name="fp8_rot_causal_s200", B=2, Hq=1, Hkv=1, S=200, causal=True),
    wl.scaled(wl.GQA_INT4, name="gqa8x2_int4_s257", Hq=8, Hkv=2, S=257),
    wl.scaled(wl.GQA_INT4, name="gqa4x1_int4_noncausal_s129", Hq=4, Hkv=1, S=129, causal=False),
    wl.scaled(wl.GQA_INT4, name="int8qk_int4v_s300", Hq=2, Hkv=2, S=300, k_qtype="int8",
              kv_block=256, kv_scale_dtype="f32"),
    wl.scaled(wl.INT8_CAUSAL, name="int8_kvblock64_s200", Hq=2, Hkv=1, S=200, kv_block=64),
    wl.scaled(wl.INT8_CAUSAL, name="int8_kvblock96_s250", Hq=2, Hkv=2, S=250, kv_block=96,
              q_block=64),
    wl.scaled(wl.INT8_CAUSAL, name="int8_s1", Hq=1, Hkv=1, S=1),
    wl.scaled(wl.INT8_CAUSAL, name="int8_s33_f16scales", Hq=2, Hkv=2, S=33, q_scale_dtype="f16",
              kv_scale_dtype="f16"),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
@pytest.mark.parametrize("layout", ["bnsd", "bsnd"])
def test_small_cases(w, layout):
    prefill_parity(w, layout=layout)


@pytest.mark.parametrize("odt", ["f32", "bf16"])
def test_output_dtypes(odt):
    prefill_parity(wl.scaled(wl.INT8_CAUSAL, name=f"int8_out_{odt}", Hq=2, Hkv=2, S=200),
                   out_dtype=odt)


def test_rectangular_noncausal():
    """Sq != Sk (non-causal): 70 queries over 333 keys."""
    say("rectangular Sq=70 Sk=333")
    g = torch.Generator().manual_seed(21)
    q = torch.randn(1, 2, 70, 128, generator=g).half()
    k = torch.randn(1, 2, 333, 128, generator=g).half()
    v = torch.randn(1, 2, 333, 128, generator=g).half()
    qc, qs = qfa.block_quant(q.cuda(), 128, "int8")
    kc, ks = qfa.block_quant(k.cuda(), 256, "int8")
    vc, vs = qfa.block_quant(v.cuda(), 256, "int8")
    out = qfa.fwd(qc, qs, kc, ks, vc, vs, q_qtype="int8", k_qtype="int8", v_qtype="int8",
                  q_block=128, kv_block=256, softmax_scale=0.09, causal=False)
    qh = oracle.dequantize(qc.cpu().numpy(), qs.cpu().numpy(), 128, "int8")
    kh = oracle.dequantize(kc.cpu().numpy(), ks.cpu().numpy(), 256, "int8")
    vh = oracle.dequantize(vc.cpu().numpy(), vs.cpu().numpy(), 256, "int8")
    ref = oracle.attention(qh, kh, vh, 0.09, causal=False)
    assert_close(out, ref, "rectangular")


def test_zero_value_block_and_zero_query_block():
    """An all-zero V block (scale 0) and an all-zero Q block (scale 0)."""
    w = wl.scaled(wl.INT8_CAUSAL, name="zeros", Hq=1, Hkv=1, S=600)
    q, k, v = wl.make_prefill_inputs(w)
    v[:, :, 256:512] = 0
    q[:, :, 128:256] = 0
    qc, qs = qfa.block_quant(q.cuda(), 128, "int8")
    kc, ks = qfa.block_quant(k.cuda(), 256, "int8")
    vc, vs = qfa.block_quant(v.cuda(), 256, "int8")
    assert float(vs[0, 0, 1]) == 0.0 and float(qs[0, 0, 1]) == 0.0
    out = qfa.fwd(qc, qs, kc, ks, vc, vs, q_qtype="int8", k_qtype="int8", v_qtype="int8",
                  q_block=128, kv_block=256, softmax_scale=w.softmax_scale, causal=True)
    deq = lambda c, s, r: oracle.dequantize(c.cpu().numpy(), s.cpu().numpy(), r, "int8")
    ref = oracle.attention(deq(qc, qs, 128), deq(kc, ks, 256), deq(vc, vs, 256),
                           w.softmax_scale, causal=True)
    assert_close(out, ref, "zero blocks")


def test_empty_query_is_noop():
    z = torch.zeros(1, 1, 0, 128, dtype=torch.int8, device="cuda")
    s = torch.zeros(1, 1, 0, device="cuda")
    out = qfa.fwd(z, s, z, s, z, s, q_qtype="int8", k_qtype="int8", v_qtype="int8", q_block=128,
                  kv_block=256, softmax_scale=0.1, causal=True)
    assert out.shape == (1, 1, 0, 128)


_ROWS = lambda S: np.unique(np.concatenate([[0, 1, 127, 128, 129, S // 2, S - 2, S - 1],
                                             np.linspace(0, S - 1, 24).astype(int)]))


@pytest.mark.parametrize("w,heads", [
    (wl.INT8_CAUSAL, [0, 13, 31]),
    (wl.FP8_ROT, [0, 23]),
    (wl.GQA_INT4, [0, 9, 63]),
    (wl.INT8QK_INT4V, [0, 17]),
], ids=lambda x: getattr(x, "name", None) or str(x))
def test_full_size_sampled_rows(w, heads):
    """The full workloads in the launch configuration the benchmark times:
    codes of the listed heads checked byte for byte, output rows sampled
    across the sequence (first, last, block edges, evenly spaced)."""
    prefill_parity(w, heads=heads, rows=_ROWS(w.S))
