"""The prepared launchers (arguments marshalled once, one ctypes call per
launch) issue the same C-ABI calls as the plain functions: their results are
bit-identical, on every repeat."""
import pytest
import torch

import block_quantized_flashattention_amd as qfa
import qfa_workloads as wl
from gpu_util import say

pytestmark = pytest.mark.gpu


def test_prepared_quant_and_fwd_match_plain_calls():
    w = wl.scaled(wl.INT8_CAUSAL, name="int8_causal_h2_s300", Hq=2, Hkv=2, S=300)
    say(f"prepared launchers, {w.name}")
    q, k, v = (t.cuda() for t in wl.make_prefill_inputs(w))
    jobs = [dict(x=q, block_rows=w.q_block, qtype=w.q_qtype),
            dict(x=k, block_rows=w.kv_block, qtype=w.k_qtype),
            dict(x=v, block_rows=w.kv_block, qtype=w.v_qtype)]
    plain = qfa.block_quant_multi(jobs)
    launch, outs = qfa.prepare_block_quant_multi(jobs)
    for _ in range(2):
        for (c, s) in outs:
            c.fill_(0)
            s.fill_(0)
        launch()
        torch.cuda.synchronize()
        for (c0, s0), (c1, s1) in zip(plain, outs):
            assert torch.equal(c0, c1) and torch.equal(s0, s1)
    (qc, qs), (kc, ks), (vc, vs) = plain
    kw = dict(q_qtype=w.q_qtype, k_qtype=w.k_qtype, v_qtype=w.v_qtype, q_block=w.q_block,
              kv_block=w.kv_block, softmax_scale=w.softmax_scale, causal=True)
    ref = qfa.fwd(qc, qs, kc, ks, vc, vs, **kw)
    attn, out = qfa.prepare_fwd(qc, qs, kc, ks, vc, vs, **kw)
    for _ in range(2):
        out.fill_(0)
        attn()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)


def test_prepared_decode_matches_plain_call():
    w = wl.scaled(wl.DECODE, name="decode_b3_h4", B=3, Hq=4, Hkv=2, S_max=1500, len_lo=700,
                  len_hi=1500)
    say(f"prepared decode, {w.name}")
    q, k, v, lens = wl.make_decode_inputs(w, device="cuda")
    kc, ks = qfa.block_quant(k, w.kv_block, w.kv_qtype, torch.float16)
    vc, vs = qfa.block_quant(v, w.kv_block, w.kv_qtype, torch.float16)
    kw = dict(kv_qtype=w.kv_qtype, kv_block=w.kv_block, softmax_scale=w.softmax_scale)
    ref = qfa.decode(q, kc, vc, ks, vs, lens, **kw)
    launch, out = qfa.prepare_decode(q, kc, vc, ks, vs, lens, **kw)
    for _ in range(2):
        out.fill_(0)
        launch()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
