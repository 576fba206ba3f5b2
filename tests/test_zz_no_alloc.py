"""The allocation-free decode entry point (qfa_decode_noalloc) against
qfa_decode through the C ABI: the same kernels write the same outputs, bit for
bit, from the library's static scratch instead of a caller's workspace. Two
calls in a row (the second smaller) check that the shared scratch keeps no
state that matters between calls."""
import ctypes

import numpy as np
import pytest
import torch

import block_quantized_flashattention_amd as qfa
import oracle
import qfa_workloads as wl
from gpu_util import assert_close, say

pytestmark = pytest.mark.gpu


def _case(B, Hq, Hkv, S_max, lo, hi, qtype, seed):
    w = wl.scaled(wl.DECODE, B=B, Hq=Hq, Hkv=Hkv, S_max=S_max, len_lo=lo, len_hi=hi,
                         seed=seed, kv_qtype=qtype)
    q, k, v, lens = wl.make_decode_inputs(w)
    kc, ks = qfa.block_quant(k.cuda(), w.kv_block, qtype, torch.float16)
    vc, vs = qfa.block_quant(v.cuda(), w.kv_block, qtype, torch.float16)
    return w, q.cuda(), kc, ks, vc, vs, lens.cuda(), (q, k, v, lens)


def _check_pair(B, Hq, Hkv, S_max, lo, hi, qtype, seed):
    say(f"no-alloc decode B={B} Hq={Hq} Hkv={Hkv} S_max={S_max} lens {lo}..{hi} {qtype}")
    w, q, kc, ks, vc, vs, lens, host = _case(B, Hq, Hkv, S_max, lo, hi, qtype, seed)
    kw = dict(kv_qtype=qtype, kv_block=w.kv_block, softmax_scale=w.softmax_scale)
    ref_out = qfa.decode(q, kc, vc, ks, vs, lens, **kw)
    out = torch.full_like(ref_out, float("nan"))
    qfa.decode_noalloc(q, kc, vc, ks, vs, lens, out=out, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), \
        "qfa_decode_noalloc differs from qfa_decode"
    # and both match the oracle to the stated tolerance
    hq, hk, hv, hl = host
    rk, rks = oracle.block_quant(hk, w.kv_block, qtype, "f16")
    rv, rvs = oracle.block_quant(hv, w.kv_block, qtype, "f16")
    ref = oracle.decode(hq.double().numpy(), oracle.dequantize(rk, rks, w.kv_block, qtype),
                        oracle.dequantize(rv, rvs, w.kv_block, qtype), hl.numpy(), w.softmax_scale)
    assert_close(out, ref, "no-alloc decode vs oracle")


def test_noalloc_matches_decode_two_calls():
    # First call: many splits per sequence; second: a smaller input.
    _check_pair(4, 8, 2, 6000, 3000, 6000, "int8", 41)
    _check_pair(2, 4, 4, 2500, 1100, 2500, "int4", 42)


def test_noalloc_rejects_oversize():
    cap = qfa.decode_noalloc_max_bytes()
    assert qfa.decode_workspace_bytes(32, 32, 16384, 128) > cap
    q = torch.zeros(32, 32, 1, 128, dtype=torch.float16, device="cuda")
    kc = torch.zeros(32, 32, 16384, 128, dtype=torch.int8, device="cuda")
    ks = torch.zeros(32, 32, 64, dtype=torch.float16, device="cuda")
    lens = torch.full((32,), 16384, dtype=torch.int32, device="cuda")
    with pytest.raises(qfa.QFAError) as e:
        qfa.decode_noalloc(q, kc, kc, ks, ks, lens, kv_qtype="int8", kv_block=256,
                           softmax_scale=0.1)
    assert e.value.status == 7
