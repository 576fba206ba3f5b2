"""GPU parity of qfa_fwd_lowp, the forward with P.V on the fp8 matrix unit and
an accuracy-gated fp16 fallback (e4m3 Q/K/V with block scales).

- Rows that kept the fp8 product are compared with the oracle's float64
  attention on the dequantized codes, to the forward's tolerance (max-abs
  1e-2, mean-abs 1e-3).
- Work items flagged by the gate must equal qfa_fwd's output bit for bit (the
  fallback recomputes them with the fp16 product); items not flagged must
  differ from it somewhere only through the fp8 product (checked via the
  tolerance above).
- The gate must flag work items whose rows are carried by a few keys
  (planted peaky rows), and must let the fp8 product through on the FP8
  workload's own inputs."""
import ctypes
import os

import numpy as np
import pytest
import torch

import block_quantized_flashattention_amd as qfa
import oracle
import qfa_workloads as wl
from block_quantized_flashattention_amd import build as qbuild
from gpu_util import SDT, assert_close, quantize_both, say

pytestmark = pytest.mark.gpu


def _items(B, Hq, Hkv, Sq, causal):
    """(batch, first head, heads, first row, rows per head) of every work item,
    from the kernel's own index functions compiled for the host."""
    if not os.path.exists(qbuild.IXCHECK_LIB):
        qbuild.build_ixcheck()
    L = ctypes.CDLL(qbuild.IXCHECK_LIB)
    L.qfa_ixcheck_fwd_item.restype = ctypes.c_long
    out = (ctypes.c_int * 5)()
    n = L.qfa_ixcheck_fwd_item(B, Hq, Hkv, Sq, int(causal), -1, out)
    items = []
    for i in range(n):
        L.qfa_ixcheck_fwd_item(B, Hq, Hkv, Sq, int(causal), i, out)
        items.append(tuple(out))
    return items


def _run(w, q, k, v, rows_per_head=None):
    """Quantize on the GPU (codes checked against the oracle for the heads
    used), run fwd and fwd_lowp, check the fallback items bit for bit and the
    sampled rows against the oracle. Returns the fraction of flagged items."""
    say(f"lowp case {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} S={w.S} D={w.D} causal={w.causal}")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    qc, qs = quantize_both(qd, w.q_block, "fp8", w.q_scale_dtype, "bnsd", "Q codes",
                           list(range(min(w.Hq, 4))))
    kc, ks = qfa.block_quant(kd, w.kv_block, "fp8", SDT[w.kv_scale_dtype])
    vc, vs = qfa.block_quant(vd, w.kv_block, "fp8", SDT[w.kv_scale_dtype])
    kw = dict(q_qtype="fp8", k_qtype="fp8", v_qtype="fp8", q_block=w.q_block,
              kv_block=w.kv_block, softmax_scale=w.softmax_scale, causal=w.causal,
              out_dtype=wl.torch_dtype(w.out_dtype))
    ref16 = qfa.fwd(qc, qs, kc, ks, vc, vs, **kw)
    out, ws = qfa.fwd_lowp(qc, qs, kc, ks, vc, vs, **kw)
    torch.cuda.synchronize()
    flags = ws.cpu().numpy()
    items = _items(w.B, w.Hq, w.Hkv, w.S, w.causal)
    assert flags.size >= 8 * len(items)
    flagged = flags[:8 * len(items)].reshape(len(items), 8).any(axis=1)
    o16, olp = ref16.cpu(), out.cpu()
    exact = torch.zeros(w.B, w.Hq, w.S, dtype=torch.bool)
    for (b, h0, nh, r0, nr), f in zip(items, flagged):
        if f:
            sl = (b, slice(h0, h0 + nh), slice(r0, min(w.S, r0 + nr)))
            assert torch.equal(olp[sl].view(torch.int16), o16[sl].view(torch.int16)), \
                f"flagged item (b={b}, h={h0}, rows {r0}..) differs from qfa_fwd"
            exact[sl] = True
    frac = float(flagged.mean())
    say(f"  flagged work items: {int(flagged.sum())} of {len(items)} ({frac:.1%})")
    # Oracle on sampled rows of a few heads (the rows may lie in either kind
    # of item), on the oracle's own K/V codes (the GPU's are checked equal).
    heads = sorted({0, w.Hq - 1} | ({w.Hq // 2} if w.Hq > 2 else set()))
    kvheads = sorted({h // (w.Hq // w.Hkv) for h in heads})
    rk, rks = oracle.block_quant(k[:, kvheads], w.kv_block, "fp8", w.kv_scale_dtype)
    rv, rvs = oracle.block_quant(v[:, kvheads], w.kv_block, "fp8", w.kv_scale_dtype)
    assert np.array_equal(kc[:, kvheads].cpu().view(torch.uint8).numpy(), rk)
    assert np.array_equal(vc[:, kvheads].cpu().view(torch.uint8).numpy(), rv)
    kh = oracle.dequantize(rk, rks, w.kv_block, "fp8")
    vh = oracle.dequantize(rv, rvs, w.kv_block, "fp8")
    rq, rqs = oracle.block_quant(q[:, heads], w.q_block, "fp8", w.q_scale_dtype)
    qh = oracle.dequantize(rq, rqs, w.q_block, "fp8")
    rows = np.arange(w.S) if rows_per_head is None else rows_per_head
    got, ref = [], []
    for b in range(w.B):
        for hi, h in enumerate(heads):
            kvi = kvheads.index(h // (w.Hq // w.Hkv))
            ref.append(oracle.attention_rows(qh[:, hi:hi + 1], kh[:, kvi:kvi + 1],
                                             vh[:, kvi:kvi + 1], w.softmax_scale, w.causal, b,
                                             0, rows))
            got.append(olp[b, h, rows].double().numpy())
    assert_close(np.concatenate(got), np.concatenate(ref), f"{w.name} lowp")
    return frac


def test_fp8_workload_full_size():
    """The FP8 workload (2 x 24 heads x 4608, rotated Q/K): the gate lets the
    fp8 product through for most work items, and sampled rows meet the
    tolerance."""
    w = wl.FP8_ROT
    q, k, v = wl.make_prefill_inputs(w)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, w.S - 1], np.linspace(0, w.S - 1, 40).astype(int)]))
    frac = _run(w, q, k, v, rows)
    assert frac < 0.5, "the fp8 product should carry most of this workload"


@pytest.mark.parametrize("S,D,causal", [(1000, 128, False), (700, 64, True), (1500, 128, True)])
def test_small_cases(S, D, causal):
    """Ragged sequence lengths, D = 64 and 128, causal and not: early causal
    rows are carried by few keys and must fall back."""
    w = wl.scaled(wl.FP8_ROT, name=f"fp8_s{S}_d{D}", B=1, Hq=2, Hkv=2, S=S, D=D, causal=causal,
                  rotate_qk=False)
    q, k, v = wl.make_prefill_inputs(w)
    frac = _run(w, q, k, v)
    if causal:
        assert frac > 0.0, "causal rows near the start have few keys and must be flagged"


def test_peaky_rows_fall_back():
    """Rows whose query is aligned with a few keys (softmax nearly one-hot)
    must flag their work items; those items equal qfa_fwd bit for bit."""
    w = wl.scaled(wl.FP8_ROT, name="fp8_peaky", B=1, Hq=2, Hkv=2, S=2048, rotate_qk=False)
    q, k, v = wl.make_prefill_inputs(w)
    qf = q.float()
    rng = np.random.default_rng(3)
    for r in rng.integers(0, w.S, 6):               # rows in a few work items of head 0
        j = int(rng.integers(0, w.S))
        qf[0, 0, r] = 0.9 * k[0, 0, j].float()      # score |k_j|^2 / sqrt(D) ~ 10
    q = qf.to(q.dtype)
    frac = _run(w, q, k, v)
    assert frac > 0.0


@pytest.mark.parametrize("causal", [False, True])
def test_bsnd_equals_bnsd(causal):
    """The layout changes addresses only: with BSND tensors the fp8 P.V forward
    gives the BNSD outputs bit for bit and the same flags, including the work
    items its workgroups recompute with the fp16 product (causal rows near the
    start are carried by few keys and flag)."""
    w = wl.scaled(wl.FP8_ROT, name=f"fp8_layouts_c{int(causal)}", B=2, Hq=4, Hkv=2, S=777,
                  causal=causal, rotate_qk=False)
    say(f"lowp layouts case {w.name}")
    q, k, v = wl.make_prefill_inputs(w)
    sdt = SDT[w.kv_scale_dtype]
    qc, qs = qfa.block_quant(q.cuda(), w.q_block, "fp8", SDT[w.q_scale_dtype])
    kc, ks = qfa.block_quant(k.cuda(), w.kv_block, "fp8", sdt)
    vc, vs = qfa.block_quant(v.cuda(), w.kv_block, "fp8", sdt)
    kw = dict(q_qtype="fp8", k_qtype="fp8", v_qtype="fp8", q_block=w.q_block,
              kv_block=w.kv_block, softmax_scale=w.softmax_scale, causal=w.causal,
              out_dtype=wl.torch_dtype(w.out_dtype))
    o1, f1 = qfa.fwd_lowp(qc, qs, kc, ks, vc, vs, layout="bnsd", **kw)
    t = lambda x: x.transpose(1, 2).contiguous()  # noqa: E731
    o2, f2 = qfa.fwd_lowp(t(qc), qs, t(kc), ks, t(vc), vs, layout="bsnd", **kw)
    torch.cuda.synchronize()
    assert torch.equal(f1.cpu(), f2.cpu()), "flags differ between layouts"
    assert torch.equal(o2.transpose(1, 2).cpu().view(torch.int16), o1.cpu().view(torch.int16)), \
        "outputs differ between layouts"
    if causal:
        assert int(f1.cpu().sum()) > 0, "causal rows near the start must flag"
