"""GPU parity of qfa_fwd against the oracle's float64 attention on the same
codes: small cases spanning several tiles with ragged tails, both layouts,
every code type, and the full-size workloads on sampled rows."""
import numpy as np
import pytest
import torch

import block_quantized_flashattention_amd as qfa
import oracle
import qfa_workloads as wl
from gpu_util import assert_close, prefill_parity, prefill_parity_every_head, say

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
    # Q blocks of 48 rows: a wavefront's 32 rows can span two Q scales.
    wl.scaled(wl.GQA_INT4, name="gqa8x2_int4_qblock48_s200", Hq=8, Hkv=2, S=200, q_block=48),
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


@pytest.mark.parametrize("w", [wl.INT8_CAUSAL, wl.FP8_ROT, wl.GQA_INT4, wl.INT8QK_INT4V],
                         ids=lambda w: w.name)
def test_full_size_every_head(w):
    """Every (batch, query head) of the full workloads: a few rows each, one of
    them the last row or one in the first two Q blocks, against the oracle's
    attention on the oracle's own codes."""
    prefill_parity_every_head(w)


@pytest.mark.parametrize("vscale", [1e4, 1e-4])
def test_per_token_path_large_and_small_v(vscale):
    """INT4 K/V with one fp16 scale per token (the GQA workload's path), V
    scaled by 1e4 and by 1e-4: the fp16 weights and staged values stay in
    range whatever the V scales' magnitude. The tolerance is stated for
    unit-variance V, so the error is compared in units of the V scale."""
    w = wl.scaled(wl.GQA_INT4, name=f"gqa8x2_int4_v{vscale:g}", Hq=8, Hkv=2, S=300)
    q, k, v = wl.make_prefill_inputs(w)
    v = (v.float() * vscale).half()
    say(f"per-token path, V x {vscale:g}: V amax {float(v.float().abs().max()):.3g}")
    qc, qs = qfa.block_quant(q.cuda(), w.q_block, "int8")
    kc, ks = qfa.block_quant(k.cuda(), 1, "int4", torch.float16)
    vc, vs = qfa.block_quant(v.cuda(), 1, "int4", torch.float16)
    out = qfa.fwd(qc, qs, kc, ks, vc, vs, q_qtype="int8", k_qtype="int4", v_qtype="int4",
                  q_block=w.q_block, kv_block=1, softmax_scale=w.softmax_scale, causal=True,
                  out_dtype=torch.float32)
    rq, rqs = oracle.block_quant(q, w.q_block, "int8")
    rk, rks = oracle.block_quant(k, 1, "int4", "f16")
    rv, rvs = oracle.block_quant(v, 1, "int4", "f16")
    assert np.array_equal(vc.cpu().numpy(), rv) and np.array_equal(vs.cpu().numpy(), rvs)
    ref = oracle.attention(oracle.dequantize(rq, rqs, w.q_block, "int8"),
                           oracle.dequantize(rk, rks, 1, "int4"),
                           oracle.dequantize(rv, rvs, 1, "int4"), w.softmax_scale, causal=True)
    assert_close(out.double().cpu().numpy() / vscale, ref / vscale, f"V x {vscale:g}")


def test_per_token_v_scales_spanning_four_decades():
    """INT4 K/V with one fp16 scale per token, V rows scaled by 10^u with u
    uniform in [-2, 2) per token: the staged values are code * sv_j / sv_ref
    with sv_ref the running maximum V scale, so early small-scale tokens are
    rescaled when a larger scale arrives and late ones are staged small. The
    tolerance is stated for unit-variance V: errors are compared in units of
    the largest V row scale."""
    w = wl.scaled(wl.GQA_INT4, name="gqa8x2_int4_vspread", Hq=8, Hkv=2, S=333)
    q, k, v = wl.make_prefill_inputs(w)
    g = torch.Generator().manual_seed(1234)
    mag = 10.0 ** (torch.rand(v.shape[0], v.shape[1], v.shape[2], 1, generator=g) * 4.0 - 2.0)
    v = (v.float() * mag).half()
    say(f"per-token path, V row magnitudes 1e-2..1e2: V amax {float(v.float().abs().max()):.3g}")
    qc, qs = qfa.block_quant(q.cuda(), w.q_block, "int8")
    kc, ks = qfa.block_quant(k.cuda(), 1, "int4", torch.float16)
    vc, vs = qfa.block_quant(v.cuda(), 1, "int4", torch.float16)
    out = qfa.fwd(qc, qs, kc, ks, vc, vs, q_qtype="int8", k_qtype="int4", v_qtype="int4",
                  q_block=w.q_block, kv_block=1, softmax_scale=w.softmax_scale, causal=True,
                  out_dtype=torch.float32)
    rq, rqs = oracle.block_quant(q, w.q_block, "int8")
    rk, rks = oracle.block_quant(k, 1, "int4", "f16")
    rv, rvs = oracle.block_quant(v, 1, "int4", "f16")
    ref = oracle.attention(oracle.dequantize(rq, rqs, w.q_block, "int8"),
                           oracle.dequantize(rk, rks, 1, "int4"),
                           oracle.dequantize(rv, rvs, 1, "int4"), w.softmax_scale, causal=True)
    unit = float(mag.max())
    assert_close(out.double().cpu().numpy() / unit, ref / unit, "V rows 1e-2..1e2")


def _sweep_cases(n=24, seed=2024):
    """Seeded random small forward configurations: code-type combination,
    D, GQA group, ragged S, causal or not, block sizes (per-key scales when
    the K/V block does not cover 64-key tiles, per-token for INT4), scale
    dtypes and layout."""
    rng = np.random.default_rng(seed)
    bases = [wl.INT8_CAUSAL, wl.FP8_ROT, wl.GQA_INT4, wl.INT8QK_INT4V]
    cases = []
    for i in range(n):
        base = bases[i % len(bases)]
        Hkv = int(rng.choice([1, 2]))
        group = int(rng.choice([1, 2, 4, 8]))
        D = int(rng.choice([64, 128]))
        S = int(rng.integers(1, 420))
        kvb = int(rng.choice([1, 16, 64, 96, 256])) if base.k_qtype == "int4" else \
            int(rng.choice([32, 64, 96, 256]))
        qb = int(rng.choice([16, 48, 64, 128]))
        sdt = str(rng.choice(["f32", "f16"]))
        w = wl.scaled(base, name=f"sweep{i}_{base.q_qtype}_{base.k_qtype}{base.v_qtype}",
                      B=int(rng.integers(1, 3)), Hq=Hkv * group, Hkv=Hkv, S=S, D=D,
                      causal=bool(rng.integers(0, 2)), q_block=qb, kv_block=kvb,
                      q_scale_dtype=sdt, kv_scale_dtype=str(rng.choice(["f32", "f16"])),
                      softmax_scale=float(np.float32(1 / np.sqrt(D))), rotate_qk=False,
                      k_outlier_channels=min(base.k_outlier_channels, 2))
        cases.append((w, str(rng.choice(["bnsd", "bsnd"]))))
    return cases


@pytest.mark.parametrize("w,layout", _sweep_cases(), ids=lambda c: getattr(c, "name", c))
def test_seeded_sweep(w, layout):
    """Random small shapes (fixed seed) against the oracle, every row."""
    prefill_parity(w, layout=layout)
