"""GPU parity of qfa_decode (split-K over the KV cache plus the merge) against
the oracle's float64 decode attention on the same cache codes."""
import numpy as np
import pytest
import torch

import block_quantized_flashattention_amd as qfa
import oracle
import qfa_workloads as wl
from gpu_util import SDT, assert_close, quantize_both, say

pytestmark = pytest.mark.gpu


def _run(w: wl.DecodeWorkload, q, k, v, lens, layout="bnsd", sample=None):
    say(f"decode case {w.name} B={q.shape[0]} Hq={w.Hq} Hkv={w.Hkv} S_max={k.shape[2]} "
        f"D={w.D} kv={w.kv_qtype} R={w.kv_block} lens={lens.tolist()[:6]}")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    B, S_max = q.shape[0], k.shape[2]
    if layout == "bsnd":
        kd, vd = kd.transpose(1, 2).contiguous(), vd.transpose(1, 2).contiguous()
    heads = None if sample is None else sorted({h for _, h in sample})
    kc, ks = quantize_both(kd, w.kv_block, w.kv_qtype, w.kv_scale_dtype, layout, "K cache", heads)
    vc, vs = quantize_both(vd, w.kv_block, w.kv_qtype, w.kv_scale_dtype, layout, "V cache", heads)
    out = qfa.decode(qd, kc, vc, ks, vs, lens.cuda(), kv_qtype=w.kv_qtype, kv_block=w.kv_block,
                     softmax_scale=w.softmax_scale, layout=layout,
                     out_dtype=wl.torch_dtype(w.out_dtype))
    torch.cuda.synchronize()
    pairs = sample or [(b, h) for b in range(B) for h in range(w.Hkv)]
    group = w.Hq // w.Hkv
    got, ref = [], []
    for b, kvh in pairs:
        L = int(lens[b])
        sl = (slice(b, b + 1), slice(kvh, kvh + 1), slice(0, L))
        if layout == "bnsd":
            kcs, vcs = kc[sl].cpu().numpy(), vc[sl].cpu().numpy()
        else:
            kcs = kc[b:b + 1, :L, kvh:kvh + 1].cpu().numpy()
            vcs = vc[b:b + 1, :L, kvh:kvh + 1].cpu().numpy()
        kss, vss = ks[b:b + 1, kvh:kvh + 1].cpu().numpy(), vs[b:b + 1, kvh:kvh + 1].cpu().numpy()
        nb = -(-L // w.kv_block)
        kh = oracle.dequantize(kcs, kss[..., :nb], w.kv_block, w.kv_qtype, layout)
        vh = oracle.dequantize(vcs, vss[..., :nb], w.kv_block, w.kv_qtype, layout)
        qs = q[b:b + 1, kvh * group:(kvh + 1) * group].double().numpy()
        ref.append(oracle.decode(qs, kh, vh, [L], w.softmax_scale))
        got.append(out[b:b + 1, kvh * group:(kvh + 1) * group].double().cpu().numpy())
    assert_close(np.concatenate(got), np.concatenate(ref), f"{w.name} decode")
    return out


SMALL = [
    # name, B, Hq, Hkv, D, S_max, lens, kv qtype, kv_block, scale dtype
    ("i8_gqa2", 3, 4, 2, 128, 3000, [1, 1024, 2999], "int8", 256, "f16"),
    ("i8_splits", 2, 2, 2, 128, 4100, [1025, 4100], "int8", 256, "f16"),
    # one head per KV head, INT8: every sequence is split into ceil(S_max/1024)
    # chunks, so very short ones leave chunks with no tokens or a few
    ("i8_short", 3, 2, 2, 128, 3000, [1, 5, 2999], "int8", 256, "f16"),
    # 128-token blocks: a wavefront's equal share spans two blocks
    ("i8_r128", 2, 2, 2, 128, 3333, [3333, 1500], "int8", 128, "f32"),
    ("i8_d64_f32s", 2, 3, 3, 64, 700, [700, 17], "int8", 64, "f32"),
    ("i4_tok", 2, 8, 2, 128, 2500, [2500, 300], "int4", 1, "f16"),
    ("i4_blk", 2, 2, 1, 128, 1500, [1200, 1500], "int4", 256, "f16"),
    ("i4_d64", 1, 4, 4, 64, 2100, [2049], "int4", 128, "f32"),
    ("i8_gqa16", 1, 16, 1, 128, 2000, [1999], "int8", 256, "f16"),
]


@pytest.mark.parametrize("name,B,Hq,Hkv,D,S_max,lens,qt,R,sdt", SMALL, ids=[c[0] for c in SMALL])
@pytest.mark.parametrize("layout", ["bnsd", "bsnd"])
def test_small_decode(name, B, Hq, Hkv, D, S_max, lens, qt, R, sdt, layout):
    w = wl.DecodeWorkload(name=name, B=B, Hq=Hq, Hkv=Hkv, D=D, S_max=S_max, len_lo=S_max,
                          len_hi=S_max, seed=40 + B + Hq, kv_qtype=qt, kv_block=R,
                          kv_scale_dtype=sdt, q_dtype="f16", out_dtype="f16",
                          softmax_scale=float(np.float32(1 / np.sqrt(D))))
    q, k, v, _ = wl.make_decode_inputs(w)
    lens_t = torch.tensor(lens, dtype=torch.int32)
    for b, L in enumerate(lens):   # rows past the length are zero in the sources
        k[b, :, L:] = 0
        v[b, :, L:] = 0
    _run(w, q, k, v, lens_t, layout=layout)



@pytest.mark.parametrize("qdt,odt", [("f32", "f32"), ("bf16", "bf16")])
@pytest.mark.parametrize("qt,R", [("int8", 256), ("int4", 256), ("int4", 1)])
def test_decode_query_dtypes(qdt, odt, qt, R):
    """fp32 and bf16 queries (the codes go to fp32 on that path) with fp32 and
    bf16 outputs, over several chunks and a ragged length."""
    w = wl.DecodeWorkload(name=f"q{qdt}_{qt}_r{R}", B=2, Hq=4, Hkv=2, D=128, S_max=2200,
                          len_lo=2200, len_hi=2200, seed=91, kv_qtype=qt, kv_block=R,
                          kv_scale_dtype="f16", q_dtype=qdt, out_dtype=odt,
                          softmax_scale=float(np.float32(1 / np.sqrt(128))))
    q, k, v, _ = wl.make_decode_inputs(w)
    lens = [2200, 777]
    for b, L in enumerate(lens):
        k[b, :, L:] = 0
        v[b, :, L:] = 0
    _run(w, q, k, v, torch.tensor(lens, dtype=torch.int32))


@pytest.mark.parametrize("w", [wl.DECODE, wl.DECODE_INT4, wl.DECODE_GQA4, wl.DECODE_GQA16_INT4],
                         ids=lambda w: w.name)
def test_full_size_decode_sampled(w):
    """The full decode workload (B=32, 32 query heads, S_max=8192, L in
    [4096, 8192]), INT8 or packed INT4 cache, one query head per KV head or
    grouped (4 and 16 per KV head, the matrix-unit kernel); inputs drawn on
    the GPU; 24 (batch, KV head) pairs, every query head of each, compared
    with the oracle."""
    say("full-size decode: generating inputs on the GPU")
    q, k, v, lens = wl.make_decode_inputs(w, device="cuda")
    rng = np.random.default_rng(7)
    sample = [(int(b), int(h)) for b, h in zip(rng.integers(0, w.B, 24), rng.integers(0, w.Hkv, 24))]
    sample[0] = (int(torch.argmax(lens)), 0)
    sample[1] = (int(torch.argmin(lens)), w.Hkv - 1)
    _run(w, q.cpu(), k, v, lens.cpu(), sample=sample)


@pytest.mark.parametrize("qt,R", [("int8", 256), ("int4", 256), ("int4", 1)])
@pytest.mark.parametrize("layout", ["bnsd", "bsnd"])
def test_rows_past_length_are_ignored(qt, R, layout):
    """Cache rows at and past each sequence's length hold stale codes (random
    bytes) and the scales of blocks that start past it are NaN: the output
    must depend on the rows before the length only."""
    w = wl.DecodeWorkload(name=f"stale_{qt}_r{R}", B=3, Hq=4, Hkv=2, D=128, S_max=2600,
                          len_lo=2600, len_hi=2600, seed=77, kv_qtype=qt, kv_block=R,
                          kv_scale_dtype="f16", q_dtype="f16", out_dtype="f16",
                          softmax_scale=float(np.float32(1 / np.sqrt(128))))
    lens = [1, 1100, 2583]
    say(f"decode stale rows {w.name} {layout} lens={lens}")
    q, k, v, _ = wl.make_decode_inputs(w)
    kd, vd = k.cuda(), v.cuda()
    if layout == "bsnd":
        kd, vd = kd.transpose(1, 2).contiguous(), vd.transpose(1, 2).contiguous()
    kc, ks = qfa.block_quant(kd, R, qt, torch.float16, layout)
    vc, vs = qfa.block_quant(vd, R, qt, torch.float16, layout)
    g = torch.Generator(device="cuda").manual_seed(5)
    for b, L in enumerate(lens):
        for c in (kc, vc):
            rows = c[b, :, L:] if layout == "bnsd" else c[b, L:]
            rows.copy_(torch.randint(-128, 128, rows.shape, generator=g, device="cuda",
                                     dtype=torch.int16).to(torch.int8))
        nb = -(-L // R)
        ks[b, :, nb:] = float("nan")
        vs[b, :, nb:] = float("nan")
    lens_t = torch.tensor(lens, dtype=torch.int32)
    out = qfa.decode(q.cuda(), kc, vc, ks, vs, lens_t.cuda(), kv_qtype=qt, kv_block=R,
                     softmax_scale=w.softmax_scale, layout=layout, out_dtype=torch.float16)
    torch.cuda.synchronize()
    got, ref = [], []
    for b, L in enumerate(lens):
        nb = -(-L // R)
        for kvh in range(w.Hkv):
            if layout == "bnsd":
                kcs = kc[b:b + 1, kvh:kvh + 1, :L].cpu().numpy()
                vcs = vc[b:b + 1, kvh:kvh + 1, :L].cpu().numpy()
            else:
                kcs = kc[b:b + 1, :L, kvh:kvh + 1].cpu().numpy()
                vcs = vc[b:b + 1, :L, kvh:kvh + 1].cpu().numpy()
            kss = ks[b:b + 1, kvh:kvh + 1, :nb].cpu().numpy()
            vss = vs[b:b + 1, kvh:kvh + 1, :nb].cpu().numpy()
            kh = oracle.dequantize(kcs, kss, R, qt, layout)
            vh = oracle.dequantize(vcs, vss, R, qt, layout)
            grp = slice(kvh * 2, kvh * 2 + 2)
            ref.append(oracle.decode(q[b:b + 1, grp].double().numpy(), kh, vh, [L], w.softmax_scale))
            got.append(out[b:b + 1, grp].double().cpu().numpy())
    assert_close(np.concatenate(got), np.concatenate(ref), f"{w.name} stale rows")


def _decode_sweep(n=16, seed=77):
    """Seeded random small decode configurations: INT8 or INT4 cache, D,
    group size 1..16, lengths anywhere in [1, S_max] (not multiples of the
    block or chunk), block or per-token scales, scale dtype and layout."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        qt = str(rng.choice(["int8", "int4"]))
        Hkv = int(rng.choice([1, 2]))
        group = int(rng.choice([1, 2, 4, 16]))
        D = int(rng.choice([64, 128]))
        S_max = int(rng.integers(2, 3500))
        B = int(rng.integers(1, 4))
        lens = [int(x) for x in rng.integers(1, S_max + 1, B)]
        R = int(rng.choice([1, 64, 128, 256])) if qt == "int4" else int(rng.choice([64, 128, 256]))
        cases.append((f"sweep{i}_{qt}_g{group}", B, Hkv * group, Hkv, D, S_max, lens, qt, R,
                      str(rng.choice(["f16", "f32"])), str(rng.choice(["bnsd", "bsnd"]))))
    return cases


_SWEEP = _decode_sweep()


@pytest.mark.parametrize("name,B,Hq,Hkv,D,S_max,lens,qt,R,sdt,layout", _SWEEP,
                         ids=[f"{c[0]}_{c[7]}_r{c[8]}_{c[10]}" for c in _SWEEP])
def test_decode_seeded_sweep(name, B, Hq, Hkv, D, S_max, lens, qt, R, sdt, layout):
    """Random small decode shapes (fixed seed) against the oracle, every head."""
    test_small_decode(name, B, Hq, Hkv, D, S_max, lens, qt, R, sdt, layout)
