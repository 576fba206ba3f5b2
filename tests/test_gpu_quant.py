"""GPU parity of qfa_block_quant: codes and scales byte for byte equal to the
oracle's, on small ragged cases, hand-computed fixtures, the e4m3 rounding
boundaries and every workload's full-size tensors."""
import numpy as np
import pytest
import torch

import block_quantized_flashattention_amd as qfa
import oracle
import qfa_workloads as wl
from golden_io import load
from gpu_util import SDT, assert_codes_equal, quantize_both, say

pytestmark = pytest.mark.gpu


def _x(shape, dtype, seed, zero=None):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(*shape, generator=g) * torch.exp(torch.randn(shape[:2] + (1, 1), generator=g))
    if zero is not None:
        x[zero] = 0
    return x.to(dtype)


CASES = [
    # qtype, rows, scale dtype, input dtype, B, N, S, D, layout
    ("int8", 128, "f32", torch.float16, 2, 3, 300, 128, "bnsd"),
    ("int8", 256, "f32", torch.float32, 1, 2, 513, 64, "bnsd"),
    ("int8", 256, "f16", torch.float16, 2, 2, 700, 128, "bsnd"),
    ("int8", 7, "f32", torch.bfloat16, 1, 2, 50, 8, "bnsd"),
    ("fp8", 128, "f32", torch.bfloat16, 2, 3, 260, 128, "bnsd"),
    ("fp8", 256, "f32", torch.bfloat16, 1, 2, 511, 128, "bsnd"),
    ("fp8", 256, "f16", torch.float32, 1, 1, 300, 64, "bnsd"),
    ("int4", 1, "f16", torch.float16, 1, 4, 37, 128, "bnsd"),
    ("int4", 1, "f16", torch.float16, 2, 3, 41, 128, "bsnd"),
    ("int4", 16, "f32", torch.float32, 1, 2, 50, 64, "bnsd"),
    ("int8", 512, "f32", torch.float16, 1, 1, 1200, 128, "bnsd"),   # 1024-thread teams
    ("int8", 1100, "f32", torch.float16, 1, 1, 2300, 128, "bnsd"),  # two-pass path
    ("fp8", 600, "f16", torch.float32, 1, 1, 1300, 128, "bsnd"),    # two-pass (fp32 input)
    ("int8", 1, "f32", torch.float16, 1, 2, 9, 1024, "bnsd"),
]


@pytest.mark.parametrize("qt,R,sdt,dt,B,N,S,D,layout", CASES)
def test_quant_matches_oracle(qt, R, sdt, dt, B, N, S, D, layout):
    say(f"quant case {qt} R={R} {sdt} {dt} B={B} N={N} S={S} D={D} {layout}")
    shape = (B, N, S, D)
    x = _x(shape, dt, seed=S * 7 + D, zero=(0, N - 1, slice(0, R)))
    if layout == "bsnd":
        x = x.transpose(1, 2).contiguous()
    quantize_both(x.cuda(), R, qt, sdt, layout, f"{qt} R={R}")


@pytest.mark.parametrize("name", ["int8_ties.txt", "int8_scale_half.txt", "e4m3_points.txt",
                                  "int4_pack.txt"])
def test_quant_golden_fixtures(name):
    """The hand-computed fixtures, channel 0 of 8 (the other channels are 0)."""
    g = load(name)
    vals = np.array(g["input"], dtype=np.float32)
    if name == "int4_pack.txt":
        x = torch.from_numpy(vals).reshape(1, 1, 1, 8)
    else:
        x = torch.zeros(1, 1, vals.size, 8)
        x[0, 0, :, 0] = torch.from_numpy(vals)
    c, s = qfa.block_quant(x.cuda(), g["block_rows"], g["qtype"],
                           torch.float16 if g["scale_dtype"] == "f16" else torch.float32)
    assert float(s.flatten()[0]) == g["scale"]
    want = np.array(g["codes"] if isinstance(g["codes"], list) else [g["codes"]]) & 0xFF
    got = c.cpu().numpy().view(np.uint8)
    got = got.ravel() if name == "int4_pack.txt" else got[0, 0, :, 0]
    assert got.astype(np.int64).tolist() == want.tolist()


def test_fp8_encoding_boundaries():
    """Blocks whose amax is 448 have scale 1, so their codes are e4m3fn(x): the
    hardware conversion must match the oracle's encoder (itself pinned to
    torch.float8_e4m3fn) at every rounding midpoint and its neighbours."""
    pos = oracle.e4m3fn_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    bits = mids.view(np.uint32).astype(np.int64)
    near = (bits[:, None] + np.arange(-64, 65)[None, :]).ravel()
    near = near[near >= 0].astype(np.uint32).view(np.float32)
    rng = np.random.default_rng(5)
    rb = rng.integers(0, 0x43E00001, size=1 << 18, dtype=np.uint32).view(np.float32)
    h = np.arange(1 << 16, dtype=np.uint16).view(np.float16).astype(np.float32)
    vals = np.concatenate([near, -near, rb, -rb, h,
                           np.array([0.0, -0.0, 448.0, -448.0], np.float32)])
    vals = vals[np.isfinite(vals) & (np.abs(vals) <= 448)]
    R, D = 64, 128
    per_block = R * D - 1
    nblk = -(-vals.size // per_block)
    x = np.zeros((nblk, R * D), np.float32)
    x[:, 0] = 448.0
    flat = x[:, 1:].reshape(-1)
    flat[:vals.size] = vals
    x[:, 1:] = flat.reshape(nblk, per_block)
    xt = torch.from_numpy(x.reshape(1, 1, nblk * R, D))
    c, s = qfa.block_quant(xt.cuda(), R, "fp8")
    assert torch.all(s == 1.0)
    rc = oracle.e4m3fn_encode(x.reshape(-1))
    got = c.cpu().numpy().view(np.uint8).reshape(-1)
    bad = np.flatnonzero(got != rc)
    assert bad.size == 0, f"{bad.size} mismatches; first x={x.reshape(-1)[bad[0]]!r} " \
                          f"gpu=0x{got[bad[0]]:02x} ref=0x{rc[bad[0]]:02x}"


def test_int8_rounding_near_ties():
    """x = (n + 0.5 +- a few ulps) * s for a block scale s that is not a power of
    two: the codes depend on the exact fp32 quotient."""
    rng = np.random.default_rng(6)
    R, D = 32, 128
    amax = np.float32(3.7)
    s = np.float32(amax / np.float32(127))
    n = rng.integers(-127, 127, size=R * D - 1).astype(np.float32)
    base = ((n + np.float32(0.5)) * s).astype(np.float32)
    jitter = rng.integers(-3, 4, size=base.size)
    xv = (base.view(np.int32) + jitter.astype(np.int32)).view(np.float32)
    xv = np.clip(xv, -amax, amax)
    x = np.concatenate([[amax], xv]).astype(np.float32).reshape(1, 1, R, D)
    xt = torch.from_numpy(x)
    c, sc = qfa.block_quant(xt.cuda(), R, "int8")
    rc, rs = oracle.block_quant(x, R, "int8")
    assert_codes_equal(c, sc, rc, rs, "int8 near ties")


@pytest.mark.parametrize("w", [wl.INT8_CAUSAL, wl.FP8_ROT, wl.GQA_INT4], ids=lambda w: w.name)
def test_quant_full_size(w):
    """Full workload tensors quantized on the GPU; every head of Q, K and V is
    compared with the oracle (K/V) or a spread of heads (Q of the largest)."""
    say(f"full-size quant {w.name}")
    q, k, v = wl.make_prefill_inputs(w)
    qheads = None if w.Hq <= 32 else list(range(0, w.Hq, 7))
    quantize_both(q.cuda(), w.q_block, w.q_qtype, w.q_scale_dtype, "bnsd", "Q", qheads)
    quantize_both(k.cuda(), w.kv_block, w.k_qtype, w.kv_scale_dtype, "bnsd", "K")
    quantize_both(v.cuda(), w.kv_block, w.v_qtype, w.kv_scale_dtype, "bnsd", "V")


def test_quant_multi_matches_oracle():
    """Every case above in one qfa_block_quant_multi call (several groups of
    input and code type, the two-pass path among them): each job's codes and
    scales equal the oracle's byte for byte."""
    say("quant multi: all small cases in one call")
    jobs, xs = [], []
    for qt, R, sdt, dt, B, N, S, D, layout in CASES:
        x = _x((B, N, S, D), dt, seed=S * 7 + D + 1, zero=(0, N - 1, slice(0, R)))
        if layout == "bsnd":
            x = x.transpose(1, 2).contiguous()
        xs.append((x, qt, R, sdt, layout))
        jobs.append(dict(x=x.cuda(), block_rows=R, qtype=qt,
                         scale_dtype=torch.float16 if sdt == "f16" else torch.float32,
                         layout=layout))
    outs = qfa.block_quant_multi(jobs)
    torch.cuda.synchronize()
    for (x, qt, R, sdt, layout), (c, s) in zip(xs, outs):
        rc, rs = oracle.block_quant(x, R, qt, sdt, layout)
        assert_codes_equal(c, s, rc, rs, f"multi {qt} R={R} {layout}")


@pytest.mark.parametrize("w", [wl.INT8_CAUSAL, wl.GQA_INT4], ids=lambda w: w.name)
def test_quant_multi_qkv_full_size(w):
    """Q, K and V of a full workload in one call (the benchmark's quantization
    step): each output equals the oracle's codes and scales byte for byte
    (every head of K and V; every head of Q, or every seventh of the largest),
    and the single-tensor calls give the same bytes."""
    say(f"quant multi full size {w.name}")
    q, k, v = wl.make_prefill_inputs(w)
    qheads = None if w.Hq <= 32 else list(range(0, w.Hq, 7))
    jobs = [(q, w.q_block, w.q_qtype, w.q_scale_dtype, "Q", qheads),
            (k, w.kv_block, w.k_qtype, w.kv_scale_dtype, "K", None),
            (v, w.kv_block, w.v_qtype, w.kv_scale_dtype, "V", None)]
    outs = qfa.block_quant_multi([dict(x=t.cuda(), block_rows=R, qtype=qt, scale_dtype=SDT[sdt])
                                  for t, R, qt, sdt, _, _ in jobs])
    torch.cuda.synchronize()
    for (t, R, qt, sdt, name, heads), (c, s) in zip(jobs, outs):
        if heads is None:
            rc, rs = oracle.block_quant(t, R, qt, sdt, "bnsd")
            assert_codes_equal(c, s, rc, rs, f"multi full size {name}")
        else:
            rc, rs = oracle.block_quant(t[:, heads], R, qt, sdt, "bnsd")
            assert_codes_equal(c[:, heads], s[:, heads], rc, rs, f"multi full size {name}")
        c1, s1 = qfa.block_quant(t.cuda(), R, qt, SDT[sdt])
        torch.cuda.synchronize()
        assert torch.equal(c.view(torch.uint8), c1.view(torch.uint8))
        assert torch.equal(s, s1)
