"""GPU parity of qfa_kv_append against the oracle: the appended cache (codes
and scales) must match byte for byte, for new blocks, rows that fit the
block's scale, rows that force a requantization, positions out of range,
INT8 and packed INT4, both layouts, and several appends in a row."""
import numpy as np
import pytest
import torch

import block_quantized_flashattention_amd as qfa
import oracle
from gpu_util import SDT, say

pytestmark = pytest.mark.gpu


def _cache(B, H, S, D, R, qtype, sdt, layout, seed):
    """A cache filled by the GPU quantizer from random rows (byte-exact with the oracle)."""
    gen = torch.Generator().manual_seed(seed)
    src = torch.randn(B, H, S, D, generator=gen).to(torch.float16)
    if layout == "bsnd":
        src = src.transpose(1, 2).contiguous()
    codes, scales = qfa.block_quant(src.cuda(), R, qtype, SDT[sdt], layout)
    return codes, scales


def _append_and_check(codes, scales, x, pos, R, qtype, layout):
    before_c, before_s = codes.cpu().numpy().copy(), scales.cpu().numpy().copy()
    qfa.kv_append(x.cuda(), torch.tensor(pos, dtype=torch.int32).cuda(), codes, scales, R, qtype,
                  layout)
    torch.cuda.synchronize()
    ref_c, ref_s = oracle.kv_append(before_c, before_s, x, pos, R, qtype,
                                    "f16" if before_s.dtype == np.float16 else "f32", layout)
    gc, gs = codes.cpu().numpy(), scales.cpu().numpy()
    np.testing.assert_array_equal(gs.view(np.uint8), ref_s.view(np.uint8))
    np.testing.assert_array_equal(gc.view(np.uint8), np.asarray(ref_c).view(np.uint8))
    changed = int((gs != before_s).sum())
    say(f"  appended {len(pos)} rows; scales changed in {changed} blocks")


@pytest.mark.parametrize("case", [
    # B, H, S_max, D, R, qtype, scale dtype, layout
    (4, 2, 600, 128, 256, "int8", "f16", "bnsd"),
    (3, 3, 300, 64, 64, "int8", "f32", "bsnd"),
    (4, 2, 600, 128, 256, "int4", "f16", "bnsd"),
    (2, 2, 100, 64, 1, "int4", "f32", "bsnd"),
], ids=lambda c: "_".join(map(str, c)))
def test_kv_append(case):
    B, H, S, D, R, qtype, sdt, layout = case
    say(f"kv append {case}")
    codes, scales = _cache(B, H, S, D, R, qtype, sdt, layout, seed=S + D)
    gen = torch.Generator().manual_seed(7)
    x = torch.randn(B, H, D, generator=gen).to(torch.float16)
    x[1] *= 40.0                      # forces a requantization of its block (unless it starts one)
    # a block start, mid-block rows, the last row, and an out-of-range position
    pos = [R * (1 if S > R else 0), min(S - 1, R + 5), S - 1, -1][:B]
    _append_and_check(codes, scales, x, pos, R, qtype, layout)


def test_kv_append_sequence_of_steps():
    """Decode-style: each step appends one row per sequence after the last."""
    B, H, S, D, R = 3, 4, 700, 128, 256
    codes, scales = _cache(B, H, S, D, R, "int8", "f16", "bnsd", seed=11)
    lens = [250, 255, 600]
    gen = torch.Generator().manual_seed(8)
    for step in range(6):
        x = torch.randn(B, H, D, generator=gen).to(torch.float16) * (1.0 + 3 * (step % 3 == 2))
        _append_and_check(codes, scales, x, [L + step for L in lens], R, "int8", "bnsd")


@pytest.mark.parametrize("qtype,layout", [("int4", "bnsd"), ("int8", "bsnd"), ("int4", "bsnd")])
def test_kv_append_requantizes_nearly_full_blocks(qtype, layout):
    """Rows 251 and 254 of 256-row blocks with a large new row: the whole
    block (hundreds of old rows) is requantized, past one pass of the
    threads' unrolled reads."""
    B, H, S, D, R = 2, 3, 600, 128, 256
    say(f"kv append requantizing nearly full blocks {qtype} {layout}")
    codes, scales = _cache(B, H, S, D, R, qtype, "f16", layout, seed=23)
    gen = torch.Generator().manual_seed(9)
    x = torch.randn(B, H, D, generator=gen).to(torch.float16) * 30.0
    _append_and_check(codes, scales, x, [251, R + 254], R, qtype, layout)


@pytest.mark.parametrize("xdt", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("qtype", ["int8", "int4"])
def test_kv_append_row_dtypes(xdt, qtype):
    """fp32 and bf16 new rows (each element read from the dword that holds
    it), one that fits its block and one that forces a requantization."""
    B, H, S, D, R = 3, 2, 600, 128, 256
    say(f"kv append row dtype {xdt} {qtype}")
    codes, scales = _cache(B, H, S, D, R, qtype, "f16", "bnsd", seed=31)
    gen = torch.Generator().manual_seed(10)
    x = torch.randn(B, H, D, generator=gen)
    x[0] *= 0.25
    x[1] *= 40.0
    _append_and_check(codes, scales, x.to(xdt), [200, R + 100, 599], R, qtype, "bnsd")


@pytest.mark.parametrize("qtype,layout,sdt", [("int8", "bnsd", "f16"), ("int4", "bsnd", "f32"),
                                              ("int4", "bnsd", "f16")])
def test_kv_append_kv_equals_two_appends(qtype, layout, sdt):
    """qfa_kv_append_kv (K and V rows of a decode step in one launch) leaves
    both caches byte-identical to two qfa_kv_append calls, with rows that fit
    their block's scale, rows that force a requantization, a new block and an
    out-of-range position, over three steps; the K cache also matches the
    oracle."""
    B, H, S, D, R = 4, 3, 600, 128, 256
    say(f"kv append K+V {qtype} {layout} {sdt}")
    kc, ks = _cache(B, H, S, D, R, qtype, sdt, layout, seed=31)
    vc, vs = _cache(B, H, S, D, R, qtype, sdt, layout, seed=32)
    kc2, ks2, vc2, vs2 = kc.clone(), ks.clone(), vc.clone(), vs.clone()
    gen = torch.Generator().manual_seed(12)
    pos0 = [R, R + 5, S - 3, -1]
    for step in range(3):
        pos = torch.tensor([p + step if p >= 0 else p for p in pos0], dtype=torch.int32).cuda()
        xk = torch.randn(B, H, D, generator=gen).to(torch.float16)
        xv = torch.randn(B, H, D, generator=gen).to(torch.float16)
        xk[step % B] *= 40.0
        xv[(step + 1) % B] *= 40.0
        before_c, before_s = kc.cpu().numpy().copy(), ks.cpu().numpy().copy()
        qfa.kv_append_kv(xk.cuda(), xv.cuda(), pos, kc, ks, vc, vs, R, qtype, layout)
        qfa.kv_append(xk.cuda(), pos, kc2, ks2, R, qtype, layout)
        qfa.kv_append(xv.cuda(), pos, vc2, vs2, R, qtype, layout)
        torch.cuda.synchronize()
        for a, b, n in ((kc, kc2, "K codes"), (ks, ks2, "K scales"), (vc, vc2, "V codes"),
                        (vs, vs2, "V scales")):
            assert torch.equal(a.cpu().view(torch.uint8) if a.element_size() == 1 else a.cpu(),
                               b.cpu().view(torch.uint8) if b.element_size() == 1 else b.cpu()), \
                f"{n} differ at step {step}"
        ref_c, ref_s = oracle.kv_append(before_c, before_s, xk, pos.cpu().tolist(), R, qtype, sdt,
                                        layout)
        np.testing.assert_array_equal(ks.cpu().numpy().view(np.uint8), ref_s.view(np.uint8))
        np.testing.assert_array_equal(kc.cpu().numpy().view(np.uint8),
                                      np.asarray(ref_c).view(np.uint8))
